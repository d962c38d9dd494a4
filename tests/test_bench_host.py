"""Host logic of bench.py that needs no GPU: the refusal of more than one GPU,
the traffic record written from two counter runs (calibration by the copy
kernel, the digest taken from the measured run), the digest gate that keeps a
record of other kernel sources out of the bench line, and the roofline
arithmetic."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM = "void tern::gemm_ternary_mfma<144, 384, 1, 4, true, 1, false, false, 6>(...)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value); rocprofv3's csv columns that
    the summary reads."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_traffic_record_from_counter_runs(tmp_path):
    # Two dispatches of the GEMM (each counted in two rows that add up), a
    # 1 GiB copy whose FETCH_SIZE reads half the bytes moved (scale 2) and
    # whose WRITE_SIZE reads all of them (scale 1).
    gib = 1 << 30
    fetch_rows = [(1, GEMM, 30000.0), (1, GEMM, 40000.0), (2, GEMM, 70000.0),
                  (3, COPY, gib / 2 / 1024)]
    write_rows = [(1, GEMM, 80000.0), (2, GEMM, 82000.0), (3, COPY, gib / 1024)]
    _counter_csv(str(tmp_path / "f" / "x" / "f_counter_collection.csv"), "FETCH_SIZE", fetch_rows)
    _counter_csv(str(tmp_path / "w" / "w_counter_collection.csv"), "WRITE_SIZE", write_rows)
    line = {"metric": "m", "config": {"m": 4608, "k": 3072, "n": 9216,
                                       "gemm_source_sha256": "abc123",
                                       "copy_calibration_bytes": gib}}
    log = tmp_path / "run.log"
    log.write_text("# a progress line\n" + json.dumps(line) + "\n")
    out = tmp_path / "rec.json"
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(log), "flux_qkv",
                            str(out))
    rec = json.loads(out.read_text())
    assert rec["kernel"] == GEMM and rec["dispatches"] == 2
    assert rec["fetch_size_kib_per_dispatch"] == pytest.approx(70000.0)
    assert rec["write_size_kib_per_dispatch"] == pytest.approx(81000.0)
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == pytest.approx(70000.0 * 1024 * 2)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(81000.0 * 1024)
    assert rec["alg_bytes_per_launch"] == 2 * 4608 * 3072 + 9216 * 3072 // 4 + 4 * 9216 + \
        2 * 4608 * 9216
    assert rec["gemm_source_sha256"] == "abc123"   # the measured run's, never the current one


def test_traffic_record_used_only_for_its_sources(tmp_path, monkeypatch):
    path = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(path))
    assert bench.load_traffic("flux_qkv") is None                 # no record
    path.write_text(json.dumps({"gemm_source_sha256": "0" * 64, "hbm_bytes_per_launch": 5.0}))
    assert bench.load_traffic("flux_qkv") is None                 # other sources
    path.write_text(json.dumps({"gemm_source_sha256": bench.source_digest(),
                                "hbm_bytes_per_launch": 5.0}))
    assert bench.load_traffic("flux_qkv") == 5.0


def test_source_digest_covers_every_gemm_source(tmp_path):
    srcs = []
    for i, text in enumerate([b"a", b"b"]):
        p = tmp_path / f"s{i}"
        p.write_bytes(text)
        srcs.append(str(p))
    d0 = bench.source_digest(srcs)
    (tmp_path / "s1").write_bytes(b"c")
    assert bench.source_digest(srcs) != d0
    assert all(os.path.exists(p) for p in bench.GEMM_SRCS)
    assert any(p.endswith("gemm_small.hip") for p in bench.GEMM_SRCS)


def test_roofline_arithmetic():
    # QKV: above the ridge, bound by the matrix cores
    flops, byts = 2 * 4608 * 3072 * 9216, bench.gemm_alg_bytes(4608, 3072, 9216)
    r = bench.roofline_of(flops, byts, 165e-6)
    assert r["bound"] == "mfma"
    assert r["pct_roofline"] == pytest.approx(100 * flops / (bench.PEAK_BF16_TFLOPS * 1e12)
                                              / 165e-6)
    assert r["tflops"] == pytest.approx(flops / 165e-6 / 1e12)
    # one token on the 16.5 MB weight: below the ridge, bound by HBM
    flops, byts = 2 * 1 * 3072 * 21504, bench.gemm_alg_bytes(1, 3072, 21504)
    r = bench.roofline_of(flops, byts, 8e-6)
    assert r["bound"] == "hbm"
    assert r["pct_roofline"] == pytest.approx(100 * byts / (bench.PEAK_HBM_GBS * 1e9) / 8e-6)
