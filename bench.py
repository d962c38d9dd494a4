#!/usr/bin/env python3
"""Throughput of the 1.58-bit linear layer on one MI355X.

One step is one pass of tern_gemm over every layer of the workload, inputs
already resident in HBM (default workload flux_qkv: bf16 X [4608, 3072] times
the packed ternary weights of a [9216, 3072] layer, fp32 per-channel scales,
bf16 Y [4608, 9216] through the fused scale epilogue).  The reported value is
tern_gemm's effective throughput, 2*M*N*K per step over the step time, in
TFLOP/s.  The weights are converted once before the timed region
(tern_quantize_pack: fp32 weights to codes, scales and packed bytes); the
conversion entry points are timed on their own afterwards and reported in
"kernels" with in_step false.  The roofline object describes tern_gemm,
timed with HIP events on the stream it is launched on; the CPU baseline is the
oracle timed on this host's cores on a bounded sample of the same step.  The
timed steps follow the W warm-up steps and further untimed steps up to
--warmup-ms of warm-up (default 100 ms): the power management lowers the
clock for a few milliseconds after matrix work starts, then settles.

After the timed steps:
  * "config3": the FLUX single-stream block set, 38 seeded (in-projection,
    out-projection) pairs, 76 tern_gemm launches back to back, timed as a
    whole sequence and per launch;
  * "sweep": tern_gemm at M = 1, 8, 16, 32, 64, 128, 256 tokens on the
    16.5 MB packed in-projection weight [21504, 3072], cycling a pool of
    distinct weights larger than every cache (the crossover from the HBM to
    the matrix-core bound); "sweep_reference": in the same setting, an almost
    empty launch and a device copy of each packed weight (per-launch floors);
  * "rows": tern_gemm on every layer shape of the five workloads, and
    tern_gemm_ex with the bias and GELU of the layers that have them;
  * "dx_rows": the input gradient (tern_gemm_dx, tern_pack_transposed) on the
    backward shapes; "dw_rows": the latent-weight gradient (tern_gemm_dw) on
    the same shapes; "a8_rows": the 8-bit-activation layer (tern_quantize_act,
    tern_gemm_a8) on the forward shapes against the int8 matrix peak.
Few-token rows cycle through a pool of distinct packed weights of at least
--pool-mib MiB, so that each launch streams its weights from HBM.  Table rows
are graph-replayed launches; each figure is the median over several replays,
taken after the row's graph has been replayed for --row-warmup-ms (default
100 ms), so that each row, like the timed steps, runs at the settled clock.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flux_qkv]

Counter summaries: python bench.py --summarize-traffic FETCH_DIR WRITE_DIR
BENCH_JSON [--workload W] reads two rocprofv3 --pmc runs of this script (one
with FETCH_SIZE, one with WRITE_SIZE, both with --copy-calibration-mib) and
the JSON line that the FETCH run printed, and writes
profiles/tern_gemm_<W>_traffic.json: the HBM bytes per tern_gemm launch,
scaled by what the counters read for the calibration copy, with the GEMM
source digest recorded by the measured run itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tern_gemm effective TFLOP/s + % of MFMA/HBM roofline, FLUX linears M=4608"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_I8_TOPS = 5000.0       # MI355X dense int8 matrix peak
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
CSRC = os.path.join(ROOT, "ternary_weight_quantized_tern_amd", "csrc")
GEMM_SRCS = [os.path.join(CSRC, f) for f in ("gemm.hip", "gemm_small.hip", "gemm_ksplit.hip", "gemm_common.h")]
W_STD = 0.02


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="after the warm-up steps, keep running untimed steps until the "
                         "warm-up has lasted this long (the clock settles under sustained load)")
    ap.add_argument("--workload", default="flux_qkv")
    ap.add_argument("--layers", type=int, default=0,
                    help="use only the first L layers of a multi-layer workload (0 = all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle's layer-output sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a device copy of this size (for counter calibration)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip every table after the timed steps")
    ap.add_argument("--rows", default="all",
                    help="comma-separated tables to time after the steps: config3, sweep, fwd, "
                         "dx, dw, a8, or all")
    ap.add_argument("--row-reps", type=int, default=30, help="launches per graph of a table row")
    ap.add_argument("--row-filter", default=None,
                    help="time only the forward rows whose name contains this text")
    ap.add_argument("--replays", type=int, default=5, help="timed graph replays per table row")
    ap.add_argument("--row-warmup-ms", type=float, default=100.0,
                    help="untimed replays of each table row's graph before its timed ones")
    ap.add_argument("--pool-mib", type=int, default=1024,
                    help="packed-weight pool cycled by the few-token rows")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="write the traffic record from two counter runs (no GPU used)")
    ap.add_argument("--traffic-out", default=None,
                    help="where --summarize-traffic writes (default: profiles/)")
    return ap.parse_args()


def gemm_alg_bytes(m, k, n):
    return 2 * m * k + n * k // 4 + 4 * n + 2 * m * n


def source_digest(paths=GEMM_SRCS):
    """sha256 over the GEMM kernel sources, in a fixed order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"tern_gemm_{workload}_traffic.json")


def load_traffic(workload):
    """HBM bytes per tern_gemm launch from the committed counter record, if it
    was measured on the current kernel sources (the record's digest is the one
    the measured run printed)."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("gemm_source_sha256") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(layers, inputs, target_s):
    """The oracle, as it stands, on all of this host's cores: the layer output
    for a leading sample of X rows, scaled to all M rows (the step is the
    layer, 2MNK per layer).  The weights are converted by the oracle first
    (not timed into the value: the step does not convert weights either)."""
    import oracle
    import tern_inputs
    cores = len(os.sched_getaffinity(0))
    t_weights = 0.0
    t_gemm = 0.0
    rows_used = []
    flops = 0
    for layer, (x, w) in zip(layers, inputs):
        t0 = time.perf_counter()
        t_ref, s_ref = oracle.oracle_quantize(w.numpy())
        p_ref = oracle.oracle_pack(t_ref)
        t_weights += time.perf_counter() - t0
        xb = tern_inputs.bf16_bits(x)
        pilot = min(8, layer.m)
        t0 = time.perf_counter()
        oracle.oracle_gemm(xb[:pilot], p_ref, s_ref, nthreads=cores)
        dt = time.perf_counter() - t0
        per_row = dt / pilot
        rows = int(max(pilot, min(layer.m, (target_s / len(layers)) / max(per_row, 1e-9))))
        if rows > pilot:
            t0 = time.perf_counter()
            oracle.oracle_gemm(xb[:rows], p_ref, s_ref, nthreads=cores)
            dt = time.perf_counter() - t0
        t_gemm += dt * layer.m / rows
        rows_used.append(rows)
        flops += 2 * layer.m * layer.n * layer.k
    return {
        "value": flops / t_gemm / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_count": os.cpu_count(),
        "affinity_cores": cores,
        "cpu_model": cpu_model(),
        "seconds_per_step_extrapolated": t_gemm,
        "weight_conversion_seconds": t_weights,
        "sample": (f"oracle layer output (fp64, scalar C, {cores} threads = all cores in this "
                   f"process's affinity) on the first {rows_used} X rows of "
                   f"M={[l.m for l in layers]}, scaled to all rows; the oracle's weight "
                   f"conversion ({t_weights:.2f} s) is not in the value"),
    }


def roofline_of(flops, byts, seconds):
    """Effective rates and the fraction of the bound that applies."""
    tf = flops / seconds / 1e12
    gbs = byts / seconds / 1e9
    bound = "mfma" if flops / byts >= RIDGE else "hbm"
    t_ideal = max(flops / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
    return {"tflops": tf, "gbs": gbs, "pct_mfma": 100 * tf / PEAK_BF16_TFLOPS,
            "pct_hbm": 100 * gbs / PEAK_HBM_GBS, "bound": bound,
            "pct_roofline": 100 * t_ideal / seconds}


ROW_WARMUP_S = 0.1  # set from --row-warmup-ms


def time_graph(torch, fn, launches, replays):
    """Seconds per call of fn() with `launches` calls captured in one HIP graph
    and replayed back to back (after one eager warm-up call on a side stream,
    then untimed replays for ROW_WARMUP_S seconds, at least one): the median
    and the minimum over `replays` timed replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(launches):
            fn()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < ROW_WARMUP_S:
        graph.replay()
        torch.cuda.synchronize()
    per = []
    for _ in range(max(1, replays)):
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        per.append(g0.elapsed_time(g1) * 1e-3 / launches)
    del graph
    return statistics.median(per), min(per)


class Cycler:
    """Calls fn(*operands[i]) for i = 0, 1, 2, ... cyclically."""

    def __init__(self, fn, operands):
        self.fn, self.operands, self.i = fn, operands, 0

    def __call__(self):
        self.fn(*self.operands[self.i % len(self.operands)])
        self.i += 1


def weight_pool(tern, torch, dev, n, k, seed, pool_mib):
    """Distinct packed weights [n, k] (seeded N(0, 0.02^2) fp32 weights drawn on
    the GPU and converted by tern_quantize_pack) totalling at least pool_mib
    MiB, as (p, s) pairs."""
    ldp = tern.packed_row_bytes(k)
    per = n * ldp + 4 * n
    count = max(1, -(-(pool_mib << 20) // per))
    gen = torch.Generator(device=dev).manual_seed(int(seed))
    ps = torch.zeros((count, n, ldp), dtype=torch.uint8, device=dev)
    ss = torch.empty((count, n), dtype=torch.float32, device=dev)
    for i in range(count):
        wi = torch.randn((n, k), generator=gen, device=dev) * W_STD
        tern.tern_quantize_pack(wi, None, ps[i], ss[i])
        del wi
    return [(ps[i], ss[i]) for i in range(count)], count * per


def time_rows(tern, tern_inputs, torch, dev, reps, replays, pool_mib, only=None):
    """The layer on every layer shape of the workloads (layer 0 inputs of each
    shape): tern_gemm, and tern_gemm_ex where the layer's consumer applies a
    bias and the tanh-form GELU (the MLP up-projections; the single-stream
    in-projection, whose GELU covers only its MLP columns from 9216 on)."""
    W = tern_inputs.WORKLOADS
    shapes = [("single", W["single"][0], None),
              ("flux_qkv", W["flux_qkv"][0], None),
              ("flux_mlp.up", W["flux_mlp"][0], None),
              ("flux_mlp.up+gelu", W["flux_mlp"][0], (False, 0)),
              ("flux_mlp.down", W["flux_mlp"][1], None),
              ("flux_single_stream.in_proj", W["flux_single_stream"][0], None),
              ("flux_single_stream.in_proj+bias+gelu[9216:]", W["flux_single_stream"][0],
               (True, 9216)),
              ("flux_single_stream.out_proj", W["flux_single_stream"][1], None)]
    for l in W["dit"]:
        shapes.append((l.name, l, None))
        if ".up." in l.name:
            shapes.append((l.name + "+bias+gelu", l, (True, 0)))
    if only:
        shapes = [sh for sh in shapes if only in sh[0]]
    rows = []
    for name, layer, epi in shapes:
        x, w = tern_inputs.draw_layer(layer)
        xd = x.to(dev)
        y = torch.empty((layer.m, layer.n), dtype=torch.bfloat16, device=dev)
        if epi is None:
            def launch(p_i, s_i, xd=xd, y=y, k=layer.k):
                tern.tern_gemm(xd, p_i, s_i, y, k)
        else:
            bias = None
            if epi[0]:
                gb = torch.Generator().manual_seed(layer.seed + 7)
                bias = (torch.randn(layer.n, generator=gb) * 0.02).to(dev)

            def launch(p_i, s_i, xd=xd, y=y, k=layer.k, bias=bias, act_from=epi[1]):
                tern.tern_gemm_ex(xd, p_i, s_i, y, bias, tern.TERN_ACT_GELU_TANH, act_from, k)
        pool = layer.m <= 64 and layer.n * layer.k >= (1 << 20)
        if pool:
            operands, pool_bytes = weight_pool(tern, torch, dev, layer.n, layer.k, layer.seed,
                                               pool_mib)
            launches = len(operands)
        else:
            operands = [tern.quantize_pack(w.to(dev))]
            launches = reps
        torch.cuda.synchronize()
        t, t_min = time_graph(torch, Cycler(launch, operands), launches, replays)
        flops = 2 * layer.m * layer.n * layer.k
        byts = gemm_alg_bytes(layer.m, layer.k, layer.n)
        if epi is not None and epi[0]:
            byts += 4 * layer.n  # the fp32 bias
        row = {"layer": name, "m": layer.m, "k": layer.k, "n": layer.n,
               "launches": launches, "us_per_launch": t * 1e6, "min_us_per_launch": t_min * 1e6,
               "alg_flops": flops, "alg_bytes": byts,
               "entry": "tern_gemm" if epi is None else "tern_gemm_ex"}
        if epi is not None:
            row["epilogue"] = {"bias": bool(epi[0]), "act": "gelu_tanh", "act_from": epi[1]}
        row.update(roofline_of(flops, byts, t))
        if pool:
            row["weight_pool_mib"] = round(pool_bytes / 2**20, 1)
        rows.append(row)
        print(f"# row {name}: {t * 1e6:.1f} us per launch, {row['tflops']:.0f} TFLOP/s, "
              f"{row['gbs']:.0f} GB/s, {row['pct_roofline']:.1f}% of roofline",
              file=sys.stderr, flush=True)
        del operands
        torch.cuda.empty_cache()
    return rows


def time_sweep(tern, torch, dev, replays, pool_mib, ms=(1, 8, 16, 32, 64, 128, 256)):
    """tern_gemm on the FLUX single-stream in-projection weight (N = 21504,
    K = 3072: 16.5 MB packed) from a few tokens to 256, cycling a pool of at
    least pool_mib MiB of distinct weights: the weight-streaming (HBM-bound)
    regime and the crossover to the matrix cores (the arithmetic intensity
    reaches the ridge near M = 45)."""
    n, k = 21504, 3072
    operands, pool_bytes = weight_pool(tern, torch, dev, n, k, 5000, pool_mib)
    rows = []
    for m in ms:
        gen = torch.Generator(device=dev).manual_seed(5100 + m)
        xd = torch.randn((m, k), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

        def launch(p_i, s_i, xd=xd, y=y):
            tern.tern_gemm(xd, p_i, s_i, y, k)

        t, t_min = time_graph(torch, Cycler(launch, operands), len(operands), replays)
        flops = 2 * m * n * k
        byts = gemm_alg_bytes(m, k, n)
        row = {"layer": f"in_proj_weight.m{m}", "m": m, "k": k, "n": n,
               "launches": len(operands), "us_per_launch": t * 1e6,
               "min_us_per_launch": t_min * 1e6, "alg_flops": flops, "alg_bytes": byts,
               "weight_pool_mib": round(pool_bytes / 2**20, 1), "entry": "tern_gemm"}
        row.update(roofline_of(flops, byts, t))
        rows.append(row)
        print(f"# sweep m={m}: {t * 1e6:.2f} us per launch, {row['gbs']:.0f} GB/s "
              f"({row['pct_hbm']:.1f}% of HBM peak), {row['tflops']:.0f} TFLOP/s, "
              f"{row['pct_roofline']:.1f}% of roofline ({row['bound']})", file=sys.stderr,
              flush=True)
    ref = sweep_reference(torch, dev, operands, replays)
    print(f"# sweep reference: an almost empty launch {ref['empty_launch_us']:.2f} us; a device "
          f"copy of the 16.5 MB weight {ref['weight_copy_us']:.2f} us per launch "
          f"({ref['weight_copy_gbs']:.0f} GB/s read + written)", file=sys.stderr, flush=True)
    del operands
    torch.cuda.empty_cache()
    return rows, ref


def sweep_reference(torch, dev, operands, replays):
    """Per-launch floors in the sweep's setting (graph replays over the same
    pool of packed weights): an almost empty launch (a one-element add) and a
    device copy of each packed weight into one buffer (torch's copy kernel,
    the weight's bytes read and written once)."""
    tiny = torch.zeros(1, device=dev)
    t_empty, _ = time_graph(torch, lambda: tiny.add_(1), len(operands), replays)
    dst = torch.empty_like(operands[0][0])

    def copy(p_i, s_i):
        dst.copy_(p_i)

    t_copy, _ = time_graph(torch, Cycler(copy, operands), len(operands), replays)
    byts = operands[0][0].numel()
    return {"empty_launch_us": t_empty * 1e6, "weight_copy_us": t_copy * 1e6,
            "weight_bytes": byts, "weight_copy_gbs": 2 * byts / t_copy / 1e9}


def time_config3(tern, tern_inputs, torch, dev, replays):
    """The 38 single-stream blocks of a FLUX-style transformer, each an
    in-projection (4608 x 3072 -> 21504) and an out-projection (4608 x 15360 ->
    3072) with fresh seeded inputs (seeds 3000 + 2l and 3000 + 2l + 1; X ~ N(0,
    1) in bf16 and W ~ N(0, 0.02^2) drawn on the GPU, W converted by
    tern_quantize_pack): the 76 tern_gemm launches back to back on one stream,
    timed as a whole (median of `replays` sequences between two events) and
    per launch (events around each launch of one more sequence)."""
    layers = list(tern_inputs.iter_layers("flux_single_stream"))
    bufs = []
    for layer in layers:
        gen = torch.Generator(device=dev).manual_seed(layer.seed)
        x = torch.randn((layer.m, layer.k), generator=gen, device=dev).to(torch.bfloat16)
        w = torch.randn((layer.n, layer.k), generator=gen, device=dev) * W_STD
        p, s = tern.quantize_pack(w)
        del w
        y = torch.empty((layer.m, layer.n), dtype=torch.bfloat16, device=dev)
        bufs.append((x, p, s, y, layer.k))
    torch.cuda.synchronize()

    def sequence():
        for x, p, s, y, k in bufs:
            tern.tern_gemm(x, p, s, y, k)

    sequence()
    torch.cuda.synchronize()
    per_seq = []
    for _ in range(max(1, replays)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sequence()
        e1.record()
        torch.cuda.synchronize()
        per_seq.append(e0.elapsed_time(e1) * 1e-3)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(bufs) + 1)]
    ev[0].record()
    for i, (x, p, s, y, k) in enumerate(bufs):
        tern.tern_gemm(x, p, s, y, k)
        ev[i + 1].record()
    torch.cuda.synchronize()
    launch_s = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(len(bufs))]
    t = statistics.median(per_seq)
    flops = sum(2 * l.m * l.n * l.k for l in layers)
    in_s = launch_s[0::2]
    out_s = launch_s[1::2]
    lin, lout = layers[0], layers[1]
    f_in, f_out = 2 * lin.m * lin.n * lin.k, 2 * lout.m * lout.n * lout.k
    out = {"layers": len(layers), "launches": len(bufs), "sequence_ms": t * 1e3,
           "sequence_min_ms": min(per_seq) * 1e3, "tflops": flops / t / 1e12,
           "pct_mfma": 100 * flops / t / 1e12 / PEAK_BF16_TFLOPS,
           "in_proj": {"m": lin.m, "k": lin.k, "n": lin.n,
                       "avg_us": 1e6 * sum(in_s) / len(in_s), "min_us": 1e6 * min(in_s),
                       "max_us": 1e6 * max(in_s),
                       "tflops": f_in / (sum(in_s) / len(in_s)) / 1e12},
           "out_proj": {"m": lout.m, "k": lout.k, "n": lout.n,
                        "avg_us": 1e6 * sum(out_s) / len(out_s), "min_us": 1e6 * min(out_s),
                        "max_us": 1e6 * max(out_s),
                        "tflops": f_out / (sum(out_s) / len(out_s)) / 1e12},
           "alg_flops": flops}
    print(f"# config3: 76 launches in {t * 1e3:.2f} ms, {out['tflops']:.0f} TFLOP/s "
          f"({out['pct_mfma']:.1f}% of the bf16 peak)", file=sys.stderr, flush=True)
    del bufs
    torch.cuda.empty_cache()
    return out


def time_dx_rows(tern, tern_inputs, torch, dev, reps, replays):
    """The input gradient of the layer, dX = bf16((dY * s) . T), on the backward
    shapes of the DiT and FLUX layers (dY [m, n] of the forward's output, dX
    [m, k]): tern_gemm_dx (the scaling pass and the ternary GEMM over n), and
    tern_pack_transposed of the layer's codes.  Seeded normal weights quantized
    on the GPU, dY ~ N(0, 1) in bf16; graph-replayed launches."""
    names = ["dit.up.m2048", "dit.down.m2048", "flux_qkv", "flux_mlp.up", "flux_mlp.down"]
    layers = {l.name: l for wl in tern_inputs.WORKLOADS.values() for l in wl}
    rows = []
    for name in names:
        layer = layers[name]
        m, k, n = layer.m, layer.k, layer.n
        _, w = tern_inputs.draw_layer(layer)
        p, s = tern.quantize_pack(w.to(dev))
        pt = torch.zeros((k, tern.packed_row_bytes(n)), dtype=torch.uint8, device=dev)
        g = torch.Generator(device=dev).manual_seed(layer.seed + 500)
        dy = torch.randn((m, n), generator=g, device=dev).to(torch.bfloat16)
        u = torch.empty_like(dy)
        dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
        tern.tern_pack_transposed(p, pt, n, k)
        t_pt, _ = time_graph(torch, lambda: tern.tern_pack_transposed(p, pt, n, k), reps, replays)
        t_dx, _ = time_graph(torch, lambda: tern.tern_gemm_dx(dy, pt, s, u, dx, k), reps, replays)
        flops = 2 * m * n * k
        # algorithmic bytes: dY, the codes, the scales and dX (the bf16 workspace
        # u, written once and read once, is the implementation's own traffic)
        byts = 2 * m * n + n * k // 4 + 4 * n + 2 * m * k
        row = {"layer": name + ".dx", "m": m, "n": n, "k": k, "us_per_launch": t_dx * 1e6,
               "alg_flops": flops, "alg_bytes": byts, "workspace_bytes": 4 * m * n,
               "entry": "tern_gemm_dx",
               "pack_transposed_us": t_pt * 1e6,
               "pack_transposed_gbs": 2 * (n * k // 4) / t_pt / 1e9}
        row.update(roofline_of(flops, byts, t_dx))
        rows.append(row)
        print(f"# dx row {name}: {t_dx * 1e6:.1f} us per launch, {row['tflops']:.0f} TFLOP/s, "
              f"{row['pct_roofline']:.1f}% of roofline; pack_transposed {t_pt * 1e6:.1f} us",
              file=sys.stderr, flush=True)
        del p, s, pt, dy, u, dx
        torch.cuda.empty_cache()
    return rows


def time_dw_rows(tern, tern_inputs, torch, dev, reps, replays):
    """The latent-weight gradient dW = dY^T . X (fp32 [n, k], straight-through
    reading) on the backward shapes of the DiT and FLUX layers: X [m, k] the
    forward layer's input (seeded as the forward), dY ~ N(0, 1) [m, n] in
    bf16; graph-replayed tern_gemm_dw launches."""
    names = ["dit.up.m2048", "dit.down.m2048", "flux_qkv", "flux_mlp.up", "flux_mlp.down",
             "single_stream0.in_proj", "single_stream0.out_proj"]
    layers = {l.name: l for wl in tern_inputs.WORKLOADS.values() for l in wl}
    rows = []
    for name in names:
        layer = layers[name]
        m, k, n = layer.m, layer.k, layer.n
        g = torch.Generator(device=dev).manual_seed(layer.seed + 900)
        x = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
        dy = torch.randn((m, n), generator=g, device=dev).to(torch.bfloat16)
        dw = torch.empty((n, k), dtype=torch.float32, device=dev)
        t, t_min = time_graph(torch, lambda: tern.tern_gemm_dw(dy, x, dw), reps, replays)
        flops = 2 * m * n * k
        byts = 2 * m * n + 2 * m * k + 4 * n * k
        row = {"layer": name + ".dw", "m": m, "n": n, "k": k, "us_per_launch": t * 1e6,
               "min_us_per_launch": t_min * 1e6, "alg_flops": flops, "alg_bytes": byts,
               "entry": "tern_gemm_dw"}
        row.update(roofline_of(flops, byts, t))
        rows.append(row)
        print(f"# dw row {name}: {t * 1e6:.1f} us per launch, {row['tflops']:.0f} TFLOP/s, "
              f"{row['pct_roofline']:.1f}% of roofline", file=sys.stderr, flush=True)
        del x, dy, dw
        torch.cuda.empty_cache()
    return rows


def time_a8_rows(tern, tern_inputs, torch, dev, reps, replays, pool_mib):
    """The 8-bit-activation layer on the forward shapes: tern_quantize_act
    (bf16 X -> int8 codes and per-token scales) and tern_gemm_a8, each
    graph-replayed, and the two together as the layer.  Rates against the
    int8 peak (5.0 POP/s) and the bf16 peak (the unquantized layer's bound).
    The few-token shapes cycle through at least pool_mib MiB of copies of the
    arranged weights, one launch per copy, so that every launch streams its
    weights from HBM; their rate is also given in GB/s."""
    W = tern_inputs.WORKLOADS
    shapes = [("flux_qkv", W["flux_qkv"][0], None),
              ("flux_mlp.up", W["flux_mlp"][0], None),
              ("flux_mlp.up+gelu", W["flux_mlp"][0], (False, 0)),
              ("flux_mlp.down", W["flux_mlp"][1], None),
              ("flux_single_stream.in_proj", W["flux_single_stream"][0], None),
              ("flux_single_stream.out_proj", W["flux_single_stream"][1], None),
              ("dit.up.m2048", W["dit"][0], None), ("dit.down.m2048", W["dit"][1], None),
              ("dit.up.m8", W["dit"][2], None), ("dit.down.m8", W["dit"][3], None)]
    rows = []
    for name, layer, epi in shapes:
        m, k, n = layer.m, layer.k, layer.n
        x, w = tern_inputs.draw_layer(layer)
        xd = x.to(dev)
        p, s = tern.quantize_pack(w.to(dev))
        p8 = tern.pack_a8(p, k)
        q, xs = tern.quantize_act(xd)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        act = tern.TERN_ACT_NONE if epi is None else tern.TERN_ACT_GELU_TANH
        af = 0 if epi is None else epi[1]

        pool = m <= 64
        p8s = [p8]
        if pool:
            count = max(1, -(-(pool_mib << 20) // (p8.numel() + 4 * n)))
            p8s = [p8.clone() for _ in range(count)]

        def gemm(p8_i):
            tern.tern_gemm_a8(q, xs, p8_i, s, y, None, act, af, k)

        def quant():
            tern.tern_quantize_act(xd, q, xs)

        def layer_fn(p8_i):
            quant()
            gemm(p8_i)

        launches = len(p8s) if pool else reps
        operands = [(t,) for t in p8s]
        t_g, _ = time_graph(torch, Cycler(gemm, operands), launches, replays)
        t_q, _ = time_graph(torch, quant, reps, replays)
        t_l, _ = time_graph(torch, Cycler(layer_fn, operands), launches, replays)
        flops = 2 * m * n * k
        byts = m * k + n * k // 4 + 4 * n + 4 * m + 2 * m * n
        q_bytes = 2 * m * k + m * k + 4 * m
        row = {"layer": name, "m": m, "k": k, "n": n, "entry": "tern_gemm_a8",
               "us_per_launch": t_g * 1e6, "tops": flops / t_g / 1e12,
               "pct_i8_peak": 100 * flops / t_g / 1e12 / PEAK_I8_TOPS,
               "pct_bf16_peak": 100 * flops / t_g / 1e12 / PEAK_BF16_TFLOPS,
               "gbs": byts / t_g / 1e9, "alg_flops": flops, "alg_bytes": byts,
               "quantize_act_us": t_q * 1e6, "quantize_act_gbs": q_bytes / t_q / 1e9,
               "layer_us": t_l * 1e6, "layer_tops": flops / t_l / 1e12}
        if epi is not None:
            row["epilogue"] = {"bias": False, "act": "gelu_tanh", "act_from": af}
        if pool:
            row["weight_pool_mib"] = round(len(p8s) * (p8.numel() + 4 * n) / 2**20, 1)
        rows.append(row)
        print(f"# a8 row {name}: gemm {t_g * 1e6:.1f} us {row['tops']:.0f} TOP/s "
              f"({row['pct_i8_peak']:.1f}% of int8 peak); quantize_act {t_q * 1e6:.1f} us "
              f"{row['quantize_act_gbs']:.0f} GB/s; layer {t_l * 1e6:.1f} us",
              file=sys.stderr, flush=True)
        del p, p8, p8s, q, xs, y, xd, operands
        torch.cuda.empty_cache()
    return rows


def time_conversion(tern, torch, layer, b, reps=10, replays=5):
    """The weight-conversion entry points on the first layer's buffers, each
    `reps` launches captured in a HIP graph and replayed (the median over
    `replays`), so that neither the host's launch latency nor a kernel's first
    launch in the process is on the GPU's clock.  Not part of the step."""
    out = {}
    w16 = b["w"].to(torch.bfloat16)
    n, k = layer.n, layer.k
    kb = (k + 3) // 4
    calls = [
        ("tern_quantize_pack", lambda: tern.tern_quantize_pack(b["w"], b["t"], b["p"], b["s"]),
         4 * n * k + n * k + n * kb + 4 * n),
        ("tern_quantize_pack.bf16_w", lambda: tern.tern_quantize_pack(w16, b["t"], b["p"], b["s"]),
         2 * n * k + n * k + n * kb + 4 * n),
        ("tern_quantize", lambda: tern.tern_quantize(b["w"], b["t"], b["s"]),
         4 * n * k + n * k + 4 * n),
        ("tern_pack", lambda: tern.tern_pack(b["t"], b["p"], k), n * k + n * kb),
        ("tern_unpack", lambda: tern.tern_unpack(b["p"], b["tu"], k), n * kb + n * k),
    ]
    for name, fn, byts in calls:
        t, _ = time_graph(torch, fn, reps, replays)
        ms = t * 1e3
        out[name] = {"avg_ms": ms, "alg_bytes": byts, "gbs": byts / (ms * 1e-3) / 1e9,
                     "in_step": False}
    del w16
    return out


def summarize_traffic(fetch_dir, write_dir, bench_json, workload, path=None):
    """Traffic record from two rocprofv3 --pmc runs of bench.py (FETCH_SIZE,
    then WRITE_SIZE, each ending with a --copy-calibration-mib copy)."""

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        by_dispatch = {}
        for path in files:
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") != counter:
                        continue
                    key = (path, r["Dispatch_Id"])
                    name = r["Kernel_Name"]
                    v = float(r["Counter_Value"])
                    if key in by_dispatch:
                        by_dispatch[key] = (name, by_dispatch[key][1] + v)
                    else:
                        by_dispatch[key] = (name, v)
        out = {}
        for name, v in by_dispatch.values():
            out.setdefault(name, []).append(v)
        return out

    with open(bench_json) as f:
        rec = [json.loads(line) for line in f if line.startswith("{")][-1]
    calib_bytes = rec["config"]["copy_calibration_bytes"]
    digest = rec["config"]["gemm_source_sha256"]
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def copy_kernel(d):
        cands = [(max(v), k) for k, v in d.items() if "copy" in k.lower()]
        return max(cands)[1]

    fk, wk = copy_kernel(fetch), copy_kernel(write)
    f_scale = calib_bytes / (max(fetch[fk]) * 1024.0)
    w_scale = calib_bytes / (max(write[wk]) * 1024.0)
    gemm = [k for k in fetch if "gemm_ternary" in k]
    if not gemm:
        raise SystemExit("no tern_gemm kernel in the counter runs")
    gk = max(gemm, key=lambda k: len(fetch[k]))
    f_kib = statistics.mean(fetch[gk])
    w_kib = statistics.mean(write[gk]) if gk in write else 0.0
    read_b = f_kib * 1024.0 * f_scale
    written_b = w_kib * 1024.0 * w_scale
    layer = rec["config"]
    alg = gemm_alg_bytes(layer["m"], layer["k"], layer["n"])
    out = {"workload": workload, "kernel": gk, "dispatches": len(fetch[gk]),
           "fetch_size_kib_per_dispatch": f_kib, "write_size_kib_per_dispatch": w_kib,
           "calibration": {"copy_bytes": calib_bytes, "fetch_kernel": fk, "write_kernel": wk,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": written_b,
           "hbm_bytes_per_launch": read_b + written_b, "alg_bytes_per_launch": alg,
           "gemm_source_sha256": digest,
           "measured_run": {"fetch_dir": fetch_dir, "write_dir": write_dir,
                            "bench_json": bench_json}}
    path = path or traffic_path(workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def main():
    global ROW_WARMUP_S
    args = parse()
    ROW_WARMUP_S = args.row_warmup_ms * 1e-3
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.workload, args.traffic_out)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the ternary linear layer is measured on one MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import tern_inputs
    import ternary_weight_quantized_tern_amd as tern

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tables = {"config3", "sweep", "fwd", "dx", "dw", "a8"} if args.rows == "all" else \
        set(args.rows.split(","))
    if args.no_rows:
        tables = set()

    layers = list(tern_inputs.iter_layers(args.workload))
    if args.layers:
        layers = layers[: args.layers]
    print(f"# workload {args.workload}: {len(layers)} layer(s), drawing inputs", file=sys.stderr,
          flush=True)
    host_inputs = [tern_inputs.draw_layer(layer) for layer in layers]

    bufs = []
    for layer, (x, w) in zip(layers, host_inputs):
        ldp = tern.packed_row_bytes(layer.k)
        b = dict(
            x=x.to(dev), w=w.to(dev),
            t=torch.empty((layer.n, layer.k), dtype=torch.int8, device=dev),
            s=torch.empty((layer.n,), dtype=torch.float32, device=dev),
            p=torch.zeros((layer.n, ldp), dtype=torch.uint8, device=dev),
            tu=torch.empty((layer.n, layer.k), dtype=torch.int8, device=dev),
            y=torch.empty((layer.m, layer.n), dtype=torch.bfloat16, device=dev),
        )
        # weight conversion, once, before the timed region
        tern.tern_quantize_pack(b["w"], b["t"], b["p"], b["s"])
        bufs.append(b)
    torch.cuda.synchronize()

    def step():
        for layer, b in zip(layers, bufs):
            tern.tern_gemm(b["x"], b["p"], b["s"], b["y"], layer.k)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Sustained-load warm-up: the chip's power management lowers the clock for
    # a few milliseconds after a burst of matrix work begins, then settles;
    # untimed steps continue until the warm-up has run --warmup-ms, so that the
    # timed steps see the settled clock of continuous operation.
    warm_steps = args.warmup
    t_warm = time.perf_counter()
    while (time.perf_counter() - t_warm) * 1e3 < args.warmup_ms:
        for _ in range(max(1, args.warmup)):
            step()
            warm_steps += 1
        torch.cuda.synchronize()

    # The timed region: K steps back to back between two events recorded on
    # the launch stream (torch's current stream, the one the binding passes to
    # the library); nothing else is queued in between, so the average launch
    # duration is the region's time over the launches.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    gemm_ms = ms_per_step / len(layers)

    flops_step = sum(2 * l.m * l.n * l.k for l in layers)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # Dominant (and only) kernel of the step: tern_gemm.  Algorithmic work per
    # launch, averaged over the workload's layers.
    gemm_flops = flops_step / len(layers)
    gemm_bytes = sum(gemm_alg_bytes(l.m, l.k, l.n) for l in layers) / len(layers)
    if gemm_flops / gemm_bytes >= RIDGE:
        achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    roof["traffic"] = load_traffic(args.workload)
    roof["kernel"] = "tern_gemm"
    roof["avg_launch_ms"] = gemm_ms
    roof["alg_flops_per_launch"] = gemm_flops
    roof["alg_bytes_per_launch"] = gemm_bytes
    roof["gbs"] = gemm_bytes / (gemm_ms * 1e-3) / 1e9

    kernels = {"tern_gemm": {"avg_ms": gemm_ms, "in_step": True, "alg_bytes": gemm_bytes,
                             "gbs": roof["gbs"],
                             "tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12}}
    kernels.update(time_conversion(tern, torch, layers[0], bufs[0]))

    calib_bytes = 0
    if args.copy_calibration_mib:
        calib_bytes = args.copy_calibration_mib << 20
        src = torch.empty(calib_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"# copy calibration: {calib_bytes} bytes read and written", file=sys.stderr)
    del bufs
    torch.cuda.empty_cache()

    out_tables = {}
    if "config3" in tables:
        print("# timing the 38 single-stream blocks back to back", file=sys.stderr, flush=True)
        out_tables["config3"] = time_config3(tern, tern_inputs, torch, dev, args.replays)
    if "sweep" in tables:
        print("# timing the few-token sweep on the 16.5 MB weight", file=sys.stderr, flush=True)
        out_tables["sweep"], out_tables["sweep_reference"] = time_sweep(
            tern, torch, dev, args.replays, args.pool_mib)
    if "fwd" in tables:
        print("# timing tern_gemm on every layer shape", file=sys.stderr, flush=True)
        out_tables["rows"] = time_rows(tern, tern_inputs, torch, dev, args.row_reps,
                                       args.replays, args.pool_mib, args.row_filter)
    if "dx" in tables:
        print("# timing the input gradient on the backward shapes", file=sys.stderr, flush=True)
        out_tables["dx_rows"] = time_dx_rows(tern, tern_inputs, torch, dev, args.row_reps,
                                             args.replays)
    if "dw" in tables:
        print("# timing the latent-weight gradient on the backward shapes", file=sys.stderr,
              flush=True)
        out_tables["dw_rows"] = time_dw_rows(tern, tern_inputs, torch, dev, args.row_reps,
                                             args.replays)
    if "a8" in tables:
        print("# timing the 8-bit-activation layer on the forward shapes", file=sys.stderr,
              flush=True)
        out_tables["a8_rows"] = time_a8_rows(tern, tern_inputs, torch, dev, args.row_reps,
                                             args.replays, args.pool_mib)

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(layers, host_inputs, args.cpu_seconds)

    shape = layers[0]
    config = {"workload": args.workload, "layers": len(layers), "m": shape.m, "k": shape.k,
              "n": shape.n, "step": "tern_gemm on every layer of the workload",
              "x": f"bf16 {shape.x_dist}", "w": "fp32 N(0, 0.02^2), converted before timing",
              "seed": shape.seed, "warmup_steps_run": warm_steps,
              "warmup_ms_min": args.warmup_ms, "row_warmup_ms": args.row_warmup_ms,
              "gemm_source_sha256": source_digest(),
              "copy_calibration_bytes": calib_bytes}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "peaks": {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                  "i8_mfma_tops": PEAK_I8_TOPS},
    }
    out.update(out_tables)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
