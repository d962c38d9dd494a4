"""The MFMAs of the tiled GEMM kernels are inline asm, so the compiler does not
pad them for hazards.  gfx950 requires two wait states between a VALU
instruction that writes a VGPR and an MFMA that reads it as its A or B
operand, and up to 19 between an MFMA and an instruction that reads its result
other than as the accumulator of the next MFMA.  The wide schedules keep
every decoded operand far from its MFMA and emit no padding, and the kernels
read their accumulators only after an explicit padding block; but the
compiler, which does not see the MFMA inside the asm, may move an
accumulator between registers right after one (it did so at the join of a
conditional block).  This test compiles the GEMM sources for gfx950 and checks
every MFMA of every kernel against the instructions that can precede it, and
every read of an accumulator register against the MFMAs before it
(fall-through and branches), so that a schedule or compiler change that breaks
either rule fails here instead of producing wrong numbers on the GPU.

CPU only: it needs hipcc, not a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

from ternary_weight_quantized_tern_amd import build as B

WAIT_STATES = 2
RESULT_WAIT_STATES = 19
SOURCES = ["gemm.hip", "gemm_small.hip", "gemm_ksplit.hip", "dw.hip"]


def _asm(src: str, tmp_path) -> str:
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.hipcc()] + B.compile_flags() + ["--cuda-device-only", "-S", "-o", str(out),
                                             os.path.join(B.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def _kernels(text: str):
    """(name, [line, ...]) for every function body in the assembly."""
    out, name, body = [], None, []
    for line in text.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None and line.startswith(".Lfunc_end"):
            out.append((name, body))
            name = None
            continue
        if name is not None:
            body.append(line)
    return out


def _vgprs(tok: str):
    tok = tok.strip()
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _parse(body):
    """Instructions and labels in order: ('label', name) or ('inst', text)."""
    items = []
    for line in body:
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            if re.match(r"^\.LBB\w+:", t):
                items.append(("label", t[:-1]))
            continue
        if t.endswith(":"):
            items.append(("label", t[:-1]))
            continue
        items.append(("inst", t))
    return items


def _hazards(items):
    """MFMAs with a VALU write of an A/B source fewer than WAIT_STATES before."""
    branches = {}  # label -> indices of branch instructions that target it
    for i, (kind, t) in enumerate(items):
        if kind == "inst" and t.startswith("s_cbranch") or kind == "inst" and t.startswith("s_branch"):
            branches.setdefault(t.split()[-1], []).append(i)
    found = []

    def walk(idx, ws, srcs, seen):
        # Walk backwards from items[idx] (exclusive) with `ws` wait states used.
        j = idx - 1
        while j >= 0 and ws < WAIT_STATES:
            kind, t = items[j]
            if kind == "label":
                for b in branches.get(t, []):
                    if (b, ws) not in seen:
                        seen.add((b, ws))
                        # the branch instruction itself is one wait state
                        walk(b, ws + 1, srcs, seen)
                j -= 1
                continue
            op = t.split()[0]
            if op == "s_nop":
                ws += int(t.split()[1], 0) + 1
                j -= 1
                continue
            if op in ("s_branch",) or op.startswith("s_endpgm"):
                return  # not a fall-through predecessor
            if op.startswith("v_") and not op.startswith(("v_mfma", "v_readfirstlane", "v_readlane",
                                                          "v_cmp")):
                dst = t.split(None, 1)[1].split(",")[0]
                if _vgprs(dst) & srcs:
                    found.append(t)
            ws += 1
            j -= 1

    count = 0
    for i, (kind, t) in enumerate(items):
        if kind != "inst" or not t.startswith("v_mfma"):
            continue
        count += 1
        ops = t.split(None, 1)[1].split(",")
        walk(i, 0, _vgprs(ops[1]) | _vgprs(ops[2]), set())
    return count, found


def _agprs(tok: str):
    tok = tok.strip()
    m = re.match(r"a\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _result_hazards(items):
    """Instructions other than MFMAs that read an accumulator register (AGPR)
    written by an MFMA fewer than RESULT_WAIT_STATES wait states before."""
    branches = {}
    for i, (kind, t) in enumerate(items):
        if kind == "inst" and (t.startswith("s_cbranch") or t.startswith("s_branch")):
            branches.setdefault(t.split()[-1], []).append(i)
    found = []

    def walk(idx, ws, srcs, seen, reader):
        j = idx - 1
        while j >= 0 and ws < RESULT_WAIT_STATES:
            kind, t = items[j]
            if kind == "label":
                for b in branches.get(t, []):
                    if (b, ws) not in seen:
                        seen.add((b, ws))
                        walk(b, ws + 1, srcs, seen, reader)
                j -= 1
                continue
            op = t.split()[0]
            if op == "s_nop":
                ws += int(t.split()[1], 0) + 1
                j -= 1
                continue
            if op in ("s_branch",) or op.startswith("s_endpgm"):
                return
            if op.startswith("v_mfma"):
                dst = t.split(None, 1)[1].split(",")[0]
                if _agprs(dst) & srcs:
                    found.append(reader)
                    return
            ws += 1
            j -= 1

    for i, (kind, t) in enumerate(items):
        if kind != "inst" or t.startswith("v_mfma") or not t.startswith("v_"):
            continue
        parts = t.split(None, 1)
        if len(parts) < 2:
            continue
        srcs = set()
        for tok in parts[1].split(",")[1:]:
            srcs |= _agprs(tok)
        if srcs:
            walk(i, 0, srcs, set(), t)
    return found


def _gemm_kernels(src, tmp_path):
    return [(n, b) for n, b in _kernels(_asm(src, tmp_path))
            if "gemm_ternary" in n or "gemm_dw" in n]


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_mfma_result_read_too_early(src, tmp_path):
    kernels = _gemm_kernels(src, tmp_path)
    assert kernels, "no GEMM kernels found in the assembly"
    for name, body in kernels:
        found = _result_hazards(_parse(body))
        assert not found, f"{name}: an MFMA result is read too early: {found[:3]}"


def test_result_checker_sees_a_planted_hazard():
    body = [
        "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]",
        "v_accvgpr_mov_b32 a12, a4",
    ]
    assert _result_hazards(_parse(body))
    padded = [body[0], "s_nop 7", "s_nop 7", "s_nop 7", body[1]]
    assert not _result_hazards(_parse(padded))
    chained = [body[0], "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]"]
    assert not _result_hazards(_parse(chained))


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_to_mfma_hazard(src, tmp_path):
    kernels = _gemm_kernels(src, tmp_path)
    assert kernels, "no GEMM kernels found in the assembly"
    total = 0
    for name, body in kernels:
        count, found = _hazards(_parse(body))
        total += count
        assert not found, f"{name}: VALU writes an MFMA source too close: {found[:3]}"
    assert total > 0


def test_checker_sees_a_planted_hazard():
    # The checker itself: a VALU write one instruction before an MFMA that
    # reads it is flagged, through a branch too; with s_nop 1 it is not.
    body = [
        "v_and_b32_e32 v5, 0xc000c000, v5",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
    ]
    assert _hazards(_parse(body))[1]
    padded = [body[0], "s_nop 1", body[1]]
    assert not _hazards(_parse(padded))[1]
    via_branch = [
        "v_perm_b32 v9, v1, v2, v3",
        "s_cbranch_scc1 .LBB0_2",
        "s_endpgm",
        ".LBB0_2:",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
    ]
    assert _hazards(_parse(via_branch))[1]
