"""The few-token kernel (gemm_ternary_few) copies the X rows of its chunks
into LDS with LDS-DMA buffer loads, then loads the packed weight words of the
same chunks, and waits with one explicit `s_waitcnt vmcnt(CPW * RB)` before
its first LDS read: since vector memory loads complete in issue order, that
wait covers exactly the copies, while the weight words keep streaming in and
are waited for one chunk at a time where they are decoded.  The wait is only
right if the compiler keeps that issue order: every copy first, then at least
CPW * RB loads, then the wait, then the first LDS read, with no wait between
the copies and the weight loads (which would stall the weight stream behind
the copies).  This test compiles gemm_small.hip for gfx950 and checks that
order in every instantiation of the kernel, so that a compiler or source
change that moves the loads past the wait fails here instead of producing
reads of X regions that have not landed.

CPU only: it needs hipcc, not a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

from ternary_weight_quantized_tern_amd import build as B

NAME = re.compile(r"gemm_ternary_fewILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)E")
VMCNT = re.compile(r"^s_waitcnt\b.*\bvmcnt\((\d+)\)")


def _few_kernels(tmp_path):
    out = tmp_path / "gemm_small.s"
    cmd = [B.hipcc()] + B.compile_flags() + ["--cuda-device-only", "-S", "-o", str(out),
                                             os.path.join(B.CSRC, "gemm_small.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    kernels, name, body = [], None, []
    for line in out.read_text().split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None and line.startswith(".Lfunc_end"):
            if NAME.search(name):
                kernels.append((name, body))
            name = None
            continue
        if name is not None:
            t = line.split(";")[0].strip()
            if t and not t.startswith(".") and not t.endswith(":"):
                body.append(t)
    return kernels


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                    reason="hipcc not available")
def test_few_kernel_waits_cover_only_the_x_copies(tmp_path):
    kernels = _few_kernels(tmp_path)
    assert kernels, "no gemm_ternary_few instantiation found"
    for name, insts in kernels:
        rb, _, cpw, _, _, _ = (int(v) for v in NAME.search(name).groups())
        first_read = next(i for i, t in enumerate(insts) if t.startswith("ds_read"))
        copies = [i for i, t in enumerate(insts[:first_read])
                  if t.startswith("buffer_load") and t.endswith(" lds")]
        assert copies, name
        first_copy, last_copy = copies[0], copies[-1]
        wait = next(i for i in range(last_copy + 1, first_read) if VMCNT.match(insts[i]))
        n = int(VMCNT.match(insts[wait]).group(1))
        loads = [i for i in range(last_copy + 1, wait) if insts[i].startswith("buffer_load")]
        # the explicit wait, with every weight load of the round before it
        assert n == cpw * rb, (name, insts[wait])
        assert len(loads) >= n, (name, len(loads), n)
        # nothing waits between the first copy and the last weight load
        waits = [insts[i] for i in range(first_copy, wait) if VMCNT.match(insts[i])]
        assert not waits, (name, waits)
