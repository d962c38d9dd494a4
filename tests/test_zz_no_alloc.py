"""tern_gemm_dx_static, the input gradient for callers that cannot allocate,
against tern_gemm_dx (the entry point with a caller workspace), through the
C-ABI on the GPU.

Both run the same kernels on the same operands, so dx must be bit-identical.
Two calls in a row exercise the library's fixed array being reused: the
second is smaller than the first, on another stream, so a stale tail of the
first call's scaled gradient would show up as a difference.  The result is
also checked against the CPU oracle, and sizes beyond the array are refused.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tern_inputs
from parity import DEV, assert_within_tolerance, bf16_to_f64, draw_grad, log, row_norms

pytestmark = pytest.mark.gpu
tern = pytest.importorskip("ternary_weight_quantized_tern_amd")


def _layer(m, n, k, seed):
    dy = draw_grad(m, n, seed)
    _, w = tern_inputs.draw(1, k, n, seed=seed + 1)
    p, s = tern.quantize_pack(w.to(DEV))
    pt = tern.pack_transposed(p, n, k)
    return dy, w, p, s, pt


def _both(dy_cpu, pt, s, k, stream=None):
    m, n = dy_cpu.shape
    dy = dy_cpu.to(DEV)
    u = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    dx_ws = torch.full((m, k), 7.0, dtype=torch.bfloat16, device=DEV)
    dx_st = torch.full((m, k), -7.0, dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_dx(dy, pt, s, u, dx_ws, k)
    torch.cuda.synchronize()
    tern.tern_gemm_dx_static(dy, pt, s, dx_st, k, stream=stream)
    torch.cuda.synchronize()
    return dx_ws, dx_st


def test_static_matches_workspace_twice_second_smaller():
    # first call: a tiled-kernel size (m > 32), then a smaller few-token one
    # on a side stream; both against the workspace entry point, bit for bit
    big = (300, 1152, 640)
    small = (8, 192, 256)
    side = torch.cuda.Stream()
    for (m, n, k), stream in ((big, None), (small, side)):
        log(f"gemm_dx_static m={m} n={n} k={k}")
        dy, w, p, s, pt = _layer(m, n, k, seed=m * 31 + n)
        dx_ws, dx_st = _both(dy, pt, s, k, stream)
        assert torch.equal(dx_st.view(torch.int16), dx_ws.view(torch.int16)), (m, n, k)
        # and the oracle's bar: dx within 8e-3 |dx_ref| + 1e-3 ||u_m||_2
        t_ref, s_ref = oracle.oracle_quantize(w.numpy())
        u_ref = oracle.oracle_scale_grad(tern_inputs.bf16_bits(dy), s_ref)
        ref = oracle.oracle_gemm_dx(u_ref, oracle.oracle_pack(t_ref), k)
        assert_within_tolerance(bf16_to_f64(dx_st), ref, np.ones(k, np.float32),
                                row_norms(u_ref), f"dx_static m={m} n={n} k={k}")


def test_static_at_a_full_backward_shape_and_the_capacity_bound():
    # the DiT up-projection's backward (m = 2048, n = 4608, k = 1152) fills an
    # eighth of the array; the FLUX single-stream in-projection's backward
    # (m * n = 99M) is beyond it and refused before any launch
    m, n, k = 2048, 4608, 1152
    log(f"gemm_dx_static m={m} n={n} k={k}")
    dy, w, p, s, pt = _layer(m, n, k, seed=77)
    dx_ws, dx_st = _both(dy, pt, s, k)
    assert torch.equal(dx_st.view(torch.int16), dx_ws.view(torch.int16))
    big_m, big_n = 4608, 21504
    assert big_m * big_n > tern.TERN_GEMM_DX_STATIC_MAX_ELEMS
    dy_big = torch.empty((big_m, big_n), dtype=torch.bfloat16, device=DEV)
    pt_big = torch.empty((64, big_n // 4), dtype=torch.uint8, device=DEV)
    s_big = torch.empty(big_n, device=DEV)
    dx_big = torch.empty((big_m, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tern.TernError) as err:
        tern.tern_gemm_dx_static(dy_big, pt_big, s_big, dx_big, 64)
    assert err.value.status == tern.TERN_ERR_SHAPE
