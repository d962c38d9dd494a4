"""GPU parity of the latent-weight gradient tern_gemm_dw against the CPU
oracle, through the C-ABI, on seeded inputs.

Bar (fp32 accumulation of exact bf16 products): every product passes through
at most 32 + ceil(m / 32) roundings in the kernel (32 within one MFMA, one per
32-token stage after it), so |dw - dw_ref| <= 2 (32 + ceil(m/32)) 2^-24
sum_m |dy[m][n] x[m][k]|, twice the first-order bound of any such summation;
dw_ref is the oracle's unrounded double result.  Small and ragged shapes are
compared on every element; the backward shapes of the DiT and FLUX layers on
sampled output channels (every column) and on the tile edges.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tern_inputs
from parity import DEV, log

pytestmark = pytest.mark.gpu
tern = pytest.importorskip("ternary_weight_quantized_tern_amd")


def draw(m, n, k, seed, x_dist="normal"):
    """dY ~ N(0, 1) [m, n] and X [m, k] (normal or Student-t), bf16, seeded."""
    g = torch.Generator().manual_seed(int(seed))
    dy = torch.randn(m, n, generator=g).to(torch.bfloat16)
    x, _ = tern_inputs.draw(m, k, 1, seed + 1, x_dist)
    return dy, x


def dev(t: torch.Tensor) -> torch.Tensor:
    """A GPU copy of a bf16 [rows, cols] matrix whose rows start 16-byte aligned
    (row pitch rounded up to 8 elements), as a view of its first cols columns."""
    rows, cols = t.shape
    buf = torch.zeros((rows, (cols + 7) // 8 * 8 if cols else 8), dtype=t.dtype, device=DEV)
    buf[:, :cols] = t.to(DEV)
    return buf[:, :cols]


def bound(dyb, xb, m):
    dyv = np.abs((dyb.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    xv = np.abs((xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    return 2.0 * (32 + -(-m // 32)) * 2.0 ** -24 * (dyv.T @ xv)


def check(dw_gpu, dy_cpu, x_cpu, what, rows=None, init=None):
    """dw_gpu [n, k] (host float) against the oracle on the given rows (all if None)."""
    dyb = tern_inputs.bf16_bits(dy_cpu)
    xb = tern_inputs.bf16_bits(x_cpu)
    m = dyb.shape[0]
    sel = np.arange(dyb.shape[1]) if rows is None else np.asarray(rows)
    ref = oracle.oracle_gemm_dw(np.ascontiguousarray(dyb[:, sel]), xb)
    if init is not None:
        ref = ref + init[sel].astype(np.float64)
    tol = bound(np.ascontiguousarray(dyb[:, sel]), xb, m)
    got = dw_gpu[sel].astype(np.float64)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside the bound, worst "
                           f"{float((err - tol).max()):.3e}")
    return float(err.max())


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (33, 130, 200), (100, 300, 257),
                                   (64, 128, 128), (257, 129, 1000), (31, 1, 5), (7, 513, 3),
                                   (2048, 256, 128),
                                   # 256 x 256 tiles (at least 256 of them), ragged k and n
                                   (64, 4100, 4224), (40, 4096, 4096)])
def test_gemm_dw_all_elements(m, n, k):
    log(f"gemm_dw m={m} n={n} k={k}")
    dy, x = draw(m, n, k, seed=m * 31 + n * 7 + k, x_dist="student_t3" if m % 2 else "normal")
    dw = tern.linear_dw(dev(dy), dev(x))
    dw2 = tern.linear_dw(dev(dy), dev(x))
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32)), "not deterministic"
    check(dw.cpu().numpy(), dy, x, f"dw {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(50, 200, 300), (96, 4096, 4160)])
def test_gemm_dw_accumulate_and_strides(m, n, k):
    # dw with a row pitch past k (columns past k untouched), dy and x as
    # strided views, accumulation into a seeded fp32 start value
    log(f"gemm_dw accumulate m={m} n={n} k={k}")
    dy, x = draw(m, n, k, seed=5 + m + n)
    g = torch.Generator().manual_seed(77)
    init = torch.randn(n, k, generator=g)
    r8 = lambda v: (v + 7) // 8 * 8
    dyg = torch.zeros((m, r8(n) + 24), dtype=torch.bfloat16, device=DEV)
    dyg[:, :n] = dy.to(DEV)
    dyg[:, n:] = float("nan")                   # never read into a stored output
    xg = torch.zeros((m, r8(k) + 40), dtype=torch.bfloat16, device=DEV)
    xg[:, :k] = x.to(DEV)
    xg[:, k:] = float("nan")
    # a row pitch of k + 13 floats (rows not 16-byte aligned: element stores)
    # for the small case, k + 12 (aligned: 16-byte stores) for the large one
    pad = 13 if n <= 256 else 12
    dwg = torch.full((n, k + pad), 5.0, dtype=torch.float32, device=DEV)
    dwg[:, :k] = init.to(DEV)
    tern.tern_gemm_dw(dyg[:, :n], xg[:, :k], dwg[:, :k], accumulate=True)
    torch.cuda.synchronize()
    out = dwg.cpu().numpy()
    assert np.all(out[:, k:] == 5.0)
    rows = None if n <= 256 else np.r_[0:3, n // 2, n - 3:n]
    check(out[:, :k], dy, x, f"dw accumulate {m}x{n}x{k}", rows=rows, init=init.numpy())


def test_gemm_dw_empty_token_range():
    n, k = 40, 72
    dw = torch.full((n, k), 3.0, device=DEV)
    dy = torch.empty((0, n), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, k), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_dw(dy, x, dw, accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(dw == 3.0)
    tern.tern_gemm_dw(dy, x, dw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0


BACKWARD = {l.name: l for wl in tern_inputs.WORKLOADS.values() for l in wl}


@pytest.mark.parametrize("name", ["dit.up.m2048", "dit.down.m2048", "flux_qkv", "flux_mlp.up",
                                  "flux_mlp.down", "single_stream0.in_proj",
                                  "single_stream0.out_proj"])
def test_gemm_dw_layer_backward_shapes(name):
    # the forward layer's input X [m, k] and a seeded output gradient dY [m, n]
    layer = BACKWARD[name]
    m, k, n = layer.m, layer.k, layer.n
    log(f"gemm_dw backward {name}: m={m} n={n} k={k}")
    x, _ = tern_inputs.draw_layer(layer)
    g = torch.Generator().manual_seed(layer.seed + 900)
    dy = torch.randn(m, n, generator=g).to(torch.bfloat16)
    dw = tern.linear_dw(dev(dy), dev(x))
    torch.cuda.synchronize()
    rng = np.random.default_rng(layer.seed)
    # every tile edge of both tile sizes, plus random channels
    edges = sorted({c for t in range(0, n, 128) for c in (t, t + 127) if c < n} | {n - 1})
    rows = np.unique(np.r_[edges[:: max(1, len(edges) // 24)], rng.integers(0, n, 24)])
    check(dw.cpu().numpy(), dy, x, f"dw {name}", rows=rows)
