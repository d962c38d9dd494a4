"""Shared helpers of the GPU parity tests: run a case through the C-ABI on the
GPU and through the CPU oracle on the same seeded inputs, then compare.

Bars (the readings behind them are documented in the design notes):
  * ternary codes, scales and packed bytes: bit-exact;
  * layer output: |y - y_ref| <= 8e-3 |y_ref| + 1e-3 s_n ||x_m||_2 for every
    compared element, y_ref being the oracle's unrounded double result.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tern_inputs
import ternary_weight_quantized_tern_amd as tern

REL_TOL = 8e-3
NORM_TOL = 1e-3
DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)


def gpu_quantize_pack(w_cpu: torch.Tensor):
    """GPU path: W -> (T, s) -> P, returned on the host."""
    w = w_cpu.to(DEV)
    t, s = tern.quantize(w)
    p = tern.pack(t)
    torch.cuda.synchronize()
    return t, s, p


def gpu_quantize_pack_fused(w_cpu: torch.Tensor, with_t: bool = True):
    """GPU path through tern_quantize_pack: W -> (T or None, s, P) on the host."""
    w = w_cpu.to(DEV)
    n, k = w.shape
    t = torch.empty((n, k), dtype=torch.int8, device=DEV) if with_t else None
    s = torch.empty((n,), dtype=torch.float32, device=DEV)
    p = torch.empty((n, tern.packed_row_bytes(k)), dtype=torch.uint8, device=DEV)
    tern.tern_quantize_pack(w, t, p, s)
    torch.cuda.synchronize()
    return t, s, p


def oracle_weights(w_cpu: torch.Tensor):
    if w_cpu.dtype == torch.bfloat16:
        t, s = oracle.oracle_quantize(tern_inputs.bf16_bits(w_cpu))
    else:
        t, s = oracle.oracle_quantize(w_cpu.numpy())
    return t, s, oracle.oracle_pack(t)


def assert_bitexact_weights(t_gpu, s_gpu, p_gpu, t_ref, s_ref, p_ref, what=""):
    k = t_ref.shape[1]
    tg = t_gpu.cpu().numpy()
    sg = s_gpu.cpu().numpy()
    pg = p_gpu.cpu().numpy()[:, : p_ref.shape[1]]
    bad_t = int(np.count_nonzero(tg[:, :k] != t_ref))
    bad_s = int(np.count_nonzero(sg.view(np.uint32) != s_ref.view(np.uint32)))
    bad_p = int(np.count_nonzero(pg != p_ref))
    assert bad_t == 0 and bad_s == 0 and bad_p == 0, \
        f"{what}: {bad_t} codes, {bad_s} scales, {bad_p} packed bytes differ"


def row_norms(x_bits: np.ndarray) -> np.ndarray:
    xv = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.sqrt(np.sum(xv * xv, axis=1))


def bf16_to_f64(y: torch.Tensor) -> np.ndarray:
    return y.cpu().float().numpy().astype(np.float64)


def assert_within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray, s: np.ndarray,
                            xnorm: np.ndarray, what=""):
    bound = REL_TOL * np.abs(y_ref) + NORM_TOL * s.astype(np.float64)[None, :] * xnorm[:, None]
    err = np.abs(y_gpu - y_ref)
    bad = err > bound
    if np.any(bad) or not np.all(np.isfinite(y_gpu)):
        idx = np.argwhere(bad | ~np.isfinite(y_gpu))
        r, c = idx[0]
        raise AssertionError(
            f"{what}: {len(idx)} of {y_ref.size} outputs outside tolerance; first at (m={r}, n={c}):"
            f" gpu={y_gpu[r, c]!r} ref={y_ref[r, c]!r} bound={bound[r, c]!r}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def edge_indices(size: int, tile: int = 256, extra: int = 0, seed: int = 0) -> np.ndarray:
    """Rows/columns at every tile and MFMA-subtile edge, plus a seeded random sample."""
    idx = set()
    for base in range(0, size, tile):
        for off in (0, 1, 31, 32, 63, 64, 127, 128, 129, 191, 255):
            if base + off < size:
                idx.add(base + off)
        if len(idx) > 4096:
            break
    for v in (size - 1, size - 2, size - 31, size - 32, size - 33):
        if 0 <= v < size:
            idx.add(v)
    if extra:
        rng = np.random.default_rng(seed)
        idx.update(rng.integers(0, size, size=extra).tolist())
    return np.array(sorted(idx), dtype=np.int64)


def gemm_gpu(x_cpu: torch.Tensor, p_gpu: torch.Tensor, s_gpu: torch.Tensor, k: int):
    x = x_cpu.to(DEV)
    y = torch.empty((x.shape[0], p_gpu.shape[0]), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm(x, p_gpu, s_gpu, y, k)
    torch.cuda.synchronize()
    return y


def check_layer(x_cpu: torch.Tensor, w_cpu: torch.Tensor, what: str, rows=None, cols=None,
                full: bool = False, repeat_check: bool = False):
    """Quantize+pack bit-exact on every weight; layer output on every element
    (``full``) or on the given rows x all columns plus all rows x given columns."""
    m, k = x_cpu.shape
    t_ref, s_ref, p_ref = oracle_weights(w_cpu)
    t_g, s_g, p_g = gpu_quantize_pack(w_cpu)
    assert_bitexact_weights(t_g, s_g, p_g, t_ref, s_ref, p_ref, what)
    # the fused conversion writes the same scales and packed bytes
    _, s_f, p_f = gpu_quantize_pack_fused(w_cpu, with_t=False)
    assert torch.equal(s_f.cpu().view(torch.int32), s_g.cpu().view(torch.int32)), f"{what}: fused s"
    assert torch.equal(p_f.cpu()[:, : p_ref.shape[1]], torch.from_numpy(p_ref)), f"{what}: fused p"
    del s_f, p_f
    # the packed codes round-trip on the GPU
    back = tern.unpack(p_g, k)
    torch.cuda.synchronize()
    assert torch.equal(back.cpu(), torch.from_numpy(t_ref)), f"{what}: unpack(pack(T)) != T"
    del back, t_g

    y = gemm_gpu(x_cpu, p_g, s_g, k)
    if repeat_check:
        y2 = gemm_gpu(x_cpu, p_g, s_g, k)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: not deterministic"
    yh = bf16_to_f64(y)
    xb = tern_inputs.bf16_bits(x_cpu)
    xnorm = row_norms(xb)
    worst = 0.0
    if full:
        y_ref = oracle.oracle_gemm(xb, p_ref, s_ref, k=k)
        worst = assert_within_tolerance(yh, y_ref, s_ref, xnorm, what)
    else:
        if rows is not None:
            y_ref = oracle.oracle_gemm(xb[rows], p_ref, s_ref, k=k)
            worst = max(worst, assert_within_tolerance(yh[rows], y_ref, s_ref, xnorm[rows],
                                                       what + " (rows)"))
        if cols is not None:
            y_ref = oracle.oracle_gemm(xb, p_ref[cols], s_ref[cols], k=k)
            worst = max(worst, assert_within_tolerance(yh[:, cols], y_ref, s_ref[cols], xnorm,
                                                       what + " (cols)"))
    return worst


# ---------------------------------------------------------------------------
# fused epilogue (tern_gemm_ex): bias and the tanh-form GELU
# ---------------------------------------------------------------------------

# Lipschitz bound of the tanh-form GELU (its slope peaks at about 1.13).
GELU_LIP = 1.2
# fp32 rounding of the product and of the bias add, relative to |z| + |b|.
EPI_ADD_TOL = 1e-5


def gemm_ex_gpu(x_cpu, p_gpu, s_gpu, k, bias_cpu=None, act=0, act_from=0):
    x = x_cpu.to(DEV)
    y = torch.empty((x.shape[0], p_gpu.shape[0]), dtype=torch.bfloat16, device=DEV)
    b = None if bias_cpu is None else torch.from_numpy(np.ascontiguousarray(bias_cpu)).to(DEV)
    tern.tern_gemm_ex(x, p_gpu, s_gpu, y, b, act, act_from, k)
    torch.cuda.synchronize()
    return y


def assert_within_tolerance_ex(y_gpu, y_lin_ref, s, xnorm, bias, act, act_from, cols=None,
                               what="", rel_tol=REL_TOL, norm_tol=NORM_TOL):
    """Epilogue output against oracle_epilogue of the unrounded linear output.

    z_ref = y_lin_ref + b.  The GPU forms z in fp32 from an fp32 sum, so
    |z - z_ref| <= 1e-3 s_n ||x_m|| (the slack of the plain layer) + 1e-5
    (|z_ref| + |b_n|) (fp32 product and add); the GELU is Lipschitz with
    constant below 1.2, and the bf16 rounding of y is covered by 8e-3 |y_ref|.
    ``cols`` are the output-column indices of y_gpu's columns (for act_from)."""
    n_cols = y_lin_ref.shape[1]
    cols = np.arange(n_cols) if cols is None else np.asarray(cols)
    b = np.zeros(n_cols) if bias is None else np.asarray(bias, np.float64)
    z_ref = y_lin_ref + b[None, :]
    act_on = (cols >= act_from) if act == oracle.ACT_GELU_TANH else np.zeros(n_cols, bool)
    # oracle_epilogue applies act to its own column indices: pass the mask as act_from 0
    # on the activated subset
    y_ref = z_ref.copy()
    if act_on.any():
        y_ref[:, act_on] = oracle.oracle_epilogue(z_ref[:, act_on], None, oracle.ACT_GELU_TANH, 0)
    lip = np.where(act_on, GELU_LIP, 1.0)[None, :]
    bound = (rel_tol * np.abs(y_ref)
             + lip * (norm_tol * s.astype(np.float64)[None, :] * xnorm[:, None]
                      + EPI_ADD_TOL * (np.abs(z_ref) + np.abs(b)[None, :])))
    err = np.abs(y_gpu - y_ref)
    bad = err > bound
    if np.any(bad) or not np.all(np.isfinite(y_gpu)):
        idx = np.argwhere(bad | ~np.isfinite(y_gpu))
        r, c = idx[0]
        raise AssertionError(
            f"{what}: {len(idx)} of {y_ref.size} outputs outside tolerance; first at (m={r}, "
            f"col={cols[c]}): gpu={y_gpu[r, c]!r} ref={y_ref[r, c]!r} bound={bound[r, c]!r}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def check_layer_ex(x_cpu, w_cpu, bias, act, act_from, what, rows=None, cols=None,
                   full=False):
    """tern_gemm_ex on every element (``full``) or on rows x all columns and all
    rows x columns; weights from the GPU quantizer (bit-exact against the
    oracle's, checked by check_layer elsewhere)."""
    m, k = x_cpu.shape
    t_ref, s_ref, p_ref = oracle_weights(w_cpu)
    _, s_g, p_g = gpu_quantize_pack(w_cpu)
    y = gemm_ex_gpu(x_cpu, p_g, s_g, k, bias, act, act_from)
    yh = bf16_to_f64(y)
    xb = tern_inputs.bf16_bits(x_cpu)
    xnorm = row_norms(xb)
    bias32 = None if bias is None else np.asarray(bias, np.float32)
    worst = 0.0
    if full:
        y_lin = oracle.oracle_gemm(xb, p_ref, s_ref, k=k)
        worst = assert_within_tolerance_ex(yh, y_lin, s_ref, xnorm, bias32, act, act_from,
                                           what=what)
    else:
        if rows is not None:
            y_lin = oracle.oracle_gemm(xb[rows], p_ref, s_ref, k=k)
            worst = max(worst, assert_within_tolerance_ex(yh[rows], y_lin, s_ref, xnorm[rows],
                                                          bias32, act, act_from,
                                                          what=what + " (rows)"))
        if cols is not None:
            y_lin = oracle.oracle_gemm(xb, p_ref[cols], s_ref[cols], k=k)
            worst = max(worst, assert_within_tolerance_ex(
                yh[:, cols], y_lin, s_ref[cols], xnorm,
                None if bias32 is None else bias32[cols], act, act_from, cols=cols,
                what=what + " (cols)"))
    return worst


# ---------------------------------------------------------------------------
# input gradient (tern_gemm_dx) and the codes packed along n
# ---------------------------------------------------------------------------

def draw_grad(m: int, n: int, seed: int) -> torch.Tensor:
    """Seeded bf16 output gradient dY [m, n] ~ N(0, 1) (CPU)."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(m, n, generator=g).to(torch.bfloat16)


def check_dx(dy_cpu: torch.Tensor, w_cpu: torch.Tensor, what: str, rows=None, cols=None,
             full=False):
    """tern_gemm_dx on the GPU against the oracle: the weights are quantized and
    packed on the GPU (bit-exact against the oracle), re-packed along n by
    tern_pack_transposed (bit-exact), the scaled gradient u compared bit for
    bit, and dx within |dx - dx_ref| <= 8e-3 |dx_ref| + 1e-3 ||u_m||_2 on every
    element (``full``) or on rows x all columns and all rows x columns."""
    m, n = dy_cpu.shape
    k = w_cpu.shape[1]
    t_ref, s_ref, p_ref = oracle_weights(w_cpu)
    t, s, p = gpu_quantize_pack(w_cpu)
    assert_bitexact_weights(t, s, p, t_ref, s_ref, p_ref, what + " (weights)")
    pt = tern.pack_transposed(p, n, k)
    pt_ref = oracle.oracle_pack_transposed(p_ref, n, k)
    nb = (n + 3) // 4
    assert np.array_equal(pt.cpu().numpy()[:, :nb], pt_ref), what + " (transposed packing)"
    dyd = dy_cpu.to(DEV)
    u = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_dx(dyd, pt, s, u, dx, k)
    torch.cuda.synchronize()
    dyb = tern_inputs.bf16_bits(dy_cpu)
    u_ref = oracle.oracle_scale_grad(dyb, s_ref)
    assert np.array_equal(tern_inputs.bf16_bits(u.cpu()), u_ref), what + " (scaled gradient)"
    unorm = row_norms(u_ref)
    dxh = bf16_to_f64(dx)
    ones = np.ones(k, np.float32)
    if full or (rows is None and cols is None):
        ref = oracle.oracle_gemm_dx(u_ref, p_ref, k)
        return assert_within_tolerance(dxh, ref, ones, unorm, what)
    worst = 0.0
    if rows is not None:
        ref = oracle.oracle_gemm_dx(u_ref[rows], p_ref, k)
        worst = max(worst, assert_within_tolerance(dxh[rows], ref, ones, unorm[rows],
                                                   what + " (rows)"))
    if cols is not None:
        # columns c of dx need column c of T: the codes of the chosen columns,
        # re-packed as a narrower layer
        t_cols = np.ascontiguousarray(t_ref[:, cols])
        ref = oracle.oracle_gemm_dx(u_ref, oracle.oracle_pack(t_cols), len(cols))
        worst = max(worst, assert_within_tolerance(dxh[:, cols], ref, ones[: len(cols)], unorm,
                                                   what + " (cols)"))
    return worst


# ---------------------------------------------------------------------------
# 8-bit activations (tern_quantize_act, tern_pack_a8, tern_gemm_a8)
# ---------------------------------------------------------------------------

# The int8 sum is exact; fp32(acc) and the two fp32 products add at most
# three roundings of 2^-24 relative, then one bf16 rounding (at most 2^-8
# relative): |y - y_ref| <= (2^-8 + 2^-21) |y_ref|.
A8_REL_TOL = 2.0 ** -8 + 2.0 ** -21


def quantize_act_gpu(x_cpu: torch.Tensor):
    q, xs = tern.quantize_act(x_cpu.to(DEV))
    torch.cuda.synchronize()
    return q, xs


def assert_act_bitexact(q_gpu, xs_gpu, q_ref, xs_ref, what=""):
    qg = q_gpu.cpu().numpy()
    xg = xs_gpu.cpu().numpy()
    bad_q = int(np.count_nonzero(qg != q_ref))
    bad_s = int(np.count_nonzero(xg.view(np.uint32) != xs_ref.view(np.uint32)))
    if bad_q or bad_s:
        idx = np.argwhere(qg != q_ref)
        first = f"; first code at {tuple(idx[0])}: gpu {qg[tuple(idx[0])]} ref " \
                f"{q_ref[tuple(idx[0])]}" if len(idx) else ""
        raise AssertionError(f"{what}: {bad_q} codes and {bad_s} scales differ{first}")


def gemm_a8_gpu(q_gpu, xs_gpu, p8_gpu, s_gpu, k, bias_cpu=None, act=0, act_from=0):
    y = torch.empty((q_gpu.shape[0], p8_gpu.shape[0]), dtype=torch.bfloat16, device=DEV)
    b = None if bias_cpu is None else torch.from_numpy(np.ascontiguousarray(bias_cpu)).to(DEV)
    tern.tern_gemm_a8(q_gpu, xs_gpu, p8_gpu, s_gpu, y, b, act, act_from, k)
    torch.cuda.synchronize()
    return y


def assert_within_tolerance_a8(y_gpu, y_ref, what=""):
    bound = A8_REL_TOL * np.abs(y_ref)
    err = np.abs(y_gpu - y_ref)
    bad = err > bound
    if np.any(bad) or not np.all(np.isfinite(y_gpu)):
        idx = np.argwhere(bad | ~np.isfinite(y_gpu))
        r, c = idx[0]
        raise AssertionError(
            f"{what}: {len(idx)} of {y_ref.size} outputs outside tolerance; first at (m={r}, n={c}):"
            f" gpu={y_gpu[r, c]!r} ref={y_ref[r, c]!r} bound={bound[r, c]!r}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def check_layer_a8(x_cpu, w_cpu, what, rows=None, cols=None, full=False, bias=None, act=0,
                   act_from=0, repeat_check=False):
    """The A8 layer end to end on the GPU (quantize and pack the weights,
    arrange them with tern_pack_a8, quantize the activations, the int8 GEMM)
    against the oracle: weights, arranged codes and activations bit-exact;
    the output within A8_REL_TOL (with the epilogue's terms for bias / GELU)
    on every element (``full``) or on rows x all columns and all rows x
    ``cols``."""
    m, k = x_cpu.shape
    t_ref, s_ref, p_ref = oracle_weights(w_cpu)
    t_g, s_g, p_g = gpu_quantize_pack(w_cpu)
    assert_bitexact_weights(t_g, s_g, p_g, t_ref, s_ref, p_ref, what)
    del t_g
    p8_ref = oracle.oracle_pack_a8(p_ref, k)
    p8_g = tern.pack_a8(p_g, k)
    torch.cuda.synchronize()
    assert torch.equal(p8_g.cpu()[:, : k // 4], torch.from_numpy(p8_ref)), f"{what}: pack_a8"
    xb = tern_inputs.bf16_bits(x_cpu)
    q_ref, xs_ref = oracle.oracle_quantize_act(xb)
    q_g, xs_g = quantize_act_gpu(x_cpu)
    assert_act_bitexact(q_g, xs_g, q_ref, xs_ref, what)
    y = gemm_a8_gpu(q_g, xs_g, p8_g, s_g, k, bias, act, act_from)
    if repeat_check:
        y2 = gemm_a8_gpu(q_g, xs_g, p8_g, s_g, k, bias, act, act_from)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"{what}: not deterministic"
    yh = bf16_to_f64(y)
    epi = bias is not None or act != 0
    bias32 = None if bias is None else np.asarray(bias, np.float32)
    zero = np.zeros(m)

    def compare(yg, q_sel, xs_sel, col_sel, tag):
        p_sel = p_ref if col_sel is None else p_ref[col_sel]
        s_sel = s_ref if col_sel is None else s_ref[col_sel]
        y_lin = oracle.oracle_gemm_a8(q_sel, xs_sel, p_sel, s_sel)
        if not epi:
            return assert_within_tolerance_a8(yg, y_lin, what + tag)
        b_sel = None if bias32 is None else (bias32 if col_sel is None else bias32[col_sel])
        return assert_within_tolerance_ex(yg, y_lin, s_sel, zero[: yg.shape[0]], b_sel, act,
                                          act_from, cols=col_sel, what=what + tag,
                                          rel_tol=A8_REL_TOL, norm_tol=0.0)

    worst = 0.0
    if full:
        worst = compare(yh, q_ref, xs_ref, None, "")
    else:
        if rows is not None:
            worst = max(worst, compare(yh[rows], q_ref[rows], xs_ref[rows], None, " (rows)"))
        if cols is not None:
            worst = max(worst, compare(yh[:, cols], q_ref, xs_ref, cols, " (cols)"))
    return worst
