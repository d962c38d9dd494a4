"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these tests retypes the oracle's own formula: each compares it with a
printed figure, a hand-worked example, a closed form, exact rational
arithmetic, brute force over every case, or a library routine.  The mutation
test at the end plants plausible mistakes in a copy of the oracle's C source
and checks that these pins catch every one.
"""
from __future__ import annotations

import math
import os
import shutil
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle as oracle_mod
import tern_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# fixtures read from tests/golden
# --------------------------------------------------------------------------

def _read_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _pages_storage():
    return {k: float(v) for k, v in (ln.split() for ln in _read_lines("pages_storage.txt"))}


def _pack_examples():
    out = []
    for ln in _read_lines("pack_examples.txt"):
        parts = ln.split()
        out.append(([int(v) for v in parts[:4]], int(parts[4], 16)))
    return out


def _quantize_examples():
    out = []
    for ln in _read_lines("quantize_examples.txt"):
        w, s, t = (part.split() for part in ln.split(";"))
        out.append((np.array([float(v) for v in w], np.float32), float(s[0]),
                    np.array([int(v) for v in t], np.int8)))
    return out


# --------------------------------------------------------------------------
# exact helpers (independent of the oracle)
# --------------------------------------------------------------------------

def _rn32(fr: Fraction) -> np.float32:
    """Round a non-negative rational to the nearest fp32 (ties to even), exactly."""
    if fr == 0:
        return np.float32(0.0)
    lo = np.float32(float(fr))  # candidate; adjust by exact comparison
    cands = sorted({lo, np.nextafter(lo, np.float32(0)), np.nextafter(lo, np.float32(np.inf))},
                   key=lambda c: (abs(Fraction(float(c)) - fr),
                                  int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(cands[0])


def _fp32_midpoint_distance(fr: Fraction) -> Fraction:
    """Relative distance from fr to the nearest point half-way between fp32 neighbours."""
    c = _rn32(fr)
    up = np.nextafter(c, np.float32(np.inf))
    dn = np.nextafter(c, np.float32(0))
    mids = [(Fraction(float(c)) + Fraction(float(up))) / 2,
            (Fraction(float(c)) + Fraction(float(dn))) / 2]
    return min(abs(fr - m) for m in mids) / fr


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# storage format
# --------------------------------------------------------------------------

def test_pack_worked_examples():
    for t, byte in _pack_examples():
        p = oracle.oracle_pack(np.array([t], np.int8))
        assert p.shape == (1, 1) and int(p[0, 0]) == byte, (t, hex(byte), hex(int(p[0, 0])))
        back = oracle.oracle_unpack(p, 4)
        assert back.tolist() == [t]


def test_pack_exhaustive_valid_quads_round_trip():
    quads = np.array([[a, b, c, d] for a in (-1, 0, 1) for b in (-1, 0, 1)
                      for c in (-1, 0, 1) for d in (-1, 0, 1)], np.int8)
    assert quads.shape == (81, 4)
    p = oracle.oracle_pack(quads)
    assert len(set(p[:, 0].tolist())) == 81           # injective
    assert np.array_equal(oracle.oracle_unpack(p, 4), quads)
    # no valid ternary value ever produces the unused code 10
    for byte in p[:, 0].tolist():
        for i in range(4):
            assert (byte >> (2 * i)) & 3 != 2


def test_pack_unpack_all_bytes_and_all_codes():
    allbytes = np.arange(256, dtype=np.uint8).reshape(256, 1)
    t = oracle.oracle_unpack(allbytes, 4)
    assert t.min() == -2 and t.max() == 1                # code 10 decodes to -2
    assert np.array_equal(oracle.oracle_pack(t), allbytes)
    quads = np.array([[a, b, c, d] for a in range(-2, 2) for b in range(-2, 2)
                      for c in range(-2, 2) for d in range(-2, 2)], np.int8)
    assert np.array_equal(oracle.oracle_unpack(oracle.oracle_pack(quads), 4), quads)


def test_pack_ragged_tail_and_layout_along_k():
    rng = np.random.default_rng(7)
    for k in (1, 2, 3, 5, 7, 13, 64, 255):
        t = rng.integers(-1, 2, size=(3, k)).astype(np.int8)
        p = oracle.oracle_pack(t)
        assert p.shape == (3, (k + 3) // 4)
        assert np.array_equal(oracle.oracle_unpack(p, k), t)
        # brute force: weight kk lives in byte kk//4 at bits 2*(kk%4)
        for r in range(3):
            for kk in range(k):
                code = (int(p[r, kk // 4]) >> (2 * (kk % 4))) & 3
                assert code == (int(t[r, kk]) & 3)
        # positions past the end of the row hold code 00
        if k % 4:
            last = int(p[0, -1])
            assert last >> (2 * (k % 4)) == 0


def test_storage_ratio_matches_pages():
    pages = _pages_storage()
    n, k = 64, 3072
    t = tern_inputs.random_ternary(n, k, seed=5).numpy()
    p = oracle.oracle_pack(t)
    bits_per_weight = 8.0 * p.nbytes / (n * k)
    assert bits_per_weight == pages["quantized_bits_stored"] == 2.0
    # per layer against 16-bit weights: exactly 8x, and 8K/(K+16) with fp32 scales
    assert (pages["source_bits"] * n * k / 8) / p.nbytes == 8.0
    with_scales = (2 * n * k) / (p.nbytes + 4 * n)
    assert with_scales == pytest.approx(8 * k / (k + 16))
    # whole model: 99.5 % of parameters at 2 bits, the rest at 16 bits
    f = pages["quantized_parameter_fraction"]
    model = pages["source_bits"] / (f * bits_per_weight + (1 - f) * pages["source_bits"])
    assert round(model, 1) == pages["model_storage_reduction"]


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

def test_quantize_worked_examples():
    for w, s_ref, t_ref in _quantize_examples():
        t, s = oracle.oracle_quantize(w.reshape(1, -1))
        assert float(s[0]) == s_ref, (w, s, s_ref)
        assert np.array_equal(t[0], t_ref), (w, t, t_ref)


def test_quantize_value_set_and_packed_codes():
    x, w = tern_inputs.draw(4, 1024, 300, seed=11)
    t, s = oracle.oracle_quantize(w.numpy())
    assert set(np.unique(t).tolist()) <= {-1, 0, 1}
    p = oracle.oracle_pack(t)
    codes = np.stack([(p >> (2 * i)) & 3 for i in range(4)])
    assert not np.any(codes == 2)
    assert np.all(s > 0)


def test_quantize_fixed_point_of_scaled_ternary():
    rng = np.random.default_rng(3)
    for k in (1, 7, 64, 3072, 32768):
        t0 = rng.integers(-1, 2, size=(4, k)).astype(np.int8)
        t0[:, 0] = 1  # at least one non-zero per row
        for c in (2.0 ** -20, 0.015625, 0.02, 1.0, 3.0e5):
            w = (np.float32(c) * t0.astype(np.float32))
            t, s = oracle.oracle_quantize(w)
            assert np.array_equal(t, t0)
            nnz = np.count_nonzero(t0, axis=1)
            exact = [Fraction(float(np.float32(c))) * int(z) / k for z in nnz]
            for si, ei in zip(s, exact):
                assert abs(Fraction(float(si)) - ei) <= ei * Fraction(1, 2 ** 23)
            # dequantize then quantize returns the same codes
            t2, _ = oracle.oracle_quantize((t.astype(np.float32) * s[:, None]).astype(np.float32))
            assert np.array_equal(t2, t0)


def test_quantize_mean_is_correctly_rounded_exact_mean():
    _, w = tern_inputs.draw(1, 3072, 64, seed=21)
    w = w.numpy()
    _, s = oracle.oracle_quantize(w)
    checked = 0
    for r in range(w.shape[0]):
        exact = sum(Fraction(float(abs(v))) for v in w[r]) / w.shape[1]
        if _fp32_midpoint_distance(exact) > Fraction(1, 2 ** 31):
            assert s[r] == _rn32(exact), r
            checked += 1
    assert checked >= 60
    # a row spanning many binades, where truncation to 2^-48 of the top binade matters least
    row = np.array([1.0, 2.0 ** -30, 2.0 ** -60, 3.0, 2.0 ** -100], np.float32)
    _, s1 = oracle.oracle_quantize(row.reshape(1, -1))
    exact = sum(Fraction(float(v)) for v in row) / len(row)
    assert abs(Fraction(float(s1[0])) - exact) <= exact * Fraction(1, 2 ** 23)


def test_quantize_matches_division_formula_away_from_ties():
    _, w = tern_inputs.draw(1, 3072, 512, seed=31)
    w = w.numpy()
    t, s = oracle.oracle_quantize(w)
    ratio = w.astype(np.float64) / s.astype(np.float64)[:, None]
    literal = np.clip(np.round(ratio), -1, 1).astype(np.int8)   # numpy rounds half to even
    bad = np.argwhere(literal != t)
    for r, c in bad:  # any disagreement must sit on the 1/2 tie, decided exactly
        exact = Fraction(float(abs(w[r, c]))) / Fraction(float(s[r]))
        assert abs(exact - Fraction(1, 2)) < Fraction(1, 2 ** 45)
    assert len(bad) <= 2


def test_quantize_gaussian_statistics():
    # T = 0 iff |w| <= s/2 with s ~ E|w| = sigma*sqrt(2/pi): P = erf(1/(2*sqrt(pi)))
    _, w = tern_inputs.draw(1, 3072, 512, seed=41)
    t, s = oracle.oracle_quantize(w.numpy())
    zero_frac = float(np.mean(t == 0))
    assert abs(zero_frac - math.erf(1.0 / (2.0 * math.sqrt(math.pi)))) < 3e-3
    assert math.erf(1.0 / (2.0 * math.sqrt(math.pi))) == pytest.approx(0.3101, abs=1e-4)
    mean_s = float(np.mean(s.astype(np.float64)))
    expect = tern_inputs.W_STD * math.sqrt(2.0 / math.pi)
    sd_row = tern_inputs.W_STD * math.sqrt(1.0 - 2.0 / math.pi) / math.sqrt(3072)
    assert abs(mean_s - expect) < 5.0 * sd_row / math.sqrt(512)
    assert abs(float(np.std(s)) - sd_row) < 0.25 * sd_row
    # signs are balanced
    assert abs(float(np.mean(t == 1)) - float(np.mean(t == -1))) < 5e-3


def test_quantize_bf16_input_equals_widened_fp32():
    _, w = tern_inputs.draw(1, 512, 40, seed=51)
    wb = w.to(torch.bfloat16)
    t1, s1 = oracle.oracle_quantize(tern_inputs.bf16_bits(wb))
    t2, s2 = oracle.oracle_quantize(wb.to(torch.float32).numpy())
    assert np.array_equal(t1, t2) and np.array_equal(s1, s2)


def test_quantize_rejects_out_of_range_k():
    with pytest.raises(ValueError):
        oracle.oracle_quantize(np.zeros((1, 32769), np.float32))
    with pytest.raises(ValueError):
        oracle.oracle_quantize(np.zeros((1, 0), np.float32))


# --------------------------------------------------------------------------
# layer output
# --------------------------------------------------------------------------

def _single_layer():
    x, w = tern_inputs.draw_layer(tern_inputs.WORKLOADS["single"][0])
    t, s = oracle.oracle_quantize(w.numpy())
    return x, t, s, oracle.oracle_pack(t)


def test_gemm_sign_sum_identity_exact():
    x, t, s, p = _single_layer()
    xb = tern_inputs.bf16_bits(x)
    y = oracle.oracle_gemm(xb, p, s)
    xv = _bf16_values(xb)
    assert y.shape == (16, 512)
    for m in range(16):
        xf = [Fraction(float(v)) for v in xv[m]]
        for n in range(0, 512, 7):
            plus = sum((xf[k] for k in range(256) if t[n, k] == 1), Fraction(0))
            minus = sum((xf[k] for k in range(256) if t[n, k] == -1), Fraction(0))
            assert y[m, n] == float(Fraction(float(s[n])) * (plus - minus)), (m, n)


def test_gemm_equals_float64_matmul_on_exact_inputs():
    rng = np.random.default_rng(61)
    m, k, n = 5, 36, 9
    xi = rng.integers(-64, 65, size=(m, k)).astype(np.float32)
    x = torch.from_numpy(xi).to(torch.bfloat16)          # small integers are exact in bf16
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    ones = np.ones(n, np.float32)
    y = oracle.oracle_gemm(tern_inputs.bf16_bits(x), oracle.oracle_pack(t), ones, k=k)
    ref = torch.matmul(torch.from_numpy(xi).double(), torch.from_numpy(t).double().T).numpy()
    assert np.array_equal(y, ref)
    # a scale per output column multiplies column n
    sc = (2.0 ** rng.integers(-3, 4, size=n)).astype(np.float32)
    y2 = oracle.oracle_gemm(tern_inputs.bf16_bits(x), oracle.oracle_pack(t), sc, k=k)
    assert np.array_equal(y2, ref * sc.astype(np.float64)[None, :])


def test_gemm_against_numpy_on_random_data():
    x, w = tern_inputs.draw(7, 384, 33, seed=71, x_dist="student_t3")
    t, s = oracle.oracle_quantize(w.numpy())
    y = oracle.oracle_gemm(tern_inputs.bf16_bits(x), oracle.oracle_pack(t), s, nthreads=3)
    ref = (x.double().numpy() @ t.astype(np.float64).T) * s.astype(np.float64)[None, :]
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_gemm_zero_row_and_zero_sizes():
    x, w = tern_inputs.draw(3, 64, 4, seed=81)
    w[2] = 0.0
    t, s = oracle.oracle_quantize(w.numpy())
    y = oracle.oracle_gemm(tern_inputs.bf16_bits(x), oracle.oracle_pack(t), s)
    assert s[2] == 0 and np.all(y[:, 2] == 0)
    y0 = oracle.oracle_gemm(np.zeros((0, 64), np.uint16), oracle.oracle_pack(t), s)
    assert y0.shape == (0, 4)


def test_gemm_thread_count_does_not_change_result():
    x, w = tern_inputs.draw(9, 256, 37, seed=91)
    t, s = oracle.oracle_quantize(w.numpy())
    p = oracle.oracle_pack(t)
    xb = tern_inputs.bf16_bits(x)
    assert np.array_equal(oracle.oracle_gemm(xb, p, s, nthreads=1),
                          oracle.oracle_gemm(xb, p, s, nthreads=5))


# --------------------------------------------------------------------------
# epilogue variant: bias and the tanh-form GELU
# --------------------------------------------------------------------------

_Z_GRID = np.concatenate([np.linspace(-12.0, 12.0, 4801), [-40.0, -20.0, -1e-8, 0.0, 1e-8, 20.0, 40.0]])


def _gelu_oracle(z):
    return oracle.oracle_epilogue(np.asarray(z, np.float64)[None, :], None,
                                  oracle.ACT_GELU_TANH, 0)[0]


def test_epilogue_gelu_equals_torch_tanh_gelu():
    # library routine: torch's GELU with approximate='tanh', in float64
    ref = torch.nn.functional.gelu(torch.from_numpy(_Z_GRID), approximate="tanh").numpy()
    got = _gelu_oracle(_Z_GRID)
    assert np.all(np.abs(got - ref) <= 1e-14 * np.maximum(1.0, np.abs(_Z_GRID)))


def test_epilogue_gelu_close_to_exact_gelu():
    # the tanh form approximates z * Phi(z) (Phi through math.erf) to a few 1e-4
    exact = np.array([0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))) for z in _Z_GRID])
    dev = np.abs(_gelu_oracle(_Z_GRID) - exact)
    assert dev.max() < 1e-3
    assert dev[np.abs(_Z_GRID) > 8].max() < 1e-12      # both saturate to 0 and z


def test_epilogue_gelu_odd_part_is_identity():
    # z/2 (1 + tanh u(z)) - (-z)/2 (1 + tanh u(-z)) = z for an odd u and tanh
    z = _Z_GRID
    assert np.all(np.abs(_gelu_oracle(z) - _gelu_oracle(-z) - z) <= 1e-15 * np.maximum(1, np.abs(z)))
    assert _gelu_oracle(np.array([0.0]))[0] == 0.0


def test_epilogue_bias_and_activated_columns():
    rng = np.random.default_rng(3)
    y = rng.normal(size=(5, 9)) * 3
    b = rng.normal(size=9).astype(np.float32)
    out = oracle.oracle_epilogue(y, b, oracle.ACT_GELU_TANH, 4)
    z = y + b.astype(np.float64)
    assert np.array_equal(out[:, :4], z[:, :4])                       # identity before act_from
    ref = torch.nn.functional.gelu(torch.from_numpy(z[:, 4:]), approximate="tanh").numpy()
    assert np.allclose(out[:, 4:], ref, rtol=0, atol=1e-14 * np.abs(z).max())
    assert np.array_equal(oracle.oracle_epilogue(y, b, oracle.ACT_NONE, 0), z)
    assert np.array_equal(oracle.oracle_epilogue(y, None, oracle.ACT_NONE, 0), y)
    assert np.array_equal(oracle.oracle_epilogue(y, None, oracle.ACT_GELU_TANH, 9), y)


def test_epilogue_rejects_bad_arguments():
    y = np.zeros((2, 3))
    for act, act_from in [(2, 0), (1, -1), (1, 4)]:
        with pytest.raises(ValueError):
            oracle.oracle_epilogue(y, None, act, act_from)


# --------------------------------------------------------------------------
# input gradient: u = bf16(dy * s), dx = u . T, and the transposed packing
# --------------------------------------------------------------------------

def _bf16_bits(a):
    return tern_inputs.bf16_bits(torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16))


def _from_bf16_bits(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_scale_grad_matches_torch_single_product_then_bf16():
    # library routine: torch's float32 product, then its round-to-nearest-even
    # conversion to bfloat16
    g = torch.Generator().manual_seed(21)
    dy = (torch.randn(37, 53, generator=g) * 3).to(torch.bfloat16)
    s = torch.rand(53, generator=g) * 0.05 + 1e-4
    ref = tern_inputs.bf16_bits((dy.float() * s).to(torch.bfloat16))
    got = oracle.oracle_scale_grad(tern_inputs.bf16_bits(dy), s.numpy())
    assert np.array_equal(got, ref)


def test_scale_grad_ties_to_even():
    # 1 * (1 + 2^-8) lies half-way between bf16 1 and 1 + 2^-7: the even one (1);
    # 1 * (1 + 3 * 2^-8) half-way between 1 + 2^-7 and 1 + 2^-6: the even one
    # (1 + 2^-6); -1 * (1 + 2^-8) rounds to -1 likewise
    dy = _bf16_bits([[1.0, 1.0, -1.0, 2.0]])
    s = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8, 0.75], np.float32)
    got = oracle.oracle_scale_grad(dy, s)
    assert got.tolist() == [[0x3F80, 0x3F82, 0xBF80, 0x3FC0]]


def test_gemm_dx_adjoint_of_the_layer_exact():
    # <dY, X T^T (.) s> = <(dY (.) s) T, X> exactly, with small integer X and
    # dY and power-of-two scales (every product and sum exact in double)
    rng = np.random.default_rng(8)
    m, k, n = 7, 72, 40
    x = rng.integers(-4, 5, size=(m, k)).astype(np.float32)
    dy = rng.integers(-3, 4, size=(m, n)).astype(np.float32)
    s = (2.0 ** rng.integers(-3, 4, size=n)).astype(np.float32)
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    p = oracle.oracle_pack(t)
    y = oracle.oracle_gemm(_bf16_bits(x), p, s)
    u = oracle.oracle_scale_grad(_bf16_bits(dy), s)
    assert np.array_equal(_from_bf16_bits(u), dy.astype(np.float64) * s)
    dx = oracle.oracle_gemm_dx(u, p, k)
    assert float((dy.astype(np.float64) * y).sum()) == float((dx * x.astype(np.float64)).sum())


def test_gemm_dx_equals_numpy_matmul():
    # exact on small-integer operands; to rounding on random bf16 operands
    rng = np.random.default_rng(9)
    m, k, n = 5, 33, 70
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    p = oracle.oracle_pack(t)
    ui = rng.integers(-8, 9, size=(m, n)).astype(np.float32)
    dx = oracle.oracle_gemm_dx(_bf16_bits(ui), p, k)
    assert np.array_equal(dx, ui.astype(np.float64) @ t.astype(np.float64))
    ur = _bf16_bits(rng.normal(size=(m, n)))
    dx = oracle.oracle_gemm_dx(ur, p, k)
    assert np.allclose(dx, _from_bf16_bits(ur) @ t.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_pack_transposed_worked_example():
    # T (5 x 2): column 0 = (1, 0, -1, 1, -1) -> codes 01 00 11 01 | 11 ->
    # bytes 0x71 0x03; column 1 = (-1, 1, 0, 1, -1) -> 11 01 00 01 | 11 ->
    # bytes 0x47 0x03
    t = np.array([[1, -1], [0, 1], [-1, 0], [1, 1], [-1, -1]], np.int8)
    pt = oracle.oracle_pack_transposed(oracle.oracle_pack(t), 5, 2)
    assert pt.tolist() == [[0x71, 0x03], [0x47, 0x03]]
    rng = np.random.default_rng(10)
    t = rng.integers(-1, 2, size=(37, 29)).astype(np.int8)
    pt = oracle.oracle_pack_transposed(oracle.oracle_pack(t), 37, 29)
    assert np.array_equal(oracle.oracle_unpack(pt, 37), t.T)


# --------------------------------------------------------------------------
# latent-weight gradient (straight-through reading): dW = dY^T . X
# --------------------------------------------------------------------------

def test_gemm_dw_worked_example():
    # dy (3 tokens x 2 channels) = [[1, 2], [3, 4], [5, 6]], x (3 x 2) =
    # [[1, 0], [0, 1], [1, 1]]: dw[n][k] = sum_m dy[m][n] x[m][k], by hand
    # [[1 + 0 + 5, 0 + 3 + 5], [2 + 0 + 6, 0 + 4 + 6]] = [[6, 8], [8, 10]]
    dy = np.array([[1, 2], [3, 4], [5, 6]], np.float32)
    x = np.array([[1, 0], [0, 1], [1, 1]], np.float32)
    dw = oracle.oracle_gemm_dw(_bf16_bits(dy), _bf16_bits(x))
    assert dw.tolist() == [[6.0, 8.0], [8.0, 10.0]]


def test_gemm_dw_adjoint_of_the_layer_exact():
    # For Y = X . (s (.) T)^T, the directional derivative of <dY, Y> along the
    # quantized weight V = s (.) T is <dY, X . V^T> = <dY, Y>; with the
    # straight-through reading it must equal <dW, V>.  Small integers and
    # power-of-two scales keep every product and sum exact in double, and Y
    # comes from the forward layer's own oracle.
    rng = np.random.default_rng(11)
    m, k, n = 9, 40, 24
    x = rng.integers(-4, 5, size=(m, k)).astype(np.float32)
    dy = rng.integers(-3, 4, size=(m, n)).astype(np.float32)
    s = (2.0 ** rng.integers(-3, 4, size=n)).astype(np.float32)
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    y = oracle.oracle_gemm(_bf16_bits(x), oracle.oracle_pack(t), s)
    dw = oracle.oracle_gemm_dw(_bf16_bits(dy), _bf16_bits(x))
    v = s.astype(np.float64)[:, None] * t.astype(np.float64)
    assert float((dw * v).sum()) == float((dy.astype(np.float64) * y).sum())
    # and along an arbitrary integer direction V: <dW, V> = <dY, X V^T>
    vv = rng.integers(-2, 3, size=(n, k)).astype(np.float64)
    lhs = float((dw * vv).sum())
    rhs = float((dy.astype(np.float64) * (x.astype(np.float64) @ vv.T)).sum())
    assert lhs == rhs


def test_gemm_dw_equals_numpy_matmul():
    # exact on small-integer operands; to rounding on random bf16 operands,
    # including a token count of one and an empty token range
    rng = np.random.default_rng(12)
    for m, n, k in ((7, 13, 19), (1, 5, 3), (64, 33, 17)):
        dy = rng.integers(-8, 9, size=(m, n)).astype(np.float32)
        x = rng.integers(-8, 9, size=(m, k)).astype(np.float32)
        dw = oracle.oracle_gemm_dw(_bf16_bits(dy), _bf16_bits(x))
        assert np.array_equal(dw, dy.T.astype(np.float64) @ x.astype(np.float64))
    dyr = _bf16_bits(rng.normal(size=(50, 21)))
    xr = _bf16_bits(rng.standard_t(3, size=(50, 30)))
    dw = oracle.oracle_gemm_dw(dyr, xr)
    assert np.allclose(dw, _from_bf16_bits(dyr).T @ _from_bf16_bits(xr), rtol=1e-12, atol=1e-12)
    dw0 = oracle.oracle_gemm_dw(np.zeros((0, 4), np.uint16), np.zeros((0, 6), np.uint16))
    assert dw0.shape == (4, 6) and not dw0.any()


# --------------------------------------------------------------------------
# 8-bit activations (per-token absmax) and the W1.58-A8 layer
# --------------------------------------------------------------------------

def _rne_int(fr: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even, exactly."""
    f = math.floor(fr)
    d = fr - f
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def test_quantize_act_worked_examples():
    # row 0: max 2 -> 127/2 = 63.5; 1 * 63.5 = 63.5 is a tie -> 64 (even),
    #        0.5 * 63.5 = 31.75 -> 32; scale 2/127
    # row 1: max 127/64 -> 127/max = 64 exactly; 0.5078125 * 64 = 32.5 -> 32
    #        (even), -0.5234375 * 64 = -33.5 -> -34 (even), 1/64 * 64 = 1;
    #        scale (127/64)/127 = 1/64
    # row 2: zeros -> codes 0; the maximum is floored at fp32(1e-5), so the
    #        scale is fp32(fp32(1e-5) / 127)
    # row 3: max 2^-20 < 1e-5 -> floored: 127 / fp32(1e-5) = 12700000 in fp32,
    #        2^-20 * 12700000 = 12.11... -> 12, -2^-21 * 12700000 = -6.06... -> -6
    x = torch.tensor([[1.0, -2.0, 0.5, 0.0],
                      [1.984375, 0.5078125, -0.5234375, 0.015625],
                      [0.0, 0.0, 0.0, 0.0],
                      [2.0 ** -20, -(2.0 ** -21), 0.0, 0.0]]).to(torch.bfloat16)
    assert torch.equal(x.float(), torch.tensor([[1.0, -2.0, 0.5, 0.0],
                                                [1.984375, 0.5078125, -0.5234375, 0.015625],
                                                [0.0, 0.0, 0.0, 0.0],
                                                [2.0 ** -20, -(2.0 ** -21), 0.0, 0.0]]))
    q, xs = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    assert q.tolist() == [[64, -127, 32, 0], [127, 32, -34, 1], [0, 0, 0, 0], [12, -6, 0, 0]]
    floor = np.float32(1e-5)
    assert xs.tolist() == [float(np.float32(2.0 / 127.0)), 0.015625,
                           float(np.float32(float(floor) / 127.0)),
                           float(np.float32(float(floor) / 127.0))]


def test_quantize_act_matches_exact_rational_rounding():
    # q = round(127 x / g), g = max(max|x|, fp32(1e-5)), away from the few
    # products that fall within fp32 rounding of a half-integer; the scale is
    # the correctly rounded fp32 quotient g / 127
    g = torch.Generator().manual_seed(91)
    x = (torch.randn(12, 200, generator=g) * torch.logspace(-3, 2, 12)[:, None]).to(torch.bfloat16)
    x[3, 17] = -x[3].abs().max() * 1.5   # a negative maximum
    x[5] = x[5] * 1e-4                   # a row below the floor
    xb = tern_inputs.bf16_bits(x)
    q, xs = oracle.oracle_quantize_act(xb)
    xv = _bf16_values(xb)
    checked = 0
    floor = Fraction(float(np.float32(1e-5)))
    for m in range(12):
        gm = max(max(Fraction(abs(float(v))) for v in xv[m]), floor)
        assert xs[m] == _rn32(gm / 127)
        assert (int(np.abs(q[m]).max()) == 127) == (gm > floor)
        for kk in range(200):
            e = Fraction(float(xv[m, kk])) * 127 / gm
            frac = abs(e - math.floor(e) - Fraction(1, 2))
            if frac > Fraction(1, 10**5):
                assert q[m, kk] == _rne_int(e), (m, kk)
                checked += 1
    assert checked > 0.99 * 12 * 200


def test_quantize_act_power_of_two_invariance_and_sign():
    x, _ = tern_inputs.draw(9, 160, 4, seed=93)
    q, xs = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    q2, xs2 = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x * 4))
    qn, xsn = oracle.oracle_quantize_act(tern_inputs.bf16_bits(-x))
    assert np.array_equal(q, q2) and np.array_equal(xs2, xs * 4)
    assert np.array_equal(qn, -q) and np.array_equal(xsn, xs)


def test_gemm_a8_integer_activations_equal_bf16_layer():
    # integer activations in [-127, 127] with a 127 in every row quantize to
    # themselves with scale 1, so the A8 layer equals the bf16 layer exactly
    rng = np.random.default_rng(95)
    m, k, n = 6, 64, 11
    xi = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    xi[np.arange(m), rng.integers(0, k, size=m)] = 127.0
    xb = tern_inputs.bf16_bits(torch.from_numpy(xi).to(torch.bfloat16))
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    s = rng.uniform(0.01, 0.1, size=n).astype(np.float32)
    p = oracle.oracle_pack(t)
    q, xs = oracle.oracle_quantize_act(xb)
    assert np.array_equal(q, xi.astype(np.int8)) and np.all(xs == 1.0)
    assert np.array_equal(oracle.oracle_gemm_a8(q, xs, p, s), oracle.oracle_gemm(xb, p, s))


def test_gemm_a8_equals_numpy_integer_matmul():
    x, w = tern_inputs.draw(7, 192, 21, seed=97, x_dist="student_t3")
    t, s = oracle.oracle_quantize(w.numpy())
    q, xs = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    y = oracle.oracle_gemm_a8(q, xs, oracle.oracle_pack(t), s)
    acc = q.astype(np.int64) @ t.astype(np.int64).T
    ref = s.astype(np.float64)[None, :] * xs.astype(np.float64)[:, None] * acc
    assert np.array_equal(y, ref)


def test_pack_a8_worked_example_and_involution():
    # codes of one word: t = 1 0 -1 1 | 0 1 1 -1 | -1 -1 0 0 | 1 1 1 0; field
    # 4i + j holds code 4j + i: fields 0-3 = codes 0, 4, 8, 12 = 1, 0, -1, 1
    # -> 01 00 11 01 (LSB first) = 0x71; fields 4-7 = codes 1, 5, 9, 13 = 0, 1,
    # -1, 1 -> 0x74; fields 8-11 = codes 2, 6, 10, 14 = -1, 1, 0, 1 -> 0x47;
    # fields 12-15 = codes 3, 7, 11, 15 = 1, -1, 0, 0 -> 0x0D
    t = np.array([[1, 0, -1, 1, 0, 1, 1, -1, -1, -1, 0, 0, 1, 1, 1, 0]], np.int8)
    p = oracle.oracle_pack(t)
    assert oracle.oracle_pack_a8(p, 16).tolist() == [[0x71, 0x74, 0x47, 0x0D]]
    # the field transposition is its own inverse
    tt = tern_inputs.random_ternary(13, 96, seed=99).numpy()
    pp = oracle.oracle_pack(tt)
    p8 = oracle.oracle_pack_a8(pp, 96)
    assert np.array_equal(oracle.oracle_pack_a8(p8, 96), pp[:, :24])
    with pytest.raises(ValueError):
        oracle.oracle_pack_a8(pp, 88)    # not whole 16-code words


# --------------------------------------------------------------------------
# mutation check: the pins above must catch plausible mistakes in the oracle
# --------------------------------------------------------------------------

MUTANTS = {
    "tie_rounds_away": ("if (2.0f * a > s)", "if (2.0f * a >= s)"),
    "sign_flipped": ("(wv < 0.0f) ? (int8_t)-1 : (int8_t)1", "(wv < 0.0f) ? (int8_t)1 : (int8_t)-1"),
    "mean_over_k_minus_1": ("/ (double)k;", "/ (double)(k > 1 ? k - 1 : 1);"),
    "mean_rescaled_wrong": ("ldexp((double)Q, E - 48)", "ldexp((double)Q, E - 47)"),
    "fixed_point_too_narrow": ("ldexp(a, 48 - E)", "ldexp(a, 12 - E)"),
    "pack_msb_first": ("byte |= code << (2 * i);", "byte |= code << (6 - 2 * i);"),
    "unpack_no_sign_extension": ("return (code & 2u) ? (int)code - 4 : (int)code;",
                                 "return (int)code;"),
    "gemm_drops_last_k": ("for (int64_t kk = 0; kk < j->k; ++kk) acc +=",
                          "for (int64_t kk = 0; kk + 1 < j->k; ++kk) acc +="),
    "gemm_no_scale": ("j->y[mm * j->ldy + n] = sn * acc;", "j->y[mm * j->ldy + n] = acc;"),
    "gemm_wrong_weight_row": ("unsigned code = (j->p[n * j->ldp + kk / 4]",
                              "unsigned code = (j->p[(n ^ 1) % (j->n_end > 0 ? j->n_end : 1) * j->ldp + kk / 4]"),
    "gemm_x_transposed_index": ("const double* xr = j->xd + mm * j->k;",
                                "const double* xr = j->xd + (mm % 2) * j->k;"),
    "gelu_cubic_coefficient": ("(z + 0.044715 * z * z * z)", "(z + 0.04715 * z * z * z)"),
    "gelu_missing_half": ("return 0.5 * z * (1.0 + tanh(u));", "return z * (1.0 + tanh(u));"),
    "gelu_inverted_sqrt": ("sqrt(2.0 / pi)", "sqrt(pi / 2.0)"),
    "epilogue_act_from_off_by_one": ("nn >= act_from", "nn > act_from"),
    "epilogue_bias_dropped": ("if (bias) v += (double)bias[nn];", "if (bias) v += 0.0;"),
    "scale_grad_truncates": ("(b + 0x7FFFu + lsb) >> 16", "b >> 16"),
    "scale_grad_ties_away": ("(b + 0x7FFFu + lsb) >> 16", "(b + 0x8000u) >> 16"),
    "scale_grad_unscaled": ("bf16_bits_to_float(dy[mm * lddy + nn]) * s[nn]",
                            "bf16_bits_to_float(dy[mm * lddy + nn])"),
    "dx_drops_last_n": ("for (int64_t nn = 0; nn < j->n; ++nn) acc +=",
                        "for (int64_t nn = 0; nn + 1 < j->n; ++nn) acc +="),
    "dx_wrong_column": ("(j->p[nn * j->ldp + kk / 4] >> (2 * (kk % 4)))",
                        "(j->p[nn * j->ldp + (kk ^ 1) / 4] >> (2 * ((kk ^ 1) % 4)))"),
    "dx_wrong_row": ("const double* ur = j->ud + mm * j->n;",
                     "const double* ur = j->ud + ((mm + 1) % j->m) * j->n;"),
    "act_ties_away": ("q[mm * ldq + kk] = (int8_t)rintf(v);", "q[mm * ldq + kk] = (int8_t)roundf(v);"),
    "act_range_128": ("const float inv = 127.0f / g;", "const float inv = 128.0f / g;"),
    "act_scale_inverted": ("xs[mm] = g / 127.0f;", "xs[mm] = 127.0f / g;"),
    "act_max_skips_first": ("for (int64_t kk = 0; kk < k; ++kk) {\n      const float a = fabsf",
                            "for (int64_t kk = 1; kk < k; ++kk) {\n      const float a = fabsf"),
    "a8_no_token_scale": ("(double)s[nn] * (double)xs[mm] * (double)acc",
                          "(double)s[nn] * (double)acc"),
    "a8_wrong_weight_index": ("acc += (int64_t)q[mm * ldq + kk] * trow[kk];",
                              "acc += (int64_t)q[mm * ldq + kk] * trow[k - 1 - kk];"),
    "pack_a8_untransposed": ("const int64_t field = 16 * w + 4 * i + j;",
                             "const int64_t field = 16 * w + 4 * j + i;"),
    "dw_drops_last_token": ("for (int64_t mm = 0; mm < j->m; ++mm) acc += g[mm] * xc[mm];",
                            "for (int64_t mm = 0; mm + 1 < j->m; ++mm) acc += g[mm] * xc[mm];"),
    "dw_wrong_gradient_column": ("dyd[nn * m + mm] = (double)bf16_bits_to_float(dy[mm * lddy + nn]);",
                                 "dyd[nn * m + mm] = (double)bf16_bits_to_float(dy[mm * lddy + (n - 1 - nn)]);"),
    "dw_wrong_input_column": ("const double* xc = j->xd + kk * j->m;",
                              "const double* xc = j->xd + ((kk + 1) % j->k) * j->m;"),
}

PIN_TESTS = [
    test_pack_worked_examples, test_pack_exhaustive_valid_quads_round_trip,
    test_pack_unpack_all_bytes_and_all_codes, test_pack_ragged_tail_and_layout_along_k,
    test_storage_ratio_matches_pages, test_quantize_worked_examples,
    test_quantize_fixed_point_of_scaled_ternary, test_quantize_mean_is_correctly_rounded_exact_mean,
    test_quantize_gaussian_statistics, test_gemm_sign_sum_identity_exact,
    test_gemm_equals_float64_matmul_on_exact_inputs, test_gemm_against_numpy_on_random_data,
    test_epilogue_gelu_equals_torch_tanh_gelu, test_epilogue_gelu_close_to_exact_gelu,
    test_epilogue_gelu_odd_part_is_identity, test_epilogue_bias_and_activated_columns,
    test_scale_grad_matches_torch_single_product_then_bf16, test_scale_grad_ties_to_even,
    test_gemm_dx_adjoint_of_the_layer_exact, test_gemm_dx_equals_numpy_matmul,
    test_pack_transposed_worked_example, test_quantize_act_worked_examples,
    test_quantize_act_matches_exact_rational_rounding,
    test_quantize_act_power_of_two_invariance_and_sign,
    test_gemm_a8_integer_activations_equal_bf16_layer, test_gemm_a8_equals_numpy_integer_matmul,
    test_pack_a8_worked_example_and_involution, test_gemm_dw_worked_example,
    test_gemm_dw_adjoint_of_the_layer_exact, test_gemm_dw_equals_numpy_matmul,
]


def test_pins_catch_planted_mistakes(monkeypatch):
    with open(oracle_mod._SRC) as f:
        src = f.read()
    tmpdir = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
            path = os.path.join(tmpdir, f"{name}.c")
            with open(path, "w") as f:
                f.write(src.replace(old, new))
            lib = oracle_mod.load(oracle_mod.build(force=True, src=path,
                                                   out=os.path.join(tmpdir, f"{name}.so")))
            caught = []
            with monkeypatch.context() as mp:
                mp.setattr(oracle_mod, "_lib", lib)
                for pin in PIN_TESTS:
                    try:
                        pin()
                    except (AssertionError, ValueError):
                        caught.append(pin.__name__)
            assert caught, f"no pin catches the planted mistake {name!r}"
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
