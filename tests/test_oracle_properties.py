"""Property-based checks of the CPU oracle (hypothesis), CPU only.

Each property follows from the definition of the method, not from the
oracle's code:
  * the mean is taken in fixed point relative to the row's largest binade, so
    permuting a row permutes its codes and leaves its scale bit-identical, and
    scaling a row by a power of two (within range) scales s by exactly that
    factor and leaves the codes unchanged;
  * a code is nonzero exactly when 2|w| > s, and then carries the sign of w
    (checked against exact rational arithmetic on the fp32 values);
  * packing and unpacking any {-1, 0, +1} matrix round-trips, and unpacking
    any byte matrix and re-packing it gives back the bytes when no field is 10;
  * per-token int8 activations: codes lie in [-127, 127], a row whose
    maximum is at least the floor 1e-5 reaches +-127 there, rounding preserves order and sign, the
    codes are odd in x and permuting the row permutes them; the field
    arrangement of the int8 layout applied twice gives back any bytes;
  * the latent-weight gradient dW = dY^T . X is a sum over tokens, so
    splitting the tokens into two batches gives the sum of the two batches'
    gradients, and permuting the tokens changes nothing (exact with
    small-integer operands).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402

SETTINGS = dict(max_examples=60, deadline=None, derandomize=True)

finite_f32 = st.floats(min_value=-1e6, max_value=1e6, allow_nan=False, allow_infinity=False,
                       width=32)
rows = st.lists(finite_f32, min_size=1, max_size=300)


@settings(**SETTINGS)
@given(rows, st.randoms(use_true_random=False))
def test_quantize_is_permutation_equivariant(vals, rnd):
    w = np.array([vals], np.float32)
    perm = list(range(w.shape[1]))
    rnd.shuffle(perm)
    t, s = oracle.oracle_quantize(w)
    tp, sp = oracle.oracle_quantize(np.ascontiguousarray(w[:, perm]))
    assert sp.view(np.uint32)[0] == s.view(np.uint32)[0]
    assert np.array_equal(tp[0], t[0][perm])


@settings(**SETTINGS)
@given(st.lists(st.floats(min_value=-8.0, max_value=8.0, allow_nan=False, width=32)
                .filter(lambda v: v == 0 or abs(v) >= 2.0 ** -60), min_size=1, max_size=200),
       st.integers(min_value=-40, max_value=40))
def test_quantize_power_of_two_scaling(vals, e):
    w = np.array([vals], np.float32)
    c = np.float32(2.0 ** e)
    t, s = oracle.oracle_quantize(w)
    tc, sc = oracle.oracle_quantize(w * c)  # exact: every value and s stay normal
    assert np.array_equal(tc, t)
    assert sc[0] == np.float32(s[0] * c)
    if s[0] != 0:
        assert sc[0] / s[0] == c


@settings(**SETTINGS)
@given(rows)
def test_quantize_decision_and_sign_exact(vals):
    w = np.array([vals], np.float32)
    t, s = oracle.oracle_quantize(w)
    sf = Fraction(float(s[0]))
    for wv, tv in zip(w[0].tolist(), t[0].tolist()):
        big = 2 * abs(Fraction(wv)) > sf
        assert (tv != 0) == big
        if tv != 0:
            assert (tv > 0) == (wv > 0)


@settings(**SETTINGS)
@given(st.integers(min_value=1, max_value=9), st.integers(min_value=1, max_value=70),
       st.integers(min_value=0, max_value=2 ** 32 - 1))
def test_pack_unpack_round_trip_any_shape(n, k, seed):
    rng = np.random.default_rng(seed)
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    p = oracle.oracle_pack(t)
    assert p.shape == (n, (k + 3) // 4)
    assert np.array_equal(oracle.oracle_unpack(p, k), t)
    # bytes without the unused code 10 re-pack to themselves
    b = rng.integers(0, 256, size=(n, (k + 3) // 4)).astype(np.uint8)
    fields = np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=-1)
    b = np.where(fields == 2, 0, fields)
    b = (b[..., 0] | (b[..., 1] << 2) | (b[..., 2] << 4) | (b[..., 3] << 6)).astype(np.uint8)
    if k % 4:
        b[:, -1] &= np.uint8((1 << (2 * (k % 4))) - 1)   # fields past k are 00
    assert np.array_equal(oracle.oracle_pack(oracle.oracle_unpack(b, k)), b)


def _bf16_row(vals):
    """bf16 bit patterns (the top halves of the fp32 encodings) and their values."""
    bits = (np.array(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits[None, :], (bits.astype(np.uint32) << 16).view(np.float32)


@settings(**SETTINGS)
@given(st.lists(st.floats(min_value=-3e4, max_value=3e4, allow_nan=False, width=32),
                min_size=1, max_size=300), st.randoms(use_true_random=False))
def test_quantize_act_range_order_sign_and_permutation(vals, rnd):
    bits, x = _bf16_row(vals)
    q, xs = oracle.oracle_quantize_act(bits)
    q = q[0].astype(np.int64)
    assert np.all(np.abs(q) <= 127)
    g = float(np.max(np.abs(x)))
    assert (int(np.max(np.abs(q))) == 127) == (g >= float(np.float32(1e-5)))
    assert (xs[0] == np.float32(float(np.float32(1e-5)) / 127)) == (g <= float(np.float32(1e-5)))
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(q[order]) >= 0)                   # monotone in x
    assert np.all(np.sign(q) * np.sign(x) >= 0)             # never the opposite sign
    qn, _ = oracle.oracle_quantize_act(np.ascontiguousarray(bits ^ np.uint16(0x8000)))
    assert np.array_equal(qn[0].astype(np.int64), -q)
    perm = list(range(len(vals)))
    rnd.shuffle(perm)
    qp, xsp = oracle.oracle_quantize_act(np.ascontiguousarray(bits[:, perm]))
    assert np.array_equal(qp[0].astype(np.int64), q[perm]) and xsp[0] == xs[0]


@settings(**SETTINGS)
@given(st.integers(min_value=1, max_value=9), st.integers(min_value=1, max_value=6),
       st.integers(min_value=0, max_value=2 ** 32 - 1))
def test_pack_a8_is_an_involution_on_any_bytes(n, words, seed):
    p = np.random.default_rng(seed).integers(0, 256, size=(n, 4 * words)).astype(np.uint8)
    p8 = oracle.oracle_pack_a8(p, 16 * words)
    assert np.array_equal(oracle.oracle_pack_a8(p8, 16 * words), p)


@settings(**SETTINGS)
@given(st.integers(min_value=1, max_value=40), st.integers(min_value=1, max_value=12),
       st.integers(min_value=1, max_value=12), st.integers(min_value=0, max_value=2**31 - 1),
       st.randoms(use_true_random=False))
def test_gemm_dw_additive_over_token_batches(m, n, k, seed, rnd):
    rng = np.random.default_rng(seed)
    bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    dy = bits(rng.integers(-9, 10, size=(m, n)))
    x = bits(rng.integers(-9, 10, size=(m, k)))
    cut = rnd.randint(0, m)
    whole = oracle.oracle_gemm_dw(dy, x)
    parts = oracle.oracle_gemm_dw(dy[:cut], x[:cut]) + oracle.oracle_gemm_dw(dy[cut:], x[cut:])
    assert np.array_equal(whole, parts)
    perm = list(range(m))
    rnd.shuffle(perm)
    assert np.array_equal(oracle.oracle_gemm_dw(dy[perm], x[perm]), whole)
