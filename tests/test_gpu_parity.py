"""GPU parity: every library entry point against the CPU oracle, through the
C-ABI, on seeded inputs.  Small cases span several 256-wide tiles and ragged
edges and are compared on every element; the five workloads run at their
full sizes with every weight compared bit-exactly and the layer output
compared on tile-edge and sampled rows and columns.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tern_inputs
from parity import (DEV, assert_bitexact_weights, assert_within_tolerance,
                    assert_within_tolerance_ex, bf16_to_f64, check_layer, check_layer_ex,
                    check_dx, draw_grad, edge_indices, gemm_ex_gpu, gemm_gpu,
                    gpu_quantize_pack, gpu_quantize_pack_fused, log, oracle_weights, row_norms)

pytestmark = pytest.mark.gpu
tern = pytest.importorskip("ternary_weight_quantized_tern_amd")


# ---------------------------------------------------------------------------
# quantize / pack / unpack on small and edge-case inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(1, 1), (3, 5), (7, 64), (33, 257), (64, 3072), (5, 32768),
                                 (300, 1000), (2, 12289), (9, 3071), (6, 3073), (11, 1152),
                                 (7, 4000)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_pack_random(n, k, dtype):
    log(f"quantize n={n} k={k} {dtype}")
    _, w = tern_inputs.draw(1, k, n, seed=1000 * n + k)
    w = w.to(dtype)
    t_ref, s_ref, p_ref = oracle_weights(w)
    t, s, p = gpu_quantize_pack(w)
    assert_bitexact_weights(t, s, p, t_ref, s_ref, p_ref, f"n={n} k={k}")


@pytest.mark.parametrize("n,k", [(1, 1), (3, 5), (7, 64), (33, 257), (64, 3072), (5, 32768),
                                 (300, 1000), (2, 12289), (9, 3071), (6, 3073), (11, 1152),
                                 (7, 4000)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("with_t", [True, False])
def test_quantize_pack_fused_random(n, k, dtype, with_t):
    log(f"quantize_pack n={n} k={k} {dtype} with_t={with_t}")
    _, w = tern_inputs.draw(1, k, n, seed=1000 * n + k + 1)
    w = w.to(dtype)
    t_ref, s_ref, p_ref = oracle_weights(w)
    t, s, p = gpu_quantize_pack_fused(w, with_t)
    if with_t:
        assert_bitexact_weights(t, s, p, t_ref, s_ref, p_ref, f"fused n={n} k={k}")
    else:
        assert_bitexact_weights(torch.from_numpy(t_ref), s, p, t_ref, s_ref, p_ref,
                                f"fused n={n} k={k}")


@pytest.mark.parametrize("k", [1, 3, 4, 5, 17, 63, 65, 255, 1153])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_pack_fused_unaligned_rows(k, dtype):
    # Row pitches that rule out vector loads and stores (the one-weight-per-
    # thread path, where four lanes combine one packed byte); bytes past
    # ceil(k/4) and codes past k must stay untouched.
    n = 21
    _, w = tern_inputs.draw(1, k, n, seed=500 + k)
    w = w.to(dtype)
    t_ref, s_ref, p_ref = oracle_weights(w)
    big = torch.zeros((n, k + 3), dtype=dtype)
    big[:, :k] = w
    wg = big.to(DEV)[:, :k]                          # pitch k + 3: no 16-byte rows
    nb = (k + 3) // 4
    t = torch.full((n, k + 5), 7, dtype=torch.int8, device=DEV)
    p = torch.full((n, nb + 9), 0xA5, dtype=torch.uint8, device=DEV)
    s = torch.empty(n, device=DEV)
    tern.tern_quantize_pack(wg, t[:, :k], p, s)
    torch.cuda.synchronize()
    th, ph = t.cpu().numpy(), p.cpu().numpy()
    assert np.array_equal(th[:, :k], t_ref)
    assert np.all(th[:, k:] == 7)
    assert np.array_equal(ph[:, :nb], p_ref)
    assert np.all(ph[:, nb:] == 0xA5)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_quantize_special_rows():
    rows = [
        [3.0, 2.0, 1.0, 0.0], [-3.0, -2.0, -1.0, -0.0], [0.0, 0.0, 0.0, 0.0],
        [-0.0, 0.0, -0.0, 0.0], [0.0, 0.0, 0.0, 8.0], [0.5, -0.5, 0.5, -0.5],
        [1.0, 1.0, 1.0, -5.0], [0.75, -1.0, -4.25, 0.0],
        [1e-45, 0.0, 0.0, 0.0],                      # subnormal maximum
        [1e-40, -3e-41, 7e-42, 0.0],                 # all subnormal
        [3e38, -3e38, 1.0, 0.0],                     # near the top of fp32
        [1.0, 2.0 ** -30, 2.0 ** -60, 2.0 ** -100],  # many binades
    ]
    w = torch.tensor(rows, dtype=torch.float32)
    t_ref, s_ref, p_ref = oracle_weights(w)
    t, s, p = gpu_quantize_pack(w)
    assert_bitexact_weights(t, s, p, t_ref, s_ref, p_ref, "special rows")


def test_quantize_strided_views_and_bf16_special():
    _, w = tern_inputs.draw(1, 200, 40, seed=7)
    big = torch.zeros(40, 264)
    big[:, :200] = w
    big[:, 200:] = 99.0                     # must be ignored
    view = big[:, :200]
    t_ref, s_ref, _ = oracle_weights(w)
    wg = big.to(DEV)[:, :200]
    t = torch.full((40, 208), 7, dtype=torch.int8, device=DEV)[:, :200]
    s = torch.empty(40, device=DEV)
    tern.tern_quantize(wg, t, s)
    torch.cuda.synchronize()
    assert view.stride(0) == 264
    assert np.array_equal(t.cpu().numpy(), t_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 15, 16, 17, 63, 64, 65, 255, 1153])
def test_pack_unpack_ragged(k):
    n = 37
    t = tern_inputs.random_ternary(n, k, seed=k).numpy()
    p_ref = oracle.oracle_pack(t)
    nb = (k + 3) // 4
    ldp = nb + 13
    tg = torch.from_numpy(t).to(DEV)
    p = torch.full((n, ldp), 0xA5, dtype=torch.uint8, device=DEV)
    tern.tern_pack(tg, p, k)
    tout = torch.full((n, k + 3), 77, dtype=torch.int8, device=DEV)
    tern.tern_unpack(p, tout, k)
    torch.cuda.synchronize()
    ph = p.cpu().numpy()
    assert np.array_equal(ph[:, :nb], p_ref)
    assert np.all(ph[:, nb:] == 0xA5)               # bytes past ceil(k/4) untouched
    th = tout.cpu().numpy()
    assert np.array_equal(th[:, :k], t)
    assert np.all(th[:, k:] == 77)


@pytest.mark.parametrize("k", [16, 16384, 16400, 50001, 65536])
def test_pack_unpack_segments_vector_pitches(k):
    # Rows of one to four 16384-weight segments with 16-byte row pitches (the
    # vector paths), ragged last groups, and a row count that is not a
    # multiple of anything; bytes and codes past the row stay untouched.
    n = 7
    t = tern_inputs.random_ternary(n, k, seed=k + 11).numpy()
    p_ref = oracle.oracle_pack(t)
    nb = (k + 3) // 4
    ldp = (nb + 15) // 16 * 16 + 16
    ldt = (k + 15) // 16 * 16 + 16
    tpad = np.full((n, ldt), 5, dtype=np.int8)
    tpad[:, :k] = t
    tg = torch.from_numpy(tpad).to(DEV)[:, :k]
    p = torch.full((n, ldp), 0xA5, dtype=torch.uint8, device=DEV)
    tern.tern_pack(tg, p, k)
    tout = torch.full((n, ldt), 77, dtype=torch.int8, device=DEV)
    tern.tern_unpack(p, tout[:, :k], k)
    torch.cuda.synchronize()
    ph = p.cpu().numpy()
    assert np.array_equal(ph[:, :nb], p_ref)
    assert np.all(ph[:, nb:] == 0xA5)
    th = tout.cpu().numpy()
    assert np.array_equal(th[:, :k], t)
    assert np.all(th[:, k:] == 77)


def test_unpack_all_byte_values():
    allb = np.tile(np.arange(256, dtype=np.uint8), (3, 1))      # [3, 256] -> k = 1024
    t_ref = oracle.oracle_unpack(allb, 1024)
    t = tern.unpack(torch.from_numpy(allb).to(DEV), 1024)
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), t_ref)
    assert t_ref.min() == -2


# ---------------------------------------------------------------------------
# layer output on small shapes (every element)
# ---------------------------------------------------------------------------

GEMM_SHAPES = [
    (1, 64, 1), (16, 256, 512), (8, 1152, 300), (300, 320, 520), (257, 128, 255),
    (513, 192, 700), (256, 64, 256), (255, 512, 257), (64, 4096, 96), (1000, 64, 33),
    # few-token path (m <= 32): ragged n, k not a multiple of the 256-wide chunk,
    # one or two MFMA row blocks, and the first size past it
    (2, 320, 50), (5, 448, 33), (16, 4608, 1152), (17, 832, 100), (31, 1088, 47),
    (32, 256, 16), (33, 576, 40), (8, 64, 4608),
    # 64 x 256 tiles (fewer than 256 big tiles, at least 512 of these): ragged m and n
    (1100, 128, 7500),
    # few-token path, every launch shape (channel blocks per workgroup 6, 3, 2
    # and 1; one, two and three chunks per wave) with one and two MFMA row
    # blocks, each with a ragged last block, and chunk slots past the last
    # chunk (3 x 1088, 4 x 704, 5 x 320)
    (3, 1088, 24536), (24, 320, 21496), (4, 704, 12280), (20, 576, 9208), (30, 448, 4600),
    (5, 320, 16400), (20, 256, 16448), (12, 576, 21520),
    # 64 x 576 tiles, one per CU; k of 3 pipeline stages (fewer than the ring)
    (1024, 192, 9216),
    # few-token kernel, K past one round of its waves (the looping form): one
    # block per workgroup with 16 and 32 tokens, six blocks with 16 and 32,
    # two and three blocks of three chunks per wave (a last round with one
    # live slot)
    (5, 8448, 100), (31, 4352, 70), (10, 4352, 21504), (17, 4160, 21512),
    (3, 6400, 16400), (7, 6400, 6150),
    # K-split kernel (at most 256 tiles of 64 tokens x 96, 144 or 192
    # channels, k >= 2048): ragged m and n (n ending inside a 4-channel group),
    # 33 and 41 K steps over four waves (a wave with one step more than the
    # others, and steps on zeros after the last), a DiT down-projection-like
    # layer with 256 whole tiles of 144 channels, and tiles of 96 and 192
    # channels
    (1000, 2112, 1700), (1300, 2624, 1702), (2048, 2048, 1152), (640, 2112, 1880),
    (100, 2112, 1002), (200, 2624, 10002),
    # K-split with one tile of 5 and of 1 channels (a single 4-channel group,
    # partly or mostly past n), 32 and 40 K steps
    (40, 2048, 5), (70, 2560, 1),
    # k just below the K-split bound: 64 x 128 tiles
    (640, 1984, 1880),
]


@pytest.mark.parametrize("m,k,n", GEMM_SHAPES)
def test_gemm_small_all_elements(m, k, n):
    log(f"gemm m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=m * 7919 + k * 31 + n,
                            x_dist="student_t3" if m % 2 else "normal")
    check_layer(x, w, f"gemm {m}x{k}x{n}", full=True, repeat_check=True)


@pytest.mark.parametrize("m", [130, 7, 20])
def test_gemm_strided_operands(m):
    k, n = 192, 140
    log(f"gemm strided m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=99 + m)
    t_ref, s_ref, p_ref = oracle_weights(w)
    xg = torch.zeros((m, k + 72), dtype=torch.bfloat16, device=DEV)
    xg[:, :k] = x.to(DEV)
    xg[:, k:] = float("nan")                          # must never be read
    pg = torch.zeros((n, 80), dtype=torch.uint8, device=DEV)
    pg[:, : k // 4] = torch.from_numpy(p_ref).to(DEV)
    pg[:, k // 4:] = 0xAA                              # would decode as -2s
    sg = torch.from_numpy(s_ref).to(DEV)
    y = torch.full((m, n + 6), 1.0, dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm(xg[:, :k], pg, sg, y[:, :n], k)
    torch.cuda.synchronize()
    yh = bf16_to_f64(y)
    assert np.all(yh[:, n:] == 1.0)                   # columns past n untouched
    xb = tern_inputs.bf16_bits(x)
    y_ref = oracle.oracle_gemm(xb, p_ref, s_ref, k=k)
    assert_within_tolerance(yh[:, :n], y_ref, s_ref, row_norms(xb), "strided")


def test_gemm_ksplit_strided_unaligned():
    # The K-split kernel with padded rows of X (NaN past k) and of the packed
    # weights (codes that would decode as -2 past k), a scale vector that is
    # not 16-byte aligned and an output whose rows do not allow 8-byte stores.
    m, k, n = 1000, 2112, 1700
    log(f"gemm ksplit strided m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=4242)
    t_ref, s_ref, p_ref = oracle_weights(w)
    xg = torch.zeros((m, k + 64), dtype=torch.bfloat16, device=DEV)
    xg[:, :k] = x.to(DEV)
    xg[:, k:] = float("nan")
    pg = torch.zeros((n, k // 4 + 48), dtype=torch.uint8, device=DEV)
    pg[:, : k // 4] = torch.from_numpy(p_ref).to(DEV)
    pg[:, k // 4:] = 0xAA
    sbuf = torch.zeros(n + 1, dtype=torch.float32, device=DEV)
    sbuf[1:] = torch.from_numpy(s_ref).to(DEV)
    ybuf = torch.full((m, n + 7), 1.0, dtype=torch.bfloat16, device=DEV)
    y = ybuf[:, 1:n + 1]
    tern.tern_gemm(xg[:, :k], pg, sbuf[1:], y, k)
    torch.cuda.synchronize()
    yh = bf16_to_f64(ybuf)
    assert np.all(yh[:, 0] == 1.0) and np.all(yh[:, n + 1:] == 1.0)
    xb = tern_inputs.bf16_bits(x)
    y_ref = oracle.oracle_gemm(xb, p_ref, s_ref, k=k)
    assert_within_tolerance(yh[:, 1:n + 1], y_ref, s_ref, row_norms(xb), "ksplit strided")


@pytest.mark.parametrize("m", [64, 128])
def test_gemm_ksplit_wide_weight(m):
    # 64 and 128 tokens on the single-stream in-projection weight (21504 x
    # 3072), the K-split kernel's 96- and 192-channel tiles at full size: every
    # row at an MFMA-block edge and sampled rows across all columns, every
    # column at a tile edge across all rows; repeated runs identical.
    k, n = 3072, 21504
    log(f"gemm ksplit wide weight m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=5100 + m)
    rows = edge_indices(m, extra=8, seed=m)
    cols = edge_indices(n, tile=96 if m == 64 else 192, extra=64, seed=m + 1)
    worst = check_layer(x, w, f"ksplit wide m={m}", rows=rows, cols=cols, repeat_check=True)
    log(f"  ok, worst error / bound = {worst:.3f}")


def test_gemm_k_zero_writes_zeros():
    m, n = 5, 7
    y = torch.full((m, n), 3.0, dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((m, 64), dtype=torch.bfloat16, device=DEV)
    p = torch.zeros((n, 16), dtype=torch.uint8, device=DEV)
    s = torch.ones(n, device=DEV)
    tern.tern_gemm(x, p, s, y, 0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()).item() == 0


def test_gemm_zero_scale_row_gives_zero_column():
    m, k, n = 40, 128, 50
    x, w = tern_inputs.draw(m, k, n, seed=5)
    w[3] = 0.0
    t, s, p = gpu_quantize_pack(w)
    y = gemm_gpu(x, p, s, k)
    assert torch.count_nonzero(y[:, 3].float()).item() == 0


def test_gemm_error_status_through_binding():
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device=DEV)
    p = torch.zeros((4, 32), dtype=torch.uint8, device=DEV)
    s = torch.ones(4, device=DEV)
    y = torch.empty((4, 4), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tern.TernError) as e:
        tern.tern_gemm(x, p, s, y, 100)
    assert e.value.status == tern.TERN_ERR_SHAPE


# ---------------------------------------------------------------------------
# fused epilogue: bias and tanh-form GELU (tern_gemm_ex)
# ---------------------------------------------------------------------------

def _bias(n, seed):
    return (np.random.default_rng(seed).normal(size=n) * 0.5).astype(np.float32)


EPI_VARIANTS = {            # (bias?, act, act_from as a function of n)
    "bias": (True, tern.TERN_ACT_NONE, lambda n: 0),
    "gelu": (False, tern.TERN_ACT_GELU_TANH, lambda n: 0),
    "bias_gelu_from_mid": (True, tern.TERN_ACT_GELU_TANH, lambda n: n // 3 + 1),
}

EPI_SHAPES = [
    (8, 256, 100), (24, 320, 210), (3, 1088, 24536),   # few-token kernel: one block, two
    (5, 320, 16400), (12, 576, 21520),                 # with three chunks a wave, three, six
    (5, 8448, 100), (7, 6400, 6150),                   # the looping form: one block, three
    (300, 320, 520), (513, 192, 700),                  # 64 x 128 tiles
    (1100, 128, 7500),                                 # 64 x 256 tiles
    (1024, 192, 9216),                                 # 64 x 576 tiles
    (1000, 2112, 1700),                                # K-split (act_from inside a 4-channel group)
    (100, 2112, 1002), (200, 2112, 10002),             # K-split, 96- and 192-channel tiles
]


@pytest.mark.parametrize("m,k,n", EPI_SHAPES)
@pytest.mark.parametrize("variant", list(EPI_VARIANTS))
def test_gemm_ex_all_elements(m, k, n, variant):
    log(f"gemm_ex {variant} m={m} k={k} n={n}")
    has_bias, act, af = EPI_VARIANTS[variant]
    x, w = tern_inputs.draw(m, k, n, seed=m * 131 + k * 7 + n + 11,
                            x_dist="student_t3" if m % 2 else "normal")
    bias = _bias(n, m + n) if has_bias else None
    check_layer_ex(x, w, bias, act, af(n), f"gemm_ex {variant} {m}x{k}x{n}", full=True)


@pytest.mark.parametrize("m,k,n", [(4608, 384, 9216), (4608, 448, 9216)])
def test_gemm_ex_big_tiles_sampled(m, k, n):
    # 144 x 384 tiles: persistent (k = 384) and one tile per workgroup (k = 448)
    log(f"gemm_ex big m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=k + 3)
    rows = edge_indices(m, extra=64, seed=k)
    cols = edge_indices(n, extra=64, seed=k + 1)
    check_layer_ex(x, w, _bias(n, k), tern.TERN_ACT_GELU_TANH, 3001, f"gemm_ex big k={k}",
                   rows=rows, cols=cols)


@pytest.mark.parametrize("m,k,n", [(4608, 384, 9216), (300, 320, 520), (8, 256, 100)])
def test_gemm_ex_without_epilogue_is_gemm(m, k, n):
    x, w = tern_inputs.draw(m, k, n, seed=m + k + n)
    _, s, p = gpu_quantize_pack(w)
    y0 = gemm_gpu(x, p, s, k)
    y1 = gemm_ex_gpu(x, p, s, k, None, tern.TERN_ACT_NONE, 0)
    y2 = gemm_ex_gpu(x, p, s, k, None, tern.TERN_ACT_GELU_TANH, n)   # empty activated range
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))


def test_gemm_ex_k_zero_is_epilogue_of_bias():
    m, n = 6, 50
    bias = _bias(n, 1)
    x = torch.zeros((m, 64), dtype=torch.bfloat16)
    p = torch.zeros((n, 16), dtype=torch.uint8, device=DEV)
    s = torch.ones(n, device=DEV)
    y = gemm_ex_gpu(x, p, s, 0, bias, tern.TERN_ACT_GELU_TANH, 17)
    ref = oracle.oracle_epilogue(np.zeros((m, n)), bias, oracle.ACT_GELU_TANH, 17)
    yh = bf16_to_f64(y)
    assert np.all(np.abs(yh - ref) <= 8e-3 * np.abs(ref) + 1e-6)


def test_allocating_conveniences():
    # quantize_pack and linear_ex allocate their outputs and call the same
    # entry points: results bit-identical to the explicit calls.
    x, w = tern_inputs.draw(64, 256, 96, seed=9)
    xd, wd = x.to(DEV), w.to(DEV)
    t, s = tern.quantize(wd)
    p = tern.pack(t)
    p2, s2 = tern.quantize_pack(wd)
    t3, p3, s3 = tern.quantize_pack(wd, with_codes=True)
    b = (torch.randn(96, generator=torch.Generator().manual_seed(5)) * 0.1).to(DEV)
    y = tern.linear_ex(xd, p, s, bias=b, gelu_from=32)
    y_ref = torch.empty_like(y)
    tern.tern_gemm_ex(xd, p, s, y_ref, b, tern.TERN_ACT_GELU_TANH, 32)
    y0 = tern.linear_ex(xd, p, s)
    torch.cuda.synchronize()
    nb = (256 + 3) // 4
    assert torch.equal(p2[:, :nb], p[:, :nb]) and torch.equal(p3[:, :nb], p[:, :nb])
    assert torch.equal(t3, t)
    assert torch.equal(s2.view(torch.int32), s.view(torch.int32))
    assert torch.equal(s3.view(torch.int32), s.view(torch.int32))
    assert torch.equal(y, y_ref)
    assert torch.equal(y0, tern.linear(xd, p, s))


def test_gemm_ex_error_status():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    p = torch.zeros((8, 16), dtype=torch.uint8, device=DEV)
    s = torch.ones(8, device=DEV)
    y = torch.empty((4, 8), dtype=torch.bfloat16, device=DEV)
    for act, af, code in [(5, 0, tern.TERN_ERR_ARG), (tern.TERN_ACT_GELU_TANH, -1, tern.TERN_ERR_ARG),
                          (tern.TERN_ACT_GELU_TANH, 9, tern.TERN_ERR_ARG)]:
        with pytest.raises(tern.TernError) as e:
            tern.tern_gemm_ex(x, p, s, y, None, act, af)
        assert e.value.status == code
    b = torch.zeros(9, device=DEV)[1:]                 # 4-byte aligned, not 16: still accepted
    tern.tern_gemm_ex(x, p, s, y, b, tern.TERN_ACT_GELU_TANH, 0)
    torch.cuda.synchronize()


def test_workload_flux_mlp_up_gelu():
    layer = tern_inputs.WORKLOADS["flux_mlp"][0]
    log(f"workload {layer.name} + GELU m={layer.m} k={layer.k} n={layer.n}")
    x, w = tern_inputs.draw_layer(layer)
    rows = edge_indices(layer.m, extra=96, seed=layer.seed)
    cols = edge_indices(layer.n, extra=96, seed=layer.seed + 1)
    check_layer_ex(x, w, None, tern.TERN_ACT_GELU_TANH, 0, layer.name + " + GELU",
                   rows=rows, cols=cols)


def test_workload_flux_single_stream_in_proj_bias_gelu_mlp_part():
    # GELU on the MLP columns only (the first 3 * 3072 columns are Q, K, V)
    layer = tern_inputs.WORKLOADS["flux_single_stream"][0]
    log(f"workload {layer.name} + bias + GELU[9216:] m={layer.m} k={layer.k} n={layer.n}")
    x, w = tern_inputs.draw_layer(layer)
    rows = edge_indices(layer.m, extra=64, seed=layer.seed)
    cols = np.unique(np.concatenate([edge_indices(layer.n, extra=96, seed=layer.seed + 1),
                                     np.arange(9200, 9232)]))
    check_layer_ex(x, w, _bias(layer.n, 5), tern.TERN_ACT_GELU_TANH, 9216,
                   layer.name + " + bias + GELU[9216:]", rows=rows, cols=cols)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

def _run_workload_layer(layer, n_extra=192, full=None):
    log(f"workload layer {layer.name} m={layer.m} k={layer.k} n={layer.n} seed={layer.seed}")
    x, w = tern_inputs.draw_layer(layer)
    rows = edge_indices(layer.m, extra=n_extra, seed=layer.seed)
    cols = edge_indices(layer.n, extra=n_extra, seed=layer.seed + 1)
    if full is None:
        full = layer.m * layer.n * layer.k <= 2 ** 26
    worst = check_layer(x, w, layer.name, rows=rows, cols=cols, full=full,
                        repeat_check=(layer.seed % 7 == 0 or layer.name == "flux_qkv"))
    log(f"  ok, worst error / bound = {worst:.3f}")


def test_workload_single():
    _run_workload_layer(tern_inputs.WORKLOADS["single"][0])


def test_workload_flux_qkv():
    _run_workload_layer(tern_inputs.WORKLOADS["flux_qkv"][0])


@pytest.mark.parametrize("i", [0, 1])
def test_workload_flux_mlp(i):
    _run_workload_layer(tern_inputs.WORKLOADS["flux_mlp"][i])


@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_workload_dit(i):
    _run_workload_layer(tern_inputs.WORKLOADS["dit"][i])


@pytest.mark.parametrize("block", range(38))
def test_workload_flux_single_stream(block):
    # every element of the first, middle and last block; tile-edge and
    # sampled rows and columns of the others
    layers = tern_inputs.WORKLOADS["flux_single_stream"]
    for layer in layers[2 * block: 2 * block + 2]:
        _run_workload_layer(layer, n_extra=64, full=block in (0, 18, 37))


def test_kernel_configurations_agree_bitwise():
    # Every tiled kernel feeds an output the same MFMA sequence over k (k-blocks
    # of 32 in ascending order into one accumulator), so the persistent 144 x 384
    # kernel (whose LDS ring streams across tiles), the one-tile-per-workgroup
    # 144 x 384 kernel, the 64 x 576 kernel and the 64 x 128 kernel (two
    # workgroups per CU) must give bit-identical outputs on the same operands.
    # A race in any of the LDS pipelines shows up as a mismatch here.  (The
    # K-split kernel sums four partial sums and is checked for repeatability
    # on its own shapes instead.)
    m, k, n = 4608, 3072, 9216
    x, w = tern_inputs.draw(m, k, n, seed=77)
    t, s, p = gpu_quantize_pack(w)
    xd = x.to(DEV)

    def run(mm, nn):
        y = torch.empty((mm, nn), dtype=torch.bfloat16, device=DEV)
        tern.tern_gemm(xd[:mm], p[:nn], s[:nn], y, k)
        return y

    full = run(m, n)            # persistent 144 x 384 (768 tiles)
    a = run(2048, n)            # 144 x 384, one tile per workgroup (m % 144 != 0)
    b = run(2048, 4608)         # 64 x 576 (exactly 256 tiles)
    c = run(512, n)             # 64 x 128, two workgroups per CU
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), full[:2048].view(torch.int16))
    assert torch.equal(b.view(torch.int16), full[:2048, :4608].view(torch.int16))
    assert torch.equal(c.view(torch.int16), full[:512].view(torch.int16))


def test_hip_graph_replays_match_eager():
    # The entry points launch kernels only (no memset or copy nodes), so a
    # captured graph must reproduce the eager results on every replay, with
    # other eager work and synchronizations between the replays.
    m, k, n = 300, 512, 640
    x, w = tern_inputs.draw(m, k, n, seed=88)
    dy = draw_grad(m, n, seed=89)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    ldp, ldpt = tern.packed_row_bytes(k), tern.packed_row_bytes(n)
    bias = (torch.randn(n, generator=torch.Generator().manual_seed(90)) * 0.1).to(DEV)

    def buffers():
        return dict(t=torch.zeros((n, k), dtype=torch.int8, device=DEV),
                    p=torch.zeros((n, ldp), dtype=torch.uint8, device=DEV),
                    s=torch.zeros(n, device=DEV),
                    tu=torch.zeros((n, k), dtype=torch.int8, device=DEV),
                    pt=torch.zeros((k, ldpt), dtype=torch.uint8, device=DEV),
                    y=torch.zeros((m, n), dtype=torch.bfloat16, device=DEV),
                    ye=torch.zeros((m, n), dtype=torch.bfloat16, device=DEV),
                    u=torch.zeros((m, n), dtype=torch.bfloat16, device=DEV),
                    dx=torch.zeros((m, k), dtype=torch.bfloat16, device=DEV))

    def work(b):
        tern.tern_quantize_pack(wd, b["t"], b["p"], b["s"])
        tern.tern_unpack(b["p"], b["tu"], k)
        tern.tern_gemm(xd, b["p"], b["s"], b["y"], k)
        tern.tern_gemm_ex(xd, b["p"], b["s"], b["ye"], bias, tern.TERN_ACT_GELU_TANH, 100, k)
        tern.tern_pack_transposed(b["p"], b["pt"], n, k)
        tern.tern_gemm_dx(dyd, b["pt"], b["s"], b["u"], b["dx"], k)

    eager = buffers()
    work(eager)
    torch.cuda.synchronize()
    cap = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(cap)                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(cap)
    for r in range(3):
        for v in cap.values():
            v.zero_()                               # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in eager:
            assert torch.equal(cap[name].view(torch.uint8), eager[name].view(torch.uint8)), \
                f"replay {r}: {name} differs from the eager result"
    del graph


def test_concurrent_streams_match_serial():
    # The entry points keep no state between calls (apart from
    # tern_gemm_dx_static's array), so calls on two streams that overlap on
    # the GPU must give the bits of the same calls made one after another:
    # the few-token kernel, the tiled kernels with and without the fused
    # epilogue, the input and the latent-weight gradients.
    gen = torch.Generator().manual_seed(91)
    xs, ws = tern_inputs.draw(8, 3072, 4608, seed=92)
    xb, wb = tern_inputs.draw(600, 1024, 2048, seed=93)
    dyb = draw_grad(600, 2048, seed=94)
    bias = (torch.randn(2048, generator=gen) * 0.1).to(DEV)
    ps, ss = tern.quantize_pack(ws.to(DEV))
    pb, sb = tern.quantize_pack(wb.to(DEV))
    ptb = tern.pack_transposed(pb, 2048, 1024)
    xsd, xbd, dybd = xs.to(DEV), xb.to(DEV), dyb.to(DEV)

    def outs():
        return dict(ys=torch.zeros((8, 4608), dtype=torch.bfloat16, device=DEV),
                    yb=torch.zeros((600, 2048), dtype=torch.bfloat16, device=DEV),
                    ye=torch.zeros((600, 2048), dtype=torch.bfloat16, device=DEV),
                    u=torch.zeros((600, 2048), dtype=torch.bfloat16, device=DEV),
                    dx=torch.zeros((600, 1024), dtype=torch.bfloat16, device=DEV),
                    dw=torch.zeros((2048, 1024), dtype=torch.float32, device=DEV))

    def work_a(o):
        tern.tern_gemm(xsd, ps, ss, o["ys"], 3072)
        tern.tern_gemm_dw(dybd, xbd, o["dw"])
        tern.tern_gemm_dx(dybd, ptb, sb, o["u"], o["dx"], 1024)

    def work_b(o):
        tern.tern_gemm(xbd, pb, sb, o["yb"], 1024)
        tern.tern_gemm_ex(xbd, pb, sb, o["ye"], bias, tern.TERN_ACT_GELU_TANH, 700, 1024)

    serial = outs()
    work_a(serial)
    work_b(serial)
    torch.cuda.synchronize()
    runs = [outs() for _ in range(4)]
    sa, sb_ = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb_.wait_stream(torch.cuda.current_stream())
    for o in runs:                                 # launches of the two streams interleave
        with torch.cuda.stream(sa):
            work_a(o)
        with torch.cuda.stream(sb_):
            work_b(o)
    torch.cuda.synchronize()
    for r, o in enumerate(runs):
        for name in serial:
            assert torch.equal(o[name].view(torch.uint8), serial[name].view(torch.uint8)), \
                f"run {r}: {name} differs from the serial result"


# ---------------------------------------------------------------------------
# input gradient: tern_pack_transposed and tern_gemm_dx
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(1, 1), (5, 2), (37, 29), (128, 128), (129, 257), (300, 515),
                                 (4608, 1152)])
@pytest.mark.parametrize("aligned", [True, False])
def test_pack_transposed(n, k, aligned):
    log(f"pack_transposed n={n} k={k} aligned={aligned}")
    t = tern_inputs.random_ternary(n, k, seed=n * 7 + k).numpy()
    p_ref = oracle.oracle_pack(t)
    pt_ref = oracle.oracle_pack_transposed(p_ref, n, k)
    kb, nb = (k + 3) // 4, (n + 3) // 4
    ldp = (kb + 15) // 16 * 16 if aligned else kb + 3
    ldpt = (nb + 15) // 16 * 16 + 16 if aligned else nb + 5
    ph = np.zeros((n, ldp), np.uint8)
    ph[:, :kb] = p_ref
    p = torch.from_numpy(ph).to(DEV)
    pt = torch.full((k, ldpt), 0xA5, dtype=torch.uint8, device=DEV)
    tern.tern_pack_transposed(p, pt, n, k)
    torch.cuda.synchronize()
    got = pt.cpu().numpy()
    assert np.array_equal(got[:, :nb], pt_ref)
    assert np.all(got[:, nb:] == 0xA5)                 # bytes past ceil(n/4) untouched


@pytest.mark.parametrize("m,n,k", [(37, 128, 90), (300, 256, 515), (33, 64, 1), (8, 448, 200),
                                   (1, 64, 64), (130, 192, 2048), (517, 320, 384)])
def test_gemm_dx_all_elements(m, n, k):
    log(f"gemm_dx m={m} n={n} k={k}")
    _, w = tern_inputs.draw(1, k, n, seed=m + 3 * n + 7 * k)
    check_dx(draw_grad(m, n, seed=m * n + k), w, f"dx m={m} n={n} k={k}", full=True)


def test_gemm_dx_n_zero_writes_zeros():
    dy = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    pt = torch.zeros((64, 16), dtype=torch.uint8, device=DEV)
    s = torch.empty(0, device=DEV)
    u = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    dx = torch.full((5, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_dx(dy, pt, s, u, dx, 64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx).item() == 0


def test_gemm_dx_error_status_and_convenience():
    dy = torch.zeros((4, 100), dtype=torch.bfloat16, device=DEV)      # n % 64 != 0
    pt = torch.zeros((8, 32), dtype=torch.uint8, device=DEV)
    s = torch.ones(100, device=DEV)
    u = torch.empty_like(dy)
    dx = torch.empty((4, 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tern.TernError) as e:
        tern.tern_gemm_dx(dy, pt, s, u, dx, 8)
    assert e.value.status == tern.TERN_ERR_SHAPE
    # linear_dx allocates the workspace and calls the same entry point
    dyc = draw_grad(40, 128, seed=5)
    _, w = tern_inputs.draw(1, 96, 128, seed=6)
    t, s, p = gpu_quantize_pack(w)
    pt = tern.pack_transposed(p, 128, 96)
    dyd = dyc.to(DEV)
    u = torch.empty_like(dyd)
    dx_ref = torch.empty((40, 96), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_dx(dyd, pt, s, u, dx_ref, 96)
    dx = tern.linear_dx(dyd, pt, s, 96)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref)


@pytest.mark.parametrize("m,n,k", [(9, 128, 77), (300, 192, 260)])
def test_gemm_dx_strided_views(m, n, k):
    # dY, the workspace and dX as views into wider rows (pitches n + 25,
    # n + 8 and k + 40): the few-token and the tiled GEMM paths, and the
    # scaling pass's element-wise path (dY's odd pitch rules out its 16-byte
    # accesses)
    _, w = tern_inputs.draw(1, k, n, seed=m + n + k)
    dy = draw_grad(m, n, seed=3 * m + n)
    t_ref, s_ref, p_ref = oracle_weights(w)
    t, s, p = gpu_quantize_pack(w)
    pt = tern.pack_transposed(p, n, k)
    dyw = torch.zeros((m, n + 25), dtype=torch.bfloat16)
    dyw[:, :n] = dy
    dyd = dyw.to(DEV)[:, :n]
    u = torch.zeros((m, n + 8), dtype=torch.bfloat16, device=DEV)[:, :n]
    dxw = torch.full((m, k + 40), 5.0, dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_dx(dyd, pt, s, u, dxw[:, :k], k)
    torch.cuda.synchronize()
    u_ref = oracle.oracle_scale_grad(tern_inputs.bf16_bits(dy), s_ref)
    assert np.array_equal(tern_inputs.bf16_bits(u.cpu().contiguous()), u_ref)
    dx_ref = oracle.oracle_gemm_dx(u_ref, p_ref, k)
    assert_within_tolerance(bf16_to_f64(dxw[:, :k].contiguous()), dx_ref, np.ones(k, np.float32),
                            row_norms(u_ref), f"dx strided m={m}")
    assert torch.all(dxw[:, k:] == 5.0)          # columns past k untouched


@pytest.mark.parametrize("m,k,n,act_from", [(5, 256, 77, 37), (20, 192, 333, 200),
                                            (31, 128, 40, 0)])
def test_gemm_ex_few_tokens_ragged_activation_boundary(m, k, n, act_from):
    # the few-token kernel with n not a multiple of 16 and the activated
    # columns starting inside a 16-channel block
    x, w = tern_inputs.draw(m, k, n, seed=m * 11 + n)
    check_layer_ex(x, w, _bias(n, m), tern.TERN_ACT_GELU_TANH, act_from,
                   f"ex few tokens m={m} n={n} from {act_from}", full=True)


@pytest.mark.parametrize("m,k", [(24, 3072), (10, 4352)])
def test_gemm_ex_few_tokens_wide_weight_looping(m, k):
    # The few-token kernel's looping form with six channel blocks per
    # workgroup and the fused epilogue, on the single-stream in-projection
    # width with bias and GELU on its MLP columns: two MFMA row blocks over 12
    # chunks on 8 waves (24 tokens), one row block over 17 chunks on 16 waves
    # (10 tokens); every element.
    n = 21504
    log(f"gemm_ex few looping m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=m * 7 + k, x_dist="student_t3")
    check_layer_ex(x, w, _bias(n, m), tern.TERN_ACT_GELU_TANH, 9216,
                   f"ex few looping m={m} k={k}", full=True)


@pytest.mark.parametrize("layer", ["dit.up.m2048", "flux_qkv", "flux_mlp.up"])
def test_workload_dx(layer):
    # the input gradients of the layers at full size: every weight and the
    # whole scaled gradient bit-exact, dx on tile-edge and sampled rows and
    # columns
    lyr = {l.name: l for wl in tern_inputs.WORKLOADS.values() for l in wl}[layer]
    log(f"dx workload {layer} m={lyr.m} n={lyr.n} k={lyr.k}")
    _, w = tern_inputs.draw_layer(lyr)
    dy = draw_grad(lyr.m, lyr.n, seed=lyr.seed + 500)
    rows = edge_indices(lyr.m, extra=24, seed=1)[:64]
    cols = edge_indices(lyr.k, extra=24, seed=2)[:96]
    check_dx(dy, w, f"dx {layer}", rows=rows, cols=cols)
