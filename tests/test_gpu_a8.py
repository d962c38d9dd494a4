"""GPU parity of the 8-bit-activation layer (tern_quantize_act, tern_pack_a8,
tern_gemm_a8) against the CPU oracle, through the C-ABI.

Bars: activation codes, per-token scales and arranged weight codes bit-exact;
the layer output within (2^-8 + 2^-21) |y_ref| of the oracle's unrounded
double result (the int32 sum is exact, so only fp32 and bf16 roundings
remain), and bit-exact where every fp32 step is exact (power-of-two scales).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tern_inputs
from parity import (DEV, assert_act_bitexact, assert_within_tolerance_a8, bf16_to_f64,
                    check_layer_a8, edge_indices, gemm_a8_gpu, log, quantize_act_gpu)
import ternary_weight_quantized_tern_amd as tern

pytestmark = pytest.mark.gpu


def _x(m, k, seed, dist="normal"):
    x, _ = tern_inputs.draw(m, k, 1, seed=seed, x_dist=dist)
    return x


# ---------------------------------------------------------------------------
# per-token activation codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 64), (7, 3072), (5, 1000), (3, 1001), (4, 8), (2, 1),
                                 (70, 520), (9, 32768), (1030, 136), (6, 15360), (5, 16384),
                                 (5, 16392), (300, 12288), (7, 1032), (6, 4104)])
@pytest.mark.parametrize("dist", ["normal", "student_t3"])
def test_quantize_act_bitexact(m, k, dist):
    log(f"quantize_act m={m} k={k} {dist}")
    x = _x(m, k, seed=m * 7 + k, dist=dist)
    # rows over many magnitudes, a row of zeros, a row with a negative maximum
    x = (x.float() * torch.logspace(-4, 3, m)[:, None]).to(torch.bfloat16)
    if m > 2:
        x[1] = 0
        x[2, k // 2] = -x[2].float().abs().max().to(torch.bfloat16) * 2
    if m > 3:
        x[3] = (x[3].float() * 1e-9).to(torch.bfloat16)      # below the floor 1e-5
    if m > 4:
        x[4] = (x[4].float() * 1e-38).to(torch.bfloat16)     # 127 / max would overflow fp32
    q_ref, xs_ref = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    q, xs = quantize_act_gpu(x)
    assert_act_bitexact(q, xs, q_ref, xs_ref, f"m={m} k={k}")


def test_quantize_act_ties_and_extremes():
    # 127/max exact (max = 127/64 -> 64): x * 64 lands on half-integers, which
    # round to even; the maximum maps to +-127
    vals = torch.tensor([127 / 64, -127 / 64] + [(j + 0.5) / 64 for j in range(-60, 60)])
    x = vals.repeat(3, 2)[:, :240].to(torch.bfloat16)
    q_ref, xs_ref = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    q, xs = quantize_act_gpu(x)
    assert_act_bitexact(q, xs, q_ref, xs_ref, "ties")
    assert int(q.abs().max()) == 127


def test_quantize_act_strided_views_and_k_zero():
    big = _x(40, 700, seed=11)
    x = big[3:33, 5:605]                       # row pitch 700, unaligned start: scalar path
    q_store = torch.full((30, 640), 55, dtype=torch.int8, device=DEV)
    xs = torch.empty(30, dtype=torch.float32, device=DEV)
    tern.tern_quantize_act(big.to(DEV)[3:33, 5:605], q_store, xs)
    torch.cuda.synchronize()
    q_ref, xs_ref = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x.contiguous()))
    assert_act_bitexact(q_store[:, :600], xs, q_ref, xs_ref, "strided")
    assert bool((q_store[:, 600:] == 55).all()), "columns past k were written"
    # k == 0: the floored scale fp32(1e-5) / 127, codes untouched
    xs0 = torch.full((4,), 7.0, device=DEV)
    q0 = torch.full((4, 16), 3, dtype=torch.int8, device=DEV)
    tern.tern_quantize_act(torch.empty((4, 16), dtype=torch.bfloat16, device=DEV), q0, xs0, k=0)
    torch.cuda.synchronize()
    floor_scale = float(np.float32(float(np.float32(1e-5)) / 127))
    assert xs0.cpu().tolist() == [floor_scale] * 4 and bool((q0 == 3).all())


# ---------------------------------------------------------------------------
# arranged weight codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(9216, 3072), (37, 48), (5, 16), (300, 1152), (64, 12288)])
def test_pack_a8_bitexact(n, k):
    t = tern_inputs.random_ternary(n, k, seed=n + k).numpy()
    p_ref = oracle.oracle_pack(t)
    p8_ref = oracle.oracle_pack_a8(p_ref, k)
    p = torch.zeros((n, tern.packed_row_bytes(k)), dtype=torch.uint8)
    p[:, : p_ref.shape[1]] = torch.from_numpy(p_ref)
    p = p.to(DEV)
    p8 = tern.pack_a8(p, k)
    torch.cuda.synchronize()
    assert torch.equal(p8.cpu()[:, : k // 4], torch.from_numpy(p8_ref))
    # in place, and back again (the arrangement is its own inverse)
    tern.tern_pack_a8(p8, p8, k)
    torch.cuda.synchronize()
    assert torch.equal(p8.cpu(), p.cpu())


def test_pack_a8_unaligned_rows_scalar_path():
    n, k = 21, 80                                  # 5 words per row, pitch 20 bytes
    t = tern_inputs.random_ternary(n, k, seed=5).numpy()
    p_ref = oracle.oracle_pack(t)
    buf = torch.zeros(n * 20 + 4, dtype=torch.uint8)
    view = buf[4:].view(n, 20)
    view[:] = torch.from_numpy(p_ref)
    dev = buf.to(DEV)
    out = torch.full((n, 24), 0xAB, dtype=torch.uint8, device=DEV)
    tern.tern_pack_a8(dev[4:].view(n, 20), out, k)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu()[:, :20], torch.from_numpy(oracle.oracle_pack_a8(p_ref, k)))
    assert bool((out[:, 20:] == 0xAB).all())


# ---------------------------------------------------------------------------
# the int8 GEMM
# ---------------------------------------------------------------------------

def _bf16_rne(v: np.ndarray) -> np.ndarray:
    # every value here is an fp32 value (exact products of small powers of two
    # and integers below 2^24), so the conversion through fp32 rounds once
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("m,k,n", [(300, 384, 520), (4608, 3072, 3072), (4608, 1152, 3072),
                                   (4600, 3072, 3000), (2304, 3072, 4608), (1, 128, 64),
                                   (33, 256, 200)])
def test_gemm_a8_power_of_two_scales_bitexact(m, k, n):
    # q uniform on [-127, 127]; with s and xs powers of two every fp32 step is
    # exact, so y must be the bf16 rounding of the exact result
    log(f"gemm_a8 exact m={m} k={k} n={n}")
    g = torch.Generator().manual_seed(m + 3 * k + 7 * n)
    q = torch.randint(-127, 128, (m, k), generator=g, dtype=torch.int8)
    xs = (2.0 ** torch.randint(-9, -3, (m,), generator=g)).float()
    s = (2.0 ** torch.randint(-8, -2, (n,), generator=g)).float()
    t = tern_inputs.random_ternary(n, k, seed=m + n).numpy()
    p = oracle.oracle_pack(t)
    p8 = oracle.oracle_pack_a8(p, k)
    p8_dev = torch.zeros((n, tern.packed_row_bytes(k)), dtype=torch.uint8)
    p8_dev[:, : k // 4] = torch.from_numpy(p8)
    y = gemm_a8_gpu(q.to(DEV), xs.to(DEV), p8_dev.to(DEV), s.to(DEV), k)
    yh = bf16_to_f64(y)
    qn, xsn, sn = q.numpy(), xs.numpy(), s.numpy()
    if m * n * k <= 2 ** 27:
        rows, cols = np.arange(m), None
    else:
        rows, cols = edge_indices(m, tile=144, extra=48, seed=m), edge_indices(n, extra=48, seed=n)
    # (the oracle's layer reads the plain packing p)
    y_ref = oracle.oracle_gemm_a8(qn[rows], xsn[rows], p, sn)
    assert np.array_equal(yh[rows], _bf16_rne(y_ref)), "rows differ"
    if cols is not None:
        y_ref_c = oracle.oracle_gemm_a8(qn, xsn, p[cols], sn[cols])
        assert np.array_equal(yh[:, cols], _bf16_rne(y_ref_c)), "columns differ"


@pytest.mark.parametrize("m,k,n", [(37, 256, 300), (300, 384, 520), (1, 128, 64),
                                   (130, 1152, 1000), (64, 128, 128), (65, 640, 129)])
def test_gemm_a8_layer_all_elements(m, k, n):
    x, w = tern_inputs.draw(m, k, n, seed=17 * m + n, x_dist="student_t3")
    worst = check_layer_a8(x, w, f"a8 m={m} k={k} n={n}", full=True)
    log(f"  worst error / bound = {worst:.3f}")


@pytest.mark.parametrize("m,k,n,act_from", [(300, 384, 520, 200), (37, 256, 300, 0),
                                            (130, 1152, 1000, 1000), (20, 128, 333, 37)])
def test_gemm_a8_epilogue_all_elements(m, k, n, act_from):
    x, w = tern_inputs.draw(m, k, n, seed=m + 5 * n)
    bias = np.random.default_rng(m).normal(0, 0.5, n).astype(np.float32)
    worst = check_layer_a8(x, w, f"a8 epi m={m} n={n}", full=True, bias=bias,
                           act=tern.TERN_ACT_GELU_TANH, act_from=act_from)
    log(f"  worst error / bound = {worst:.3f}")


def test_gemm_a8_epilogue_big_tiles_sampled():
    m, k, n = 4608, 384, 9216
    x, w = tern_inputs.draw(m, k, n, seed=77)
    bias = np.random.default_rng(3).normal(0, 0.5, n).astype(np.float32)
    rows = edge_indices(m, tile=144, extra=32, seed=1)
    cols = np.unique(np.concatenate([edge_indices(n, extra=64, seed=2), np.arange(8990, 9010)]))
    check_layer_a8(x, w, "a8 epi 4608x9216", rows=rows, cols=cols, bias=bias,
                   act=tern.TERN_ACT_GELU_TANH, act_from=9000)


def test_gemm_a8_persistent_epilogue_sampled():
    # The FLUX MLP up-projection shape: 1024 tiles of 144 x 384 with K / 128 = 24
    # steps, a multiple of the four-stage ring, a 16-byte aligned output, scale
    # and bias: the persistent kernel with the fused epilogue (its staging
    # through the ring's last stage while the next tile's stages are in flight).
    # act_from inside a tile and inside a 16-channel block.
    m, k, n = 4608, 3072, 12288
    x, w = tern_inputs.draw(m, k, n, seed=81)
    bias = np.random.default_rng(7).normal(0, 0.5, n).astype(np.float32)
    act_from = 6002
    rows = edge_indices(m, tile=144, extra=24, seed=8)
    cols = np.unique(np.concatenate([edge_indices(n, tile=384, extra=48, seed=9),
                                     np.arange(act_from - 10, act_from + 10)]))
    check_layer_a8(x, w, "a8 epi persistent 4608x12288", rows=rows, cols=cols, bias=bias,
                   act=tern.TERN_ACT_GELU_TANH, act_from=act_from, repeat_check=True)


def test_gemm_a8_persistent_and_direct_epilogues_agree_bitwise():
    # The same fused layer through the persistent kernel (its epilogue staged in
    # LDS) and, with the output misaligned, through the one-tile-per-workgroup
    # kernel with the direct epilogue: the same formula on the same int32 sums.
    m, k, n = 4608, 3072, 12288
    g = torch.Generator().manual_seed(13)
    q = torch.randint(-127, 128, (m, k), generator=g, dtype=torch.int8).to(DEV)
    xs = (torch.rand(m, generator=g) * 0.05).to(DEV)
    s = (torch.rand(n, generator=g) * 0.05).to(DEV)
    bias = (torch.randn(n, generator=g) * 0.5).to(DEV)
    t = tern_inputs.random_ternary(n, k, seed=14).numpy()
    p8 = torch.from_numpy(oracle.oracle_pack_a8(oracle.oracle_pack(t), k)).to(DEV)
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_a8(q, xs, p8, s, y1, bias, tern.TERN_ACT_GELU_TANH, 6002)
    buf = torch.empty(m * n + 1, dtype=torch.bfloat16, device=DEV)
    y2 = buf[1:].view(m, n)
    tern.tern_gemm_a8(q, xs, p8, s, y2, bias, tern.TERN_ACT_GELU_TANH, 6002)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_gemm_a8_one_tile_per_cu_epilogue_sampled():
    # M = 2048, N = 4608: the 64 x 576 tiles, one per CU
    m, k, n = 2048, 1152, 4608
    x, w = tern_inputs.draw(m, k, n, seed=79, x_dist="student_t3")
    bias = np.random.default_rng(4).normal(0, 0.5, n).astype(np.float32)
    rows = edge_indices(m, tile=64, extra=32, seed=5)
    cols = np.unique(np.concatenate([edge_indices(n, tile=576, extra=64, seed=6),
                                     np.arange(2290, 2310)]))
    check_layer_a8(x, w, "a8 epi 2048x4608", rows=rows, cols=cols, bias=bias,
                   act=tern.TERN_ACT_GELU_TANH, act_from=2300)


@pytest.mark.parametrize("m,k,n", [(32, 3072, 3072), (17, 256, 1000), (5, 4608, 1152),
                                   (16, 1152, 4608), (2, 15360, 520)])
def test_gemm_a8_few_tokens_all_elements(m, k, n):
    x, w = tern_inputs.draw(m, k, n, seed=3 * m + n, x_dist="student_t3")
    worst = check_layer_a8(x, w, f"a8 few m={m} k={k} n={n}", full=True)
    log(f"  worst error / bound = {worst:.3f}")


def test_gemm_a8_few_token_and_tiled_kernels_agree_bitwise():
    # m = 32 runs the weight-streaming kernel, m = 33 the tiled one; both
    # apply the same formula to the same exact int32 sums
    k, n = 1152, 4608
    g = torch.Generator().manual_seed(8)
    q = torch.randint(-127, 128, (33, k), generator=g, dtype=torch.int8).to(DEV)
    xs = (torch.rand(33, generator=g) * 0.05).to(DEV)
    s = (torch.rand(n, generator=g) * 0.05).to(DEV)
    t = tern_inputs.random_ternary(n, k, seed=12).numpy()
    p8 = torch.from_numpy(oracle.oracle_pack_a8(oracle.oracle_pack(t), k)).to(DEV)
    bias = torch.linspace(-1, 1, n).to(DEV)
    for act, act_from, b in ((tern.TERN_ACT_NONE, 0, None), (tern.TERN_ACT_GELU_TANH, 1000, bias)):
        y33 = torch.empty((33, n), dtype=torch.bfloat16, device=DEV)
        y32 = torch.empty((32, n), dtype=torch.bfloat16, device=DEV)
        tern.tern_gemm_a8(q, xs, p8, s, y33, b, act, act_from)
        tern.tern_gemm_a8(q[:32], xs[:32], p8, s, y32, b, act, act_from)
        torch.cuda.synchronize()
        assert torch.equal(y32.view(torch.int16), y33[:32].view(torch.int16)), f"act={act}"


def test_gemm_a8_k_zero_and_strided_operands():
    # k == 0: bf16(gelu(bias))
    n = 40
    bias = torch.linspace(-2, 2, n)
    y = torch.full((5, n), 9.0, dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_a8(torch.empty((5, 128), dtype=torch.int8, device=DEV),
                      torch.ones(5, device=DEV), torch.zeros((n, 32), dtype=torch.uint8, device=DEV),
                      torch.ones(n, device=DEV), y, bias.to(DEV), tern.TERN_ACT_GELU_TANH, 0, k=0)
    torch.cuda.synchronize()
    ref = oracle.oracle_epilogue(np.zeros((5, n)), bias.numpy(), oracle.ACT_GELU_TANH, 0)
    assert np.allclose(bf16_to_f64(y), ref, rtol=2.0 ** -8, atol=1e-6)
    # views: q rows of pitch 400 bytes, y rows of pitch 310, p8 rows of 112 bytes
    m, k, n = 70, 384, 300
    x, w = tern_inputs.draw(m, k, n, seed=23)
    t_ref, s_ref = oracle.oracle_quantize(w.numpy())
    p_ref = oracle.oracle_pack(t_ref)
    q_ref, xs_ref = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    qb = torch.zeros((m, 400), dtype=torch.int8)
    qb[:, :k] = torch.from_numpy(q_ref)
    pb = torch.zeros((n, 112), dtype=torch.uint8)
    pb[:, : k // 4] = torch.from_numpy(p_ref)
    p8 = torch.zeros_like(pb).to(DEV)
    tern.tern_pack_a8(pb.to(DEV), p8, k)
    yb = torch.zeros((m, 310), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_a8(qb.to(DEV)[:, :k], torch.from_numpy(xs_ref).to(DEV), p8,
                      torch.from_numpy(s_ref).to(DEV), yb[:, :n], k=k)
    torch.cuda.synchronize()
    y_ref = oracle.oracle_gemm_a8(q_ref, xs_ref, p_ref, s_ref)
    assert_within_tolerance_a8(bf16_to_f64(yb[:, :n]), y_ref, "strided")
    assert bool((yb[:, n:] == 0).all())


def test_gemm_a8_launch_paths_agree_bitwise():
    # the persistent 144 x 384 kernel (whole tiles, 16-byte aligned y, K / 128
    # a multiple of its four-stage ring) and the one-tile-per-workgroup kernel
    # with the direct epilogue (y misaligned) compute the same formula
    m, k, n = 4608, 1024, 4608
    g = torch.Generator().manual_seed(5)
    q = torch.randint(-127, 128, (m, k), generator=g, dtype=torch.int8).to(DEV)
    xs = (torch.rand(m, generator=g) * 0.05).to(DEV)
    s = (torch.rand(n, generator=g) * 0.05).to(DEV)
    t = tern_inputs.random_ternary(n, k, seed=9).numpy()
    p8 = torch.from_numpy(oracle.oracle_pack_a8(oracle.oracle_pack(t), k)).to(DEV)
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    tern.tern_gemm_a8(q, xs, p8, s, y1)
    buf = torch.empty(m * n + 1, dtype=torch.bfloat16, device=DEV)
    y2 = buf[1:].view(m, n)
    tern.tern_gemm_a8(q, xs, p8, s, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_gemm_a8_max_k_sums_do_not_overflow():
    # K = 2^18, the largest the entry point accepts: with every code at +-127
    # and every weight +-1 the sums reach 127 * 2^18 (64x that in the kernel's
    # int32 accumulator, just below 2^31); power-of-two scales keep every fp32
    # step exact, so y must equal the bf16 rounding of the exact sum
    m, k, n = 3, 2 ** 18, 128
    q = torch.full((m, k), 127, dtype=torch.int8)
    q[1] = -127
    q[2, 1::2] = -127                    # alternating: the sum cancels to 0 for t = +1
    t = np.ones((n, k), np.int8)
    t[1::2] = -1                         # odd channels all -1
    t[5, : k // 2] = 0                   # a channel half zero
    p = oracle.oracle_pack(t)
    p8 = torch.from_numpy(oracle.oracle_pack_a8(p, k))
    xs = torch.tensor([2.0 ** -10, 2.0 ** -8, 2.0 ** -4])
    s = torch.full((n,), 2.0 ** -6)
    y = gemm_a8_gpu(q.to(DEV), xs.to(DEV), p8.to(DEV), s.to(DEV), k)
    y_ref = oracle.oracle_gemm_a8(q.numpy(), xs.numpy(), p, s.numpy())
    assert np.array_equal(bf16_to_f64(y), _bf16_rne(y_ref))
    assert y_ref[0, 0] == 127 * k * 2.0 ** -16 and y_ref[1, 1] == 127 * k * 2.0 ** -14


def test_a8_layer_in_a_hip_graph_matches_eager():
    m, k, n = 300, 384, 520
    x, w = tern_inputs.draw(m, k, n, seed=41)
    xd = x.to(DEV)
    p, s = tern.quantize_pack(w.to(DEV))
    p8 = tern.pack_a8(p, k)
    q = torch.empty((m, k), dtype=torch.int8, device=DEV)
    xs = torch.empty(m, dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)

    def layer():
        tern.tern_quantize_act(xd, q, xs)
        tern.tern_gemm_a8(q, xs, p8, s, y)

    layer()
    torch.cuda.synchronize()
    eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    for i in range(4):
        y.zero_()
        q.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


def test_linear_a8_convenience_and_errors():
    m, k, n = 50, 256, 96
    x, w = tern_inputs.draw(m, k, n, seed=31)
    p, s = tern.quantize_pack(w.to(DEV))
    y = tern.linear_a8(x.to(DEV), tern.pack_a8(p, k), s)
    torch.cuda.synchronize()
    t_ref, s_ref = oracle.oracle_quantize(w.numpy())
    q_ref, xs_ref = oracle.oracle_quantize_act(tern_inputs.bf16_bits(x))
    assert_within_tolerance_a8(bf16_to_f64(y), oracle.oracle_gemm_a8(
        q_ref, xs_ref, oracle.oracle_pack(t_ref), s_ref), "linear_a8")
    with pytest.raises(tern.TernError) as e:
        tern.linear_a8(x[:, :192].contiguous().to(DEV), tern.pack_a8(p, k), s)   # k % 128 != 0
    assert e.value.status == tern.TERN_ERR_SHAPE


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,i", [("single", 0), ("flux_qkv", 0), ("flux_mlp", 0),
                                    ("flux_mlp", 1), ("dit", 0), ("dit", 1), ("dit", 2),
                                    ("dit", 3)])
def test_workload_a8(name, i):
    layer = tern_inputs.WORKLOADS[name][i]
    log(f"a8 workload {layer.name} m={layer.m} k={layer.k} n={layer.n}")
    x, w = tern_inputs.draw_layer(layer)
    full = layer.m * layer.n * layer.k <= 2 ** 26
    rows = edge_indices(layer.m, tile=144, extra=96, seed=layer.seed)
    cols = edge_indices(layer.n, extra=96, seed=layer.seed + 1)
    worst = check_layer_a8(x, w, layer.name, rows=rows, cols=cols, full=full,
                           repeat_check=layer.name == "flux_qkv")
    log(f"  ok, worst error / bound = {worst:.3f}")
