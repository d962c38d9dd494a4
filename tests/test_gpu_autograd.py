"""GPU parity of the straight-through autograd wrapper (ternary_linear) against
the CPU oracle: the forward output is the tern_gemm result on the weights
quantized and packed on the GPU (bit for bit), the input gradient meets the
tern_gemm_dx bar against the oracle's (dY * s) . T, and the latent-weight
gradient the tern_gemm_dw bar against the oracle's dY^T . X.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tern_inputs
from parity import (DEV, assert_within_tolerance, bf16_to_f64, draw_grad, log, oracle_weights,
                    row_norms)
from test_gpu_dw import check as check_dw

pytestmark = pytest.mark.gpu
tern = pytest.importorskip("ternary_weight_quantized_tern_amd")


@pytest.mark.parametrize("m,k,n", [(40, 128, 192), (300, 256, 128), (8, 192, 320),
                                   (2048, 1152, 256)])
def test_ternary_linear_forward_and_straight_through_gradients(m, k, n):
    log(f"ternary_linear m={m} k={k} n={n}")
    x, w = tern_inputs.draw(m, k, n, seed=m + 3 * k + 7 * n)
    dy = draw_grad(m, n, seed=m + k + n)
    xg = x.to(DEV).requires_grad_()
    wg = w.to(DEV).requires_grad_()
    y = tern.ternary_linear(xg, wg)
    y.backward(dy.to(DEV))
    torch.cuda.synchronize()

    p, s = tern.quantize_pack(w.to(DEV))
    y_ref = tern.linear(x.to(DEV), p, s)
    assert torch.equal(y.detach().view(torch.int16), y_ref.view(torch.int16))

    _, s_ref, p_ref = oracle_weights(w)
    dyb = tern_inputs.bf16_bits(dy)
    u_ref = oracle.oracle_scale_grad(dyb, s_ref)
    dx_ref = oracle.oracle_gemm_dx(u_ref, p_ref, k)
    assert xg.grad.dtype == torch.bfloat16
    assert_within_tolerance(bf16_to_f64(xg.grad), dx_ref, np.ones(k, np.float32),
                            row_norms(u_ref), f"dx {m}x{k}x{n}")
    assert wg.grad.dtype == torch.float32 and tuple(wg.grad.shape) == (n, k)
    check_dw(wg.grad.cpu().numpy(), dy, x, f"dw {m}x{k}x{n}")


def test_ternary_linear_gradient_of_one_input_only():
    m, k, n = 64, 128, 128
    x, w = tern_inputs.draw(m, k, n, seed=5)
    dy = draw_grad(m, n, seed=6).to(DEV)
    xg, wg = x.to(DEV), w.to(DEV).requires_grad_()
    tern.ternary_linear(xg, wg).backward(dy)
    assert xg.grad is None and wg.grad is not None
    xg2, wg2 = x.to(DEV).requires_grad_(), w.to(DEV)
    tern.ternary_linear(xg2, wg2).backward(dy)
    assert wg2.grad is None and xg2.grad is not None
    torch.cuda.synchronize()
    assert torch.equal(wg.grad, tern.linear_dw(dy, x.to(DEV)))


def test_ternary_linear_bf16_latent_weights():
    m, k, n = 32, 64, 64
    x, w = tern_inputs.draw(m, k, n, seed=9)
    wb = w.to(torch.bfloat16).to(DEV).requires_grad_()
    dy = draw_grad(m, n, seed=10).to(DEV)
    y = tern.ternary_linear(x.to(DEV), wb)
    y.backward(dy)
    torch.cuda.synchronize()
    assert wb.grad.dtype == torch.bfloat16
    dw32 = tern.linear_dw(dy, x.to(DEV))
    assert torch.equal(wb.grad, dw32.to(torch.bfloat16))
    p, s = tern.quantize_pack(wb.detach())
    assert torch.equal(y.detach().view(torch.int16), tern.linear(x.to(DEV), p, s).view(torch.int16))
