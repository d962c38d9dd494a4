"""The ternary linear layer as a torch autograd function, for training the
latent full-precision weights in the loop (quantization-aware training as in
"TerDiT: Ternary Diffusion Models with Transformers", abstract).

Forward: the latent weights w [n, k] (fp32 or bf16) are ternarized and packed
(tern_quantize_pack) and the layer runs on the packed codes (tern_gemm):
Y = bf16((X . T^T) * s).  Backward, with the straight-through reading of the
quantizer (its gradient passed unchanged to w): the input gradient
dX = bf16((dY * s) . T) (tern_pack_transposed + tern_gemm_dx) and the
latent-weight gradient dW = dY^T . X in fp32 (tern_gemm_dw).  Every step is a
libternary entry point; this module only marshals the tensors.
"""
from __future__ import annotations

import torch

from . import _binding as _b


class TernaryLinearFunction(torch.autograd.Function):
    """Y = TernaryLinear(X, W): X bf16 [m, k], W fp32 or bf16 [n, k] (the
    latent weights).  k must be a multiple of 64 (tern_gemm) and n a multiple of
    64 when the input gradient is needed (tern_gemm_dx).  The gradient of W has
    W's dtype from an fp32 product; the gradient of X is bf16."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
        n, k = w.shape
        p, s = _b.quantize_pack(w.detach())
        y = _b.linear(x.detach(), p, s)
        ctx.save_for_backward(x.detach(), p, s)
        ctx.nk = (n, k)
        ctx.w_dtype = w.dtype
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, p, s = ctx.saved_tensors
        n, k = ctx.nk
        dy = dy.to(torch.bfloat16).contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0]:
            pt = _b.pack_transposed(p, n, k)
            dx = _b.linear_dx(dy, pt, s, k)
        if ctx.needs_input_grad[1]:
            dw = _b.linear_dw(dy, x.contiguous())
            if ctx.w_dtype != torch.float32:
                dw = dw.to(ctx.w_dtype)
        return dx, dw


def ternary_linear(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """The ternary linear layer with straight-through gradients (see
    TernaryLinearFunction)."""
    return TernaryLinearFunction.apply(x, w)
