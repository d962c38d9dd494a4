"""Seeded synthetic inputs for the 1.58-bit linear layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark, so it holds no arithmetic of the method itself: it only draws
activations and full-precision weights and lists the layer shapes.

Recipe (one linear layer):
  * one ``torch.Generator`` on the CPU, ``manual_seed(seed)``;
  * activations first: X fp32 [M, K] ~ N(0, 1), or Student-t with 3 degrees of
    freedom built as Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from the same
    generator; then cast to bf16 (round to nearest even);
  * weights second: W fp32 [N, K] ~ N(0, 0.02^2).

The shapes stand in for the linear layers of a FLUX-style vision transformer
(hidden size 3072, 4096 image + 512 text tokens for one 1024x1024 image) and of
a small DiT (hidden size 1152), the workloads that "1.58-bit FLUX" (Table 3 and
section 3.1 Settings) and "TerDiT" (abstract) describe.  No dataset items or
trained weights are used.
"""
from __future__ import annotations

import dataclasses
from typing import Iterator, List

import numpy as np
import torch

W_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Linear:
    """One ternary linear layer: X [m, k] times ternary W [n, k]^T."""
    name: str
    m: int
    k: int
    n: int
    seed: int
    x_dist: str = "normal"  # "normal" or "student_t3"


def _layers_config3() -> List[Linear]:
    out = []
    for layer in range(38):
        out.append(Linear(f"single_stream{layer}.in_proj", 4608, 3072, 21504, 3000 + 2 * layer))
        out.append(Linear(f"single_stream{layer}.out_proj", 4608, 15360, 3072, 3000 + 2 * layer + 1))
    return out


# Workload table.  Seeds: 0 for the single small layer, else 1000*i + j for the
# j-th linear of workload i in the order listed.
WORKLOADS = {
    "single": [Linear("single", 16, 256, 512, 0)],
    "flux_qkv": [Linear("flux_qkv", 4608, 3072, 9216, 1000)],
    "flux_mlp": [Linear("flux_mlp.up", 4608, 3072, 12288, 2000),
                 Linear("flux_mlp.down", 4608, 12288, 3072, 2001)],
    "flux_single_stream": _layers_config3(),
    "dit": [Linear("dit.up.m2048", 2048, 1152, 4608, 4000, "student_t3"),
            Linear("dit.down.m2048", 2048, 4608, 1152, 4001, "student_t3"),
            Linear("dit.up.m8", 8, 1152, 4608, 4002, "student_t3"),
            Linear("dit.down.m8", 8, 4608, 1152, 4003, "student_t3")],
}
WORKLOAD_ORDER = ["single", "flux_qkv", "flux_mlp", "flux_single_stream", "dit"]


def draw(m: int, k: int, n: int, seed: int, x_dist: str = "normal", w_dtype=torch.float32):
    """Return ``(x_bf16 [m,k], w [n,k])`` as CPU tensors, drawn X first then W."""
    g = torch.Generator().manual_seed(int(seed))
    if x_dist == "normal":
        x = torch.randn(m, k, generator=g, dtype=torch.float32)
    elif x_dist == "student_t3":
        z = torch.randn(m, k, generator=g, dtype=torch.float32)
        c = torch.zeros(m, k, dtype=torch.float32)
        for _ in range(3):
            zi = torch.randn(m, k, generator=g, dtype=torch.float32)
            c += zi * zi
        x = z / torch.sqrt(c / 3.0)
    else:
        raise ValueError(f"unknown activation distribution {x_dist!r}")
    x = x.to(torch.bfloat16)
    w = torch.randn(n, k, generator=g, dtype=torch.float32) * W_STD
    if w_dtype != torch.float32:
        w = w.to(w_dtype)
    return x, w


def draw_layer(layer: Linear, w_dtype=torch.float32):
    return draw(layer.m, layer.k, layer.n, layer.seed, layer.x_dist, w_dtype)


def iter_layers(workload: str) -> Iterator[Linear]:
    return iter(WORKLOADS[workload])


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """bf16 CPU tensor -> numpy uint16 array of its bit patterns."""
    assert x.dtype == torch.bfloat16
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def random_ternary(n: int, k: int, seed: int, p_zero: float = 1.0 / 3.0) -> torch.Tensor:
    """A seeded int8 [n, k] array over {-1, 0, +1} (for pack/unpack tests)."""
    g = torch.Generator().manual_seed(int(seed))
    u = torch.rand(n, k, generator=g)
    sign = torch.where(torch.rand(n, k, generator=g) < 0.5, -1, 1).to(torch.int8)
    return torch.where(u < p_zero, torch.zeros_like(sign), sign)
