"""CPU oracle for the 1.58-bit linear layer (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does.
"""
from .oracle import (  # noqa: F401
    ACT_GELU_TANH,
    ACT_NONE,
    build,
    library_path,
    oracle_epilogue,
    oracle_gemm,
    oracle_gemm_a8,
    oracle_gemm_dw,
    oracle_gemm_dx,
    oracle_pack,
    oracle_pack_a8,
    oracle_pack_transposed,
    oracle_quantize,
    oracle_quantize_act,
    oracle_scale_grad,
    oracle_unpack,
)
