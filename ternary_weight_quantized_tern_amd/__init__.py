"""libternary: the 1.58-bit (ternary-weight) linear layer on AMD MI355X (gfx950).

The compute lives in ``libternary.so`` (hand-written HIP kernels behind the C
ABI of ``include/ternary.h``); this package is its ctypes binding.  Importing it
fails if the library has not been built: there is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    TERN_ACT_GELU_TANH,
    TERN_ACT_NONE,
    TERN_BF16,
    TERN_ERR_ALIGN,
    TERN_ERR_ARG,
    TERN_ERR_DTYPE,
    TERN_ERR_HIP,
    TERN_ERR_NULL,
    TERN_ERR_SHAPE,
    TERN_ERR_STRIDE,
    TERN_F32,
    TERN_OK,
    TERN_QUANTIZE_MAX_K,
    TernError,
    library,
    linear,
    linear_dx,
    linear_ex,
    pack,
    pack_transposed,
    packed_row_bytes,
    quantize,
    quantize_pack,
    tern_gemm,
    tern_gemm_dx,
    tern_gemm_ex,
    tern_pack,
    tern_pack_transposed,
    tern_quantize,
    tern_quantize_pack,
    tern_status_string,
    tern_unpack,
    unpack,
)
