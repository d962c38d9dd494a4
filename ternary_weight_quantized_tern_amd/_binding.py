"""ctypes binding of libternary: argument marshalling only.

Each ``tern_*`` function here has the name of the C entry point declared in
``include/ternary.h`` and takes its tensors in the same order.  It checks that the torch
tensors it is given are on the GPU with the documented dtypes and unit column
stride, reads their device pointers, leading dimensions and the current HIP
stream, and calls the library.  All arithmetic runs in the library's kernels;
nothing here computes any part of the layer, and there is no fallback: if
``libternary.so`` is missing or cannot be loaded, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TERN_LIB", os.path.join(_PKG_DIR, "libternary.so"))

TERN_OK = 0
TERN_ERR_NULL = 1
TERN_ERR_SHAPE = 2
TERN_ERR_ALIGN = 3
TERN_ERR_STRIDE = 4
TERN_ERR_DTYPE = 5
TERN_ERR_HIP = 6
TERN_ERR_ARG = 7
TERN_ACT_NONE = 0
TERN_ACT_GELU_TANH = 1
TERN_F32 = 0
TERN_BF16 = 1
TERN_QUANTIZE_MAX_K = 32768

TERN_GEMM_DX_STATIC_MAX_ELEMS = 67108864

EXPORTED = ("tern_quantize", "tern_quantize_pack", "tern_pack", "tern_unpack", "tern_gemm",
            "tern_gemm_ex", "tern_pack_transposed", "tern_gemm_dx", "tern_gemm_dx_static",
            "tern_gemm_dw", "tern_quantize_act", "tern_pack_a8", "tern_gemm_a8",
            "tern_status_string")


class TernError(RuntimeError):
    """A libternary call returned a status other than TERN_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {tern_status_string(status)}")


def _load(path: str):
    if not os.path.exists(path):
        raise ImportError(
            f"libternary.so not found at {path}; build it with "
            "`python ternary_weight_quantized_tern_amd/build.py` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.tern_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, vp, vp]
    lib.tern_quantize_pack.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, vp, i64, vp, vp]
    lib.tern_pack.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    lib.tern_unpack.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    lib.tern_gemm.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, vp, i64, vp]
    lib.tern_gemm_ex.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, vp, ctypes.c_int, i64, vp,
                                 i64, vp]
    lib.tern_pack_transposed.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    lib.tern_gemm_dx.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, vp, i64, vp, i64, vp]
    lib.tern_gemm_dx_static.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, vp, i64, vp]
    lib.tern_gemm_dw.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, i64, ctypes.c_int, vp]
    lib.tern_quantize_act.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
    lib.tern_pack_a8.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    lib.tern_gemm_a8.argtypes = [vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, ctypes.c_int, i64,
                                 vp, i64, vp]
    for name in ("tern_quantize", "tern_quantize_pack", "tern_pack", "tern_unpack", "tern_gemm",
                 "tern_gemm_ex", "tern_pack_transposed", "tern_gemm_dx", "tern_gemm_dx_static",
                 "tern_gemm_dw", "tern_quantize_act", "tern_pack_a8", "tern_gemm_a8"):
        getattr(lib, name).restype = ctypes.c_int
    lib.tern_status_string.argtypes = [ctypes.c_int]
    lib.tern_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load(LIB_PATH)


def library():
    """The loaded ``ctypes.CDLL`` (for ABI tests)."""
    return _lib


def tern_status_string(status: int) -> str:
    return _lib.tern_status_string(int(status)).decode()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _mat(a: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(a, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if a.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor, got {a.device}")
    if a.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {a.dtype}, expected one of {dtypes}")
    if a.dim() != 2 or (a.shape[1] > 1 and a.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D row-major view (unit column stride)")
    if a.shape[0] > 1:
        return a.stride(0)
    # With a single row the leading dimension is never used to step between
    # rows; report the row length rounded up to 16 elements.
    return (a.shape[1] + 15) // 16 * 16


def _vec(a: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(a, torch.Tensor) or a.device.type != "cuda" or a.dtype != dtype:
        raise TypeError(f"{name} must be a GPU tensor of dtype {dtype}")
    if a.dim() != 1 or (a.numel() > 1 and a.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous 1-D tensor")


def _check(fn: str, status: int) -> None:
    if status != TERN_OK:
        raise TernError(fn, status)


def tern_quantize(w: torch.Tensor, t: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """Absmean-ternarize ``w`` [n, k] (fp32 or bf16) into ``t`` int8 [n, >=k] and ``s`` fp32 [n]."""
    ldw = _mat(w, "w", (torch.float32, torch.bfloat16))
    ldt = _mat(t, "t", (torch.int8,))
    _vec(s, "s", torch.float32)
    n, k = w.shape
    if t.shape[0] != n or t.shape[1] < k or s.shape[0] != n:
        raise ValueError("t must be [n, >=k] and s [n]")
    dt = TERN_F32 if w.dtype == torch.float32 else TERN_BF16
    _check("tern_quantize", _lib.tern_quantize(w.data_ptr(), dt, n, k, ldw, t.data_ptr(), ldt,
                                               s.data_ptr(), _stream(stream)))


def tern_quantize_pack(w: torch.Tensor, t, p: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """``tern_quantize`` and ``tern_pack`` of its result in one pass: ``w`` [n, k]
    (fp32 or bf16) -> ``p`` uint8 [n, >=ceil(k/4)], ``s`` fp32 [n], and ``t`` int8
    [n, >=k] unless ``t`` is None."""
    ldw = _mat(w, "w", (torch.float32, torch.bfloat16))
    ldp = _mat(p, "p", (torch.uint8,))
    _vec(s, "s", torch.float32)
    n, k = w.shape
    if p.shape[0] != n or p.shape[1] < (k + 3) // 4 or s.shape[0] != n:
        raise ValueError("p must be [n, >=ceil(k/4)] and s [n] for w [n, k]")
    t_ptr, ldt = None, 0
    if t is not None:
        ldt = _mat(t, "t", (torch.int8,))
        if t.shape[0] != n or t.shape[1] < k:
            raise ValueError("t must be [n, >=k]")
        t_ptr = t.data_ptr()
    dt = TERN_F32 if w.dtype == torch.float32 else TERN_BF16
    _check("tern_quantize_pack", _lib.tern_quantize_pack(w.data_ptr(), dt, n, k, ldw, t_ptr, ldt,
                                                         p.data_ptr(), ldp, s.data_ptr(),
                                                         _stream(stream)))


def tern_pack(t: torch.Tensor, p: torch.Tensor, k: int | None = None, stream=None) -> None:
    """Pack int8 ``t`` [n, k] into ``p`` uint8 [n, >=ceil(k/4)]."""
    ldt = _mat(t, "t", (torch.int8,))
    ldp = _mat(p, "p", (torch.uint8,))
    n = t.shape[0]
    k = t.shape[1] if k is None else int(k)
    if p.shape[0] != n or k > t.shape[1] or p.shape[1] < (k + 3) // 4:
        raise ValueError("p must be [n, >=ceil(k/4)] for t [n, k]")
    _check("tern_pack", _lib.tern_pack(t.data_ptr(), n, k, ldt, p.data_ptr(), ldp, _stream(stream)))


def tern_unpack(p: torch.Tensor, t: torch.Tensor, k: int | None = None, stream=None) -> None:
    """Unpack ``p`` uint8 [n, >=ceil(k/4)] into int8 ``t`` [n, >=k] (k defaults to t's width)."""
    ldp = _mat(p, "p", (torch.uint8,))
    ldt = _mat(t, "t", (torch.int8,))
    n = p.shape[0]
    k = t.shape[1] if k is None else int(k)
    if t.shape[0] != n or t.shape[1] < k or p.shape[1] < (k + 3) // 4:
        raise ValueError("t must be [n, >=k] and p [n, >=ceil(k/4)]")
    _check("tern_unpack", _lib.tern_unpack(p.data_ptr(), n, int(k), ldp, t.data_ptr(), ldt,
                                           _stream(stream)))


def tern_gemm(x: torch.Tensor, p: torch.Tensor, s: torch.Tensor, y: torch.Tensor,
              k: int | None = None, stream=None) -> None:
    """``y`` [m, n] bf16 = bf16((x [m, k] . T^T) * s), T decoded from ``p`` [n, >=k/4].

    k defaults to x's width.
    """
    ldx = _mat(x, "x", (torch.bfloat16,))
    ldp = _mat(p, "p", (torch.uint8,))
    ldy = _mat(y, "y", (torch.bfloat16,))
    _vec(s, "s", torch.float32)
    m = x.shape[0]
    k = x.shape[1] if k is None else int(k)
    n = p.shape[0]
    if k > x.shape[1] or p.shape[1] < k // 4 or s.shape[0] != n or tuple(y.shape[:1]) != (m,) \
            or y.shape[1] < n:
        raise ValueError("shapes must be x [m, k], p [n, >=k/4], s [n], y [m, >=n]")
    _check("tern_gemm", _lib.tern_gemm(x.data_ptr(), m, k, ldx, p.data_ptr(), n, ldp,
                                       s.data_ptr(), y.data_ptr(), ldy, _stream(stream)))


def tern_gemm_ex(x: torch.Tensor, p: torch.Tensor, s: torch.Tensor, y: torch.Tensor,
                 bias: torch.Tensor | None = None, act: int = TERN_ACT_NONE, act_from: int = 0,
                 k: int | None = None, stream=None) -> None:
    """``tern_gemm`` with a fused epilogue: ``y = bf16(f_n(x . T^T * s + bias))``,
    ``f_n`` the tanh-form GELU for columns ``n >= act_from`` when ``act`` is
    ``TERN_ACT_GELU_TANH``, else the identity; ``bias`` fp32 [n] or None."""
    ldx = _mat(x, "x", (torch.bfloat16,))
    ldp = _mat(p, "p", (torch.uint8,))
    ldy = _mat(y, "y", (torch.bfloat16,))
    _vec(s, "s", torch.float32)
    m = x.shape[0]
    k = x.shape[1] if k is None else int(k)
    n = p.shape[0]
    if k > x.shape[1] or p.shape[1] < k // 4 or s.shape[0] != n or tuple(y.shape[:1]) != (m,) \
            or y.shape[1] < n:
        raise ValueError("shapes must be x [m, k], p [n, >=k/4], s [n], y [m, >=n]")
    b_ptr = None
    if bias is not None:
        _vec(bias, "bias", torch.float32)
        if bias.shape[0] != n:
            raise ValueError("bias must be [n]")
        b_ptr = bias.data_ptr()
    _check("tern_gemm_ex", _lib.tern_gemm_ex(x.data_ptr(), m, k, ldx, p.data_ptr(), n, ldp,
                                             s.data_ptr(), b_ptr, int(act), int(act_from),
                                             y.data_ptr(), ldy, _stream(stream)))


def tern_pack_transposed(p: torch.Tensor, pt: torch.Tensor, n: int | None = None,
                         k: int | None = None, stream=None) -> None:
    """Re-pack the codes of ``p`` uint8 [n, >=ceil(k/4)] (packed along k) along n
    into ``pt`` uint8 [k, >=ceil(n/4)]; n defaults to p's rows, k to pt's rows."""
    ldp = _mat(p, "p", (torch.uint8,))
    ldpt = _mat(pt, "pt", (torch.uint8,))
    n = p.shape[0] if n is None else int(n)
    k = pt.shape[0] if k is None else int(k)
    if n > p.shape[0] or k > pt.shape[0] or p.shape[1] < (k + 3) // 4 or pt.shape[1] < (n + 3) // 4:
        raise ValueError("p must be [>=n, >=ceil(k/4)] and pt [>=k, >=ceil(n/4)]")
    _check("tern_pack_transposed",
           _lib.tern_pack_transposed(p.data_ptr(), n, k, ldp, pt.data_ptr(), ldpt, _stream(stream)))


def tern_gemm_dx(dy: torch.Tensor, pt: torch.Tensor, s: torch.Tensor, u: torch.Tensor,
                 dx: torch.Tensor, k: int | None = None, stream=None) -> None:
    """Input gradient of the layer: ``u = bf16(dy * s)`` into the workspace ``u``
    (bf16 [m, >=n]), then ``dx = bf16(u . T)`` with ``pt`` the codes packed
    along n (uint8 [k, >=n/4]); dy bf16 [m, n], s fp32 [n], dx bf16 [m, >=k]."""
    lddy = _mat(dy, "dy", (torch.bfloat16,))
    ldpt = _mat(pt, "pt", (torch.uint8,))
    ldu = _mat(u, "u", (torch.bfloat16,))
    lddx = _mat(dx, "dx", (torch.bfloat16,))
    _vec(s, "s", torch.float32)
    m, n = dy.shape
    k = pt.shape[0] if k is None else int(k)
    if (s.shape[0] != n or k > pt.shape[0] or pt.shape[1] < n // 4 or tuple(u.shape[:1]) != (m,)
            or u.shape[1] < n or tuple(dx.shape[:1]) != (m,) or dx.shape[1] < k):
        raise ValueError("shapes must be dy [m, n], pt [>=k, >=n/4], s [n], u [m, >=n], dx [m, >=k]")
    _check("tern_gemm_dx", _lib.tern_gemm_dx(dy.data_ptr(), m, n, lddy, pt.data_ptr(), k, ldpt,
                                             s.data_ptr(), u.data_ptr(), ldu, dx.data_ptr(), lddx,
                                             _stream(stream)))


def tern_gemm_dx_static(dy: torch.Tensor, pt: torch.Tensor, s: torch.Tensor, dx: torch.Tensor,
                        k: int | None = None, stream=None) -> None:
    """``tern_gemm_dx`` with the scaled gradient in the library's fixed device
    array instead of a caller workspace (m * n <= TERN_GEMM_DX_STATIC_MAX_ELEMS);
    calls that overlap in time on one GPU race on that array."""
    lddy = _mat(dy, "dy", (torch.bfloat16,))
    ldpt = _mat(pt, "pt", (torch.uint8,))
    lddx = _mat(dx, "dx", (torch.bfloat16,))
    _vec(s, "s", torch.float32)
    m, n = dy.shape
    k = pt.shape[0] if k is None else int(k)
    if (s.shape[0] != n or k > pt.shape[0] or pt.shape[1] < n // 4 or tuple(dx.shape[:1]) != (m,)
            or dx.shape[1] < k):
        raise ValueError("shapes must be dy [m, n], pt [>=k, >=n/4], s [n], dx [m, >=k]")
    _check("tern_gemm_dx_static",
           _lib.tern_gemm_dx_static(dy.data_ptr(), m, n, lddy, pt.data_ptr(), k, ldpt,
                                    s.data_ptr(), dx.data_ptr(), lddx, _stream(stream)))


def tern_gemm_dw(dy: torch.Tensor, x: torch.Tensor, dw: torch.Tensor, accumulate: bool = False,
                 stream=None) -> None:
    """Latent-weight gradient of the layer (straight-through reading):
    ``dw [n, >=k] fp32 (+)= dy^T . x`` with ``dy`` bf16 [m, n] and ``x`` bf16
    [m, k]; with ``accumulate`` the product is added into ``dw``."""
    lddy = _mat(dy, "dy", (torch.bfloat16,))
    ldx = _mat(x, "x", (torch.bfloat16,))
    lddw = _mat(dw, "dw", (torch.float32,))
    m, n = dy.shape
    mx, k = x.shape
    if mx != m or dw.shape[0] != n or dw.shape[1] < k:
        raise ValueError("shapes must be dy [m, n], x [m, k], dw [n, >=k]")
    _check("tern_gemm_dw", _lib.tern_gemm_dw(dy.data_ptr(), m, n, lddy, x.data_ptr(), k, ldx,
                                             dw.data_ptr(), lddw, 1 if accumulate else 0,
                                             _stream(stream)))


def tern_quantize_act(x: torch.Tensor, q: torch.Tensor, xs: torch.Tensor, k: int | None = None,
                      stream=None) -> None:
    """Per-token int8 activations of bf16 ``x`` [m, k]: codes into ``q`` int8
    [m, >=k], scales max|x|/127 into ``xs`` fp32 [m]."""
    ldx = _mat(x, "x", (torch.bfloat16,))
    ldq = _mat(q, "q", (torch.int8,))
    _vec(xs, "xs", torch.float32)
    m = x.shape[0]
    k = x.shape[1] if k is None else int(k)
    if k > x.shape[1] or tuple(q.shape[:1]) != (m,) or q.shape[1] < k or xs.shape[0] != m:
        raise ValueError("shapes must be x [m, k], q [m, >=k], xs [m]")
    _check("tern_quantize_act", _lib.tern_quantize_act(x.data_ptr(), m, k, ldx, q.data_ptr(), ldq,
                                                       xs.data_ptr(), _stream(stream)))


def tern_pack_a8(p: torch.Tensor, p8: torch.Tensor, k: int, n: int | None = None,
                 stream=None) -> None:
    """Arrange the codes of ``p`` uint8 [n, >=k/4] for the int8 GEMM into
    ``p8`` uint8 [n, >=k/4] (k % 16 == 0); ``p8`` may be ``p`` itself."""
    ldp = _mat(p, "p", (torch.uint8,))
    ldp8 = _mat(p8, "p8", (torch.uint8,))
    n = p.shape[0] if n is None else int(n)
    k = int(k)
    if n > p.shape[0] or n > p8.shape[0] or p.shape[1] < k // 4 or p8.shape[1] < k // 4:
        raise ValueError("p and p8 must be [>=n, >=k/4]")
    _check("tern_pack_a8", _lib.tern_pack_a8(p.data_ptr(), n, k, ldp, p8.data_ptr(), ldp8,
                                             _stream(stream)))


def tern_gemm_a8(q: torch.Tensor, xs: torch.Tensor, p8: torch.Tensor, s: torch.Tensor,
                 y: torch.Tensor, bias: torch.Tensor | None = None, act: int = TERN_ACT_NONE,
                 act_from: int = 0, k: int | None = None, stream=None) -> None:
    """The layer on int8 activations: ``y = bf16(f_n(s_n * xs_m * (q . T^T) +
    bias))`` with ``q`` int8 [m, k], ``xs`` fp32 [m], ``p8`` from tern_pack_a8,
    ``s`` fp32 [n], bias and act as ``tern_gemm_ex``."""
    ldq = _mat(q, "q", (torch.int8,))
    ldp8 = _mat(p8, "p8", (torch.uint8,))
    ldy = _mat(y, "y", (torch.bfloat16,))
    _vec(xs, "xs", torch.float32)
    _vec(s, "s", torch.float32)
    m = q.shape[0]
    k = q.shape[1] if k is None else int(k)
    n = p8.shape[0]
    if k > q.shape[1] or xs.shape[0] != m or p8.shape[1] < k // 4 or s.shape[0] != n \
            or tuple(y.shape[:1]) != (m,) or y.shape[1] < n:
        raise ValueError("shapes must be q [m, k], xs [m], p8 [n, >=k/4], s [n], y [m, >=n]")
    b_ptr = None
    if bias is not None:
        _vec(bias, "bias", torch.float32)
        if bias.shape[0] != n:
            raise ValueError("bias must be [n]")
        b_ptr = bias.data_ptr()
    _check("tern_gemm_a8", _lib.tern_gemm_a8(q.data_ptr(), m, k, ldq, xs.data_ptr(), p8.data_ptr(),
                                             n, ldp8, s.data_ptr(), b_ptr, int(act), int(act_from),
                                             y.data_ptr(), ldy, _stream(stream)))


# ---------------------------------------------------------------------------
# allocating conveniences (torch allocates the outputs; the library computes)
# ---------------------------------------------------------------------------

def quantize(w: torch.Tensor, stream=None):
    """Return ``(t, s)`` for full-precision weights ``w`` [n, k]."""
    n, k = w.shape
    t = torch.empty((n, k), dtype=torch.int8, device=w.device)
    s = torch.empty((n,), dtype=torch.float32, device=w.device)
    tern_quantize(w, t, s, stream)
    return t, s


def packed_row_bytes(k: int) -> int:
    """Row pitch used for packed weights: ceil(k/4) rounded up to 16 bytes."""
    return ((k + 3) // 4 + 15) // 16 * 16


def pack(t: torch.Tensor, stream=None) -> torch.Tensor:
    n, k = t.shape
    p = torch.zeros((n, packed_row_bytes(k)), dtype=torch.uint8, device=t.device)
    tern_pack(t, p, k, stream)
    return p


def quantize_pack(w: torch.Tensor, with_codes: bool = False, stream=None):
    """Full-precision weights ``w`` [n, k] -> ``(p, s)`` (packed codes and
    scales) in one pass, or ``(t, p, s)`` with the int8 codes as well."""
    n, k = w.shape
    p = torch.zeros((n, packed_row_bytes(k)), dtype=torch.uint8, device=w.device)
    s = torch.empty((n,), dtype=torch.float32, device=w.device)
    t = torch.empty((n, k), dtype=torch.int8, device=w.device) if with_codes else None
    tern_quantize_pack(w, t, p, s, stream)
    return (t, p, s) if with_codes else (p, s)


def unpack(p: torch.Tensor, k: int, stream=None) -> torch.Tensor:
    t = torch.empty((p.shape[0], k), dtype=torch.int8, device=p.device)
    tern_unpack(p, t, k, stream)
    return t


def linear(x: torch.Tensor, p: torch.Tensor, s: torch.Tensor, stream=None) -> torch.Tensor:
    """Ternary linear layer: bf16 ``x`` [m, k] -> bf16 [m, n]."""
    y = torch.empty((x.shape[0], p.shape[0]), dtype=torch.bfloat16, device=x.device)
    tern_gemm(x, p, s, y, None, stream)
    return y


def linear_ex(x: torch.Tensor, p: torch.Tensor, s: torch.Tensor, bias: torch.Tensor | None = None,
              gelu_from: int | None = None, stream=None) -> torch.Tensor:
    """The layer with a fused epilogue: plus ``bias`` (fp32 [n]) if given, then
    the tanh-form GELU on output columns ``>= gelu_from`` if given."""
    y = torch.empty((x.shape[0], p.shape[0]), dtype=torch.bfloat16, device=x.device)
    act = TERN_ACT_NONE if gelu_from is None else TERN_ACT_GELU_TANH
    tern_gemm_ex(x, p, s, y, bias, act, 0 if gelu_from is None else int(gelu_from), None, stream)
    return y


def pack_transposed(p: torch.Tensor, n: int, k: int, stream=None) -> torch.Tensor:
    """The codes of packed weights ``p`` (n rows, row length k) packed along n:
    uint8 [k, ceil(n/4) rounded up to 16]."""
    pt = torch.zeros((k, packed_row_bytes(n)), dtype=torch.uint8, device=p.device)
    tern_pack_transposed(p, pt, n, k, stream)
    return pt


def linear_dx(dy: torch.Tensor, pt: torch.Tensor, s: torch.Tensor, k: int, stream=None):
    """Input gradient ``bf16((dy * s) . T)`` [m, k] of the layer; ``pt`` from
    pack_transposed.  Allocates the bf16 workspace for the scaled gradient."""
    u = torch.empty_like(dy, memory_format=torch.contiguous_format)
    dx = torch.empty((dy.shape[0], k), dtype=torch.bfloat16, device=dy.device)
    tern_gemm_dx(dy, pt, s, u, dx, k, stream)
    return dx


def linear_dw(dy: torch.Tensor, x: torch.Tensor, stream=None) -> torch.Tensor:
    """Latent-weight gradient ``dy^T . x`` (fp32 [n, k]) of the layer for bf16
    ``dy`` [m, n] and ``x`` [m, k] (straight-through reading)."""
    dw = torch.empty((dy.shape[1], x.shape[1]), dtype=torch.float32, device=dy.device)
    tern_gemm_dw(dy, x, dw, False, stream)
    return dw


def quantize_act(x: torch.Tensor, stream=None):
    """Return ``(q, xs)``: int8 codes [m, k] (rows 16-byte aligned) and fp32
    per-token scales [m] of bf16 activations ``x`` [m, k]."""
    m, k = x.shape
    q = torch.empty((m, (k + 15) // 16 * 16), dtype=torch.int8, device=x.device)[:, :k]
    xs = torch.empty((m,), dtype=torch.float32, device=x.device)
    tern_quantize_act(x, q, xs, None, stream)
    return q, xs


def pack_a8(p: torch.Tensor, k: int, stream=None) -> torch.Tensor:
    """Packed weights ``p`` (row length k) arranged for the int8 GEMM (same shape)."""
    p8 = torch.zeros_like(p)
    tern_pack_a8(p, p8, k, None, stream)
    return p8


def linear_a8(x: torch.Tensor, p8: torch.Tensor, s: torch.Tensor, bias: torch.Tensor | None = None,
              gelu_from: int | None = None, stream=None) -> torch.Tensor:
    """The layer with 8-bit activations: bf16 ``x`` [m, k] quantized per token,
    then the int8 GEMM with ``p8`` from pack_a8 (and the optional fused bias and
    GELU of linear_ex).  Returns bf16 [m, n]."""
    q, xs = quantize_act(x, stream)
    y = torch.empty((x.shape[0], p8.shape[0]), dtype=torch.bfloat16, device=x.device)
    act = TERN_ACT_NONE if gelu_from is None else TERN_ACT_GELU_TANH
    tern_gemm_a8(q, xs, p8, s, y, bias, act, 0 if gelu_from is None else int(gelu_from), None,
                 stream)
    return y
