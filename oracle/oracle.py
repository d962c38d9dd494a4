"""ctypes front end of the C oracle in ``oracle.c`` (test infrastructure only).

The C source is compiled with gcc at -O2, without fast-math, into
``liboracle.so`` next to it, on first use or whenever the source is newer than
the library.  Arguments are numpy arrays in host memory; the wrappers only
check shapes and pass pointers.  What each function computes, and the reading
of the pages behind it, is documented in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math) and return its path."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out))
    os.close(fd)
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-pthread", "-o", tmp, src, "-lm"]
    try:
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        os.replace(tmp, out)
    except subprocess.CalledProcessError as e:
        os.unlink(tmp)
        raise RuntimeError(f"oracle build failed:\n{e.stderr}") from e
    return out


def load(path: str | None = None):
    """Load (building first if needed) and type the oracle's entry points."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    lib = ctypes.CDLL(path or build())
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, vp]
    lib.oracle_pack.argtypes = [vp, i64, i64, i64, vp, i64]
    lib.oracle_unpack.argtypes = [vp, i64, i64, i64, vp, i64]
    lib.oracle_gemm.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, vp, i64, ctypes.c_int]
    lib.oracle_epilogue.argtypes = [vp, i64, i64, i64, vp, ctypes.c_int, i64]
    lib.oracle_scale_grad.argtypes = [vp, i64, i64, i64, vp, vp, i64]
    lib.oracle_gemm_dx.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, i64, ctypes.c_int]
    lib.oracle_quantize_act.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    lib.oracle_gemm_a8.argtypes = [vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, i64]
    lib.oracle_pack_a8.argtypes = [vp, i64, i64, i64, vp, i64]
    lib.oracle_gemm_dw.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, i64, ctypes.c_int]
    for f in (lib.oracle_quantize, lib.oracle_pack, lib.oracle_unpack, lib.oracle_gemm,
              lib.oracle_epilogue, lib.oracle_scale_grad, lib.oracle_gemm_dx,
              lib.oracle_quantize_act, lib.oracle_gemm_a8, lib.oracle_pack_a8,
              lib.oracle_gemm_dw):
        f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"{name}: bad arguments (oracle returned {rc})")


def oracle_quantize(w: np.ndarray, lib=None):
    """Absmean-ternarize each row of ``w`` (float32, or bf16 given as uint16 bits).

    Returns ``(t, s)``: int8 ``[N, K]`` in {-1, 0, 1} and float32 ``[N]``.
    """
    lib = lib or load()
    w = np.ascontiguousarray(w)
    if w.dtype == np.float32:
        dt = 0
    elif w.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("w must be float32 or bf16 bits as uint16")
    n, k = w.shape
    t = np.empty((n, k), np.int8)
    s = np.empty((n,), np.float32)
    _check(lib.oracle_quantize(_ptr(w), dt, n, k, k, _ptr(t), k, _ptr(s)), "oracle_quantize")
    return t, s


def oracle_pack(t: np.ndarray, lib=None) -> np.ndarray:
    """Pack int8 ``[N, K]`` into uint8 ``[N, ceil(K/4)]`` (2-bit codes, LSB first)."""
    lib = lib or load()
    t = np.ascontiguousarray(t, dtype=np.int8)
    n, k = t.shape
    nb = (k + 3) // 4
    p = np.empty((n, nb), np.uint8)
    _check(lib.oracle_pack(_ptr(t), n, k, k, _ptr(p), nb), "oracle_pack")
    return p


def oracle_unpack(p: np.ndarray, k: int, lib=None) -> np.ndarray:
    """Unpack uint8 ``[N, >=ceil(K/4)]`` into int8 ``[N, K]`` (sign-extended 2-bit codes)."""
    lib = lib or load()
    p = np.ascontiguousarray(p, dtype=np.uint8)
    n, ldp = p.shape
    t = np.empty((n, k), np.int8)
    _check(lib.oracle_unpack(_ptr(p), n, k, ldp, _ptr(t), k), "oracle_unpack")
    return t


def oracle_gemm(x_bf16_bits: np.ndarray, p: np.ndarray, s: np.ndarray, k: int | None = None,
                nthreads: int | None = None, lib=None) -> np.ndarray:
    """Unrounded layer output ``y = s_n * sum_k x[m,k] * T[n,k]`` in float64 ``[M, N]``.

    ``x_bf16_bits`` holds the bf16 activations as uint16 bit patterns ``[M, K]``.
    """
    lib = lib or load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    p = np.ascontiguousarray(p, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    m, kx = x.shape
    k = kx if k is None else k
    n, ldp = p.shape
    if s.shape != (n,):
        raise ValueError("s must have one entry per weight row")
    y = np.empty((m, n), np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    _check(lib.oracle_gemm(_ptr(x), m, k, kx, _ptr(p), n, ldp, _ptr(s), _ptr(y), n, nthreads),
           "oracle_gemm")
    return y


ACT_NONE = 0
ACT_GELU_TANH = 1


def oracle_epilogue(y: np.ndarray, bias: np.ndarray | None = None, act: int = ACT_NONE,
                    act_from: int = 0, lib=None) -> np.ndarray:
    """Bias and activation on an unrounded layer output (float64 ``[M, N]``):
    ``f_n(y + b_n)`` with ``f_n`` the tanh-form GELU for ``n >= act_from`` when
    ``act`` is ``ACT_GELU_TANH``, else the identity.  Returns a new array."""
    lib = lib or load()
    out = np.array(y, dtype=np.float64, order="C", copy=True)
    m, n = out.shape
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
        if b.shape != (n,):
            raise ValueError("bias must have one entry per output column")
    _check(lib.oracle_epilogue(_ptr(out), m, n, n, None if b is None else _ptr(b), int(act),
                               int(act_from)), "oracle_epilogue")
    return out


def oracle_pack_transposed(p: np.ndarray, n: int, k: int, lib=None) -> np.ndarray:
    """The codes of packed weights ``p`` (rows n, packed along k) packed along n
    instead: uint8 ``[K, ceil(N/4)]`` whose row k holds T[0..N-1, k]."""
    t = oracle_unpack(np.ascontiguousarray(p)[:n], k, lib=lib)
    return oracle_pack(np.ascontiguousarray(t.T), lib=lib)


def oracle_scale_grad(dy_bf16_bits: np.ndarray, s: np.ndarray, lib=None) -> np.ndarray:
    """``u = bf16(fp32(dy) * s_n)`` (single-precision product, then round to
    nearest even) as uint16 bf16 bit patterns ``[M, N]``."""
    lib = lib or load()
    dy = np.ascontiguousarray(dy_bf16_bits, dtype=np.uint16)
    s = np.ascontiguousarray(s, dtype=np.float32)
    m, n = dy.shape
    if s.shape != (n,):
        raise ValueError("s must have one entry per gradient column")
    u = np.empty((m, n), np.uint16)
    _check(lib.oracle_scale_grad(_ptr(dy), m, n, n, _ptr(s), _ptr(u), n), "oracle_scale_grad")
    return u


def oracle_gemm_dx(u_bf16_bits: np.ndarray, p: np.ndarray, k: int, n: int | None = None,
                   nthreads: int | None = None, lib=None) -> np.ndarray:
    """Unrounded input gradient ``dx[m,k] = sum_n u[m,n] * T[n,k]`` in float64
    ``[M, K]``; ``p`` the forward's packed weights (rows n, packed along k)."""
    lib = lib or load()
    u = np.ascontiguousarray(u_bf16_bits, dtype=np.uint16)
    p = np.ascontiguousarray(p, dtype=np.uint8)
    m, nu = u.shape
    n = nu if n is None else n
    if p.shape[0] < n:
        raise ValueError("p must have a row per gradient column")
    ldp = p.shape[1]
    dx = np.empty((m, k), np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    _check(lib.oracle_gemm_dx(_ptr(u), m, n, nu, _ptr(p), k, ldp, _ptr(dx), k, nthreads),
           "oracle_gemm_dx")
    return dx


def oracle_quantize_act(x_bf16_bits: np.ndarray, lib=None):
    """Per-token absmax int8 activations: ``(q int8 [M, K], xs float32 [M])``."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    xs = np.empty((m,), np.float32)
    _check(lib.oracle_quantize_act(_ptr(x), m, k, k, _ptr(q), k, _ptr(xs)), "oracle_quantize_act")
    return q, xs


def oracle_gemm_a8(q: np.ndarray, xs: np.ndarray, p: np.ndarray, s: np.ndarray, lib=None):
    """Unrounded 8-bit-activation layer ``s_n * xs_m * sum_k q[m,k] T[n,k]``
    in float64 ``[M, N]`` (the integer sum exact)."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    p = np.ascontiguousarray(p, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    m, k = q.shape
    n, ldp = p.shape
    y = np.empty((m, n), np.float64)
    _check(lib.oracle_gemm_a8(_ptr(q), m, k, k, _ptr(xs), _ptr(p), n, ldp, _ptr(s), _ptr(y), n),
           "oracle_gemm_a8")
    return y


def oracle_pack_a8(p: np.ndarray, k: int, lib=None) -> np.ndarray:
    """Field-transposed packing of the codes of ``p`` (row length k, a
    multiple of 16): ``[N, k / 4]`` uint8."""
    lib = lib or load()
    p = np.ascontiguousarray(p, dtype=np.uint8)
    n, ldp = p.shape
    nb = k // 4
    out = np.empty((n, nb), np.uint8)
    _check(lib.oracle_pack_a8(_ptr(p), n, k, ldp, _ptr(out), nb), "oracle_pack_a8")
    return out


def oracle_gemm_dw(dy_bf16_bits: np.ndarray, x_bf16_bits: np.ndarray,
                   nthreads: int | None = None, lib=None) -> np.ndarray:
    """Unrounded latent-weight gradient ``dw[n,k] = sum_m dy[m,n] * x[m,k]`` in
    float64 ``[N, K]`` (straight-through reading); ``dy`` ``[M, N]`` and ``x``
    ``[M, K]`` as bf16 bit patterns."""
    lib = lib or load()
    dy = np.ascontiguousarray(dy_bf16_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    m, n = dy.shape
    mx, k = x.shape
    if mx != m:
        raise ValueError("dy and x must have the same number of rows (tokens)")
    dw = np.empty((n, k), np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    _check(lib.oracle_gemm_dw(_ptr(dy), m, n, n, _ptr(x), k, k, _ptr(dw), k, nthreads),
           "oracle_gemm_dw")
    return dw
