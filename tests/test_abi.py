"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

The library must load, export every function ``include/ternary.h`` declares,
and reject bad arguments with the documented status before touching the GPU.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ternary.h")

tern = pytest.importorskip("ternary_weight_quantized_tern_amd",
                           reason="libternary.so not built")
lib = tern.library()


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tern_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(tern.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", tern.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tern_[a-z0-9_]+)\b", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c_and_matches_enum_values(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(
        '#include "ternary.h"\n#include <stdio.h>\n'
        "int main(void){printf(\"%d %d %d %d %d %d %d %d %d %d\\n\", TERN_OK, TERN_ERR_NULL,"
        " TERN_ERR_SHAPE, TERN_ERR_ALIGN, TERN_ERR_STRIDE, TERN_ERR_DTYPE, TERN_ERR_HIP,"
        " TERN_F32, TERN_BF16, TERN_QUANTIZE_MAX_K); return 0;}\n")
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}",
                    str(src), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals == [tern.TERN_OK, tern.TERN_ERR_NULL, tern.TERN_ERR_SHAPE, tern.TERN_ERR_ALIGN,
                    tern.TERN_ERR_STRIDE, tern.TERN_ERR_DTYPE, tern.TERN_ERR_HIP, tern.TERN_F32,
                    tern.TERN_BF16, tern.TERN_QUANTIZE_MAX_K]


def test_status_strings():
    seen = set()
    for code in range(8):
        sstr = tern.tern_status_string(code)
        assert sstr and sstr not in seen
        seen.add(sstr)
    assert "unknown" in tern.tern_status_string(99)


# Fake but well-aligned, non-null device addresses: every call below is
# rejected (or is a no-op) during host validation, so nothing is dereferenced
# and no HIP call is made.
A = 1 << 20
NULL = None


def test_quantize_validation():
    q = lib.tern_quantize
    assert q(A, 7, 4, 64, 64, A, 64, A, NULL) == tern.TERN_ERR_DTYPE
    assert q(A, 0, -1, 64, 64, A, 64, A, NULL) == tern.TERN_ERR_SHAPE
    assert q(A, 0, 4, 32769, 32769, A, 32769, A, NULL) == tern.TERN_ERR_SHAPE
    assert q(A, 0, 4, 0, 64, A, 64, A, NULL) == tern.TERN_ERR_SHAPE
    assert q(NULL, 0, 0, 64, 64, NULL, 64, NULL, NULL) == tern.TERN_OK   # n == 0: no-op
    assert q(NULL, 0, 4, 64, 64, A, 64, A, NULL) == tern.TERN_ERR_NULL
    assert q(A, 0, 4, 64, 64, NULL, 64, A, NULL) == tern.TERN_ERR_NULL
    assert q(A, 0, 4, 64, 64, A, 64, NULL, NULL) == tern.TERN_ERR_NULL
    assert q(A, 0, 4, 64, 63, A, 64, A, NULL) == tern.TERN_ERR_STRIDE
    assert q(A, 0, 4, 64, 64, A, 63, A, NULL) == tern.TERN_ERR_STRIDE
    assert q(A + 2, 0, 4, 64, 64, A, 64, A, NULL) == tern.TERN_ERR_ALIGN  # fp32 needs 4 bytes
    assert q(A, 0, 4, 64, 64, A, 64, A + 1, NULL) == tern.TERN_ERR_ALIGN


def test_quantize_pack_validation():
    q = lib.tern_quantize_pack

    def call(w=A, dt=0, n=4, k=64, ldw=64, t=A, ldt=64, p=A, ldp=16, s=A):
        return q(w, dt, n, k, ldw, t, ldt, p, ldp, s, NULL)

    assert call(dt=7) == tern.TERN_ERR_DTYPE
    assert call(n=-1) == tern.TERN_ERR_SHAPE
    assert call(k=32769, ldw=32769, ldt=32769, ldp=8193) == tern.TERN_ERR_SHAPE
    assert call(k=0) == tern.TERN_ERR_SHAPE
    assert call(n=0, w=NULL, t=NULL, p=NULL, s=NULL) == tern.TERN_OK   # n == 0: no-op
    for name in ("w", "p", "s"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(ldw=63) == tern.TERN_ERR_STRIDE
    assert call(ldt=63) == tern.TERN_ERR_STRIDE
    # t NULL: ldt is ignored (strides are checked before alignment, so a
    # rejected alignment shows that ldt = 0 passed)
    assert call(t=NULL, ldt=0, s=A + 1) == tern.TERN_ERR_ALIGN
    assert call(ldp=15) == tern.TERN_ERR_STRIDE                  # < ceil(k/4)
    assert call(k=65, ldw=65, ldt=65, ldp=16) == tern.TERN_ERR_STRIDE
    assert call(w=A + 2) == tern.TERN_ERR_ALIGN                  # fp32 needs 4 bytes
    assert call(s=A + 1) == tern.TERN_ERR_ALIGN


def test_pack_unpack_validation():
    for fn in (lib.tern_pack, lib.tern_unpack):
        assert fn(A, -1, 8, 8, A, 2, NULL) == tern.TERN_ERR_SHAPE
        assert fn(A, 3, -8, 8, A, 2, NULL) == tern.TERN_ERR_SHAPE
        assert fn(NULL, 0, 8, 8, NULL, 2, NULL) == tern.TERN_OK
        assert fn(NULL, 3, 0, 8, NULL, 2, NULL) == tern.TERN_OK
        assert fn(NULL, 3, 8, 8, A, 8, NULL) == tern.TERN_ERR_NULL
        assert fn(A, 3, 8, 8, NULL, 8, NULL) == tern.TERN_ERR_NULL
    assert lib.tern_pack(A, 3, 9, 8, A, 3, NULL) == tern.TERN_ERR_STRIDE     # ldt < k
    assert lib.tern_pack(A, 3, 9, 9, A, 2, NULL) == tern.TERN_ERR_STRIDE     # ldp < ceil(k/4)
    assert lib.tern_unpack(A, 3, 9, 2, A, 9, NULL) == tern.TERN_ERR_STRIDE
    assert lib.tern_unpack(A, 3, 9, 3, A, 8, NULL) == tern.TERN_ERR_STRIDE


def test_gemm_validation():
    g = lib.tern_gemm
    ok = dict(x=A, m=8, k=128, ldx=128, p=A, n=16, ldp=32, s=A, y=A, ldy=16)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["x"], a["m"], a["k"], a["ldx"], a["p"], a["n"], a["ldp"], a["s"], a["y"],
                 a["ldy"], NULL)

    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(k=100, ldx=128) == tern.TERN_ERR_SHAPE        # k % 64 != 0
    assert call(n=2 ** 31) == tern.TERN_ERR_SHAPE
    assert call(m=2 ** 30, n=2 ** 20, ldy=2 ** 20) == tern.TERN_ERR_SHAPE  # 2^24 * 2^13 tiles
    assert call(m=0, x=NULL, p=NULL, s=NULL, y=NULL) == tern.TERN_OK
    assert call(n=0, x=NULL, p=NULL, s=NULL, y=NULL) == tern.TERN_OK
    for name in ("x", "p", "s", "y"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(ldx=120) == tern.TERN_ERR_STRIDE
    assert call(ldp=16) == tern.TERN_ERR_STRIDE                # < k/4
    assert call(ldy=15) == tern.TERN_ERR_STRIDE
    assert call(ldx=1 << 23) == tern.TERN_ERR_STRIDE           # beyond 32-bit block offsets
    assert call(ldp=1 << 24) == tern.TERN_ERR_STRIDE
    assert call(x=A + 8) == tern.TERN_ERR_ALIGN
    assert call(p=A + 4) == tern.TERN_ERR_ALIGN
    assert call(ldx=132) == tern.TERN_ERR_ALIGN
    assert call(ldp=40) == tern.TERN_ERR_ALIGN
    assert call(y=A + 1) == tern.TERN_ERR_ALIGN
    assert call(s=A + 2) == tern.TERN_ERR_ALIGN


def test_gemm_ex_validation():
    g = lib.tern_gemm_ex
    ok = dict(x=A, m=8, k=128, ldx=128, p=A, n=16, ldp=32, s=A, b=A, act=1, af=0, y=A, ldy=16)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["x"], a["m"], a["k"], a["ldx"], a["p"], a["n"], a["ldp"], a["s"], a["b"],
                 a["act"], a["af"], a["y"], a["ldy"], NULL)

    assert call(act=2) == tern.TERN_ERR_ARG
    assert call(act=2, m=-1) == tern.TERN_ERR_ARG              # the kind is checked first
    assert call(af=-1) == tern.TERN_ERR_ARG
    assert call(af=17) == tern.TERN_ERR_ARG                    # act_from > n
    assert call(act=0, af=99, ldx=120) == tern.TERN_ERR_STRIDE  # act_from ignored without act
    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(k=100, ldx=128) == tern.TERN_ERR_SHAPE
    assert call(m=0, x=NULL, p=NULL, s=NULL, y=NULL) == tern.TERN_OK
    for name in ("x", "p", "s", "y"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(b=A + 2) == tern.TERN_ERR_ALIGN               # bias needs 4 bytes
    assert call(b=A + 4, x=A + 8) == tern.TERN_ERR_ALIGN


def test_pack_transposed_validation():
    f = lib.tern_pack_transposed
    assert f(A, -1, 8, 2, A, 2, NULL) == tern.TERN_ERR_SHAPE
    assert f(A, 8, 2 ** 31, 2 ** 29, A, 2, NULL) == tern.TERN_ERR_SHAPE
    assert f(NULL, 0, 8, 2, NULL, 2, NULL) == tern.TERN_OK
    assert f(NULL, 8, 0, 2, NULL, 2, NULL) == tern.TERN_OK
    assert f(NULL, 8, 8, 2, A, 2, NULL) == tern.TERN_ERR_NULL
    assert f(A, 8, 8, 2, NULL, 2, NULL) == tern.TERN_ERR_NULL
    assert f(A, 9, 9, 2, A, 3, NULL) == tern.TERN_ERR_STRIDE     # ldp < ceil(k/4)
    assert f(A, 9, 9, 3, A, 2, NULL) == tern.TERN_ERR_STRIDE     # ldpt < ceil(n/4)


def test_gemm_dx_validation():
    g = lib.tern_gemm_dx
    ok = dict(dy=A, m=8, n=128, lddy=128, pt=A, k=16, ldpt=32, s=A, u=A, ldu=128, dx=A, lddx=16)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["dy"], a["m"], a["n"], a["lddy"], a["pt"], a["k"], a["ldpt"], a["s"], a["u"],
                 a["ldu"], a["dx"], a["lddx"], NULL)

    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(n=100, lddy=128, ldu=128) == tern.TERN_ERR_SHAPE   # n % 64 != 0
    assert call(k=2 ** 31) == tern.TERN_ERR_SHAPE
    assert call(m=0, dy=NULL, pt=NULL, s=NULL, u=NULL, dx=NULL) == tern.TERN_OK
    assert call(k=0, dy=NULL, pt=NULL, s=NULL, u=NULL, dx=NULL) == tern.TERN_OK
    for name in ("dy", "pt", "s", "u", "dx"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(n=0, pt=NULL) == tern.TERN_ERR_NULL
    assert call(n=0, dx=NULL) == tern.TERN_ERR_NULL
    assert call(n=0, dy=NULL, s=NULL, u=NULL, lddx=15) == tern.TERN_ERR_STRIDE  # not read at n = 0
    assert call(lddy=120) == tern.TERN_ERR_STRIDE
    assert call(ldu=120) == tern.TERN_ERR_STRIDE
    assert call(ldpt=16) == tern.TERN_ERR_STRIDE                  # < n/4
    assert call(lddx=15) == tern.TERN_ERR_STRIDE
    assert call(ldu=1 << 23) == tern.TERN_ERR_STRIDE
    assert call(ldpt=1 << 24) == tern.TERN_ERR_STRIDE
    assert call(u=A + 8) == tern.TERN_ERR_ALIGN
    assert call(ldu=132) == tern.TERN_ERR_ALIGN
    assert call(pt=A + 4) == tern.TERN_ERR_ALIGN
    assert call(ldpt=40) == tern.TERN_ERR_ALIGN
    assert call(dy=A + 1) == tern.TERN_ERR_ALIGN
    assert call(dx=A + 1) == tern.TERN_ERR_ALIGN
    assert call(s=A + 2) == tern.TERN_ERR_ALIGN


def test_gemm_dx_static_validation():
    # Every rejection below happens before any HIP call (in particular before
    # the array's address is looked up), so it runs without a GPU.
    g = lib.tern_gemm_dx_static
    ok = dict(dy=A, m=8, n=128, lddy=128, pt=A, k=16, ldpt=32, s=A, dx=A, lddx=16)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["dy"], a["m"], a["n"], a["lddy"], a["pt"], a["k"], a["ldpt"], a["s"], a["dx"],
                 a["lddx"], NULL)

    cap = tern.TERN_GEMM_DX_STATIC_MAX_ELEMS
    assert cap == 1 << 26
    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(n=100, lddy=128) == tern.TERN_ERR_SHAPE   # n % 64 != 0
    assert call(k=2 ** 31) == tern.TERN_ERR_SHAPE
    # the array's capacity: m * n above it is refused, exactly at it passes
    # validation (shown by a later check failing instead)
    assert call(m=cap // 128 + 1) == tern.TERN_ERR_SHAPE
    assert call(m=4608, n=21504, lddy=21504, ldpt=5376) == tern.TERN_ERR_SHAPE
    assert call(m=cap // 128, lddx=15) == tern.TERN_ERR_STRIDE
    assert call(m=0, dy=NULL, pt=NULL, s=NULL, dx=NULL) == tern.TERN_OK
    assert call(k=0, dy=NULL, pt=NULL, s=NULL, dx=NULL) == tern.TERN_OK
    for name in ("dy", "pt", "s", "dx"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(n=0, pt=NULL) == tern.TERN_ERR_NULL
    assert call(n=0, dy=NULL, s=NULL, lddx=15) == tern.TERN_ERR_STRIDE  # not read at n = 0
    assert call(lddy=120) == tern.TERN_ERR_STRIDE
    assert call(ldpt=16) == tern.TERN_ERR_STRIDE                  # < n/4
    assert call(lddx=15) == tern.TERN_ERR_STRIDE
    assert call(ldpt=1 << 24) == tern.TERN_ERR_STRIDE
    assert call(pt=A + 4) == tern.TERN_ERR_ALIGN
    assert call(ldpt=40) == tern.TERN_ERR_ALIGN
    assert call(dy=A + 1) == tern.TERN_ERR_ALIGN
    assert call(dx=A + 1) == tern.TERN_ERR_ALIGN
    assert call(s=A + 2) == tern.TERN_ERR_ALIGN


def test_gemm_dw_validation():
    g = lib.tern_gemm_dw
    ok = dict(dy=A, m=64, n=256, lddy=256, x=A, k=128, ldx=128, dw=A, lddw=128, acc=0)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["dy"], a["m"], a["n"], a["lddy"], a["x"], a["k"], a["ldx"], a["dw"], a["lddw"],
                 a["acc"], NULL)

    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(n=-1) == tern.TERN_ERR_SHAPE
    assert call(k=2 ** 31) == tern.TERN_ERR_SHAPE
    assert call(n=0, dy=NULL, x=NULL, dw=NULL) == tern.TERN_OK       # no-op
    assert call(k=0, dy=NULL, x=NULL, dw=NULL) == tern.TERN_OK
    assert call(dw=NULL) == tern.TERN_ERR_NULL
    assert call(dy=NULL) == tern.TERN_ERR_NULL
    assert call(x=NULL) == tern.TERN_ERR_NULL
    assert call(m=0, dy=NULL, x=NULL, lddy=0, ldx=0, dw=A + 1) == tern.TERN_ERR_ALIGN  # m = 0: not read
    assert call(lddy=255) == tern.TERN_ERR_STRIDE
    assert call(ldx=127) == tern.TERN_ERR_STRIDE
    assert call(lddw=127) == tern.TERN_ERR_STRIDE
    assert call(m=1 << 20, lddy=4096) == tern.TERN_ERR_SHAPE        # a stage's span past 2^31
    assert call(dy=A + 2) == tern.TERN_ERR_ALIGN
    assert call(x=A + 8) == tern.TERN_ERR_ALIGN
    assert call(lddy=260) == tern.TERN_ERR_ALIGN
    assert call(ldx=132) == tern.TERN_ERR_ALIGN
    assert call(dw=A + 2) == tern.TERN_ERR_ALIGN


def test_quantize_act_validation():
    f = lib.tern_quantize_act
    ok = dict(x=A, m=8, k=64, ldx=64, q=A, ldq=64, xs=A)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["m"], a["k"], a["ldx"], a["q"], a["ldq"], a["xs"], NULL)

    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(k=2 ** 31) == tern.TERN_ERR_SHAPE
    assert call(m=0, x=NULL, q=NULL, xs=NULL) == tern.TERN_OK
    for name in ("x", "q", "xs"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(k=0, x=NULL, q=NULL, xs=NULL) == tern.TERN_ERR_NULL   # xs is written
    assert call(k=0, x=NULL, q=NULL, ldx=0, ldq=0, xs=A + 1) == tern.TERN_ERR_ALIGN  # x, q not read
    assert call(ldx=63) == tern.TERN_ERR_STRIDE
    assert call(ldq=63) == tern.TERN_ERR_STRIDE
    assert call(x=A + 1) == tern.TERN_ERR_ALIGN
    assert call(xs=A + 2) == tern.TERN_ERR_ALIGN


def test_pack_a8_validation():
    f = lib.tern_pack_a8
    assert f(A, -1, 16, 4, A, 4, NULL) == tern.TERN_ERR_SHAPE
    assert f(A, 8, 24, 8, A, 8, NULL) == tern.TERN_ERR_SHAPE      # k % 16 != 0
    assert f(A, 8, 2 ** 31, 2 ** 29, A, 2 ** 29, NULL) == tern.TERN_ERR_SHAPE
    assert f(NULL, 0, 16, 4, NULL, 4, NULL) == tern.TERN_OK
    assert f(NULL, 8, 0, 4, NULL, 4, NULL) == tern.TERN_OK
    assert f(NULL, 8, 16, 4, A, 4, NULL) == tern.TERN_ERR_NULL
    assert f(A, 8, 16, 4, NULL, 4, NULL) == tern.TERN_ERR_NULL
    assert f(A, 8, 32, 4, A, 8, NULL) == tern.TERN_ERR_STRIDE     # ldp < k/4
    assert f(A, 8, 32, 8, A, 4, NULL) == tern.TERN_ERR_STRIDE     # ldp8 < k/4
    assert f(A + 2, 8, 16, 4, A, 4, NULL) == tern.TERN_ERR_ALIGN
    assert f(A, 8, 16, 4, A + 2, 4, NULL) == tern.TERN_ERR_ALIGN
    assert f(A, 8, 16, 6, A, 4, NULL) == tern.TERN_ERR_ALIGN
    assert f(A, 8, 16, 4, A, 6, NULL) == tern.TERN_ERR_ALIGN


def test_gemm_a8_validation():
    g = lib.tern_gemm_a8
    ok = dict(q=A, m=8, k=128, ldq=128, xs=A, p=A, n=16, ldp=32, s=A, b=NULL, act=0, af=0, y=A,
              ldy=16)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["q"], a["m"], a["k"], a["ldq"], a["xs"], a["p"], a["n"], a["ldp"], a["s"],
                 a["b"], a["act"], a["af"], a["y"], a["ldy"], NULL)

    assert call(act=2) == tern.TERN_ERR_ARG
    assert call(act=1, af=17) == tern.TERN_ERR_ARG
    assert call(act=1, af=-1, m=-1) == tern.TERN_ERR_ARG         # the kind is checked first
    assert call(m=-1) == tern.TERN_ERR_SHAPE
    assert call(k=64, ldq=128) == tern.TERN_ERR_SHAPE            # k % 128 != 0
    assert call(k=2 ** 18 + 128, ldq=2 ** 18 + 128, ldp=2 ** 16 + 32) == tern.TERN_ERR_SHAPE
    assert call(m=2 ** 30, n=2 ** 20, ldy=2 ** 20) == tern.TERN_ERR_SHAPE
    assert call(m=0, q=NULL, xs=NULL, p=NULL, s=NULL, y=NULL) == tern.TERN_OK
    assert call(n=0, q=NULL, xs=NULL, p=NULL, s=NULL, y=NULL) == tern.TERN_OK
    for name in ("q", "xs", "p", "s", "y"):
        assert call(**{name: NULL}) == tern.TERN_ERR_NULL
    assert call(ldq=112) == tern.TERN_ERR_STRIDE
    assert call(ldp=16) == tern.TERN_ERR_STRIDE                   # < k/4
    assert call(ldy=15) == tern.TERN_ERR_STRIDE
    assert call(ldq=1 << 24) == tern.TERN_ERR_STRIDE
    assert call(ldp=1 << 24) == tern.TERN_ERR_STRIDE
    assert call(q=A + 8) == tern.TERN_ERR_ALIGN
    assert call(ldq=136) == tern.TERN_ERR_ALIGN
    assert call(p=A + 4) == tern.TERN_ERR_ALIGN
    assert call(ldp=40) == tern.TERN_ERR_ALIGN
    assert call(y=A + 1) == tern.TERN_ERR_ALIGN
    assert call(xs=A + 2) == tern.TERN_ERR_ALIGN
    assert call(s=A + 2) == tern.TERN_ERR_ALIGN
    assert call(b=A + 2) == tern.TERN_ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        tern.tern_gemm(x, torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(4),
                       torch.zeros(4, 4, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        tern.quantize(torch.zeros(4, 64))


def test_missing_library_fails_loudly(tmp_path):
    env = dict(os.environ, TERN_LIB=str(tmp_path / "nope.so"))
    r = subprocess.run(["python", "-c", "import ternary_weight_quantized_tern_amd"], cwd=ROOT,
                       env=env, capture_output=True, text=True)
    assert r.returncode != 0 and "no CPU fallback" in r.stderr
