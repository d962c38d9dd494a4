"""Build libternary.so in-tree with hipcc for gfx950.

``python ternary_weight_quantized_tern_amd/build.py`` (or ``build_library()``)
compiles every ``csrc/*.hip`` into one shared library next to this file.  Run
it by path: importing the package would first try to load the library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libternary.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = os.environ.get("TERN_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags(arch: str = ARCH) -> list:
    return [
        f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC",
        # Packed fp32 VALU instructions are kept out of every kernel.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile_one(src: str, obj: str, extra: list) -> None:
    cmd = [hipcc()] + compile_flags() + extra + ["-c", "-o", obj, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({r.returncode}):\n{r.stderr}")


def build_library(out: str = LIB_PATH, extra: list | None = None, verbose: bool = False) -> str:
    """Compile all HIP sources into ``out`` (atomically replaced).  Each source
    is compiled to an object file of its own, in parallel, then linked."""
    from concurrent.futures import ThreadPoolExecutor

    extra = list(extra or [])
    srcs = sources()
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=os.path.dirname(out))
    os.close(fd)
    with tempfile.TemporaryDirectory(prefix="tern_build_") as objdir:
        objs = [os.path.join(objdir, os.path.basename(f) + ".o") for f in srcs]
        if verbose:
            print(" ".join([hipcc()] + compile_flags() + extra + ["-c", "<each of>"] + srcs),
                  flush=True)
        jobs = max(1, min(len(srcs), os.cpu_count() or 1))
        try:
            with ThreadPoolExecutor(max_workers=jobs) as pool:
                for f in [pool.submit(_compile_one, s, o, extra) for s, o in zip(srcs, objs)]:
                    f.result()
            cmd = [hipcc()] + compile_flags() + extra + ["-shared", "-o", tmp] + objs
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"link failed ({r.returncode}):\n{r.stderr}")
            # A kernel whose host stub was not emitted shows up as an undefined
            # symbol only when the library is loaded: load it in a child process.
            chk = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r})"],
                                 capture_output=True, text=True)
            if chk.returncode != 0:
                raise RuntimeError(f"built library does not load:\n{chk.stderr}")
            os.replace(tmp, out)
        finally:
            if os.path.exists(tmp):
                os.unlink(tmp)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
