"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/csrc/oracle_driver.c calls every oracle entry point on small and
edge-case shapes with exactly sized buffers; built with gcc
-fsanitize=address,undefined and -fno-sanitize-recover, any out-of-bounds
access, use after free, signed overflow or misaligned access in the oracle
makes the run fail.  CPU only (gcc, no GPU).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "csrc", "oracle_driver.c"),
           "-o", str(exe), "-lm", "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver ok" in r.stdout
