"""Host sanitizers on the oracle: the C oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only), and every oracle pin run
against that build in a child process.

An out-of-bounds read or write of an operand (a wrong stride, a halo index
off by one at the image border, a pool window past the last row) or
undefined arithmetic (signed overflow of an index) stops the child with a
sanitizer report instead of silently reading neighbouring memory.
"""
import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.cpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                    reason="gcc with the address sanitizer runtime is needed")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env.update(FC_ORACLE_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
