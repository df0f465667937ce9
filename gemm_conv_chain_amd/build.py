"""Build libfusedchain.so (HIP, gfx950) in-tree with hipcc.

``python -m gemm_conv_chain_amd.build`` or ``build()``.  Every HIP source in
csrc/ is compiled for gfx950 only and linked into
``gemm_conv_chain_amd/libfusedchain.so``.  Packed-FP32 instruction selection is
disabled (-packed-fp32-ops).

The same sources are also built with ``-DFC_DEBUG_POISON`` into
``libfusedchain_poison.so``: the debug build whose kernels fill LDS buffers
with a poison pattern whenever a buffer is released, so that a read racing
its producer shows up in the results (tests load it through
``gemm_conv_chain_amd.poison_build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfusedchain.so")
POISON_LIB = os.path.join(HERE, "libfusedchain_poison.so")
POISON_DEFINE = "-DFC_DEBUG_POISON"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src, poison: bool = False):
    odir = os.path.join(BUILD, "poison") if poison else BUILD
    obj = os.path.join(odir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ([POISON_DEFINE] if poison else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False, poison: bool = True) -> str:
    """Compile and link libfusedchain.so (and, with poison, the debug build
    libfusedchain_poison.so); returns the product library's path."""
    os.makedirs(os.path.join(BUILD, "poison"), exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = [(s, False) for s in srcs] + ([(s, True) for s in srcs] if poison else [])
    # longest sources first, so the slowest compiles do not start last
    jobs.sort(key=lambda j: -os.path.getsize(j[0]))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        done = dict(zip(jobs, ex.map(lambda j: _compile(*j), jobs)))
    _link([done[(s, False)] for s in srcs], LIB)
    if verbose:
        print("built", LIB)
    if poison:
        _link([done[(s, True)] for s in srcs], POISON_LIB)
        if verbose:
            print("built", POISON_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
