"""Build libtern.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m packed_bit_gemv_tern_amd.build

Each .hip file is compiled to an object under ``_build/`` (in parallel), then
linked into ``packed_bit_gemv_tern_amd/libtern.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtern.so")
SOURCES = ["tern_api.hip", "tern_pack.hip", "tern_valu.hip", "tern_mfma.hip", "tern_gemm.hip",
           "tern_head.hip", "tern_quant.hip", "tern_block.hip", "tern_packed5.hip", "tern_probe.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # no packed fp32 instructions in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every fp32 product and sum rounded as written: no fused multiply-adds
    # formed from separate operations
    "-ffp-contract=off",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
