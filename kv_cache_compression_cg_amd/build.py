"""Builds libcg.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m kv_cache_compression_cg_amd.build

Float rules for bit-exact parity with the CPU reference: no contraction of a*b+c into
fma unless written (-ffp-contract=off), no fast-math, correctly rounded fp32 division
and square root (HIP's default).  Packed fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libcg.so")
# counter-calibration kernels used by the benchmark only (not part of the codec's ABI)
CALIB_LIB = os.path.join(LIB_DIR, "libcg_calib.so")
CALIB_SOURCES = [os.path.join(CSRC, "cg_calib.hip")]
SOURCES = [os.path.join(CSRC, "cg_kernels_encode.hip"), os.path.join(CSRC, "cg_kernels_decode.hip"),
           os.path.join(CSRC, "cg_api.cpp")]
ARCH = os.environ.get("CG_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-ffp-contract=off",
            "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _link(sources, lib, verbose):
    """Each source compiled to its own object in parallel (the kernels of one file call no
    device code of another), then one shared library linked from them."""
    tmp = lib + ".tmp%d" % os.getpid()
    objs = [tmp + ".%d.o" % i for i in range(len(sources))]
    cmds = [[hipcc()] + flags() + ["-c", "-x", "hip", src, "-o", obj]
            for src, obj in zip(sources, objs)]
    try:
        with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc()] + flags() + ["-shared"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, lib)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    _link(SOURCES, LIB, verbose)
    _link(CALIB_SOURCES, CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
