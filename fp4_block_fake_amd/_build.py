"""Compile libnvfp4.so (and libnvfp4_probe.so, the benchmark's HBM stream probes)
in-tree with hipcc for gfx950.

Kept free of package imports so it can run before the library exists:
``python fp4_block_fake_amd/_build.py``.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "nvfp4.hip")
LIB = os.path.join(PKG, "libnvfp4.so")
PROBE_SRC = os.path.join(PKG, "csrc", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "libnvfp4_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # bit-exact numerics: no a*b+c contraction, IEEE divide, no fast-math
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _compile(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _compile(SRC, LIB, verbose)
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
