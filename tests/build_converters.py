"""Test-only GPU libraries, built with hipcc for gfx950 by __graft_entry__.build():

* tests/libconverters_gpu.so from tests/converters_gpu.hip (the conversion
  instructions applied to every input);
* tests/libnvfp4_exact_path.so: libnvfp4's own source built with every
  quantizing wave on the exact-quotient code path (NVFP4_EXACT_PATH=2), so the
  parity tests can run that path under every scale byte, not only in waves
  that hold a block whose multiplier is not certified.

The GPU tests load them and fail if they are missing.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "converters_gpu.hip")
LIB = os.path.join(HERE, "libconverters_gpu.so")
EXACT_LIB = os.path.join(HERE, "libnvfp4_exact_path.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    build_exact_path(verbose)
    return LIB


def build_exact_path(verbose: bool = False) -> str:
    root = os.path.dirname(HERE)
    tmp = EXACT_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wall", "-DNVFP4_EXACT_PATH=2", "-I", os.path.join(root, "include"), "-o", tmp,
           os.path.join(root, "fp4_block_fake_amd", "csrc", "nvfp4.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, EXACT_LIB)
    return EXACT_LIB


if __name__ == "__main__":
    print(build(verbose=True))
