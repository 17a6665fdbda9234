"""Test-only GPU libraries, built with hipcc for gfx950 by __graft_entry__.build():

* tests/libconverters_gpu.so from tests/converters_gpu.hip (the conversion
  instructions applied to every input);
* tests/libnvfp4_test_paths.so: libnvfp4's own source built with the code paths
  that ordinary shapes rarely or never reach switched on for everything: every
  quantizing wave on the exact-quotient path (NVFP4_EXACT_PATH=2), not only
  waves that hold a block whose multiplier is not certified, and every ragged
  shape through the one-lane-per-block kernels (NVFP4_HALF_ROWS_MAX_BLOCKS=0),
  which the library otherwise keeps for tensors of 2^31 blocks and more, and the
  linear layer's tile rounds (the re-tiled last round of 256 x 256 tiles, the 256 x
  128 tiles of 129-256 rows) planned for 6 CUs (NVFP4_LIN_RETILE_CUS=6), so that small
  layers reach every narrower tile.

The GPU tests load them and fail if they are missing.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "converters_gpu.hip")
LIB = os.path.join(HERE, "libconverters_gpu.so")
TEST_PATHS_LIB = os.path.join(HERE, "libnvfp4_test_paths.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    build_test_paths(verbose)
    return LIB


def build_test_paths(verbose: bool = False) -> str:
    root = os.path.dirname(HERE)
    tmp = TEST_PATHS_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wall", "-DNVFP4_EXACT_PATH=2", "-DNVFP4_HALF_ROWS_MAX_BLOCKS=0",
           "-DNVFP4_LIN_RETILE_CUS=6", "-I", os.path.join(root, "include"), "-o", tmp,
           os.path.join(root, "fp4_block_fake_amd", "csrc", "nvfp4.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, TEST_PATHS_LIB)
    return TEST_PATHS_LIB


if __name__ == "__main__":
    print(build(verbose=True))
