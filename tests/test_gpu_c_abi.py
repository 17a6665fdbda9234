"""The C ABI from a plain C program (tests/c_abi_gpu.c): HIP runtime memory and a
stream, libnvfp4 for the work, the CPU oracle linked in for the expected bytes; no
Python or torch between the caller and the library.  Each shape must come out bit for
bit equal to the oracle for the fused fake-quant (plain and workspace), the fused
quantize-pack, the dequant-unpack and the one-call observe step.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

PKG = os.path.join(ROOT, "fp4_block_fake_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP headers are missing")
    if not os.path.exists(os.path.join(PKG, "libnvfp4.so")):
        pytest.fail("libnvfp4.so is not built")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_gpu")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_gpu.c"),
           os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-ffp-contract=off", "-fno-fast-math",
           "-o", exe, "-L", PKG, "-lnvfp4", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    return exe


# empty, ragged rows (their own kernels and the reduction launch), a single block,
# whole-block rows (the two-launch workspace path), and a tensor with many workgroups
@pytest.mark.parametrize("rows,cols", [(0, 16), (3, 20), (1, 16), (64, 4096), (1037, 144), (2048, 2064)])
def test_c_program_bit_exact(program, rows, cols):
    print("[gpu-parity] C ABI program %dx%d" % (rows, cols), flush=True)
    r = subprocess.run([program, str(rows), str(cols), str(1000 + rows + cols)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "all bit-exact" in r.stdout, r.stdout + r.stderr
