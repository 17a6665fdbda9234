"""The gfx950 conversion instructions the kernels rely on, checked against the CPU oracle
on every input they can receive (tests/converters_gpu.hip applies each to a range of
binary32 bit patterns; NaN patterns are left out):

* v_cvt_scalef32_pk_fp4_f32 with scale 1.0, on every binary32 of either sign up to
  the infinities: the E2M1 index of the oracle's rounding of min(|v|, 6), with code
  bit 3 equal to the sign bit of v.  The quantizing kernels feed it fl(x * r) where a
  per-scale-byte certificate says that gives the exact quotient's code, and clear
  the sign of -0.0 first (the method signs a code only when the quotient is below
  zero), so this is exactly the property they need.
* v_cvt_pk_bf16_f32 (the float2 -> bf16x2 conversion the kernels write), on every
  binary32 of either sign up to the infinities: the oracle's round-to-nearest-even.
* v_cvt_pk_fp8_f32 on every non-negative binary32 up to +inf, followed by the
  kernels' min(byte, 0x7E): the oracle's saturating E4M3 encode.
* v_cvt_scalef32_pk_f32_fp4 with scale 1.0 on every byte under every selector: the
  oracle's E2M1 values, -0 for code 8 included.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from conftest import ROOT

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

LIB = os.path.join(ROOT, "tests", "libconverters_gpu.so")
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
CHUNK = 1 << 26
POS_END = 0x7F800002          # +0 .. +inf (and one NaN, masked)
NEG = 0x80000000
NEG_END = 0xFF800002          # -0 .. -inf (and one NaN, masked)


@pytest.fixture(scope="module")
def conv():
    if not os.path.exists(LIB):
        pytest.fail("tests/libconverters_gpu.so is not built (run __graft_entry__.build())")
    torch.cuda.init()
    lib = ctypes.CDLL(LIB)
    lib.conv_run.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p]
    lib.conv_run.restype = ctypes.c_int
    return lib


def run(lib, which, first, n):
    out = np.empty(n // 2 if which == 0 else n, dtype=np.uint16 if which == 1 else np.uint8)
    rc = lib.conv_run(which, first, n, out.ctypes.data)
    assert rc == 0, "conv_run(%d, %#x, %d) returned HIP error %d" % (which, first, n, rc)
    return out


def sweep(lib, which, lo, hi, check):
    """Converter `which` over the bit patterns [lo, hi) in chunks; check(bits, got) compares
    one slice (even-aligned) with the oracle and returns the bit patterns that differ, on
    THREADS host threads (the oracle's C calls release the GIL)."""
    bad = 0
    print("[gpu-parity] converter %d over [%#x, %#x)" % (which, lo, hi), flush=True)
    with ThreadPoolExecutor(THREADS) as pool:
        for first in range(lo, hi, CHUNK):
            n = min(CHUNK, hi - first)
            got = run(lib, which, first, n)
            step = -(-n // THREADS // 2) * 2
            jobs = []
            for a in range(0, n, step):
                b = min(n, a + step)
                bits = np.arange(first + a, first + b, dtype=np.uint64).astype(np.uint32)
                part = got[a // 2:b // 2] if which == 0 else got[a:b]
                jobs.append(pool.submit(check, bits, part))
            for j in jobs:
                miss = j.result()
                if miss.size:
                    print("[gpu-parity] converter %d differs at %s" % (which, [hex(int(m)) for m in miss[:8]]),
                          flush=True)
                bad += int(miss.size)
    return bad


def not_nan(bits):
    return (bits & 0x7FFFFFFF) <= 0x7F800000


def check_fp4(bits, got):
    v = bits.view(np.float32)
    keep = not_nan(bits)
    want = oracle.e2m1_round_array(np.minimum(np.abs(np.where(keep, v, 0)), np.float32(6)))
    want |= ((bits >> 28) & 8).astype(np.uint8)
    codes = np.empty(bits.size, np.uint8)
    codes[0::2] = got & 0x0F
    codes[1::2] = got >> 4
    return bits[(codes != want) & keep]


def check_bf16(bits, got):
    keep = not_nan(bits)
    want = oracle.f32_to_bf16_array(np.where(keep, bits, 0).view(np.float32))
    return bits[(got != want) & keep]


def check_fp8(bits, got):
    keep = not_nan(bits)
    want = oracle.e4m3_encode_array(np.where(keep, bits, 0).view(np.float32))
    clamped = np.minimum(got, np.uint8(0x7E))
    return bits[((clamped != want) | (got > 0x7F)) & keep]


@pytest.mark.parametrize("lo,hi", [(0, POS_END), (NEG, NEG_END)], ids=["positive", "negative"])
def test_fp4_converter_every_binary32(conv, lo, hi):
    assert sweep(conv, 0, lo, hi, check_fp4) == 0


@pytest.mark.parametrize("lo,hi", [(0, POS_END), (NEG, NEG_END)], ids=["positive", "negative"])
def test_bf16_converter_every_binary32(conv, lo, hi):
    assert sweep(conv, 1, lo, hi, check_bf16) == 0


def test_fp8_converter_every_non_negative_binary32(conv):
    assert sweep(conv, 2, 0, POS_END, check_fp8) == 0


def test_fp4_decode_every_byte_and_selector(conv):
    out = np.empty(2048, np.float32)
    assert conv.conv_run(3, 0, 0, out.ctypes.data) == 0
    # the oracle's value of every code: an unpack of all 256 bytes at block scale 1.0
    # (E4M3 0x38) and gs 1
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    vals = oracle.dequantize(packed, np.full((1, 32), 0x38, np.uint8), 1.0, 512)[0]
    want = (vals.astype(np.uint32) << 16).view(np.float32)
    for sel in range(4):
        got = out[sel * 512:(sel + 1) * 512]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "selector %d" % sel
