"""Arithmetic facts the kernels' fast paths rest on that the CPU can check exhaustively
(no GPU): binary64 arithmetic is IEEE on both sides, so the same expression gives the
same bits here and on the GPU.
"""
import numpy as np


def test_divide_by_six_through_binary64_is_exact_for_every_bf16():
    """The kernels form bamax / 6 as float(double(bamax) * (1/6)) instead of a binary32
    divide.  A bf16 value has 8 significant bits, so its quotient by 3 never falls close
    enough to a binary32 rounding mid-point for the double rounding to matter: checked
    here for every finite bf16 value of either sign, subnormals included."""
    b = np.arange(0, 0x10000, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]                              # finite
    x = (b << 16).view(np.float32)
    fast = (x.astype(np.float64) * (1.0 / 6.0)).astype(np.float32)
    ieee = x / np.float32(6.0)
    assert np.array_equal(fast.view(np.uint32), ieee.view(np.uint32))
