"""Pins for the oracle's MXFP4 variant (no GPU): 32-element blocks, one binary32 block
scale block_amax / 6, no per-tensor factor (VideoX-Fun page, module constants, the
block-size comment, which names 32-element blocks with a single-precision scale as the
MXFP4 form).

Checked against constructed tensors whose every output is known, the E2M1 values and
tie directions the pages print (tests/golden/), special cases, and an independent
re-derivation from numpy float32 arithmetic, torch's bf16 cast and brute-force
nearest-value rounding.
"""
import numpy as np
import pytest

import oracle
import synth
from cases import log_uniform_bf16
from synth import bits_to_f32
from test_oracle_pins import nearest_index, signed_lut, torch_bf16, unpack_codes

EPS32 = np.float32(1e-12)


def mx_scales_5bit():
    """Block scales m * 2^e with a 5-bit m, above the 1e-12 clamp: every E2M1 value times
    s is bf16-exact and fl(6s / 6) = s, so the expected outputs are the inputs themselves."""
    m = np.arange(16, 32, dtype=np.float64)
    e = np.arange(-38, 100, 5, dtype=np.float64)
    return (m[None, :] * 2.0 ** e[:, None]).reshape(-1)


def test_every_code_times_many_scales(golden):
    s = mx_scales_5bit()
    lut = signed_lut(golden)
    x = np.concatenate([lut, lut[::-1]])[None, :] * s[:, None]          # 32 per block: +-6s present
    bits = torch_bf16(x.astype(np.float32))
    assert np.array_equal(bits_to_f32(bits).astype(np.float64), x)
    packed, scales = oracle.mx_quantize(bits)
    assert packed.shape == (s.size, 16) and scales.shape == (s.size, 1)
    assert np.array_equal(scales[:, 0].astype(np.float64), s)
    codes = np.concatenate([np.arange(16), np.arange(16)[::-1]]).astype(np.uint8)
    want = np.tile(codes, (s.size, 1))
    want[want == 8] = 0                                     # -0.0 has no sign after the divide
    assert np.array_equal(unpack_codes(packed), want)
    y = oracle.mx_fake_quant(bits)
    want_y = bits.copy()
    want_y[want_y == 0x8000] = 0
    assert np.array_equal(y, want_y)


def test_exact_ties(golden):
    t = np.array([float(v[0]) for v in golden("e2m1_boundaries.txt")])
    tie_idx = np.array([int(i) for _, i, _ in golden("e2m1_ties.txt")], np.uint8)
    s = mx_scales_5bit()[::3]
    row = np.concatenate([[6.0], t, -t, [-6.0], np.ones(8), np.full(8, 0.5)])
    assert row.size == 32
    x = row[None, :] * s[:, None]
    bits = torch_bf16(x.astype(np.float32))
    assert np.array_equal(bits_to_f32(bits).astype(np.float64), x)
    packed, scales = oracle.mx_quantize(bits)
    assert np.array_equal(scales[:, 0].astype(np.float64), s)
    codes = unpack_codes(packed)
    assert np.array_equal(codes[:, 1:8], np.tile(tie_idx, (s.size, 1)))
    assert np.array_equal(codes[:, 8:15], np.tile(tie_idx + 8, (s.size, 1)))
    assert np.all(codes[:, 0] == 7) and np.all(codes[:, 15] == 15)


def test_scales_below_the_clamp(golden):
    """A block whose scale is below 1e-12 divides its elements by 1e-12 (the clamp) but
    still multiplies the codes back by its own scale."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 3e-12                                         # scale 5e-13 < 1e-12
    x[0, 1] = 1.2e-12                                       # quotient 1.2 -> index 2 (1.0)
    x[0, 2] = -2.4e-12                                      # quotient -2.4 -> index 4 (2.0), negative
    bits = torch_bf16(x)
    packed, scales = oracle.mx_quantize(bits)
    v = bits_to_f32(bits)[0]
    assert scales[0, 0] == v[0] / np.float32(6)
    q = v[:3] / EPS32
    codes = unpack_codes(packed)[0]
    assert list(codes[:3]) == [int(nearest_index(np.abs(q[i:i + 1]), golden)[0]) + 8 * int(q[i] < 0)
                               for i in range(3)]
    y = bits_to_f32(oracle.mx_fake_quant(bits))[0]
    lut = signed_lut(golden).astype(np.float32)
    assert np.array_equal(y[:3], bits_to_f32(torch_bf16(lut[codes[:3]] * scales[0, 0])))


def test_zero_block_negative_zero_and_underflow():
    x = np.zeros((1, 96), np.float32)
    x[0, 32] = -0.0
    x[0, 64] = 3.0e38                                       # scale 5e37
    x[0, 65] = -1e-40                                       # quotient underflows to -0: code 0
    x[0, 66] = -1e-6                                        # quotient -2e-44 rounds to -0: code 8
    x[0, 67] = 1e-6
    bits = torch_bf16(x)
    bits[0, 32] = 0x8000
    packed, scales = oracle.mx_quantize(bits)
    codes = unpack_codes(packed)[0]
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and not codes[:64].any()
    assert scales[0, 2] == np.float32(bits_to_f32(bits[0, 64:65])[0]) / np.float32(6)
    assert codes[64] == 7 and codes[65] == 0 and codes[66] == 8 and codes[67] == 0
    y = oracle.mx_fake_quant(bits)[0]
    assert not y[:64].any()
    assert y[65] == 0 and y[66] == 0x8000 and y[67] == 0


def test_unpack_of_every_byte(golden):
    lut = signed_lut(golden)
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    scales = np.ones((1, 16), np.float32)
    y = bits_to_f32(oracle.mx_dequantize(packed, scales, 512))[0].astype(np.float64)
    b = np.arange(256)
    assert np.array_equal(y[0::2], lut[b & 15]) and np.array_equal(y[1::2], lut[b >> 4])


def test_pack_unpack_round_trip():
    codes = [c for c in range(16) if c != 8]
    pairs = np.array([lo | (hi << 4) for lo in codes for hi in codes], np.uint8)
    per_block = 15
    pad = (-len(pairs)) % per_block
    pairs = np.concatenate([pairs, np.full(pad, 0x11, np.uint8)]).reshape(-1, per_block)
    packed = np.concatenate([np.full((len(pairs), 1), 0x77, np.uint8), pairs], 1).reshape(1, -1)
    cols = packed.shape[1] * 2
    scales = np.full((1, cols // 32), 0.75, np.float32)        # block max 6 * 0.75 = 4.5
    y = oracle.mx_dequantize(packed, scales, cols)
    p2, s2 = oracle.mx_quantize(y)
    assert np.array_equal(s2, scales) and np.array_equal(p2, packed)


def mx_rederive(xbits, golden):
    """Every MXFP4 step again from numpy float32 arithmetic, torch's bf16 cast and
    brute-force nearest-value rounding (cols a multiple of 32)."""
    x = bits_to_f32(xbits)
    rows, cols = x.shape
    b = x.reshape(rows, cols // 32, 32)
    s = np.abs(b).max(-1) / np.float32(6.0)
    sq = np.maximum(s, EPS32)
    with np.errstate(over="ignore"):
        q = np.clip(b / sq[..., None], np.float32(-6.0), np.float32(6.0))
    code = nearest_index(np.abs(q), golden) + 8 * (q < 0)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).reshape(rows, cols // 2).astype(np.uint8)
    y = torch_bf16(signed_lut(golden).astype(np.float32)[code] * s[..., None]).reshape(rows, cols)
    return packed, s, y


CASES = {
    "c1": lambda: synth.c1_weight(),
    "c5_rows": lambda: synth.c5_weight(rows=48),
    "c4_act_rows": lambda: synth.c4_activation(0, tokens=64),
    "log_uniform": lambda: log_uniform_bf16(1, (64, 512), -130, 120),
    "log_uniform_small": lambda: log_uniform_bf16(2, (32, 256), -140, -100),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_whole_path_rederived_independently(case, golden):
    x = CASES[case]()
    packed, scales = oracle.mx_quantize(x)
    p2, s2, y2 = mx_rederive(x, golden)
    assert np.array_equal(scales.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(packed, p2)
    assert np.array_equal(oracle.mx_fake_quant(x), y2)
    assert np.array_equal(oracle.mx_dequantize(packed, scales, x.shape[1]), y2)


def test_ragged_rows_are_zero_padded():
    x = synth.c1_weight()[:8, :40]
    pad = np.zeros((8, 64), np.uint16)
    pad[:, :40] = x
    p1, s1 = oracle.mx_quantize(x)
    p2, s2 = oracle.mx_quantize(pad)
    assert p1.shape == (8, 32) and s1.shape == (8, 2)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
    assert np.array_equal(oracle.mx_dequantize(p1, s1, 40), oracle.mx_dequantize(p2, s2, 64)[:, :40])


def test_rounding_error_within_half_gap():
    x = synth.c1_weight()
    packed, scales = oracle.mx_quantize(x)
    q = bits_to_f32(x).reshape(256, -1, 32) / np.maximum(scales, EPS32)[..., None]
    codes = unpack_codes(packed).reshape(256, -1, 32)
    g = np.float64([0, .5, 1, 1.5, 2, 3, 4, 6])
    got = g[codes & 7] * np.where(codes & 8, -1, 1)
    half_gap = np.where(np.abs(q) < 2, 0.25, np.where(np.abs(q) < 4, 0.5, 1.0))
    assert np.all(np.abs(q - got) <= half_gap)


def test_block_of_32_not_16():
    """Two 16-element halves with different maxima share one scale."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0
    x[0, 16] = 0.75
    x[0, 17] = 0.5
    packed, scales = oracle.mx_quantize(torch_bf16(x))
    assert scales[0, 0] == 1.0
    codes = unpack_codes(packed)[0]
    assert codes[0] == 7 and codes[16] == 2 and codes[17] == 1     # 0.75 ties up to 1.0
