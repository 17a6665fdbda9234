"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: values the pages
print (tests/golden/, each file citing its page), library routines whose
definition coincides with a step (torch's float8_e4m3fn and bfloat16 CPU
casts, numpy's IEEE float32 arithmetic), brute-force nearest-value search,
closed forms and constructed tensors whose every output is known in advance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from cases import log_uniform_bf16, scale_straddle_cases, straddle_block, torch_fp8_decode, torch_fp8_encode
from synth import bits_to_f32

EPS32 = np.float32(1e-12)


# ---------------------------------------------------------------- helpers

def torch_bf16(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def grid(golden):
    return np.array([float(m) for _, m in golden("e2m1_grid.txt")])


def signed_lut(golden):
    g = grid(golden)
    return np.concatenate([g, -g])


def nearest_index(a, golden):
    """Brute force: the magnitude index nearest to a (float64 distances), ties to the even index."""
    g = grid(golden)
    a = np.minimum(np.asarray(a, dtype=np.float64), g[-1])   # beyond the top value: the top value
    d = np.abs(a[..., None] - g)                       # exact for these operands
    dmin = d.min(-1, keepdims=True)
    cand = d == dmin
    first = np.argmax(cand, -1)                       # lowest candidate
    two = cand.sum(-1) == 2
    # of two equally near neighbours, take the even index
    return np.where(two & (first % 2 == 1), first + 1, first).astype(np.uint8)


def unpack_codes(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def f32_bits(lo, hi):
    return np.arange(lo, hi, dtype=np.uint32).view(np.float32)


def windows(centres_f32, half):
    """All float32 patterns within +-half ulps of each (non-negative) centre."""
    c = np.asarray(centres_f32, dtype=np.float32).view(np.uint32).astype(np.int64)
    off = np.arange(-half, half + 1, dtype=np.int64)
    p = (c[:, None] + off[None, :]).reshape(-1)
    p = p[(p >= 0) & (p < 0x7F800000)]
    return np.unique(p).astype(np.uint32).view(np.float32)


# ---------------------------------------------------------------- E2M1 grid

def test_grid_and_lut_match_pages(golden):
    # every code 0..15 once, decoded with block scale 1 (E4M3 0x38 = 1.0, gs = 1)
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).reshape(1, 8)
    scales = np.array([[0x38]], np.uint8)
    assert torch_fp8_decode(scales)[0, 0] == 1.0
    y = oracle.dequantize(packed, scales, 1.0, 16)
    assert np.array_equal(bits_to_f32(y[0]).astype(np.float64), signed_lut(golden))
    # code 8 is negative zero
    assert y[0, 8] == 0x8000 and y[0, 0] == 0x0000


def test_boundaries_are_midpoints(golden):
    g = grid(golden)
    b = np.array([float(v[0]) for v in golden("e2m1_boundaries.txt")])
    assert np.array_equal(b, (g[:-1] + g[1:]) / 2)


def test_tie_table(golden):
    for value, index, _src in golden("e2m1_ties.txt"):
        assert oracle.e2m1_round(float(value)) == int(index), value


def test_printed_compare_chain():
    # verl QATLinear page, section 1: <=0.25 -> 0.0, <0.75 -> 0.5, <=1.25 -> 1.0
    a = windows([0.25, 0.75, 1.25], 64)
    a = a[a <= np.float32(1.25) + np.float32(1e-6)]
    got = oracle.e2m1_round_array(a)
    want = np.where(a <= 0.25, 0, np.where(a < 0.75, 1, np.where(a <= 1.25, 2, 3)))
    assert np.array_equal(got, want)


def test_e2m1_brute_force_near_every_decision_point(golden):
    g = grid(golden).astype(np.float32)
    b = np.array([float(v[0]) for v in golden("e2m1_boundaries.txt")], np.float32)
    a = windows(np.concatenate([g, b]), 1 << 16)
    a = np.concatenate([a, f32_bits(0, 0x40C00001)[::4099], np.float32([6.5, 7, 100, 3e38, np.inf])])
    assert np.array_equal(oracle.e2m1_round_array(a), nearest_index(a, golden))


def test_e2m1_monotone_over_every_float_in_range():
    # Every binary32 in [0, 6]: the rounded index never decreases.  With the
    # decision windows above this fixes the rounding for every input.
    top = int(np.float32(6.0).view(np.uint32)) + 1
    step = 1 << 26
    prev = 0
    for lo in range(0, top, step):
        hi = min(lo + step, top)
        r = oracle.e2m1_round_array(f32_bits(lo, hi))
        assert r[0] >= prev
        assert np.all(np.diff(r.astype(np.int16)) >= 0)
        prev = r[-1]
    assert prev == 7


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_all_bytes_vs_torch(golden):
    b = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_decode_array(b), torch_fp8_decode(b)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    facts = {k: float(v) for k, v in golden("e4m3.txt")}
    assert ours[:0x7F].max() == facts["max"] == oracle.e4m3_decode(0x7E)


def test_e4m3_encode_vs_torch_cast():
    vals = oracle.e4m3_decode_array(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    lim = np.float32(464.0).view(np.uint32)
    v = np.concatenate([windows(np.concatenate([vals, mids]).astype(np.float32), 4096),
                        f32_bits(0, int(lim) + 1)[::101]])
    v = v[v <= 464.0]
    assert np.array_equal(oracle.e4m3_encode_array(v), torch_fp8_encode(v))


def test_e4m3_encode_saturates_and_underflows():
    big = np.float32([448.0, 448.5, 463.9, 464.0, 464.1, 480.0, 1e6, 3e38, np.inf])
    assert np.all(oracle.e4m3_encode_array(big) == 0x7E)
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00          # tie to the even code 0
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 0x01
    assert oracle.e4m3_encode(2.0 ** -9) == 0x01
    assert oracle.e4m3_encode(1e-40) == 0x00
    assert oracle.e4m3_encode(0.0) == 0x00


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_vs_torch_cast():
    hi = np.arange(0, 0x10000, dtype=np.uint32)
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF]
    rng = np.random.default_rng(7)
    pats = [(hi << 16) | l for l in lows] + [(hi << 16) | rng.integers(0, 0x10000, hi.size, dtype=np.uint32)]
    p = np.concatenate(pats)
    finite = (p & 0x7F800000) != 0x7F800000
    f = p[finite].view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16_array(f), torch_bf16(f))


# ---------------------------------------------------------------- steps 1, 2

def test_amax_is_the_max_magnitude():
    for x in (synth.c1_weight(), synth.c5_weight(rows=64)):
        assert oracle.amax(x) == np.abs(bits_to_f32(x)).max()
    z = np.array([0x8000, 0x0000, 0x8000], np.uint16)            # -0, +0
    assert oracle.amax(z) == 0.0 and not np.signbit(oracle.amax(z))


def test_shared_sibling_amax():
    q, k, v = (s[:256] for s in synth.c3_siblings())
    want = max(np.abs(bits_to_f32(t)).max() for t in (q, k, v))
    assert oracle.amax_group([q, k, v]) == want
    assert oracle.amax_group([q, k, v]) == max(oracle.amax(q), oracle.amax(k), oracle.amax(v))


def test_global_scale_is_ieee_quotient():
    rng = np.random.default_rng(3)
    a = np.concatenate([np.float32([0.0, 1e-30, 1e-12, 2e-12, 1.0, 2.625, 448.0, 3.3e38]),
                        np.exp(rng.uniform(-60, 80, 20000)).astype(np.float32)])
    want = np.float32(2688.0) / np.maximum(a, EPS32)
    got = np.array([oracle.global_scale(float(x)) for x in a], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- constructed tensors

def all_codes_all_scales(k, golden):
    """Row i (S = i+1 = 0x01..0x7E) holds LUT[c] * dec(S) / 2**k for c = 0..15."""
    s = torch_fp8_decode(np.arange(1, 127, dtype=np.uint8)).astype(np.float64) / 2.0 ** k
    x = signed_lut(golden)[None, :] * s[:, None]
    bits = torch_bf16(x.astype(np.float32))
    assert np.array_equal(bits_to_f32(bits).astype(np.float64), x)       # every value exact
    return bits


@pytest.mark.parametrize("k", [4, 10, 12])
def test_all_codes_times_all_scales(k, golden):
    x = all_codes_all_scales(k, golden)
    assert oracle.amax(x) == 2688.0 * 2.0 ** -k
    packed, scales, gs = oracle.quantize(x)
    assert gs == 2.0 ** k
    assert np.array_equal(scales[:, 0], np.arange(1, 127))
    want = np.tile(np.arange(16, dtype=np.uint8), (126, 1))
    want[:, 8] = 0                                    # -0.0 has no sign after the divide
    assert np.array_equal(unpack_codes(packed), want)
    y = oracle.fake_quant(x)
    want_y = x.copy()
    want_y[:, 8] = 0
    assert np.array_equal(y, want_y)


def tie_tensor(k, golden):
    """Blocks +6s | +t s (t = each boundary) | -t s | -6s, s over even-mantissa E4M3 values, gs = 2**k."""
    t = np.array([float(v[0]) for v in golden("e2m1_boundaries.txt")])
    even = np.arange(2, 127, 2, dtype=np.uint8)
    s = torch_fp8_decode(even).astype(np.float64) / 2.0 ** k
    row = np.concatenate([[6.0], t, -t, [-6.0]])
    x = row[None, :] * s[:, None]
    bits = torch_bf16(x.astype(np.float32))
    assert np.array_equal(bits_to_f32(bits).astype(np.float64), x)
    return bits, even


@pytest.mark.parametrize("k", [4, 10])
def test_exact_ties(k, golden):
    x, even = tie_tensor(k, golden)
    packed, scales, gs = oracle.quantize(x)
    assert gs == 2.0 ** k
    assert np.array_equal(scales[:, 0], even)
    tie_idx = np.array([int(i) for _, i, _ in golden("e2m1_ties.txt")], np.uint8)
    want = np.concatenate([[7], tie_idx, tie_idx + 8, [15]]).astype(np.uint8)
    assert np.array_equal(unpack_codes(packed), np.tile(want, (len(even), 1)))


def test_c2_injected_blocks_are_exact_ties(golden):
    x = synth.c2_weight()
    blocks, scale, k = synth.c2_tie_info()
    packed, scales, gs = oracle.quantize(x)
    assert gs == 2.0 ** k
    codes = unpack_codes(packed).reshape(-1, 16)[blocks]
    xb = bits_to_f32(x).reshape(-1, 16)[blocks].astype(np.float64)
    ratio = xb / scale.astype(np.float64)[:, None]
    assert np.array_equal(ratio * 4, np.round(ratio * 4))              # quarter steps
    want = nearest_index(np.abs(ratio), golden) + 8 * (ratio < 0)
    assert np.array_equal(codes, want)
    on_mid = np.isin(np.abs(ratio), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert on_mid.sum(1).min() >= 8


# ---------------------------------------------------------------- pack / unpack

def test_unpack_of_every_byte(golden):
    lut = signed_lut(golden)
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    scales = np.full((1, 32), 0x38, np.uint8)                         # block scale 1.0
    y = bits_to_f32(oracle.dequantize(packed, scales, 1.0, 512))[0].astype(np.float64)
    b = np.arange(256)
    assert np.array_equal(y[0::2], lut[b & 15]) and np.array_equal(y[1::2], lut[b >> 4])


def test_pack_unpack_round_trip():
    # every ordered pair of codes, except code 8 (-0 re-quantizes to +0), in blocks
    # whose first byte is 0x77 (+6, +6): block amax 6 -> gs 448, S 0x7E, scale 1.
    codes = [c for c in range(16) if c != 8]
    pairs = np.array([lo | (hi << 4) for lo in codes for hi in codes], np.uint8)
    per_block = 7
    pad = (-len(pairs)) % per_block
    pairs = np.concatenate([pairs, np.full(pad, 0x11, np.uint8)]).reshape(-1, per_block)
    packed = np.concatenate([np.full((len(pairs), 1), 0x77, np.uint8), pairs], 1).reshape(1, -1)
    cols = packed.shape[1] * 2
    scales = np.full((1, cols // 16), 0x7E, np.uint8)
    y = oracle.dequantize(packed, scales, 448.0, cols)
    p2, s2, gs2 = oracle.quantize(y)
    assert gs2 == 448.0
    assert np.array_equal(s2, scales) and np.array_equal(p2, packed)


# ---------------------------------------------------------------- observer

def test_observer_sentinel_and_static():
    seq = np.float32([3.0, 2.0, 5.5, 5.0, 7.25, 1.0, 7.25, 9.0, 0.5, 8.0])
    for mode in (oracle.OBS_STATIC_MINMAX, oracle.OBS_EMA):
        assert oracle.observer(-1.0, 3.0, mode, 0.01) == 3.0
    s, got = -1.0, []
    for c in seq:
        s = oracle.observer(s, float(c), oracle.OBS_STATIC_MINMAX)
        got.append(s)
    assert np.array_equal(np.float32(got), np.maximum.accumulate(seq))


def test_observer_ema_closed_forms():
    assert oracle.observer(2.0, 4.0, oracle.OBS_EMA, 0.5) == 3.0
    assert oracle.observer(4.0, 8.0, oracle.OBS_EMA, 0.25) == 5.0       # 0.75*4 + 0.25*8
    assert oracle.observer(123.0, 7.5, oracle.OBS_EMA, 1.0) == 7.5
    assert oracle.observer(7.5, 123.0, oracle.OBS_EMA, 0.0) == 7.5


def test_observer_ema_within_rounding_of_exact_recurrence():
    rng = np.random.default_rng(11)
    cur = rng.uniform(10, 60, 10).astype(np.float32)
    s, exact = -1.0, None
    for c in cur:
        s = oracle.observer(s, float(c), oracle.OBS_EMA, 0.01)
        d = float(np.float32(0.01))
        exact = float(c) if exact is None else (1 - d) * exact + d * float(c)
    assert abs(s - exact) <= 10 * 3 * 2.0 ** -24 * exact


# The EMA update of the verl QATLinear page, section 5 (_update_input_global_scale):
# new = (1 - d) * old + d * cur on float32 buffers.  Evaluated as torch evaluates it on
# float32 tensors, every operation rounds to float32 on its own: 1 - d, both products,
# then the sum.  numpy float32 scalar arithmetic does exactly that (it never fuses).

def ema_step_f32(state, cur, d):
    """One update in numpy float32, each operation rounded separately (the -1 sentinel
    start stores cur)."""
    state, cur, d = np.float32(state), np.float32(cur), np.float32(d)
    if state < 0:
        return cur
    keep = np.float32(np.float32(1.0) - d)
    return np.float32(np.float32(keep * state) + np.float32(d * cur))


def round_f32(q):
    """An exact rational -> the nearest float32, ties to the even significand."""
    from fractions import Fraction
    f = np.float32(float(q))                          # within one float32 step of q
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    dist = [abs(Fraction(float(c)) - q) for c in cands]
    best = min(dist)
    near = [c for c, e in zip(cands, dist) if e == best]
    return near[0] if len(near) == 1 else [c for c in near if not (int(c.view(np.uint32)) & 1)][0]


def ema_lerp_f32(state, cur, d):
    """A plausible mistake: the lerp form old + d * (cur - old), each step rounded."""
    state, cur, d = np.float32(state), np.float32(cur), np.float32(d)
    if state < 0:
        return cur
    return np.float32(state + np.float32(d * np.float32(cur - state)))


def ema_fma_f32(state, cur, d):
    """A plausible mistake: (1 - d) * old + (d * cur) as one fused multiply-add."""
    from fractions import Fraction
    state, cur, d = np.float32(state), np.float32(cur), np.float32(d)
    if state < 0:
        return cur
    keep = np.float32(np.float32(1.0) - d)
    return round_f32(Fraction(float(keep)) * Fraction(float(state)) + Fraction(float(np.float32(d * cur))))


def ema_sequences():
    """(decay, amax sequence) pairs: the c4 activations' ten step maxima, and seeded random
    sequences over several decades, each starting from the -1 sentinel."""
    c4 = np.float32([oracle.amax(synth.c4_activation(t)) for t in range(10)])
    rng = np.random.default_rng(23)
    seqs = [(0.01, c4)]
    for d in (0.01, 0.25, 0.3, 0.5, 1.0):
        for k in range(4):
            seqs.append((d, np.exp(rng.uniform(-8, 12, 40)).astype(np.float32)))
    return seqs


def test_observer_ema_bit_exact_float32_recurrence():
    """The oracle's EMA equals the float32 step-by-step recurrence bit for bit, and the
    sequences are chosen so that the lerp and fused-multiply-add orders are told apart."""
    lerp_differs = fma_differs = 0
    for d, seq in ema_sequences():
        df = float(np.float32(d))
        s = -1.0
        want = np.float32(-1.0)
        for c in seq:
            prev = want
            s = oracle.observer(s, float(c), oracle.OBS_EMA, df)
            want = ema_step_f32(prev, c, df)
            assert np.float32(s).view(np.uint32) == want.view(np.uint32), (d, c)
            lerp_differs += ema_lerp_f32(prev, c, df) != want
            fma_differs += ema_fma_f32(prev, c, df) != want
    assert lerp_differs > 10 and fma_differs > 10, (lerp_differs, fma_differs)


def test_observer_ema_from_a_prior_state():
    """A state carried over (not the sentinel) steps with the same float32 recurrence."""
    rng = np.random.default_rng(29)
    for d in (0.01, 0.3, 0.7):
        s = np.float32(rng.uniform(1, 100))
        for c in np.exp(rng.uniform(-3, 6, 25)).astype(np.float32):
            got = np.float32(oracle.observer(float(s), float(c), oracle.OBS_EMA, float(np.float32(d))))
            want = ema_step_f32(s, c, float(np.float32(d)))
            assert got.view(np.uint32) == want.view(np.uint32)
            s = want


# ---------------------------------------------------------------- special cases

def test_all_zero_tensor():
    x = np.zeros((4, 64), np.uint16)
    x[1] = 0x8000                                                     # -0.0 row
    assert oracle.amax(x) == 0.0
    packed, scales, gs = oracle.quantize(x)
    assert gs == np.float32(2688.0) / EPS32
    assert not packed.any() and not scales.any()
    assert not oracle.fake_quant(x).any()


def test_zero_block_underflow_block_and_negative_zero_codes():
    x = np.zeros((1, 64), np.float32)
    x[0, 0] = 1.0                                     # amax 1 -> gs 2688
    x[0, 16:32] = 0.0                                 # all-zero block
    x[0, 32:48] = 1e-9                                # block scale underflows to 0x00
    x[0, 33] = -1e-9
    x[0, 48] = 6.0 * 0.0625                           # anchor: scale exactly 0.0625
    x[0, 49] = -0.0625 * 0.1                          # rounds to -0 (code 8)
    x[0, 50] = 0.0625 * 0.1
    bits = torch_bf16(x)
    packed, scales, gs = oracle.quantize(bits, amax_value=1.0)
    codes = unpack_codes(packed)[0]
    assert scales[0, 1] == 0 and not codes[16:32].any()
    assert scales[0, 2] == 0 and codes[32] == 7 and codes[33] == 15 and np.all(codes[34:48] == 7)
    assert codes[49] == 8 and codes[50] == 0
    y = oracle.fake_quant(bits, amax_value=1.0)[0]
    assert np.all(y[32:48] & 0x7FFF == 0) and y[33] == 0x8000 and y[32] == 0x0000
    assert y[49] == 0x8000 and y[50] == 0x0000


# ---------------------------------------------------------------- whole-path re-derivation

def rederive(xbits, amax_value, golden):
    """Every step again from numpy float32 arithmetic, torch's casts and brute-force rounding."""
    x = bits_to_f32(xbits)
    rows, cols = x.shape
    b = x.reshape(rows, cols // 16, 16)
    gs = np.float32(2688.0) / np.maximum(np.float32(amax_value), EPS32)
    v = (np.abs(b).max(-1) / np.float32(6.0)) * gs
    s8 = np.where(v >= 448.0, np.uint8(0x7E), torch_fp8_encode(np.minimum(v, 448.0)))
    sd = torch_fp8_decode(s8) / gs
    sq = np.maximum(sd, EPS32)
    with np.errstate(over="ignore"):
        q = np.clip(b / sq[..., None], np.float32(-6.0), np.float32(6.0))
    code = nearest_index(np.abs(q), golden) + 8 * (q < 0)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).reshape(rows, cols // 2).astype(np.uint8)
    y = torch_bf16(signed_lut(golden).astype(np.float32)[code] * sd[..., None]).reshape(rows, cols)
    return packed, s8.reshape(rows, cols // 16), gs, y


CASES = {
    "c1": lambda: (synth.c1_weight(), None),
    "c2_rows": lambda: (synth.c2_weight()[:96], float(oracle.amax(synth.c2_weight()))),
    "c4_act_low_amax": lambda: (synth.c4_activation(0, tokens=64), 40.0),  # EMA-like: saturating blocks
    "c5_rows": lambda: (synth.c5_weight(rows=48), None),
    "log_uniform": lambda: (log_uniform_bf16(1, (64, 512), -130, 120), None),
    "log_uniform_small_amax": lambda: (log_uniform_bf16(2, (32, 256), -140, -100), None),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_whole_path_rederived_independently(case, golden):
    x, a = CASES[case]()
    a = oracle.amax(x) if a is None else a
    packed, scales, gs = oracle.quantize(x, a)
    p2, s2, gs2, y2 = rederive(x, a, golden)
    assert gs == gs2
    assert np.array_equal(scales, s2)
    assert np.array_equal(packed, p2)
    assert np.array_equal(oracle.fake_quant(x, a), y2)
    assert np.array_equal(oracle.dequantize(packed, scales, gs, x.shape[1]), y2)


def test_rounding_error_within_half_gap():
    x = synth.c1_weight()
    packed, scales, gs = oracle.quantize(x)
    sd = torch_fp8_decode(scales) / gs
    q = bits_to_f32(x).reshape(256, -1, 16) / np.maximum(sd, EPS32)[..., None]
    codes = unpack_codes(packed).reshape(256, -1, 16)
    g = np.float64([0, .5, 1, 1.5, 2, 3, 4, 6])
    got = g[codes & 7] * np.where(codes & 8, -1, 1)
    half_gap = np.where(np.abs(q) < 2, 0.25, np.where(np.abs(q) < 4, 0.5, 1.0))
    assert np.all(np.abs(q - got) <= half_gap)


def test_ragged_columns_are_zero_padded():
    x = synth.c1_weight()[:8, :40]
    pad = np.zeros((8, 48), np.uint16)
    pad[:, :40] = x
    p1, s1, g1 = oracle.quantize(x)
    p2, s2, g2 = oracle.quantize(pad)
    assert p1.shape == (8, 24) and s1.shape == (8, 3)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2) and g1 == g2
    assert np.array_equal(oracle.dequantize(p1, s1, g1, 40), oracle.dequantize(p2, s2, g2, 48)[:, :40])


def test_block_scale_divides_by_six(golden):
    cases = scale_straddle_cases()
    assert len(cases) >= 32
    for a, bmax in cases:
        x = straddle_block(bmax)
        packed, scales, gs = oracle.quantize(x, a)
        p2, s2, gs2, _ = rederive(x, a, golden)
        assert gs == gs2 and scales[0, 0] == s2[0, 0] and np.array_equal(packed, p2)
        wrong = torch_fp8_encode(np.float32([np.float32(bmax) * (np.float32(1) / np.float32(6)) * gs]))
        assert wrong[0] != scales[0, 0]


# ---------------------------------------------------------------- linear over a packed weight

def _packed_weight(n, k, seed):
    rng = np.random.default_rng(seed)
    w = synth.to_bf16_bits((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    return oracle.quantize(w)


def test_linear_one_hot_rows_read_back_the_weight_columns():
    """x = identity: row i of y is column i of dq(W) plus the bias (no transpose, no offset)."""
    n, k = 48, 64
    packed, scales, gs = _packed_weight(n, k, 3)
    bias = synth.to_bf16_bits(np.linspace(-1, 1, n).astype(np.float32))
    eye = np.where(np.eye(k, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    w = oracle.bf16_array_to_f64(oracle.dequantize(packed, scales, gs, k))
    y = oracle.linear(eye, packed, scales, gs, k, bias)
    assert y.shape == (k, n)
    assert np.array_equal(y, w.T + oracle.bf16_array_to_f64(bias)[None, :])
    assert np.array_equal(oracle.linear(eye, packed, scales, gs, k), w.T)


def test_linear_matches_brute_force_loops():
    m, n, k = 3, 5, 32
    packed, scales, gs = _packed_weight(n, k, 4)
    rng = np.random.default_rng(5)
    x = synth.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    bias = synth.to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    wbits = oracle.dequantize(packed, scales, gs, k)
    got = oracle.linear(x, packed, scales, gs, k, bias)
    mag = oracle.linear_magnitude(x, packed, scales, gs, k, bias)
    for i in range(m):
        for j in range(n):
            acc = oracle.bf16_to_f32(int(bias[j]))
            s = abs(acc)
            for t in range(k):
                p = oracle.bf16_to_f32(int(x[i, t])) * oracle.bf16_to_f32(int(wbits[j, t]))
                acc += p
                s += abs(p)
            assert abs(got[i, j] - acc) <= 1e-13 * s
            assert abs(mag[i, j] - s) <= 1e-13 * s


def test_linear_is_linear_in_x():
    n, k = 16, 96
    packed, scales, gs = _packed_weight(n, k, 6)
    rng = np.random.default_rng(7)
    x = synth.to_bf16_bits(rng.standard_normal((4, k)).astype(np.float32))
    twice = (x.astype(np.uint32) + (1 << 7)).astype(np.uint16)      # exponent + 1: exactly 2x
    assert np.array_equal(oracle.bf16_array_to_f64(twice), 2 * oracle.bf16_array_to_f64(x))
    assert np.array_equal(oracle.linear(twice, packed, scales, gs, k),
                          2 * oracle.linear(x, packed, scales, gs, k))
