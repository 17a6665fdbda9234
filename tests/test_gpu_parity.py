"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, bit for bit.

Tolerance is 0: every amax, global scale, scale byte, code nibble and bf16
output must equal the oracle's.  Workloads are the five seeded configurations,
each compared whole at full size (the large ones against the oracle run over row
shards on the host's cores), and edge tensors: empty, single block, ragged tails of the grid,
all-zero and negative-zero data, underflowing and saturating blocks, every
code times every scale byte, exact ties, a sweep of every bf16 magnitude around
every decision threshold, in-place calls and fused-sibling groups.
"""
import numpy as np
import pytest

import oracle
import synth
from cases import log_uniform_bf16, scale_straddle_cases, straddle_block

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import fp4_block_fake_amd as nv  # noqa: E402

EPS32 = np.float32(1e-12)


# ---------------------------------------------------------------- helpers

from gpu_util import (DEV, assert_same, dev, fbits, host, oracle_amax, oracle_dequantize,  # noqa: E402
                      oracle_fake_quant, oracle_quantize, say, scalar)


def check_all_ops(x, amax_in=None, what=""):
    """fused/cached fake-quant, quantize-pack and dequant-unpack vs the oracle, whole tensor."""
    say("all ops %s %s amax_in=%s" % (what, x.shape, amax_in))
    xt = dev(x)
    a = oracle.amax(x) if amax_in is None else amax_in
    a_in = None if amax_in is None else scalar(amax_in)
    a_out = scalar(-7.0)
    y = nv.nvfp4_fake_quant(xt, amax_in=a_in, amax_out=a_out)
    a_out2 = scalar(-7.0)
    packed, scales, gs = nv.nvfp4_quantize_pack(xt, amax_in=a_in, amax_out=a_out2)
    yd = nv.nvfp4_dequant_unpack(packed, scales, gs, cols=x.shape[1])
    torch.cuda.synchronize()
    p_ref, s_ref, g_ref = oracle.quantize(x, a)
    y_ref = oracle.fake_quant(x, a)
    if amax_in is None:
        assert fbits(a_out.item()) == fbits(a), what + " amax (fake-quant)"
        assert fbits(a_out2.item()) == fbits(a), what + " amax (quantize-pack)"
    assert fbits(gs.item()) == fbits(g_ref), what + " global scale"
    assert_same(scales.cpu().numpy(), s_ref, what + " scales")
    assert_same(packed.cpu().numpy(), p_ref, what + " packed")
    assert_same(host(y), y_ref, what + " fake-quant")
    assert_same(host(yd), y_ref, what + " dequant-unpack")
    return y


# ---------------------------------------------------------------- the five configurations

def test_c1_fused_fake_quant():
    check_all_ops(synth.c1_weight(), what="c1")


def test_c2_all_ops_and_invariant():
    x = synth.c2_weight()
    y = check_all_ops(x, what="c2")
    # the same bytes again (determinism), and in place
    xt = dev(x)
    y2 = nv.nvfp4_fake_quant(xt, amax_out=scalar(0.0))
    nv.nvfp4_fake_quant(xt, y=xt, amax_out=scalar(0.0))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(xt.view(torch.int16), y.view(torch.int16))


def test_c3_shared_sibling_amax():
    sibs = synth.c3_siblings()
    say("c3 grouped amax over %s" % [s.shape for s in sibs])
    ts = [dev(s) for s in sibs]
    shared = nv.nvfp4_amax(ts)
    a_ref = oracle.amax_group(list(sibs))
    assert fbits(shared.item()) == fbits(a_ref)
    assert a_ref == max(oracle.amax(s) for s in sibs)
    for i, (s, t) in enumerate(zip(sibs, ts)):
        y = nv.nvfp4_fake_quant(t, amax_in=shared)
        torch.cuda.synchronize()
        assert_same(host(y), oracle.fake_quant(s, a_ref), "c3 sibling %d" % i)


def test_c4_activation_observers_and_weight():
    state_s, state_e = scalar(-1.0), scalar(-1.0)
    ref_s = ref_e = -1.0
    for step in range(10):
        x = synth.c4_activation(step)
        say("c4 step %d" % step)
        xt = dev(x)
        cur = nv.nvfp4_amax(xt)
        nv.nvfp4_observer_update(state_s, cur, nv.OBS_STATIC_MINMAX)
        nv.nvfp4_observer_update(state_e, cur, nv.OBS_EMA, 0.01)
        y_s = nv.nvfp4_fake_quant(xt, amax_in=state_s)
        y_e = nv.nvfp4_fake_quant(xt, amax_in=state_e)
        torch.cuda.synchronize()
        a = oracle.amax(x)
        ref_s = oracle.observer(ref_s, a, oracle.OBS_STATIC_MINMAX)
        ref_e = oracle.observer(ref_e, a, oracle.OBS_EMA, np.float32(0.01))
        assert fbits(cur.item()) == fbits(a), "step %d amax" % step
        assert fbits(state_s.item()) == fbits(ref_s), "step %d static state" % step
        assert fbits(state_e.item()) == fbits(ref_e), "step %d ema state" % step
        assert_same(host(y_s), oracle_fake_quant(x, ref_s), "step %d static fq" % step)
        assert_same(host(y_e), oracle_fake_quant(x, ref_e), "step %d ema fq" % step)
    w = synth.c4_weight()
    say("c4 weight %s" % (w.shape,))
    amax = scalar(0.0)
    y = nv.nvfp4_fake_quant(dev(w), amax_out=amax)
    torch.cuda.synchronize()
    a = oracle_amax(w)
    assert fbits(amax.item()) == fbits(a)
    assert_same(host(y), oracle_fake_quant(w, a), "c4 weight fq")


def test_c5_large_weight_full_path():
    w = synth.c5_weight()
    say("c5 %s" % (w.shape,))
    xt = dev(w)
    a_q, a_f = scalar(0.0), scalar(0.0)
    packed, scales, gs = nv.nvfp4_quantize_pack(xt, amax_out=a_q)
    yd = nv.nvfp4_dequant_unpack(packed, scales, gs)
    y = nv.nvfp4_fake_quant(xt, amax_out=a_f)
    torch.cuda.synchronize()
    a = oracle_amax(w)
    assert fbits(a_q.item()) == fbits(a) and fbits(a_f.item()) == fbits(a)
    p_ref, s_ref, g_ref = oracle_quantize(w, a)
    assert fbits(gs.item()) == fbits(g_ref)
    assert_same(packed.cpu().numpy(), p_ref, "c5 packed")
    assert_same(scales.cpu().numpy(), s_ref, "c5 scales")
    del packed, scales
    y_ref = oracle_fake_quant(w, a)
    assert_same(host(y), y_ref, "c5 fake-quant")
    assert_same(host(yd), y_ref, "c5 dequant-unpack of the device codes")
    del y, yd
    # the unpack alone, on the oracle's own codes and scales
    yo = nv.nvfp4_dequant_unpack(torch.from_numpy(p_ref).to(DEV), torch.from_numpy(s_ref).to(DEV), scalar(g_ref))
    torch.cuda.synchronize()
    assert_same(host(yo), oracle_dequantize(p_ref, s_ref, g_ref, w.shape[1]), "c5 dequant-unpack of the oracle's codes")


def test_c5_row_shards_with_the_all_reduced_amax():
    """c5 under 8-way row sharding ([3584, 8192] per rank), the part one GPU can show:
    each shard's amax, their maximum (the all-reduce), then each shard quantized with
    it through the cached-amax calls gives exactly the rows of the whole tensor's
    result."""
    w = synth.c5_weight()
    say("c5 row shards %s" % (w.shape,))
    xt = dev(w)
    packed, scales, gs = nv.nvfp4_quantize_pack(xt)
    y = nv.nvfp4_fake_quant(xt)
    rows = w.shape[0] // 8
    shard_amax = [nv.nvfp4_amax(xt[r * rows:(r + 1) * rows]) for r in range(8)]
    global_amax = scalar(-1.0)
    for a in shard_amax:                       # the MAX all-reduce of one fp32 per rank
        torch.maximum(global_amax, a, out=global_amax)
    torch.cuda.synchronize()
    assert fbits(global_amax.item()) == fbits(oracle.amax(w))
    for r in (0, 3, 7):
        shard = xt[r * rows:(r + 1) * rows]
        p_s, s_s, g_s = nv.nvfp4_quantize_pack(shard, amax_in=global_amax)
        y_s = nv.nvfp4_fake_quant(shard, amax_in=global_amax)
        torch.cuda.synchronize()
        assert fbits(g_s.item()) == fbits(gs.item())
        assert torch.equal(p_s, packed[r * rows:(r + 1) * rows])
        assert torch.equal(s_s, scales[r * rows:(r + 1) * rows])
        assert torch.equal(y_s.view(torch.int16), y[r * rows:(r + 1) * rows].view(torch.int16))
    assert_same(host(y[7 * rows:]), oracle_fake_quant(w[7 * rows:], oracle_amax(w)), "shard 7 against the oracle")


# ---------------------------------------------------------------- edge tensors

@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (5, 15), (4, 17), (33, 40), (9, 1000), (2, 4097),
                                   (130, 24), (1000, 33), (2, 2), (7, 18), (64, 4100), (1025, 30), (17, 1006),
                                   (300, 62), (513, 8)])
def test_ragged_columns_zero_padded(shape):
    """Rows not a multiple of 16: zero-padded blocks, padded code/scale layout, cols outputs.
    Both go through the half-block kernels, with element-wise accesses for odd lengths and
    dword accesses for even ones (a half may lie wholly in the padding, as for 18 or 8
    columns)."""
    rng = np.random.default_rng(shape[0] * 131 + shape[1])
    x = synth.to_bf16_bits((rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, shape))).astype(np.float32))
    check_all_ops(x, what="ragged cols")
    check_all_ops(x, amax_in=float(np.float32(0.75)), what="ragged cols, cached amax")
    xt = dev(x)
    nv.nvfp4_fake_quant(xt, y=xt, amax_out=scalar(0.0))          # in place
    torch.cuda.synchronize()
    assert_same(host(xt), oracle.fake_quant(x), "ragged in place")


@pytest.mark.parametrize("shape", [(1, 16), (7, 48), (3, 16000), (1037, 144), (515, 16)])
def test_ragged_grid_tails(shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    x = synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.05)
    check_all_ops(x, what="ragged")


def test_empty_tensor():
    say("empty")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    a = scalar(-3.0)
    y = nv.nvfp4_fake_quant(x, amax_out=a)
    packed, scales, gs = nv.nvfp4_quantize_pack(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and packed.shape == (0, 32) and scales.shape == (0, 4)
    assert fbits(a.item()) == 0
    assert fbits(gs.item()) == fbits(oracle.global_scale(0.0))
    z = nv.nvfp4_amax([torch.empty(0, dtype=torch.bfloat16, device=DEV)])
    torch.cuda.synchronize()
    assert fbits(z.item()) == 0


def test_zero_and_negative_zero_tensor():
    x = np.zeros((5, 64), np.uint16)
    x[1::2] = 0x8000
    check_all_ops(x, what="zeros")


def test_underflow_and_negative_zero_codes():
    v = np.zeros((2, 64), np.float32)
    v[0, 0] = 1.0
    v[0, 32:48] = 1e-9
    v[0, 33] = -1e-9
    v[0, 48] = 6.0 * 0.0625
    v[0, 49] = -0.0625 * 0.1
    v[1, :16] = -1e-30
    v[1, 16:32] = np.float32(-2.0) ** -np.arange(120, 136)
    check_all_ops(synth.to_bf16_bits(v), what="underflow")


@pytest.mark.parametrize("k", [4, 10, 12])
def test_every_code_times_every_scale(k):
    s = oracle.e4m3_decode_array(np.arange(1, 127, dtype=np.uint8)).astype(np.float64) / 2.0 ** k
    lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    x = np.concatenate([lut, -lut])[None, :] * s[:, None]
    check_all_ops(synth.to_bf16_bits(x.astype(np.float32)), what="codes x scales k=%d" % k)


def test_exact_ties():
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    even = np.arange(2, 127, 2, dtype=np.uint8)
    s = oracle.e4m3_decode_array(even).astype(np.float64) / 1024.0
    row = np.concatenate([[6.0], t, -t, [-6.0]])
    check_all_ops(synth.to_bf16_bits((row[None, :] * s[:, None]).astype(np.float32)), what="ties")


@pytest.mark.parametrize("seed,lo,hi", [(1, -133, 120), (2, -140, -100), (3, 60, 127), (4, -30, 10)])
def test_wide_dynamic_range(seed, lo, hi):
    check_all_ops(log_uniform_bf16(seed, (96, 512), lo, hi), what="log-uniform %d" % seed)


@pytest.mark.parametrize("amax_in", [1e-20, 3e-12, 0.01, 0.37, 6.0, 12345.6, 5e20, 3.3e38])
def test_cached_amax_saturation_and_clamp(amax_in):
    x = synth.c2_weight()[:256]
    check_all_ops(x, amax_in=float(np.float32(amax_in)), what="cached amax")


def threshold_sweep(amax_value):
    """Blocks whose other 15 elements walk every bf16 magnitude around the seven decision
    thresholds (and the zero threshold) of each scale byte, with that byte's block max first."""
    mags = np.arange(1, 0x7F80, dtype=np.uint16)
    single = np.zeros((mags.size, 16), np.uint16)
    single[:, 0] = mags
    _, s_of, gs = oracle.quantize(single, amax_value)
    s_of = s_of[:, 0]
    rng = np.random.default_rng(int(fbits(amax_value)) & 0xFFFF)
    blocks = []
    for s in np.unique(s_of):
        anchor = int(mags[np.flatnonzero(s_of == s)[-1]])
        sd = np.float32(oracle.e4m3_decode(int(s))) / gs
        sq = max(sd, EPS32)
        lo = int(synth.to_bf16_bits(np.float32([sq * 0.2]))[0])
        hi = int(synth.to_bf16_bits(np.float32([min(sq * 6.5, 3e38)]))[0])
        sweep = np.arange(lo, min(hi, anchor) + 1)
        sweep = np.concatenate([sweep, np.arange(max(0, anchor - 64), anchor + 1), np.arange(0, 40)])
        sweep = sweep[sweep <= anchor].astype(np.uint16)
        sweep = sweep | np.where(rng.random(sweep.size) < 0.5, 0x8000, 0).astype(np.uint16)
        pad = (-sweep.size) % 15
        sweep = np.concatenate([sweep, np.zeros(pad, np.uint16)]).reshape(-1, 15)
        first = np.full((sweep.shape[0], 1), anchor, np.uint16)
        blocks.append(np.concatenate([first, sweep], 1))
    return np.concatenate(blocks)


@pytest.mark.parametrize("amax_value", [2.625, 2688.0 / 16, 1.0, 0.37, 1.7e-5, 12345.6, 5e20, 3e-11,
                                        196.0, 5.5, 1000.0, 7.0])
def test_every_magnitude_around_every_threshold(amax_value):
    """The last four amax values give global scales under which 1 / sq rounded fails
    the fast-path check for 14-47 of the 126 scale bytes, so the kernels use a
    neighbouring multiplier there (196 is the c4 activations' amax)."""
    a = float(np.float32(amax_value))
    x = threshold_sweep(a)
    check_all_ops(x, amax_in=a, what="threshold sweep")


SWEEP_AMAX = [2.625, 2688.0 / 16, 1.0, 0.37, 1.7e-5, 12345.6, 5e20, 3e-11, 196.0, 5.5, 1000.0, 7.0]


@pytest.mark.parametrize("amax_value", SWEEP_AMAX)
def test_every_bf16_magnitude_as_a_block(amax_value):
    """Each finite bf16 magnitude as the largest element of its own block (the other 15
    elements zero), with random signs, under a given amax: the block's scale byte runs
    the binary64 divide by 6 and the E4M3 converter on every possible block maximum, and
    its code the element path, all against the oracle."""
    a = float(np.float32(amax_value))
    mags = np.arange(1, 0x7F80, dtype=np.uint16)
    rng = np.random.default_rng(int(fbits(a)) & 0xFFFF)
    x = np.zeros((mags.size, 16), np.uint16)
    x[:, 0] = mags | np.where(rng.random(mags.size) < 0.5, 0x8000, 0).astype(np.uint16)
    x[:, 9] = (mags >> 1) | 0x8000
    check_all_ops(x, amax_in=a, what="every bf16 magnitude")


# ---------------------------------------------------------------- amax groups and observers

def test_amax_groups_tails_and_accumulate():
    rng = np.random.default_rng(9)
    sizes = [1, 7, 8, 9, 0, 4095, 4096 * 3 + 5, 16, 100003, 3, 64, 1 << 18]
    arrs = [synth.to_bf16_bits(rng.standard_normal(n).astype(np.float32) * (1 + i)) for i, n in enumerate(sizes)]
    arrs[5][-1] = 0x4480   # a large value in a tail element
    ts = [dev(a) for a in arrs]
    say("amax group of %d tensors" % len(ts))
    got = nv.nvfp4_amax(ts)
    prior = scalar(-1.0)
    nv.nvfp4_amax(ts, amax=prior, accumulate=True)
    big = scalar(1e30)
    nv.nvfp4_amax(ts, amax=big, accumulate=True)
    torch.cuda.synchronize()
    want = oracle.amax_group(arrs)
    assert fbits(got.item()) == fbits(want)
    assert fbits(prior.item()) == fbits(want)
    assert fbits(big.item()) == fbits(np.float32(1e30))
    for a, t in zip(arrs, ts):
        one = nv.nvfp4_amax(t)
        torch.cuda.synchronize()
        assert fbits(one.item()) == fbits(oracle.amax(a))


def test_amax_buffer_reused_after_a_larger_result():
    """A workgroup skips its atomic when the buffer already holds at least its own
    maximum; a result left by an earlier call must never count as such a value."""
    rng = np.random.default_rng(19)
    big = synth.to_bf16_bits(rng.standard_normal((2048, 4096)).astype(np.float32) * 8)
    small = synth.to_bf16_bits(rng.standard_normal((2048, 4096)).astype(np.float32) * 0.01)
    tb, ts = dev(big), dev(small)
    buf = scalar(0.0)
    say("amax buffer reuse, 2048x4096")
    for _ in range(3):
        nv.nvfp4_amax(tb, amax=buf)
        nv.nvfp4_amax(ts, amax=buf)
        torch.cuda.synchronize()
        assert fbits(buf.item()) == fbits(oracle.amax(small))
        nv.nvfp4_amax(tb, amax=buf)
        y = nv.nvfp4_fake_quant(ts, amax_out=buf)
        torch.cuda.synchronize()
        assert fbits(buf.item()) == fbits(oracle.amax(small))
        assert_same(host(y), oracle.fake_quant(small, oracle.amax(small)), "fake-quant after reuse")
        nv.nvfp4_amax(tb, amax=buf)
        _, _, gs = nv.nvfp4_quantize_pack(ts, amax_out=buf)
        torch.cuda.synchronize()
        assert fbits(buf.item()) == fbits(oracle.amax(small))
        assert fbits(gs.item()) == fbits(oracle.global_scale(oracle.amax(small)))


@pytest.mark.parametrize("decay", [0.01, 0.3, 1.0])
def test_observer_sequences(decay):
    cur = np.float32([3.5, 2.0, 7.25, 1e-3, 40.0, 39.0, 0.0, 55.5, 12.0, 13.0])
    st_s, st_e = scalar(-1.0), scalar(-1.0)
    rs = re = -1.0
    for c in cur:
        ct = scalar(float(c))
        nv.nvfp4_observer_update(st_s, ct, nv.OBS_STATIC_MINMAX)
        nv.nvfp4_observer_update(st_e, ct, nv.OBS_EMA, decay)
        torch.cuda.synchronize()
        rs = oracle.observer(rs, float(c), oracle.OBS_STATIC_MINMAX)
        re = oracle.observer(re, float(c), oracle.OBS_EMA, float(np.float32(decay)))
        assert fbits(st_s.item()) == fbits(rs)
        assert fbits(st_e.item()) == fbits(re)


def test_ste_backward_is_identity():
    x = dev(synth.c1_weight()).requires_grad_(True)
    y = nv.FakeQuantSTE.apply(x)
    g = torch.randn_like(y)
    y.backward(g)
    torch.cuda.synchronize()
    assert torch.equal(x.grad.view(torch.int16), g.view(torch.int16))
    assert_same(host(y.detach()), oracle.fake_quant(synth.c1_weight()), "ste forward")


def test_block_scale_divide_by_six_straddles():
    """Blocks where an IEEE divide by 6 and a reciprocal multiply give different E4M3 bytes."""
    cases = scale_straddle_cases()
    assert len(cases) >= 32
    for a, bmax in cases:
        check_all_ops(straddle_block(bmax), amax_in=a, what="straddle")


def test_more_than_2pow31_elements():
    """64-bit indexing: 67000 x 32768 bf16 (2.2e9 elements, 4.4 GB), whole against the oracle
    in chunks of rows."""
    rows, cols = 67000, 32768
    rng = np.random.default_rng(77)
    tile = synth.normal_bf16(77, (64, cols), 0.02)
    x = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, 64):                      # the tile, with a per-chunk exponent shift
        n = min(64, rows - r0)
        shift = np.uint16(int(rng.integers(0, 8)) << 7)
        x[r0:r0 + n] = np.where((tile[:n] & 0x7FFF) != 0, tile[:n] + shift, tile[:n])
    say("2^31+ elements: %dx%d" % (rows, cols))
    xt = dev(x)
    amax = scalar(0.0)
    y = nv.nvfp4_fake_quant(xt, amax_out=amax)
    packed, scales, gs = nv.nvfp4_quantize_pack(xt, amax_in=amax)
    torch.cuda.synchronize()
    a = oracle_amax(x)
    assert fbits(amax.item()) == fbits(a)
    assert fbits(gs.item()) == fbits(oracle.global_scale(a))
    step = 4096
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        say("2^31+ rows %d..%d" % (r0, r1))
        p_ref, s_ref, _ = oracle_quantize(x[r0:r1], a)
        assert_same(packed[r0:r1].cpu().numpy(), p_ref, "2^31+ packed rows %d.." % r0)
        assert_same(scales[r0:r1].cpu().numpy(), s_ref, "2^31+ scale rows %d.." % r0)
        assert_same(host(y[r0:r1]), oracle_fake_quant(x[r0:r1], a), "2^31+ fake-quant rows %d.." % r0)
