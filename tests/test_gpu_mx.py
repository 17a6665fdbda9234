"""GPU parity of the MXFP4 variant (32-element blocks, one binary32 scale each, no global
scale) against the oracle, bit for bit: packed codes, the scales' bits and the bf16
outputs of fake-quant and unpack.  Every configuration tensor is compared whole; edge
tensors cover empty and ragged rows, every code times many scales, exact ties, zero,
-0 and underflowing quotients, the 1e-12 clamp, wide dynamic ranges, and a sweep of
every bf16 magnitude around every decision boundary for a range of block maxima.
"""
import numpy as np
import pytest

import oracle
import synth
from cases import log_uniform_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import fp4_block_fake_amd as nv  # noqa: E402
from gpu_util import DEV, assert_same, dev, host, oracle_mx_fake_quant, oracle_mx_quantize, say  # noqa: E402


def check_mx(x, what, big=False):
    """fake-quant, quantize-pack and unpack of x against the oracle, whole tensor."""
    say("mx %s %s" % (what, x.shape))
    xt = dev(x)
    y = nv.nvfp4_mx_fake_quant(xt)
    packed, scales = nv.nvfp4_mx_quantize_pack(xt)
    yd = nv.nvfp4_mx_dequant_unpack(packed, scales, cols=x.shape[1])
    torch.cuda.synchronize()
    if big:
        p_ref, s_ref = oracle_mx_quantize(x)
        y_ref = oracle_mx_fake_quant(x)
    else:
        p_ref, s_ref = oracle.mx_quantize(x)
        y_ref = oracle.mx_fake_quant(x)
    assert_same(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32), what + " scales")
    assert_same(packed.cpu().numpy(), p_ref, what + " packed")
    assert_same(host(y), y_ref, what + " fake-quant")
    assert_same(host(yd), y_ref, what + " dequant-unpack")
    return xt, y


def test_c1_c2_c3():
    check_mx(synth.c1_weight(), "c1")
    check_mx(synth.c2_weight(), "c2", big=True)
    for i, s in enumerate(synth.c3_siblings()):
        check_mx(s, "c3 sibling %d" % i, big=True)


def test_c4_activation_and_weight():
    check_mx(synth.c4_activation(0), "c4 activation step 0", big=True)
    check_mx(synth.c4_weight(), "c4 weight", big=True)


def test_c5_weight_whole():
    x = synth.c5_weight()
    xt, y = check_mx(x, "c5", big=True)
    y2 = nv.nvfp4_mx_fake_quant(xt)                     # determinism
    nv.nvfp4_mx_fake_quant(xt, y=xt)                    # in place
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y.view(torch.int16), xt.view(torch.int16))


MX_RAGGED = [(1, 1), (3, 7), (5, 16), (4, 31), (33, 33), (9, 40), (2, 1000), (7, 4097), (130, 48), (1000, 65),
             (513, 100), (257, 4099)]


@pytest.mark.parametrize("shape", MX_RAGGED)
def test_ragged_rows_zero_padded(shape):
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    x = synth.to_bf16_bits((rng.standard_normal(shape) * np.exp(rng.uniform(-4, 4, shape))).astype(np.float32))
    xt, _ = check_mx(x, "ragged")
    nv.nvfp4_mx_fake_quant(xt, y=xt)
    torch.cuda.synchronize()
    assert_same(host(xt), oracle.mx_fake_quant(x), "ragged in place")


@pytest.mark.parametrize("shape", [(1, 32), (7, 64), (3, 16000), (1037, 160), (515, 32), (64, 8192)])
def test_whole_block_grid_tails(shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    check_mx(synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * 0.05), "tails")


def test_empty():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    y = nv.nvfp4_mx_fake_quant(x)
    packed, scales = nv.nvfp4_mx_quantize_pack(x)
    yd = nv.nvfp4_mx_dequant_unpack(packed, scales)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and packed.shape == (0, 32) and scales.shape == (0, 2) and yd.shape == (0, 64)


def test_every_code_times_many_scales():
    m = np.arange(16, 32, dtype=np.float64)
    e = np.arange(-140, 120, 3, dtype=np.float64)
    s = (m[None, :] * 2.0 ** e[:, None]).reshape(-1)
    lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    row = np.concatenate([lut, -lut, lut[::-1], -lut[::-1]])
    x = np.clip(row[None, :] * s[:, None], -3e38, 3e38)
    check_mx(synth.to_bf16_bits(x.astype(np.float32)), "codes x scales")


def test_ties_zero_and_underflow():
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    s = np.exp2(np.arange(-60, 60, 2, dtype=np.float64)) * 1.25
    row = np.concatenate([[6.0], t, -t, [-6.0], np.zeros(8), np.full(8, -0.0)])
    x = synth.to_bf16_bits((row[None, :] * s[:, None]).astype(np.float32))
    z = np.zeros((4, 96), np.float32)
    z[1, 40] = 3.0e38
    z[1, 41], z[1, 42], z[1, 43] = -1e-40, -1e-6, 1e-6
    z[2, :] = -1e-30
    z[3, 0], z[3, 1], z[3, 2] = 3e-12, 1.2e-12, -2.4e-12
    zb = synth.to_bf16_bits(z)
    zb[0, 5] = 0x8000
    check_mx(x, "ties")
    check_mx(zb, "zero, -0, underflow, clamp")


@pytest.mark.parametrize("seed,lo,hi", [(1, -133, 120), (2, -140, -100), (3, 60, 127), (4, -30, 10)])
def test_wide_dynamic_range(seed, lo, hi):
    check_mx(log_uniform_bf16(seed, (96, 512), lo, hi), "log-uniform %d" % seed)


def boundary_sweep(seed):
    """Blocks whose 31 other elements walk every bf16 magnitude from about 0.2 s to the
    block maximum (s = max / 6), for block maxima over the whole bf16 range, with
    random signs: every decision boundary of every such scale is crossed."""
    rng = np.random.default_rng(seed)
    maxima = np.unique(np.concatenate([
        rng.integers(0x0001, 0x7F80, 120).astype(np.uint16),        # any finite magnitude
        np.arange(0x2B00, 0x2C00, 17, dtype=np.uint16),             # around the 1e-12 clamp
        np.uint16([0x0001, 0x0080, 0x3F80, 0x40C0, 0x7F7F])]))
    blocks = []
    for bm in maxima:
        b = float((np.uint32(bm) << 16).view(np.float32))
        sq = max(np.float32(b) / np.float32(6), np.float32(1e-12))
        lo = int(synth.to_bf16_bits(np.float32([sq * 0.2]))[0]) if sq * 0.2 > 1e-45 else 0
        sweep = np.arange(lo, int(bm) + 1, dtype=np.int64)
        sweep = np.concatenate([sweep, np.arange(0, 40)]).astype(np.uint16)
        sweep = sweep | np.where(rng.random(sweep.size) < 0.5, 0x8000, 0).astype(np.uint16)
        pad = (-sweep.size) % 31
        sweep = np.concatenate([sweep, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        first = np.full((sweep.shape[0], 1), bm, np.uint16)
        blocks.append(np.concatenate([first, sweep], 1))
    return np.concatenate(blocks)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_every_magnitude_around_every_boundary(seed):
    x = boundary_sweep(seed)
    check_mx(x, "boundary sweep %d" % seed, big=True)


def test_every_bf16_magnitude_as_a_block():
    mags = np.arange(1, 0x7F80, dtype=np.uint16)
    rng = np.random.default_rng(8)
    x = np.zeros((mags.size, 32), np.uint16)
    x[:, 0] = mags | np.where(rng.random(mags.size) < 0.5, 0x8000, 0).astype(np.uint16)
    x[:, 17] = (mags >> 1) | 0x8000
    x[:, 31] = np.maximum(mags, 0x0100) - 0x0080
    check_mx(x, "every bf16 magnitude", big=True)


def every_max_and_smaller(lo, hi):
    """Blocks [bm, -0, -m1, -m2, ...] for the bf16 block maxima bm in [lo, hi): after each
    bm come every bf16 magnitude from 0 to bm, negated, 31 per block (zeros pad the last
    block of each bm).  Negative elements exercise the sign rule; a positive element has
    the same magnitude code."""
    bm = np.arange(lo, hi, dtype=np.int64)
    nblk = -(-(bm + 1) // 31)
    owner = np.repeat(bm, nblk)
    first = np.repeat(np.cumsum(nblk) - nblk, nblk)
    k = np.arange(owner.size, dtype=np.int64) - first           # block index within its bm
    mag = k[:, None] * 31 + np.arange(31, dtype=np.int64)[None, :]
    mag = np.where(mag <= owner[:, None], mag, 0).astype(np.uint16) | np.uint16(0x8000)
    return np.concatenate([owner.astype(np.uint16)[:, None], mag], 1)


@pytest.mark.parametrize("lo,hi", [(1, 0x2000), (0x2000, 0x3000), (0x3000, 0x3800), (0x3800, 0x4000),
                                   (0x4000, 0x4800), (0x4800, 0x5000), (0x5000, 0x5800), (0x5800, 0x6000),
                                   (0x6000, 0x6800), (0x6800, 0x7000), (0x7000, 0x7800), (0x7800, 0x7F80)])
def test_every_block_max_with_every_smaller_magnitude(lo, hi):
    """Exhaustive over the element path: every (finite bf16 block maximum, magnitude not
    above it) pair, about 5.3e8 elements over the twelve ranges."""
    x = every_max_and_smaller(lo, hi)
    say("mx exhaustive block maxima [%#x, %#x): %d blocks" % (lo, hi, x.shape[0]))
    xt = dev(x)
    y = nv.nvfp4_mx_fake_quant(xt)
    packed, scales = nv.nvfp4_mx_quantize_pack(xt)
    torch.cuda.synchronize()
    del xt
    p_ref, s_ref = oracle_mx_quantize(x)
    assert_same(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32), "scales")
    assert_same(packed.cpu().numpy(), p_ref, "packed")
    del packed, p_ref
    assert_same(host(y), oracle_mx_fake_quant(x), "fake-quant")


def test_binding_rejects_bad_arguments():
    x = dev(synth.c1_weight())
    with pytest.raises(ValueError):
        nv.nvfp4_mx_fake_quant(x, y=torch.empty((255, 1024), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        nv.nvfp4_mx_quantize_pack(x, scales=torch.empty((256, 32), dtype=torch.float32))
    packed, scales = nv.nvfp4_mx_quantize_pack(x)
    with pytest.raises(ValueError):
        nv.nvfp4_mx_dequant_unpack(packed, scales.cpu())
    with pytest.raises(ValueError):
        nv.nvfp4_mx_dequant_unpack(packed, scales, cols=1100)           # 35 blocks, not 32
    torch.cuda.synchronize()
