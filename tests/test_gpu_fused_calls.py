"""GPU parity of the one-launch calls against the CPU oracle, bit for bit.

nvfp4_fake_quant_group must give, for every member, the oracle's fake-quant of
that member with the shared amax of the whole group (verl QATLinear page,
section 4); nvfp4_fake_quant_dual must give the oracle's fake-quant of x under
each of its two amaxes (section 5).  The oracle has no notion of launches, so
these are the same expected values as for one call per tensor.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import fp4_block_fake_amd as nv  # noqa: E402
from gpu_util import DEV, assert_same, dev, fbits, host, oracle_fake_quant, say, scalar  # noqa: E402


def random_bf16(rng, shape, spread=3.0):
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, shape))
    return synth.to_bf16_bits(x.astype(np.float32))


# ---------------------------------------------------------------- group

def test_group_c3_siblings_shared_amax():
    sibs = list(synth.c3_siblings())
    say("group fake-quant c3 %s" % [s.shape for s in sibs])
    ts = [dev(s) for s in sibs]
    a_ref = oracle.amax_group(sibs)
    amax = scalar(-3.0)
    ys = nv.nvfp4_fake_quant_group(ts, amax_out=amax)
    torch.cuda.synchronize()
    assert fbits(amax.item()) == fbits(a_ref)
    for i, (s, y) in enumerate(zip(sibs, ys)):
        assert_same(host(y), oracle.fake_quant(s, a_ref), "c3 group member %d" % i)
    # the same with the amax given, into preallocated outputs
    ys2 = [torch.empty_like(t) for t in ts]
    nv.nvfp4_fake_quant_group(ts, ys=ys2, amax_in=amax)
    torch.cuda.synchronize()
    for y, y2 in zip(ys, ys2):
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


# Shapes chosen to exercise: chunk boundaries (a chunk is 1024 blocks), tensors
# smaller than one chunk, empty members, ragged rows (their own launches), more
# members than one launch takes, and an in-place member.
MIXED = [(64, 256), (0, 32), (1, 16), (3, 20), (1024, 16), (1025, 16), (37, 4096), (5, 33), (512, 48),
         (2, 16), (129, 1024), (7, 1), (300, 160)]


@pytest.mark.parametrize("given", [False, True])
def test_group_mixed_members(given):
    rng = np.random.default_rng(77 + given)
    xs = [random_bf16(rng, s) for s in MIXED]
    xs[6][5, 7] = 0x4500          # 2048: the group maximum sits in one member
    a_ref = oracle.amax_group(xs) if not given else float(np.float32(0.5))
    say("group of %d mixed members, amax %s" % (len(xs), "given" if given else "computed"))
    ts = [dev(x) for x in xs]
    ys = [torch.empty_like(t) for t in ts]
    ys[4] = ts[4]                 # in place
    amax = scalar(a_ref) if given else scalar(0.0)
    nv.nvfp4_fake_quant_group(ts, ys=ys, amax_in=amax if given else None,
                              amax_out=None if given else amax)
    torch.cuda.synchronize()
    assert fbits(amax.item()) == fbits(a_ref)
    for i, (x, y) in enumerate(zip(xs, ys)):
        assert_same(host(y), oracle.fake_quant(x, a_ref), "member %d %s" % (i, x.shape))


def test_group_of_one_equals_single_call():
    rng = np.random.default_rng(5)
    x = random_bf16(rng, (333, 512))
    t = dev(x)
    (yg,) = nv.nvfp4_fake_quant_group([t])
    y1 = nv.nvfp4_fake_quant(t)
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int16), y1.view(torch.int16))
    assert_same(host(yg), oracle.fake_quant(x), "group of one")


# ---------------------------------------------------------------- dual

def test_dual_c4_activation_two_observers():
    """Steps 0 and 1 of the c4 activation stream with both observers; the fake-quant of
    step 1 under the two states comes from one read of x."""
    x0, x1 = synth.c4_activation(0), synth.c4_activation(1)
    say("dual fake-quant c4 %s" % (x1.shape,))
    rs = re = -1.0
    for x in (x0, x1):
        a = oracle.amax(x)
        rs = oracle.observer(rs, a, oracle.OBS_STATIC_MINMAX)
        re = oracle.observer(re, a, oracle.OBS_EMA, np.float32(0.01))
    assert rs != re
    xt = dev(x1)
    y_s, y_e = nv.nvfp4_fake_quant_dual(xt, scalar(rs), scalar(re))
    torch.cuda.synchronize()
    assert_same(host(y_s), oracle_fake_quant(x1, rs), "dual static")
    assert_same(host(y_e), oracle_fake_quant(x1, re), "dual ema")
    # whole tensors against the single-output kernel
    z_s = nv.nvfp4_fake_quant(xt, amax_in=scalar(rs))
    z_e = nv.nvfp4_fake_quant(xt, amax_in=scalar(re))
    torch.cuda.synchronize()
    assert torch.equal(y_s.view(torch.int16), z_s.view(torch.int16))
    assert torch.equal(y_e.view(torch.int16), z_e.view(torch.int16))


@pytest.mark.parametrize("shape", [(1, 16), (3, 20), (515, 16), (64, 4096), (33, 40), (1037, 144)])
@pytest.mark.parametrize("inplace", [None, 0, 1])
def test_dual_shapes_and_in_place(shape, inplace):
    rng = np.random.default_rng(shape[0] * 3 + shape[1] + 11 * (inplace or 0))
    x = random_bf16(rng, shape)
    a0 = oracle.amax(x)
    a1 = float(np.float32(a0 * 0.3))          # below the max: saturated blocks
    say("dual %s in place %s" % (shape, inplace))
    xt = dev(x)
    y0 = xt if inplace == 0 else torch.empty_like(xt)
    y1 = xt if inplace == 1 else torch.empty_like(xt)
    nv.nvfp4_fake_quant_dual(xt, scalar(a0), scalar(a1), y0=y0, y1=y1)
    torch.cuda.synchronize()
    assert_same(host(y0), oracle.fake_quant(x, a0), "dual y0")
    assert_same(host(y1), oracle.fake_quant(x, a1), "dual y1")


def test_dual_rejects_shared_output():
    t = torch.zeros((4, 16), dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(t)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_fake_quant_dual(t, scalar(1.0), scalar(1.0), y0=y, y1=y)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_fake_quant_dual(t, scalar(1.0), scalar(1.0), y0=t, y1=t)
