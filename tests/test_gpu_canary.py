"""Canary bytes around every output buffer, for every call that writes device memory.

Each output is a view into a larger buffer whose guard zones before and after hold
seeded random bytes; the view starts at the smallest alignment the call accepts (so a
16-byte aligned output is not 32-byte aligned, a scale array starts at an odd address).
Before the call the output itself holds garbage.  After it the guard bytes must be
unchanged (no stray or out-of-bounds write, also on the ragged tails), and the output
must be the oracle's, bit for bit; the linear layer, whose expected value is a rounding
bound, must equal an unguarded call of the same shape instead (the same kernel, so the
same bits).  Scalars (amax, gs, observer states) and the workspace are guarded the same
way.
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
from gpu_util import DEV, assert_same, dev, fbits, host, say  # noqa: E402

GUARD = 4096        # bytes of canary on each side


class Guarded:
    """A device byte buffer: canary, then `nbytes` of output starting `skew` bytes past a
    512-byte boundary (torch's allocations are 512-byte aligned), then canary."""

    def __init__(self, nbytes, skew, seed):
        self.lo = GUARD + skew
        self.nbytes = nbytes
        total = self.lo + nbytes + GUARD
        rng = np.random.default_rng(seed)
        self.canary = rng.integers(0, 256, total, dtype=np.uint8)
        self.canary[self.lo:self.lo + nbytes] = 0xFF          # garbage in the output itself
        self.buf = torch.from_numpy(self.canary.copy()).to(DEV)

    def view(self, dtype, shape):
        inner = self.buf[self.lo:self.lo + self.nbytes]
        return inner.view(dtype).view(shape)

    def check(self, what):
        got = self.buf.cpu().numpy()
        want = self.canary
        before = np.flatnonzero(got[:self.lo] != want[:self.lo])
        after = np.flatnonzero(got[self.lo + self.nbytes:] != want[self.lo + self.nbytes:])
        assert before.size == 0, "%s: %d canary bytes changed before the output, nearest %d bytes before it" % (
            what, before.size, self.lo - before[-1])
        assert after.size == 0, "%s: %d canary bytes changed after the output, first %d bytes after it" % (
            what, after.size, after[0])


def bf16_out(shape, seed, skew=16):
    g = Guarded(2 * shape[0] * shape[1], skew, seed)
    return g, g.view(torch.bfloat16, shape)


def u8_out(shape, seed, skew):
    g = Guarded(shape[0] * shape[1], skew, seed)
    return g, g.view(torch.uint8, shape)


def f32_out(seed, fill=None):
    g = Guarded(4, 4, seed)
    t = g.view(torch.float32, (1,))
    if fill is not None:
        t.fill_(fill)
    return g, t


def random_bf16(rng, shape, spread=3.0):
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, shape))
    return synth.to_bf16_bits(x.astype(np.float32))


# ragged rows (cols % 16 != 0, and cols < 16; odd lengths, whose odd rows start on an
# odd element, among them ending the tensor), chunk edges, a single block, wide rows,
# a tensor large enough for the persistent multi-workgroup grids, and empty tensors
SHAPES = [(1, 16), (3, 20), (7, 1), (33, 40), (1025, 16), (1037, 144), (64, 4096), (2048, 2064), (0, 16),
          (5, 18), (129, 4100), (6, 17), (66, 1001), (130, 4097)]


def inputs(shape, seed):
    rng = np.random.default_rng(seed)
    x = random_bf16(rng, shape)
    return x, dev(x)


@pytest.mark.parametrize("shape", SHAPES)
def test_fake_quant_calls(shape):
    x, xt = inputs(shape, 1000 + shape[0] + shape[1])
    a = oracle.amax(x) if x.size else 0.0
    want = oracle.fake_quant(x, a) if x.size else x
    say("canary fake_quant %s" % (shape,))

    gy, y = bf16_out(shape, 1)
    ga, amax = f32_out(2)
    nv.nvfp4_fake_quant(xt, y=y, amax_out=amax)
    torch.cuda.synchronize()
    gy.check("fake_quant y")
    ga.check("fake_quant amax_out")
    assert fbits(amax.item()) == fbits(a)
    assert_same(host(y), want, "fake_quant")

    gy, y = bf16_out(shape, 3)
    nv.nvfp4_fake_quant(xt, y=y, amax_in=oracle_amax_dev(a))
    torch.cuda.synchronize()
    gy.check("fake_quant (amax given) y")
    assert_same(host(y), want, "fake_quant, amax given")

    gy, y = bf16_out(shape, 4)
    ga, amax = f32_out(5)
    gw = Guarded(nv.WORKSPACE_BYTES, 0, 6)
    ws = gw.view(torch.uint8, (nv.WORKSPACE_BYTES,))
    nv.nvfp4_fake_quant_ws(xt, y=y, amax_out=amax, workspace=ws)
    torch.cuda.synchronize()
    gy.check("fake_quant_ws y")
    ga.check("fake_quant_ws amax_out")
    gw.check("fake_quant_ws workspace")
    assert fbits(amax.item()) == fbits(a)
    assert_same(host(y), want, "fake_quant_ws")


def oracle_amax_dev(a):
    return torch.tensor([a], dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_pack_and_unpack(shape):
    x, xt = inputs(shape, 2000 + shape[0] + shape[1])
    a = oracle.amax(x) if x.size else 0.0
    p_ref, s_ref, g_ref = oracle.quantize(x, a)
    nbr = nv.blocks_per_row(shape[1])
    say("canary quantize_pack / dequant_unpack %s" % (shape,))

    for ws_call in (False, True):
        what = "quantize_pack_ws" if ws_call else "quantize_pack"
        gp, packed = u8_out((shape[0], 8 * nbr), 10 + ws_call, skew=8)
        gsc, scales = u8_out((shape[0], nbr), 12 + ws_call, skew=1)
        gg, gs = f32_out(14 + ws_call)
        ga, amax = f32_out(16 + ws_call)
        if ws_call:
            gw = Guarded(nv.WORKSPACE_BYTES, 0, 18)
            ws = gw.view(torch.uint8, (nv.WORKSPACE_BYTES,))
            nv.nvfp4_quantize_pack_ws(xt, amax_out=amax, packed=packed, scales=scales, global_scale=gs,
                                      workspace=ws)
        else:
            nv.nvfp4_quantize_pack(xt, amax_out=amax, packed=packed, scales=scales, global_scale=gs)
        torch.cuda.synchronize()
        for g, name in ((gp, "packed"), (gsc, "scales"), (gg, "global_scale"), (ga, "amax_out")):
            g.check("%s %s" % (what, name))
        if ws_call:
            gw.check("%s workspace" % what)
        assert fbits(amax.item()) == fbits(a) and fbits(gs.item()) == fbits(g_ref)
        assert_same(packed.cpu().numpy(), p_ref, what + " packed")
        assert_same(scales.cpu().numpy(), s_ref, what + " scales")

    gy, y = bf16_out(shape, 20)
    nv.nvfp4_dequant_unpack(packed, scales, gs, y=y, cols=shape[1])
    torch.cuda.synchronize()
    gy.check("dequant_unpack y")
    if x.size:
        assert_same(host(y), oracle.dequantize(p_ref, s_ref, g_ref, shape[1]), "dequant_unpack")


@pytest.mark.parametrize("shape", [(3, 20), (1037, 144), (2048, 2064), (0, 16)])
def test_dual_and_observe(shape):
    x, xt = inputs(shape, 3000 + shape[0] + shape[1])
    a = oracle.amax(x) if x.size else 0.0
    a0, a1 = float(np.float32(2.0 * a + 1.0)), float(np.float32(0.5 * a + 0.25))
    say("canary dual / observe %s" % (shape,))

    g0, y0 = bf16_out(shape, 30)
    g1, y1 = bf16_out(shape, 31)
    nv.nvfp4_fake_quant_dual(xt, oracle_amax_dev(a0), oracle_amax_dev(a1), y0=y0, y1=y1)
    torch.cuda.synchronize()
    g0.check("dual y0")
    g1.check("dual y1")
    if x.size:
        assert_same(host(y0), oracle.fake_quant(x, a0), "dual y0")
        assert_same(host(y1), oracle.fake_quant(x, a1), "dual y1")

    d = float(np.float32(0.25))
    gs0, s0 = f32_out(32, fill=a0)
    gs1, s1 = f32_out(33, fill=a1)
    gc, cur = f32_out(34)
    g0, y0 = bf16_out(shape, 35)
    g1, y1 = bf16_out(shape, 36)
    gw = Guarded(nv.WORKSPACE_BYTES, 0, 37)
    ws = gw.view(torch.uint8, (nv.WORKSPACE_BYTES,))
    nv.nvfp4_observe_fake_quant(xt, s0, nv.OBS_STATIC_MINMAX, 0.0, s1, nv.OBS_EMA, 0.25, y0=y0, y1=y1,
                                cur=cur, workspace=ws)
    torch.cuda.synchronize()
    r0 = oracle.observer(a0, a, oracle.OBS_STATIC_MINMAX)
    r1 = oracle.observer(a1, a, oracle.OBS_EMA, d)
    for g, name in ((g0, "y0"), (g1, "y1"), (gc, "cur"), (gw, "workspace"), (gs0, "state0"), (gs1, "state1")):
        g.check("observe " + name)
    assert fbits(cur.item()) == fbits(a)
    assert fbits(s0.item()) == fbits(r0) and fbits(s1.item()) == fbits(r1)
    if x.size:
        assert_same(host(y0), oracle.fake_quant(x, r0), "observe y0")
        assert_same(host(y1), oracle.fake_quant(x, r1), "observe y1")

    gs0, s0 = f32_out(38, fill=a0)
    gc, cur2 = f32_out(39, fill=a)
    nv.nvfp4_observer_update(s0, cur2, nv.OBS_EMA, 0.25)
    torch.cuda.synchronize()
    gc.check("observer_update cur")
    want = oracle.observer(a0, a, oracle.OBS_EMA, d)
    assert fbits(s0.item()) == fbits(want)
    gs0.check("observer_update state")


GROUP = [(64, 256), (0, 32), (3, 20), (1025, 16), (37, 4096), (5, 33), (512, 48), (7, 1)]


@pytest.mark.parametrize("ws_call", [False, True])
def test_group_and_amax(ws_call):
    rng = np.random.default_rng(4000 + ws_call)
    xs = [random_bf16(rng, shape) for shape in GROUP]
    ts = [dev(x) for x in xs]
    a = oracle.amax_group(xs)
    say("canary group (workspace %s)" % ws_call)
    outs = [bf16_out(shape, 40 + i, skew=16 * (1 + i % 3)) for i, shape in enumerate(GROUP)]
    ga, amax = f32_out(50)
    if ws_call:
        gw = Guarded(nv.WORKSPACE_BYTES, 0, 51)
        ws = gw.view(torch.uint8, (nv.WORKSPACE_BYTES,))
        nv.nvfp4_fake_quant_group_ws(ts, ys=[y for _, y in outs], amax_out=amax, workspace=ws)
    else:
        nv.nvfp4_fake_quant_group(ts, ys=[y for _, y in outs], amax_out=amax)
    torch.cuda.synchronize()
    ga.check("group amax_out")
    if ws_call:
        gw.check("group workspace")
    assert fbits(amax.item()) == fbits(a)
    for i, ((g, y), x) in enumerate(zip(outs, xs)):
        g.check("group member %d" % i)
        assert_same(host(y), oracle.fake_quant(x, a) if x.size else x, "group member %d" % i)

    ga, amax = f32_out(52)
    nv.nvfp4_amax(ts, amax)
    torch.cuda.synchronize()
    ga.check("amax")
    assert fbits(amax.item()) == fbits(a)


@pytest.mark.parametrize("m,n,k", [(1, 40, 64), (5, 33, 96), (64, 100, 256), (65, 70, 128), (200, 130, 512)])
def test_linear(m, n, k):
    rng = np.random.default_rng(5000 + m + n + k)
    w = synth.to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = synth.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    b = synth.to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    p, s, g = oracle.quantize(w)
    pt = torch.from_numpy(p).to(DEV)
    st = torch.from_numpy(s).to(DEV)
    gt = oracle_amax_dev(g)
    xt, bt = dev(x), dev(b)
    say("canary linear m=%d n=%d k=%d" % (m, n, k))
    plain = nv.nvfp4_linear(xt, pt, st, gt, bias=bt)
    gy, y = bf16_out((m, n), 60, skew=2)
    nv.nvfp4_linear(xt, pt, st, gt, bias=bt, y=y)
    torch.cuda.synchronize()
    gy.check("linear y")
    assert torch.equal(y.view(torch.int16), plain.view(torch.int16))
