"""GPU parity of nvfp4_observe_fake_quant against the CPU oracle, bit for bit.

One call makes the activation step of a W4A4 layer (verl QATLinear page,
section 5): the step amax, the observer update of each state on it, and the
fake-quant of x with each new state.  The oracle runs the same three steps
(amax, observer, fake_quant); states and the step amax must match bit for bit
on every step, outputs on every element (sampled rows for the full-size c4
activations, where the whole tensors are also compared with the dual call).
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

S, E = oracle.OBS_STATIC_MINMAX, oracle.OBS_EMA


def random_bf16(rng, shape, spread=3.0):
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, shape))
    return synth.to_bf16_bits(x.astype(np.float32))


def test_c4_ten_steps_two_observers():
    """The c4 activation stream: ten steps with a static-minmax and an EMA (decay 0.01)
    observer, one call per step."""
    s_static, s_ema = scalar(-1.0), scalar(-1.0)
    cur = scalar(0.0)
    rs = re = -1.0
    d = float(np.float32(0.01))
    y0 = y1 = None
    for t in range(10):
        x = synth.c4_activation(t)
        say("observe c4 step %d %s" % (t, x.shape))
        xt = dev(x)
        if y0 is None:
            y0, y1 = torch.empty_like(xt), torch.empty_like(xt)
        nv.nvfp4_observe_fake_quant(xt, s_static, nv.OBS_STATIC_MINMAX, 0.0, s_ema, nv.OBS_EMA, 0.01,
                                    y0=y0, y1=y1, cur=cur)
        torch.cuda.synchronize()
        a = oracle.amax(x)
        rs = oracle.observer(rs, a, S)
        re = oracle.observer(re, a, E, d)
        assert fbits(cur.item()) == fbits(a), "step %d amax" % t
        assert fbits(s_static.item()) == fbits(rs), "step %d static state" % t
        assert fbits(s_ema.item()) == fbits(re), "step %d ema state" % t
        assert_same(host(y0), oracle_fake_quant(x, rs), "step %d static" % t)
        assert_same(host(y1), oracle_fake_quant(x, re), "step %d ema" % t)
        if t in (0, 1, 9):
            z0, z1 = nv.nvfp4_fake_quant_dual(xt, scalar(rs), scalar(re))
            torch.cuda.synchronize()
            assert torch.equal(y0.view(torch.int16), z0.view(torch.int16))
            assert torch.equal(y1.view(torch.int16), z1.view(torch.int16))
    assert rs != re


# chunk edges, ragged rows (their own passes), a single value, wide rows, empty
SHAPES = [(1, 16), (3, 20), (7, 1), (1025, 16), (64, 4096), (33, 40), (1037, 144), (0, 16), (0, 24),
          (65, 4100)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("inplace", [None, 0, 1])
def test_two_observers_shapes(shape, inplace):
    rng = np.random.default_rng(shape[0] * 11 + shape[1] + 5 * (inplace or 0))
    xs = [random_bf16(rng, shape, spread=1.0 + step) for step in range(3)]
    say("observe two %s in place %s" % (shape, inplace))
    s0, s1 = scalar(-1.0), scalar(-1.0)
    cur = scalar(-9.0)
    r0 = r1 = -1.0
    d = float(np.float32(0.25))
    for step, x in enumerate(xs):
        xt = dev(x)
        y0 = xt if inplace == 0 else torch.empty_like(xt)
        y1 = xt if inplace == 1 else torch.empty_like(xt)
        nv.nvfp4_observe_fake_quant(xt, s0, nv.OBS_EMA, 0.25, s1, nv.OBS_STATIC_MINMAX, 0.0,
                                    y0=y0, y1=y1, cur=cur)
        torch.cuda.synchronize()
        a = oracle.amax(x) if x.size else 0.0
        r0 = oracle.observer(r0, a, E, d)
        r1 = oracle.observer(r1, a, S)
        assert fbits(cur.item()) == fbits(a)
        assert fbits(s0.item()) == fbits(r0) and fbits(s1.item()) == fbits(r1), "step %d" % step
        if x.size:
            assert_same(host(y0), oracle.fake_quant(x, r0), "step %d y0" % step)
            assert_same(host(y1), oracle.fake_quant(x, r1), "step %d y1" % step)


@pytest.mark.parametrize("shape", [(1, 16), (3, 20), (515, 16), (64, 4096), (33, 40), (0, 16)])
@pytest.mark.parametrize("mode", [nv.OBS_STATIC_MINMAX, nv.OBS_EMA])
@pytest.mark.parametrize("inplace", [False, True])
def test_one_observer(shape, mode, inplace):
    rng = np.random.default_rng(shape[0] + 3 * shape[1] + mode + 7 * inplace)
    say("observe one %s mode %d in place %s" % (shape, mode, inplace))
    state = scalar(-1.0)
    r = -1.0
    for step in range(3):
        x = random_bf16(rng, shape, spread=1.0 + step)
        xt = dev(x)
        y = nv.nvfp4_observe_fake_quant(xt, state, mode, 0.5, y0=xt if inplace else None)
        torch.cuda.synchronize()
        a = oracle.amax(x) if x.size else 0.0
        r = oracle.observer(r, a, mode, float(np.float32(0.5)))
        assert fbits(state.item()) == fbits(r), "step %d state" % step
        if x.size:
            assert_same(host(y), oracle.fake_quant(x, r), "step %d y" % step)


def test_prior_state_and_saturation():
    """A prior state above the step amax (static keeps it, so blocks saturate nothing,
    EMA moves towards the step amax) and one below it."""
    rng = np.random.default_rng(19)
    x = random_bf16(rng, (96, 512))
    a = oracle.amax(x)
    for prior in (4.0 * a, 0.25 * a):
        prior = float(np.float32(prior))
        s0, s1 = scalar(prior), scalar(prior)
        say("observe prior %g (amax %g)" % (prior, a))
        y0, y1 = nv.nvfp4_observe_fake_quant(dev(x), s0, nv.OBS_STATIC_MINMAX, 0.0, s1, nv.OBS_EMA, 0.01)
        torch.cuda.synchronize()
        r0 = oracle.observer(prior, a, S)
        r1 = oracle.observer(prior, a, E, float(np.float32(0.01)))
        assert fbits(s0.item()) == fbits(r0) and fbits(s1.item()) == fbits(r1)
        assert_same(host(y0), oracle.fake_quant(x, r0), "prior %g static" % prior)
        assert_same(host(y1), oracle.fake_quant(x, r1), "prior %g ema" % prior)


def test_matches_the_separate_calls():
    """The one call equals amax, two observer updates and the dual fake-quant."""
    rng = np.random.default_rng(17)
    x = dev(random_bf16(rng, (777, 512)))
    a_s, b_s = scalar(3.0), scalar(3.0)
    a_e, b_e = scalar(0.5), scalar(0.5)
    say("observe vs separate calls")
    y0, y1 = nv.nvfp4_observe_fake_quant(x, a_s, nv.OBS_STATIC_MINMAX, 0.0, a_e, nv.OBS_EMA, 0.01)
    cur = nv.nvfp4_amax(x)
    nv.nvfp4_observer_update(b_s, cur, nv.OBS_STATIC_MINMAX)
    nv.nvfp4_observer_update(b_e, cur, nv.OBS_EMA, 0.01)
    z0, z1 = nv.nvfp4_fake_quant_dual(x, b_s, b_e)
    torch.cuda.synchronize()
    assert fbits(a_s.item()) == fbits(b_s.item()) and fbits(a_e.item()) == fbits(b_e.item())
    assert torch.equal(y0.view(torch.int16), z0.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), z1.view(torch.int16))


def test_workspace_is_reused_and_its_contents_do_not_matter():
    """One workspace for calls of different sizes, filled with garbage before each."""
    rng = np.random.default_rng(29)
    ws = nv.new_workspace(DEV)
    state = scalar(-1.0)
    r = -1.0
    for step, shape in enumerate([(2048, 4096), (3, 48), (1024, 1024), (0, 16)]):
        x = random_bf16(rng, shape, spread=2.0)
        ws.fill_(0x5A + step)
        say("observe reused workspace %s" % (shape,))
        y = nv.nvfp4_observe_fake_quant(dev(x), state, nv.OBS_EMA, 0.25, workspace=ws)
        torch.cuda.synchronize()
        a = oracle.amax(x) if x.size else 0.0
        r = oracle.observer(r, a, E, float(np.float32(0.25)))
        assert fbits(state.item()) == fbits(r), "step %d" % step
        if x.size:
            assert_same(host(y), oracle.fake_quant(x, r), "step %d y" % step)


def test_rejects_shared_state_and_bad_mode():
    t = torch.zeros((4, 16), dtype=torch.bfloat16, device=DEV)
    s = scalar(-1.0)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_observe_fake_quant(t, s, nv.OBS_STATIC_MINMAX, 0.0, s, nv.OBS_EMA, 0.01)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_observe_fake_quant(t, s, 7)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_observe_fake_quant(t, s, nv.OBS_EMA, 0.0)


def test_replays_in_a_graph():
    """Captured once, the step replays with the states advancing on every replay."""
    rng = np.random.default_rng(23)
    xs = [random_bf16(rng, (512, 1024), spread=1.0 + i) for i in range(4)]
    xt = dev(xs[0])
    s0, s1, cur = scalar(-1.0), scalar(-1.0), scalar(0.0)
    y0, y1 = torch.empty_like(xt), torch.empty_like(xt)

    ws = nv.new_workspace(DEV)

    def step():
        nv.nvfp4_observe_fake_quant(xt, s0, nv.OBS_STATIC_MINMAX, 0.0, s1, nv.OBS_EMA, 0.01, y0=y0, y1=y1,
                                    cur=cur, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    s0.fill_(-1.0)
    s1.fill_(-1.0)
    r0 = r1 = -1.0
    for replay, x in enumerate(xs):
        xt.copy_(dev(x))
        y0.fill_(float(replay + 1))
        y1.fill_(float(replay + 1))
        cur.fill_(-5.0)
        ws.fill_(0xA5 + replay)
        torch.cuda.synchronize()
        say("observe graph replay %d" % replay)
        graph.replay()
        torch.cuda.synchronize()
        a = oracle.amax(x)
        r0 = oracle.observer(r0, a, S)
        r1 = oracle.observer(r1, a, E, float(np.float32(0.01)))
        assert fbits(cur.item()) == fbits(a)
        assert fbits(s0.item()) == fbits(r0) and fbits(s1.item()) == fbits(r1)
        assert_same(host(y0), oracle.fake_quant(x, r0), "replay %d y0" % replay)
        assert_same(host(y1), oracle.fake_quant(x, r1), "replay %d y1" % replay)
