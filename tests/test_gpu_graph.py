"""The library's calls under HIP graph capture.

Every call only enqueues kernels on the caller's stream (no allocation, no memset, no
host synchronisation), so a caller may capture a sequence of them in a graph and replay
it.  Each replay here runs after eager work that overwrites every output and amax, and
must reproduce the eager results bit for bit.
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
from gpu_util import DEV, assert_same, dev, fbits, host, say, scalar  # noqa: E402


def test_captured_sequence_replays_exactly():
    rng = np.random.default_rng(61)
    x = synth.to_bf16_bits((rng.standard_normal((512, 1024)) * 0.05).astype(np.float32))
    sibs = [synth.to_bf16_bits((rng.standard_normal((r, 256)) * s).astype(np.float32))
            for r, s in ((256, 0.02), (64, 0.03), (64, 0.01))]
    xt, st = dev(x), [dev(s) for s in sibs]
    y = torch.empty_like(xt)
    ys = [torch.empty_like(t) for t in st]
    packed = torch.empty((512, 512), dtype=torch.uint8, device=DEV)
    scales = torch.empty((512, 64), dtype=torch.uint8, device=DEV)
    a_fq, a_qp, a_grp, gs = scalar(0.0), scalar(0.0), scalar(0.0), scalar(0.0)
    yd = torch.empty_like(xt)
    state = scalar(-1.0)
    xl = dev(synth.to_bf16_bits(rng.standard_normal((8, 1024)).astype(np.float32)))
    yl = torch.empty((8, 512), dtype=torch.bfloat16, device=DEV)

    def sequence():
        nv.nvfp4_fake_quant(xt, y=y, amax_out=a_fq)
        nv.nvfp4_quantize_pack(xt, amax_out=a_qp, packed=packed, scales=scales, global_scale=gs)
        nv.nvfp4_dequant_unpack(packed, scales, gs, y=yd)
        nv.nvfp4_fake_quant_group(st, ys=ys, amax_out=a_grp)
        nv.nvfp4_observer_update(state, a_fq, nv.OBS_EMA, 0.25)
        nv.nvfp4_linear(xl, packed[:, :], scales, gs, y=yl)

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sequence()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence()
    torch.cuda.synchronize()

    a = oracle.amax(x)
    y_ref = oracle.fake_quant(x, a)
    p_ref, s_ref, g_ref = oracle.quantize(x, a)
    a_group = oracle.amax_group(sibs)
    for replay in range(4):
        # eager work between replays overwrites everything the graph writes
        for t in (y, yd, yl, *ys):
            t.fill_(float(replay + 1))
        packed.fill_(0xFF)
        scales.fill_(0x7F)
        for s in (a_fq, a_qp, a_grp, gs):
            s.fill_(-5.0)
        state.fill_(-1.0)
        torch.cuda.synchronize()
        say("graph replay %d" % replay)
        graph.replay()
        torch.cuda.synchronize()
        assert fbits(a_fq.item()) == fbits(a) and fbits(a_qp.item()) == fbits(a)
        assert fbits(gs.item()) == fbits(g_ref)
        assert fbits(state.item()) == fbits(oracle.observer(-1.0, a, oracle.OBS_EMA, 0.25))
        assert_same(host(y), y_ref, "replayed fake-quant")
        assert_same(packed.cpu().numpy(), p_ref, "replayed codes")
        assert_same(scales.cpu().numpy(), s_ref, "replayed scales")
        assert_same(host(yd), y_ref, "replayed unpack")
        assert fbits(a_grp.item()) == fbits(a_group)
        for i, (s, t) in enumerate(zip(sibs, ys)):
            assert_same(host(t), oracle.fake_quant(s, a_group), "replayed sibling %d" % i)
        y_lin = oracle.linear(host(xl), p_ref, s_ref, g_ref, 1024)
        got = oracle.bf16_array_to_f64(host(yl))
        mag = oracle.linear_magnitude(host(xl), p_ref, s_ref, g_ref, 1024)
        assert np.all(np.abs(got - y_lin) <= 2.0 ** -8 * np.abs(y_lin) + 2 * 1032 * 2.0 ** -24 * mag + 2.0 ** -133)


def test_captured_other_calls_replay_exactly():
    """The MXFP4 calls (whole-block and ragged rows), the no-allocation fake-quant, the
    dual fake-quant, odd-length ragged rows, and the linear layer on its LDS-staged
    tiles (128 and 512 rows of x), captured together and replayed after eager work
    that overwrites every output."""
    rng = np.random.default_rng(67)
    x = synth.to_bf16_bits((rng.standard_normal((256, 1024)) * 0.05).astype(np.float32))
    xr = synth.to_bf16_bits((rng.standard_normal((65, 1001)) * 0.05).astype(np.float32))
    xt, xrt = dev(x), dev(xr)
    y_mx, y_mxr, y_na, y_odd = (torch.empty_like(xt), torch.empty_like(xrt), torch.empty_like(xt),
                                torch.empty_like(xrt))
    y0, y1 = torch.empty_like(xt), torch.empty_like(xt)
    p_mx, s_mx = nv.nvfp4_mx_quantize_pack(xt)
    p_mxr, s_mxr = nv.nvfp4_mx_quantize_pack(xrt)
    y_mxd = torch.empty_like(xt)
    a_na, a0, a1 = scalar(0.0), scalar(0.0), scalar(0.0)
    packed, scales, gs = nv.nvfp4_quantize_pack(xt)
    torch.cuda.synchronize()
    p_ref, s_ref, g_ref = oracle.quantize(x, oracle.amax(x))
    xl = {m: dev(synth.to_bf16_bits(rng.standard_normal((m, 1024)).astype(np.float32))) for m in (128, 512)}
    yl = {m: torch.empty((m, 256), dtype=torch.bfloat16, device=DEV) for m in (128, 512)}
    st0, st1 = 0.5, 2.0

    def sequence():
        nv.nvfp4_mx_fake_quant(xt, y=y_mx)
        nv.nvfp4_mx_quantize_pack(xt, packed=p_mx, scales=s_mx)
        nv.nvfp4_mx_dequant_unpack(p_mx, s_mx, y=y_mxd)
        nv.nvfp4_mx_fake_quant(xrt, y=y_mxr)
        nv.nvfp4_mx_quantize_pack(xrt, packed=p_mxr, scales=s_mxr)
        nv.nvfp4_fake_quant_noalloc(xt, y=y_na, amax_out=a_na)
        nv.nvfp4_fake_quant_dual(xt, a0, a1, y0=y0, y1=y1)
        nv.nvfp4_fake_quant(xrt, y=y_odd)
        for m in (128, 512):
            nv.nvfp4_linear(xl[m], packed, scales, gs, y=yl[m])

    def set_amaxes():
        a0.fill_(st0)
        a1.fill_(st1)

    set_amaxes()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sequence()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence()
    torch.cuda.synchronize()

    p_mx_ref, s_mx_ref = oracle.mx_quantize(x)
    p_mxr_ref, s_mxr_ref = oracle.mx_quantize(xr)
    a = oracle.amax(x)
    for replay in range(3):
        for t in (y_mx, y_mxr, y_na, y_odd, y0, y1, y_mxd, *yl.values()):
            t.fill_(float(replay + 3))
        for t in (p_mx, p_mxr):
            t.fill_(0xEE)
        for t in (s_mx, s_mxr):
            t.fill_(-9.0)
        a_na.fill_(-5.0)
        set_amaxes()
        torch.cuda.synchronize()
        say("graph replay (other calls) %d" % replay)
        graph.replay()
        torch.cuda.synchronize()
        assert_same(host(y_mx), oracle.mx_fake_quant(x), "replayed mx fake-quant")
        assert_same(p_mx.cpu().numpy(), p_mx_ref, "replayed mx codes")
        assert_same(s_mx.cpu().numpy().view(np.uint32), s_mx_ref.view(np.uint32), "replayed mx scales")
        assert_same(host(y_mxd), oracle.mx_dequantize(p_mx_ref, s_mx_ref, 1024), "replayed mx unpack")
        assert_same(host(y_mxr), oracle.mx_fake_quant(xr), "replayed mx ragged fake-quant")
        assert_same(p_mxr.cpu().numpy(), p_mxr_ref, "replayed mx ragged codes")
        assert fbits(a_na.item()) == fbits(a)
        assert_same(host(y_na), oracle.fake_quant(x, a), "replayed no-allocation fake-quant")
        assert_same(host(y0), oracle.fake_quant(x, st0), "replayed dual 0")
        assert_same(host(y1), oracle.fake_quant(x, st1), "replayed dual 1")
        assert_same(host(y_odd), oracle.fake_quant(xr), "replayed odd-length rows")
        for m in (128, 512):
            y_lin = oracle.linear(host(xl[m]), p_ref, s_ref, g_ref, 1024)
            got = oracle.bf16_array_to_f64(host(yl[m]))
            mag = oracle.linear_magnitude(host(xl[m]), p_ref, s_ref, g_ref, 1024)
            assert np.all(np.abs(got - y_lin) <= 2.0 ** -8 * np.abs(y_lin) + 2 * 1032 * 2.0 ** -24 * mag
                          + 2.0 ** -133), "replayed linear m=%d" % m
