"""GPU parity of the workspace calls against the CPU oracle, bit for bit.

nvfp4_fake_quant_ws and nvfp4_quantize_pack_ws must give the oracle's fake-quant
and quantize-pack of x with its own amax (VideoX-Fun page, the tensor-wide amax
and the divide-by-gs convention), and max|x| in amax_out; nvfp4_fake_quant_group_ws
the fake-quant of every member with the group's shared amax (verl QATLinear page,
section 4).  The workspace is
reused between calls of different sizes and is filled with garbage before most
calls: its contents on entry must not matter.
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
from gpu_util import (DEV, assert_same, dev, fbits, host, oracle_amax, oracle_fake_quant,  # noqa: E402
                      oracle_quantize, say, scalar)

WS = nv.new_workspace(DEV)      # one workspace for the whole module: calls reuse it


def random_bf16(rng, shape, spread=3.0):
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, shape))
    return synth.to_bf16_bits(x.astype(np.float32))


def dirty_workspace():
    """Fill the workspace with garbage: the calls must not depend on its contents."""
    WS.fill_(0xA5)


# shapes: one half block short of a chunk, chunk edges, ragged rows, a single value,
# wide rows, and the empty tensor
SHAPES = [(1, 16), (3, 20), (7, 1), (1023, 16), (1025, 16), (64, 4096), (33, 40), (1037, 144), (0, 16),
          (0, 5), (0, 18), (2, 18), (257, 4100), (4096, 4100), (5, 17), (129, 4097)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("inplace", [False, True])
def test_fake_quant_ws(shape, inplace):
    rng = np.random.default_rng(shape[0] * 7 + shape[1] + inplace)
    x = random_bf16(rng, shape)
    say("fake_quant_ws %s in place %s" % (shape, inplace))
    dirty_workspace()
    xt = dev(x)
    y = xt if inplace else torch.empty_like(xt)
    amax = scalar(-7.0)
    nv.nvfp4_fake_quant_ws(xt, y=y, amax_out=amax, workspace=WS)
    torch.cuda.synchronize()
    a = oracle.amax(x) if x.size else 0.0
    assert fbits(amax.item()) == fbits(a)
    assert_same(host(y), oracle.fake_quant(x, a) if x.size else x, "fake_quant_ws")


@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_pack_ws(shape):
    rng = np.random.default_rng(shape[0] * 5 + shape[1])
    x = random_bf16(rng, shape)
    say("quantize_pack_ws %s" % (shape,))
    dirty_workspace()
    xt = dev(x)
    amax = scalar(-7.0)
    packed, scales, gs = nv.nvfp4_quantize_pack_ws(xt, amax_out=amax, workspace=WS)
    torch.cuda.synchronize()
    a = oracle.amax(x) if x.size else 0.0
    p_ref, s_ref, g_ref = oracle.quantize(x, a)
    assert fbits(amax.item()) == fbits(a)
    assert fbits(gs.item()) == fbits(g_ref)
    assert_same(packed.cpu().numpy(), p_ref, "packed")
    assert_same(scales.cpu().numpy(), s_ref, "scales")


def test_amax_out_may_be_omitted():
    rng = np.random.default_rng(5)
    x = random_bf16(rng, (129, 1024))
    xt = dev(x)
    say("workspace calls without amax_out")
    y = nv.nvfp4_fake_quant_ws(xt, workspace=WS)
    packed, scales, gs = nv.nvfp4_quantize_pack_ws(xt, workspace=WS)
    torch.cuda.synchronize()
    p_ref, s_ref, g_ref = oracle.quantize(x)
    assert_same(host(y), oracle.fake_quant(x), "fake_quant_ws, no amax_out")
    assert_same(packed.cpu().numpy(), p_ref, "packed, no amax_out")
    assert_same(scales.cpu().numpy(), s_ref, "scales, no amax_out")
    assert fbits(gs.item()) == fbits(g_ref)


def test_c2_weight_whole():
    x = synth.c2_weight()
    say("workspace calls c2 %s" % (x.shape,))
    xt = dev(x)
    a_fq, a_qp = scalar(0.0), scalar(0.0)
    y = nv.nvfp4_fake_quant_ws(xt, amax_out=a_fq, workspace=WS)
    packed, scales, gs = nv.nvfp4_quantize_pack_ws(xt, amax_out=a_qp, workspace=WS)
    torch.cuda.synchronize()
    a = oracle.amax(x)
    p_ref, s_ref, g_ref = oracle.quantize(x, a)
    assert fbits(a_fq.item()) == fbits(a) and fbits(a_qp.item()) == fbits(a)
    assert fbits(gs.item()) == fbits(g_ref)
    assert_same(host(y), oracle.fake_quant(x, a), "c2 fake_quant_ws")
    assert_same(packed.cpu().numpy(), p_ref, "c2 packed")
    assert_same(scales.cpu().numpy(), s_ref, "c2 scales")


def test_c5_weight_whole():
    """The c5 weight at full size, in the launch configuration the benchmark times, whole
    against the oracle."""
    x = synth.c5_weight()
    say("workspace calls c5 %s" % (x.shape,))
    xt = dev(x)
    a_fq, a_qp = scalar(0.0), scalar(0.0)
    y = nv.nvfp4_fake_quant_ws(xt, amax_out=a_fq, workspace=WS)
    packed, scales, gs = nv.nvfp4_quantize_pack_ws(xt, amax_out=a_qp, workspace=WS)
    torch.cuda.synchronize()
    a = oracle_amax(x)
    assert fbits(a_fq.item()) == fbits(a) and fbits(a_qp.item()) == fbits(a)
    p_ref, s_ref, g_ref = oracle_quantize(x, a)
    assert fbits(gs.item()) == fbits(g_ref)
    assert_same(packed.cpu().numpy(), p_ref, "c5 packed")
    assert_same(scales.cpu().numpy(), s_ref, "c5 scales")
    assert_same(host(y), oracle_fake_quant(x, a), "c5 fake_quant_ws")


def test_workspace_reuse_large_then_small():
    """A large call leaves many partial maxima behind; a small call after it on the
    same workspace must read only its own."""
    rng = np.random.default_rng(9)
    big = random_bf16(rng, (2048, 4096), spread=8.0)
    small = random_bf16(rng, (3, 48), spread=0.5)
    say("workspace reuse")
    bt, st = dev(big), dev(small)
    a_big, a_small = scalar(0.0), scalar(0.0)
    nv.nvfp4_fake_quant_ws(bt, amax_out=a_big, workspace=WS)
    y = nv.nvfp4_fake_quant_ws(st, amax_out=a_small, workspace=WS)
    torch.cuda.synchronize()
    assert fbits(a_big.item()) == fbits(oracle.amax(big)) > fbits(oracle.amax(small))
    assert fbits(a_small.item()) == fbits(oracle.amax(small))
    assert_same(host(y), oracle.fake_quant(small), "small after large")


def test_group_ws_c3_siblings():
    sibs = list(synth.c3_siblings())
    say("group ws c3")
    ts = [dev(x) for x in sibs]
    amax = scalar(-3.0)
    dirty_workspace()
    ys = nv.nvfp4_fake_quant_group_ws(ts, amax_out=amax, workspace=WS)
    torch.cuda.synchronize()
    a = oracle.amax_group(sibs)
    assert fbits(amax.item()) == fbits(a)
    for i, (x, y) in enumerate(zip(sibs, ys)):
        assert_same(host(y), oracle.fake_quant(x, a), "c3 group ws member %d" % i)


# up to 8 members: chunk edges, an empty member, ragged rows (their own launches), an
# in-place member
GROUP = [(64, 256), (0, 32), (3, 20), (1025, 16), (37, 4096), (5, 33), (512, 48), (7, 1)]


@pytest.mark.parametrize("k", [1, 3, 8])
def test_group_ws_members(k):
    rng = np.random.default_rng(90 + k)
    xs = [random_bf16(rng, shape) for shape in GROUP[:k]]
    say("group ws %d members" % k)
    ts = [dev(x) for x in xs]
    ys = [t if i == 0 else torch.empty_like(t) for i, t in enumerate(ts)]     # member 0 in place
    dirty_workspace()
    nv.nvfp4_fake_quant_group_ws(ts, ys=ys, workspace=WS)
    torch.cuda.synchronize()
    a = oracle.amax_group(xs) if any(x.size for x in xs) else 0.0
    for i, (x, y) in enumerate(zip(xs, ys)):
        assert_same(host(y), oracle.fake_quant(x, a) if x.size else x, "member %d" % i)


def test_group_ws_rejects_more_than_eight():
    ts = [torch.zeros((1, 16), dtype=torch.bfloat16, device=DEV) for _ in range(9)]
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_fake_quant_group_ws(ts, workspace=WS)


def test_workspace_calls_replay_in_a_graph():
    """The workspace calls enqueue kernels only (no memset), so a captured sequence
    replays exactly, here after the workspace and every output were overwritten."""
    rng = np.random.default_rng(23)
    w = random_bf16(rng, (256, 2048))
    wt = dev(w)
    yw = torch.empty_like(wt)
    packed = torch.empty((256, 1024), dtype=torch.uint8, device=DEV)
    scales = torch.empty((256, 128), dtype=torch.uint8, device=DEV)
    aw, ap, gs = scalar(0.0), scalar(0.0), scalar(0.0)

    def sequence():
        nv.nvfp4_fake_quant_ws(wt, y=yw, amax_out=aw, workspace=WS)
        nv.nvfp4_quantize_pack_ws(wt, amax_out=ap, packed=packed, scales=scales, global_scale=gs, workspace=WS)

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

    a = oracle.amax(w)
    p_ref, s_ref, g_ref = oracle.quantize(w, a)
    for replay in range(4):
        yw.fill_(float(replay + 1))
        packed.fill_(0xFF)
        scales.fill_(0x7F)
        for t in (aw, ap, gs):
            t.fill_(-5.0)
        WS.fill_(0x5A + replay)
        torch.cuda.synchronize()
        say("workspace graph replay %d" % replay)
        graph.replay()
        torch.cuda.synchronize()
        assert fbits(aw.item()) == fbits(a) and fbits(ap.item()) == fbits(a)
        assert fbits(gs.item()) == fbits(g_ref)
        assert_same(host(yw), oracle.fake_quant(w, a), "replay %d fake-quant" % replay)
        assert_same(packed.cpu().numpy(), p_ref, "replay %d packed" % replay)
        assert_same(scales.cpu().numpy(), s_ref, "replay %d scales" % replay)
