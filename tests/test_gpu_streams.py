"""Concurrent use of the library: calls on several streams, from several host threads.

The C ABI keeps no state between calls, so calls on different streams whose buffers
do not overlap may run at the same time, and host threads may call it concurrently
(ctypes releases the GIL during a call).  Every result must still be the oracle's,
bit for bit.
"""
import threading

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


def random_bf16(rng, shape, sigma):
    return synth.to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def test_calls_on_two_streams_overlap_correctly():
    rng = np.random.default_rng(71)
    xs = [random_bf16(rng, (1024, 2048), s) for s in (0.02, 3.0)]
    ts = [dev(x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ys = [torch.empty_like(t) for t in ts]
    amax = [torch.empty(1, dtype=torch.float32, device=DEV) for _ in ts]
    packs = [None, None]
    ws = [nv.new_workspace(DEV) for _ in ts]
    torch.cuda.synchronize()
    say("two streams, interleaved fused calls")
    for it in range(8):
        for i, (t, st) in enumerate(zip(ts, streams)):
            with torch.cuda.stream(st):
                if it % 2:
                    nv.nvfp4_fake_quant_ws(t, y=ys[i], amax_out=amax[i], workspace=ws[i])
                else:
                    nv.nvfp4_fake_quant(t, y=ys[i], amax_out=amax[i])
                packs[i] = nv.nvfp4_quantize_pack(t)
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        a = oracle.amax(x)
        p_ref, s_ref, g_ref = oracle.quantize(x, a)
        assert fbits(amax[i].item()) == fbits(a)
        assert_same(host(ys[i]), oracle.fake_quant(x, a), "stream %d fake-quant" % i)
        assert_same(packs[i][0].cpu().numpy(), p_ref, "stream %d codes" % i)
        assert_same(packs[i][1].cpu().numpy(), s_ref, "stream %d scales" % i)
        assert fbits(packs[i][2].item()) == fbits(g_ref)


def test_host_threads_each_with_a_stream():
    rng = np.random.default_rng(73)
    n = 4
    xs = [random_bf16(rng, (256 + 64 * i, 1024), 0.01 * (i + 1)) for i in range(n)]
    ts = [dev(x) for x in xs]
    results = [None] * n
    errors = []
    torch.cuda.synchronize()

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                y = None
                for _ in range(20):
                    y = nv.nvfp4_fake_quant(ts[i])
                    packed, scales, gs = nv.nvfp4_quantize_pack(ts[i])
                    back = nv.nvfp4_dequant_unpack(packed, scales, gs)
                st.synchronize()
                results[i] = (y, back)
        except Exception as e:                      # reported by the main thread
            errors.append(e)

    say("four host threads")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(n)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for i, x in enumerate(xs):
        want = oracle.fake_quant(x)
        y, back = results[i]
        assert_same(host(y), want, "thread %d fake-quant" % i)
        assert_same(host(back), want, "thread %d unpack" % i)
