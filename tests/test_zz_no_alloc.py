"""nvfp4_fake_quant_noalloc (the fused fake-quant on the library's own per-GPU scratch)
against nvfp4_fake_quant_ws (the same call on a caller's workspace) and the oracle,
bit for bit, through the C ABI.  Two calls in a row, the second with a smaller
input, so the second runs on the scratch exactly as the first left it; then a
ragged shape (its amax reduced by one workgroup into the scratch when no amax_out
is given) and an empty tensor.
"""
import ctypes

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


def noalloc_raw(x, y, amax_out):
    """The entry point called with raw device pointers (no binding logic in between)."""
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    return nv.lib.nvfp4_fake_quant_noalloc(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), x.shape[0], x.shape[1],
        None if amax_out is None else ctypes.c_void_p(amax_out.data_ptr()), stream)


def check_against_ws(x, what, with_amax=True):
    say("noalloc %s %s" % (what, x.shape))
    xt = dev(x)
    y = torch.full_like(xt, 7.0)
    a = scalar(-5.0) if with_amax else None
    assert noalloc_raw(xt, y, a) == 0
    y_ws = nv.nvfp4_fake_quant_ws(xt, amax_out=scalar(-5.0) if with_amax else None)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16)), what + ": noalloc vs workspace call"
    a_ref = oracle.amax(x)
    if with_amax:
        assert fbits(a.item()) == fbits(a_ref), what + " amax"
    assert_same(host(y), oracle.fake_quant(x, a_ref), what + " vs oracle")


def test_two_calls_in_a_row_then_smaller():
    big = synth.c2_weight()                                        # 4096 x 4096
    small = synth.normal_bf16(91, (1000, 2048), 0.3)
    check_against_ws(big, "c2 weight")
    check_against_ws(small, "smaller, second call")
    check_against_ws(small[:37], "smaller again, no amax_out", with_amax=False)


def test_ragged_and_empty():
    rng = np.random.default_rng(92)
    x = synth.to_bf16_bits((rng.standard_normal((333, 100)) * 3).astype(np.float32))
    check_against_ws(x, "ragged rows")
    check_against_ws(x, "ragged rows, no amax_out", with_amax=False)
    empty = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    a = scalar(-5.0)
    y = nv.nvfp4_fake_quant_noalloc(empty, amax_out=a)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and fbits(a.item()) == 0


def test_binding_and_in_place():
    x = synth.c1_weight()
    xt = dev(x)
    a = scalar(0.0)
    nv.nvfp4_fake_quant_noalloc(xt, y=xt, amax_out=a)               # in place
    torch.cuda.synchronize()
    assert_same(host(xt), oracle.fake_quant(x), "in place")
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_noalloc(dev(x), y=torch.empty((255, 1024), dtype=torch.bfloat16, device=DEV))
