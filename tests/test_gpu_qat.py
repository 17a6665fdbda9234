"""QAT glue on the GPU (verl QATLinear page, sections 2-5).

Every fake-quantized operand the layer feeds to its matmul must equal the
oracle's fake-quant of that operand (weight: own amax, or the fused siblings'
shared amax; activation: the observer state of that step), bit for bit.  The
matmul itself is torch's; the layer's output and gradients are compared with
the same torch ops applied to the oracle's operands, so they must match exactly
too.  Matmuls here are 2-D (plain mm), and reference gradients come from the
same 2-D ops.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import torch.nn.functional as F  # noqa: E402

from fp4_block_fake_amd import qat  # noqa: E402
from gpu_util import DEV, assert_same, dev, fbits, host, say  # noqa: E402


def bits(t):
    return host(t.detach().contiguous())


def rand_bf16(rng, shape, sigma):
    return synth.to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def layer_from(w_bits, b_bits=None, **kw):
    out_f, in_f = w_bits.shape
    lin = qat.QATLinear(in_f, out_f, bias=b_bits is not None, device=DEV, **kw)
    with torch.no_grad():
        lin.weight.copy_(dev(w_bits))
        if b_bits is not None:
            lin.bias.copy_(dev(b_bits))
    return lin


def test_w4a16_forward_uses_the_fake_quantized_weight():
    rng = np.random.default_rng(31)
    w, b, x = rand_bf16(rng, (256, 512), 0.02), rand_bf16(rng, (256,), 0.1), rand_bf16(rng, (64, 512), 1.0)
    lin = layer_from(w, b, mode="w4a16")
    say("qat w4a16 forward")
    w_fq = oracle.fake_quant(w)
    assert_same(bits(lin.fake_quantized_weight()), w_fq, "weight fake-quant")
    out = lin(dev(x))
    ref = F.linear(dev(x), dev(w_fq), dev(b))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("observer", ["static_minmax", "minmax"])
def test_w4a4_observer_steps_and_forward(observer):
    rng = np.random.default_rng(41)
    w = rand_bf16(rng, (128, 256), 0.02)
    lin = layer_from(w, None, mode="w4a4", activation_observer=observer, ema_decay=0.1)
    lin.train()
    w_fq = oracle.fake_quant(w)
    mode = oracle.OBS_STATIC_MINMAX if observer == "static_minmax" else oracle.OBS_EMA
    state = -1.0
    for step, scale in enumerate([1.0, 3.0, 0.5, 2.0]):
        x = rand_bf16(rng, (96, 256), scale)
        say("qat w4a4 %s step %d" % (observer, step))
        out = lin(dev(x))
        torch.cuda.synchronize()
        state = oracle.observer(state, oracle.amax(x), mode, float(np.float32(0.1)))
        assert fbits(lin.input_amax.item()) == fbits(state), "step %d state" % step
        x_fq = oracle.fake_quant(x, state)
        ref = F.linear(dev(x_fq), dev(w_fq))
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "step %d output" % step
    # evaluation keeps the state and fake-quantizes with it
    lin.eval()
    x = rand_bf16(rng, (32, 256), 5.0)
    out = lin(dev(x))
    torch.cuda.synchronize()
    assert fbits(lin.input_amax.item()) == fbits(state)
    ref = F.linear(dev(oracle.fake_quant(x, state)), dev(w_fq))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_activation_of_any_leading_shape_is_blocked_along_features():
    rng = np.random.default_rng(43)
    lin = layer_from(rand_bf16(rng, (64, 48), 0.05), None, mode="w4a4")
    x = rand_bf16(rng, (2, 5, 48), 1.0)                       # 48 = 3 blocks per row
    xt = dev(x)
    got = lin.fake_quantized_input(xt)
    torch.cuda.synchronize()
    assert got.shape == xt.shape
    assert_same(bits(got).reshape(10, 48), oracle.fake_quant(x.reshape(10, 48), oracle.amax(x)),
                "3-D activation")


def test_fused_siblings_share_the_group_amax():
    torch.manual_seed(0)

    class Attn(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.q_proj = torch.nn.Linear(128, 128, bias=False)
            self.k_proj = torch.nn.Linear(128, 64, bias=False)
            self.v_proj = torch.nn.Linear(128, 64, bias=False)
            self.o_proj = torch.nn.Linear(128, 128, bias=False)

    m = Attn().to(device=DEV, dtype=torch.bfloat16)
    with torch.no_grad():
        m.k_proj.weight.mul_(7.0)                               # k holds the group maximum
    qat.apply_qat(m, mode="w4a16")
    ws = {n: bits(getattr(m, n).weight) for n in ("q_proj", "k_proj", "v_proj", "o_proj")}
    a_group = oracle.amax_group([ws["q_proj"], ws["k_proj"], ws["v_proj"]])
    assert a_group == oracle.amax(ws["k_proj"]) > oracle.amax(ws["q_proj"])
    say("qat fused siblings")
    for n in ("q_proj", "k_proj", "v_proj"):
        assert_same(bits(getattr(m, n).fake_quantized_weight()), oracle.fake_quant(ws[n], a_group), n)
    assert_same(bits(m.o_proj.fake_quantized_weight()), oracle.fake_quant(ws["o_proj"]), "o_proj alone")
    # a weight update is seen by the next forward of every sibling
    with torch.no_grad():
        m.v_proj.weight.data.mul_(16.0)                         # through .data: no version bump
    ws["v_proj"] = bits(m.v_proj.weight)
    a2 = oracle.amax_group([ws["q_proj"], ws["k_proj"], ws["v_proj"]])
    assert a2 != a_group
    assert_same(bits(m.q_proj.fake_quantized_weight()), oracle.fake_quant(ws["q_proj"], a2), "q after update")


def test_gradients_pass_straight_through():
    rng = np.random.default_rng(47)
    w, b = rand_bf16(rng, (96, 160), 0.03), rand_bf16(rng, (96,), 0.1)
    x, g = rand_bf16(rng, (40, 160), 1.0), rand_bf16(rng, (40, 96), 1.0)
    lin = layer_from(w, b, mode="w4a4")
    lin.train()
    xt = dev(x).requires_grad_(True)
    out = lin(xt)
    out.backward(dev(g))
    torch.cuda.synchronize()
    # the same 2-D ops on the oracle's operands, as leaves
    state = oracle.observer(-1.0, oracle.amax(x), oracle.OBS_STATIC_MINMAX)
    x_fq = dev(oracle.fake_quant(x, state)).requires_grad_(True)
    w_fq = dev(oracle.fake_quant(w)).requires_grad_(True)
    b_ref = dev(b).requires_grad_(True)
    ref = F.linear(x_fq, w_fq, b_ref)
    ref.backward(dev(g))
    torch.cuda.synchronize()
    say("qat straight-through gradients")
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(xt.grad.view(torch.int16), x_fq.grad.view(torch.int16))
    assert torch.equal(lin.weight.grad.view(torch.int16), w_fq.grad.view(torch.int16))
    assert torch.equal(lin.bias.grad.view(torch.int16), b_ref.grad.view(torch.int16))


def test_disabled_layer_is_plain_linear():
    rng = np.random.default_rng(53)
    w, x = rand_bf16(rng, (32, 64), 0.05), rand_bf16(rng, (8, 64), 1.0)
    lin = layer_from(w, None)
    lin.fake_quant_enabled = False
    out = lin(dev(x))
    assert torch.equal(out.view(torch.int16), F.linear(dev(x), dev(w)).view(torch.int16))
    assert lin.input_amax.item() == -1.0                        # no observation happened
