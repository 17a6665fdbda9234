"""QAT glue host logic (no GPU): layer replacement, sibling fusion, options and errors
(verl QATLinear page, sections 3-5)."""
import pytest

torch = pytest.importorskip("torch")
nv = pytest.importorskip("fp4_block_fake_amd")
from fp4_block_fake_amd import qat  # noqa: E402

nn = torch.nn


class Block(nn.Module):
    def __init__(self, d=64, f=128):
        super().__init__()
        self.q_proj, self.k_proj, self.v_proj = nn.Linear(d, d), nn.Linear(d, d // 2), nn.Linear(d, d // 2)
        self.o_proj = nn.Linear(d, d, bias=False)
        self.gate_proj, self.up_proj = nn.Linear(d, f), nn.Linear(d, f)
        self.down_proj = nn.Linear(f, d)
        self.norm = nn.LayerNorm(d)


class Model(nn.Module):
    def __init__(self):
        super().__init__()
        self.layers = nn.ModuleList([Block(), Block()])
        self.lm_head = nn.Linear(64, 100)


def test_apply_qat_replaces_linears_over_the_same_parameters():
    m = Model().to(torch.bfloat16)
    before = {n: p for n, p in m.named_parameters()}
    qat.apply_qat(m, mode="w4a4", activation_observer="minmax", ema_decay=0.05)
    after = dict(m.named_parameters())
    assert before.keys() == after.keys()
    assert all(before[n] is after[n] for n in before)       # same tensors, not copies
    for i in range(2):
        blk = m.layers[i]
        for name in ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"):
            layer = getattr(blk, name)
            assert isinstance(layer, qat.QATLinear), name
            assert layer.mode is qat.QATMode.W4A4 and layer.ema_decay == 0.05
            assert layer.activation_observer == "minmax"
            assert layer.input_amax.tolist() == [-1.0]
        assert blk.o_proj.bias is None
        assert isinstance(blk.norm, nn.LayerNorm)
    assert type(m.lm_head) is nn.Linear                        # excluded by name


def test_siblings_fused_per_parent_only():
    m = qat.apply_qat(Model().to(torch.bfloat16), mode=qat.QATMode.W4A16)
    b0, b1 = m.layers
    g = b0.q_proj.fusion
    assert g is b0.k_proj.fusion is b0.v_proj.fusion
    assert g.modules == [b0.q_proj, b0.k_proj, b0.v_proj]
    assert b0.gate_proj.fusion is b0.up_proj.fusion is not g
    assert b0.o_proj.fusion is None and b0.down_proj.fusion is None
    assert b1.q_proj.fusion is not g                           # another layer, another group
    assert not hasattr(b0.q_proj, "input_amax")                # W4A16 keeps no observer
    assert "input_amax" not in dict(m.named_buffers())


def test_state_dict_round_trip_keeps_observer_state():
    m = qat.apply_qat(Model().to(torch.bfloat16))
    m.layers[0].q_proj.input_amax.fill_(3.5)
    sd = m.state_dict()
    assert "layers.0.q_proj.input_amax" in sd
    m2 = qat.apply_qat(Model().to(torch.bfloat16))
    m2.load_state_dict(sd)
    assert m2.layers[0].q_proj.input_amax.item() == 3.5


def test_options_are_checked():
    with pytest.raises(ValueError):
        qat.QATLinear(32, 32, group_size=32)
    with pytest.raises(ValueError):
        qat.QATLinear(32, 32, activation_observer="percentile")
    with pytest.raises(ValueError):
        qat.QATLinear(32, 32, ema_decay=0.0)
    with pytest.raises(ValueError):
        qat.QATLinear(32, 32, mode="w8a8")
    with pytest.raises(TypeError):
        qat.fuse(qat.QATLinear(32, 32), nn.Linear(32, 32))


def test_forward_needs_bf16_on_the_gpu_unless_disabled():
    lin = qat.QATLinear(32, 16)
    x = torch.randn(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lin(x)                                   # CPU tensors: no fallback
    lin32 = qat.QATLinear(32, 16, dtype=torch.float32)
    with pytest.raises(TypeError):
        lin32(x.float())
    lin.fake_quant_enabled = False               # plain nn.Linear behaviour
    assert torch.equal(lin(x), torch.nn.functional.linear(x, lin.weight, lin.bias))
