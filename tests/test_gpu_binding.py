"""The Python binding rejects, before any launch, every caller-given tensor the C ABI
cannot take as is: a wrong shape, dtype or device, or a host tensor whose pointer
would otherwise reach a kernel.  Each case raises ValueError and leaves the other
buffers untouched.
"""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import fp4_block_fake_amd as nv  # noqa: E402
from gpu_util import DEV, say  # noqa: E402


def gpu(*shape, dtype=torch.bfloat16, fill=1.0):
    return torch.full(shape, fill, dtype=dtype, device=DEV)


def f32(v=0.0, device=DEV):
    return torch.full((1,), v, dtype=torch.float32, device=device)


def untouched(*ts):
    """Snapshots, compared after the rejected call."""
    return [(t, t.clone()) for t in ts]


def still(snaps):
    torch.cuda.synchronize()
    for t, c in snaps:
        assert torch.equal(t.view(torch.uint8) if t.dtype == torch.uint8 else t.view(torch.int16)
                           if t.dtype == torch.bfloat16 else t, c.view(torch.uint8) if c.dtype == torch.uint8
                           else c.view(torch.int16) if c.dtype == torch.bfloat16 else c)


def test_fake_quant_outputs_and_scalars():
    say("binding: fake_quant rejections")
    x = gpu(64, 32)
    small = gpu(63, 32, fill=3.0)
    snaps = untouched(small)
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant(x, y=small)                          # y smaller than x
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant(x, y=gpu(32, 64))                    # same size, other shape
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant(x, amax_out=f32(device="cpu"))       # host amax_out
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant(x, amax_in=f32(device="cpu"))        # host amax_in
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant(x, amax_in=torch.ones(1, dtype=torch.float64, device=DEV))
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_ws(x, y=small)
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_ws(x, amax_out=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_ws(x, workspace=torch.empty(nv.WORKSPACE_BYTES, dtype=torch.uint8))
    still(snaps)


def test_quantize_pack_and_unpack():
    say("binding: quantize_pack / dequant_unpack rejections")
    x = gpu(64, 32)
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_pack(x, amax_in=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_pack(x, amax_out=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_pack(x, global_scale=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_pack(x, packed=torch.empty((64, 16), dtype=torch.uint8))     # host packed
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_pack_ws(x, scales=torch.empty((64, 2), dtype=torch.uint8))  # host scales
    packed, scales, gs = nv.nvfp4_quantize_pack(x)
    y = gpu(64, 32, fill=5.0)
    snaps = untouched(y)
    with pytest.raises(ValueError):
        nv.nvfp4_dequant_unpack(packed, scales.cpu(), gs, y=y)                           # host scales
    with pytest.raises(ValueError):
        nv.nvfp4_dequant_unpack(packed, scales, gs.cpu(), y=y)
    with pytest.raises(ValueError):
        nv.nvfp4_dequant_unpack(packed, scales, gs, y=gpu(63, 32))                       # y too small
    with pytest.raises(ValueError):
        nv.nvfp4_dequant_unpack(packed, scales, gs, y=gpu(64, 16))
    still(snaps)


def test_group_dual_observers_and_linear():
    say("binding: group, dual, observer and linear rejections")
    x = gpu(64, 32)
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_group([x, gpu(16, 32)], amax_out=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_group([x], ys=[gpu(64, 16)])
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_group_ws([x], amax_out=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_dual(x, f32(1.0), f32(1.0, device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant_dual(x, f32(1.0), f32(1.0), y1=gpu(32, 32))
    with pytest.raises(ValueError):
        nv.nvfp4_observer_update(f32(-1.0), f32(2.0, device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_observe_fake_quant(x, f32(-1.0), cur=f32(device="cpu"))
    with pytest.raises(ValueError):
        nv.nvfp4_observe_fake_quant(x, f32(-1.0), y0=gpu(64, 16))
    with pytest.raises(ValueError):
        nv.nvfp4_amax([x, torch.zeros(16, dtype=torch.bfloat16)])
    w = gpu(48, 64)
    packed, scales, gs = nv.nvfp4_quantize_pack(w)
    xm = gpu(4, 64)
    with pytest.raises(ValueError):
        nv.nvfp4_linear(xm, packed, scales.cpu(), gs)
    with pytest.raises(ValueError):
        nv.nvfp4_linear(xm, packed, scales, gs, bias=torch.zeros(48, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        nv.nvfp4_linear(xm, packed, scales, gs, y=gpu(4, 47))
    torch.cuda.synchronize()
