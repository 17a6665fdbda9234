"""Python binding of libnvfp4.so: NVFP4 two-level block quantization on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels in ``csrc/``; torch supplies device memory and the current
stream.  The functions carry the C ABI's names and semantics (see
``include/nvfp4.h``); outputs that are not passed in are allocated here with
torch.  Importing this package fails when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "NVFP4Error", "OBS_STATIC_MINMAX", "OBS_EMA", "lib", "library_path",
    "nvfp4_amax", "nvfp4_fake_quant", "nvfp4_fake_quant_group", "nvfp4_fake_quant_dual",
    "nvfp4_quantize_pack", "nvfp4_dequant_unpack", "nvfp4_linear", "nvfp4_observer_update",
    "nvfp4_strerror", "FakeQuantSTE", "blocks_per_row", "nvfp4_observe_fake_quant",
    "WORKSPACE_BYTES", "new_workspace", "nvfp4_fake_quant_ws", "nvfp4_quantize_pack_ws",
    "nvfp4_fake_quant_group_ws", "nvfp4_fake_quant_noalloc",
    "MX_BLOCK", "mx_blocks_per_row", "nvfp4_mx_fake_quant", "nvfp4_mx_quantize_pack", "nvfp4_mx_dequant_unpack",
]

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")

OBS_STATIC_MINMAX = 0
OBS_EMA = 1
WORKSPACE_BYTES = 2304        # NVFP4_WORKSPACE_BYTES
MX_BLOCK = 32                 # NVFP4_MX_BLOCK

_EXPORTS = ("nvfp4_amax", "nvfp4_fake_quant", "nvfp4_fake_quant_group", "nvfp4_fake_quant_dual",
            "nvfp4_quantize_pack", "nvfp4_dequant_unpack", "nvfp4_linear", "nvfp4_observer_update",
            "nvfp4_observe_fake_quant", "nvfp4_fake_quant_ws", "nvfp4_quantize_pack_ws",
            "nvfp4_fake_quant_group_ws", "nvfp4_fake_quant_noalloc", "nvfp4_mx_fake_quant",
            "nvfp4_mx_quantize_pack", "nvfp4_mx_dequant_unpack", "nvfp4_strerror")


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, nvfp4_strerror(status), status))
        self.status = status


def _load(path: str = library_path) -> ctypes.CDLL:
    """The library at `path` with every export's argument types set (the tests also
    load a build of the same source with other compile-time settings this way)."""
    if not os.path.exists(path):
        raise ImportError("%s is not built; run "
                          "`python fp4_block_fake_amd/_build.py` or __graft_entry__.build()" % path)
    so = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    so.nvfp4_amax.argtypes = [P, P, I, P, I, P]
    so.nvfp4_fake_quant.argtypes = [P, P, I64, I64, P, P, P]
    so.nvfp4_fake_quant_group.argtypes = [P, P, P, P, I, P, P, P]
    so.nvfp4_fake_quant_dual.argtypes = [P, I64, I64, P, P, P, P, P]
    so.nvfp4_quantize_pack.argtypes = [P, I64, I64, P, P, P, P, P, P]
    so.nvfp4_dequant_unpack.argtypes = [P, P, P, I64, I64, P, P]
    so.nvfp4_linear.argtypes = [P, I64, I64, P, P, P, I64, P, P, P]
    so.nvfp4_observer_update.argtypes = [P, P, I, ctypes.c_float, P]
    F = ctypes.c_float
    so.nvfp4_observe_fake_quant.argtypes = [P, I64, I64, P, P, I, F, P, P, I, F, P, P, P]
    so.nvfp4_fake_quant_ws.argtypes = [P, P, I64, I64, P, P, P]
    so.nvfp4_quantize_pack_ws.argtypes = [P, I64, I64, P, P, P, P, P, P]
    so.nvfp4_fake_quant_group_ws.argtypes = [P, P, P, P, I, P, P, P]
    so.nvfp4_fake_quant_noalloc.argtypes = [P, P, I64, I64, P, P]
    so.nvfp4_mx_fake_quant.argtypes = [P, P, I64, I64, P]
    so.nvfp4_mx_quantize_pack.argtypes = [P, I64, I64, P, P, P]
    so.nvfp4_mx_dequant_unpack.argtypes = [P, P, I64, I64, P, P]
    so.nvfp4_strerror.argtypes = [I]
    so.nvfp4_strerror.restype = ctypes.c_char_p
    for name in _EXPORTS:
        if name != "nvfp4_strerror":
            getattr(so, name).restype = I
    return so


lib = _load()


def nvfp4_strerror(status: int) -> str:
    return lib.nvfp4_strerror(status).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise NVFP4Error(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> ctypes.c_void_p:
    # torch's current stream on the device; the raw accessor skips building a Stream
    # object (about 2 us per call), with the public API as the fallback
    if _raw_stream is not None:
        index = device.index if device.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(index))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _same_device(t: torch.Tensor, device, name: str) -> None:
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError("%s must be a CUDA tensor on %s" % (name, device if device is not None else "the GPU"))


def _matrix(x: torch.Tensor, name: str, device=None, shape=None):
    """A contiguous 2-D bf16 tensor on `device` (and of `shape`, when given) -> its shape."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("%s must be a contiguous 2-D bfloat16 CUDA tensor" % name)
    _same_device(x, device, name)
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(x.shape)))
    return x.shape


def _bytes(t: torch.Tensor, name: str, shape, device) -> None:
    """A contiguous uint8 tensor of `shape` on `device`."""
    if t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous uint8 tensor of shape %s" % (name, tuple(shape)))
    _same_device(t, device, name)


def _scalar(device, t=None, fill=None, name="scalar"):
    if t is None:
        t = torch.empty(1, dtype=torch.float32, device=device)
        if fill is not None:
            t.fill_(fill)
    elif t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError("%s must be a 1-element float32 CUDA tensor" % name)
    else:
        _same_device(t, device, name)
    return t


def nvfp4_amax(tensors, amax: torch.Tensor | None = None, accumulate: bool = False) -> torch.Tensor:
    """max|x| over one bf16 tensor or a list of fused siblings -> 1-element fp32 device tensor."""
    if isinstance(tensors, torch.Tensor):
        tensors = [tensors]
    if not tensors:
        raise ValueError("nvfp4_amax needs at least one tensor")
    dev = tensors[0].device
    for i, t in enumerate(tensors):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("amax inputs must be contiguous bfloat16 CUDA tensors")
        _same_device(t, dev, "tensors[%d]" % i)
    amax = _scalar(dev, amax, name="amax")
    ptrs = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    ns = (ctypes.c_int64 * len(tensors))(*[t.numel() for t in tensors])
    _check(lib.nvfp4_amax(ptrs, ns, len(tensors), _ptr(amax), int(bool(accumulate)), _stream(dev)),
           "nvfp4_amax")
    return amax


def nvfp4_fake_quant(x: torch.Tensor, y: torch.Tensor | None = None,
                     amax_in: torch.Tensor | None = None,
                     amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [R, C] -> fake-quantized bf16 [R, C].  Without amax_in the amax of x is
    computed first, into amax_out (a scratch scalar when not given)."""
    rows, cols = _matrix(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _matrix(y, "y", x.device, x.shape)
    if amax_in is not None:
        _scalar(x.device, amax_in, name="amax_in")
    if amax_out is not None:
        _scalar(x.device, amax_out, name="amax_out")
    elif amax_in is None:
        amax_out = _scalar(x.device)
    _check(lib.nvfp4_fake_quant(_ptr(x), _ptr(y), rows, cols, _ptr(amax_in), _ptr(amax_out),
                                _stream(x.device)), "nvfp4_fake_quant")
    return y


def _group_args(xs, ys, what):
    xs = list(xs)
    if not xs:
        raise ValueError("%s needs at least one tensor" % what)
    shapes = [_matrix(x, "xs[%d]" % i) for i, x in enumerate(xs)]
    dev = xs[0].device
    ys = [torch.empty_like(x) for x in xs] if ys is None else list(ys)
    if len(ys) != len(xs):
        raise ValueError("ys must have one output per input")
    for i, (x, y) in enumerate(zip(xs, ys)):
        _same_device(x, dev, "xs[%d]" % i)
        _matrix(y, "ys[%d]" % i, dev, x.shape)
    n = len(xs)
    arrays = ((ctypes.c_void_p * n)(*[x.data_ptr() for x in xs]), (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys]),
              (ctypes.c_int64 * n)(*[r for r, _ in shapes]), (ctypes.c_int64 * n)(*[c for _, c in shapes]), n)
    return dev, ys, arrays


def nvfp4_fake_quant_group(xs, ys=None, amax_in: torch.Tensor | None = None,
                           amax_out: torch.Tensor | None = None):
    """Fake-quantize fused siblings with one shared amax -> list of bf16 outputs.
    Without amax_in the amax over all of xs is computed first, into amax_out."""
    dev, ys, arrays = _group_args(xs, ys, "nvfp4_fake_quant_group")
    if amax_in is not None:
        _scalar(dev, amax_in, name="amax_in")
    if amax_out is not None:
        _scalar(dev, amax_out, name="amax_out")
    elif amax_in is None:
        amax_out = _scalar(dev)
    _check(lib.nvfp4_fake_quant_group(*arrays, _ptr(amax_in), _ptr(amax_out), _stream(dev)),
           "nvfp4_fake_quant_group")
    return ys


def nvfp4_fake_quant_group_ws(xs, ys=None, amax_out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None):
    """nvfp4_fake_quant_group with the shared amax computed from xs (at most 8 tensors),
    through a workspace."""
    dev, ys, arrays = _group_args(xs, ys, "nvfp4_fake_quant_group_ws")
    if amax_out is not None:
        _scalar(dev, amax_out, name="amax_out")
    ws = _workspace(dev, workspace)
    _check(lib.nvfp4_fake_quant_group_ws(*arrays, _ptr(amax_out), _ptr(ws), _stream(dev)),
           "nvfp4_fake_quant_group_ws")
    return ys


def nvfp4_fake_quant_dual(x: torch.Tensor, amax0: torch.Tensor, amax1: torch.Tensor,
                          y0: torch.Tensor | None = None, y1: torch.Tensor | None = None):
    """One read of x fake-quantized under two amaxes (two observers) -> (y0, y1)."""
    rows, cols = _matrix(x, "x")
    _scalar(x.device, amax0, name="amax0")
    _scalar(x.device, amax1, name="amax1")
    y0 = torch.empty_like(x) if y0 is None else y0
    y1 = torch.empty_like(x) if y1 is None else y1
    for name, y in (("y0", y0), ("y1", y1)):
        _matrix(y, name, x.device, x.shape)
    _check(lib.nvfp4_fake_quant_dual(_ptr(x), rows, cols, _ptr(amax0), _ptr(y0), _ptr(amax1), _ptr(y1),
                                     _stream(x.device)), "nvfp4_fake_quant_dual")
    return y0, y1


def blocks_per_row(cols: int) -> int:
    """16-element blocks per row; a ragged row is zero-padded to a whole block."""
    return -(-cols // 16)


def nvfp4_quantize_pack(x: torch.Tensor, amax_in: torch.Tensor | None = None,
                        amax_out: torch.Tensor | None = None, packed: torch.Tensor | None = None,
                        scales: torch.Tensor | None = None,
                        global_scale: torch.Tensor | None = None):
    """bf16 [R, C] -> (packed uint8 [R, 8*nbr], E4M3 scale bytes uint8 [R, nbr], fp32 gs [1]),
    nbr = ceil(C / 16)."""
    rows, cols = _matrix(x, "x")
    dev = x.device
    nbr = blocks_per_row(cols)
    if packed is None:
        packed = torch.empty((rows, 8 * nbr), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, nbr), dtype=torch.uint8, device=dev)
    global_scale = _scalar(dev, global_scale, name="global_scale")
    if amax_in is not None:
        _scalar(dev, amax_in, name="amax_in")
    if amax_out is not None:
        _scalar(dev, amax_out, name="amax_out")
    elif amax_in is None:
        amax_out = _scalar(dev)
    _bytes(packed, "packed", (rows, 8 * nbr), dev)
    _bytes(scales, "scales", (rows, nbr), dev)
    _check(lib.nvfp4_quantize_pack(_ptr(x), rows, cols, _ptr(amax_in), _ptr(amax_out), _ptr(packed),
                                   _ptr(scales), _ptr(global_scale), _stream(dev)),
           "nvfp4_quantize_pack")
    return packed, scales, global_scale


def nvfp4_dequant_unpack(packed: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                         y: torch.Tensor | None = None, cols: int | None = None) -> torch.Tensor:
    """(packed [R, 8*nbr], scales [R, nbr], gs) -> bf16 [R, cols]; cols defaults to 16*nbr."""
    if packed.dtype != torch.uint8 or packed.dim() != 2 or not packed.is_cuda or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous 2-D uint8 CUDA tensor")
    if packed.shape[1] % 8:
        raise ValueError("packed rows hold 8 bytes per 16-element block")
    rows, nbr = packed.shape[0], packed.shape[1] // 8
    if cols is None:
        cols = 16 * nbr
    if blocks_per_row(cols) != nbr:
        raise ValueError("cols=%d does not match %d packed blocks per row" % (cols, nbr))
    _bytes(scales, "scales", (rows, nbr), packed.device)
    _scalar(packed.device, global_scale, name="global_scale")
    if y is None:
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=packed.device)
    _matrix(y, "y", packed.device, (rows, cols))
    _check(lib.nvfp4_dequant_unpack(_ptr(packed), _ptr(scales), _ptr(global_scale), rows, cols,
                                    _ptr(y), _stream(packed.device)), "nvfp4_dequant_unpack")
    return y


def nvfp4_linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                 global_scale: torch.Tensor, bias: torch.Tensor | None = None,
                 y: torch.Tensor | None = None) -> torch.Tensor:
    """x bf16 [M, K] times the packed weight [N, K] (transposed), plus bias -> bf16 [M, N].
    packed / scales / global_scale as nvfp4_quantize_pack returns them; K % 32 == 0."""
    m, k = _matrix(x, "x")
    if packed.dtype != torch.uint8 or packed.dim() != 2 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous 2-D uint8 CUDA tensor")
    _same_device(packed, x.device, "packed")
    n = packed.shape[0]
    if packed.shape[1] * 2 != k:
        raise ValueError("packed holds %d codes per row, x has %d columns" % (packed.shape[1] * 2, k))
    _bytes(scales, "scales", (n, k // 16), x.device)
    _scalar(x.device, global_scale, name="global_scale")
    if bias is not None:
        if bias.dtype != torch.bfloat16 or tuple(bias.shape) != (n,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous bfloat16 CUDA tensor of %d elements" % n)
        _same_device(bias, x.device, "bias")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _matrix(y, "y", x.device, (m, n))
    _check(lib.nvfp4_linear(_ptr(x), m, k, _ptr(packed), _ptr(scales), _ptr(global_scale), n, _ptr(bias),
                            _ptr(y), _stream(x.device)), "nvfp4_linear")
    return y


def nvfp4_observer_update(state: torch.Tensor, cur: torch.Tensor, mode: int = OBS_STATIC_MINMAX,
                          decay: float = 0.01) -> torch.Tensor:
    """One observer step on device scalars, in place on ``state`` (initialise it to -1)."""
    _scalar(state.device, state, name="state")
    _scalar(state.device, cur, name="cur")
    _check(lib.nvfp4_observer_update(_ptr(state), _ptr(cur), int(mode), float(decay),
                                     _stream(state.device)), "nvfp4_observer_update")
    return state


def nvfp4_observe_fake_quant(x: torch.Tensor, state0: torch.Tensor, mode0: int = OBS_STATIC_MINMAX,
                             decay0: float = 0.01, state1: torch.Tensor | None = None,
                             mode1: int = OBS_EMA, decay1: float = 0.01,
                             y0: torch.Tensor | None = None, y1: torch.Tensor | None = None,
                             cur: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """One activation step: cur = max|x|, each observer state steps on cur (in place),
    and x is fake-quantized with each new state -> y0, or (y0, y1) with two observers.
    workspace: as for the *_ws calls (a fresh one when not given)."""
    rows, cols = _matrix(x, "x")
    dev = x.device
    _scalar(dev, state0, name="state0")
    if state1 is not None:
        _scalar(dev, state1, name="state1")
    cur = _scalar(dev, cur, name="cur")
    y0 = torch.empty_like(x) if y0 is None else y0
    if state1 is not None and y1 is None:
        y1 = torch.empty_like(x)
    for name, y in (("y0", y0), ("y1", y1)):
        if y is not None:
            _matrix(y, name, dev, x.shape)
    ws = _workspace(dev, workspace)
    _check(lib.nvfp4_observe_fake_quant(_ptr(x), rows, cols, _ptr(cur), _ptr(state0), int(mode0),
                                        float(decay0), _ptr(y0), _ptr(state1), int(mode1), float(decay1),
                                        _ptr(y1), _ptr(ws), _stream(dev)), "nvfp4_observe_fake_quant")
    return y0 if state1 is None else (y0, y1)


def new_workspace(device) -> torch.Tensor:
    """A workspace for the *_ws calls (torch's allocations are 512-byte aligned).
    Reuse it for calls on one stream."""
    return torch.empty(WORKSPACE_BYTES, dtype=torch.uint8, device=device)


def _workspace(device, ws):
    if ws is None:
        return new_workspace(device)
    if ws.dtype != torch.uint8 or ws.numel() < WORKSPACE_BYTES or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor of at least %d bytes"
                         % WORKSPACE_BYTES)
    _same_device(ws, device, "workspace")
    return ws


def nvfp4_fake_quant_ws(x: torch.Tensor, y: torch.Tensor | None = None,
                        amax_out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_fake_quant with the amax computed from x, through a workspace."""
    rows, cols = _matrix(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _matrix(y, "y", x.device, x.shape)
    if amax_out is not None:
        _scalar(x.device, amax_out, name="amax_out")
    ws = _workspace(x.device, workspace)
    _check(lib.nvfp4_fake_quant_ws(_ptr(x), _ptr(y), rows, cols, _ptr(amax_out), _ptr(ws),
                                   _stream(x.device)), "nvfp4_fake_quant_ws")
    return y


def nvfp4_fake_quant_noalloc(x: torch.Tensor, y: torch.Tensor | None = None,
                             amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_fake_quant_ws on the library's own per-GPU scratch instead of a workspace:
    the call allocates nothing (pass y to allocate nothing here either).  Calls on one
    GPU must not overlap in time."""
    rows, cols = _matrix(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _matrix(y, "y", x.device, x.shape)
    if amax_out is not None:
        _scalar(x.device, amax_out, name="amax_out")
    _check(lib.nvfp4_fake_quant_noalloc(_ptr(x), _ptr(y), rows, cols, _ptr(amax_out), _stream(x.device)),
           "nvfp4_fake_quant_noalloc")
    return y


def nvfp4_quantize_pack_ws(x: torch.Tensor, amax_out: torch.Tensor | None = None,
                           packed: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                           global_scale: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None):
    """nvfp4_quantize_pack with the amax computed from x, through a workspace."""
    rows, cols = _matrix(x, "x")
    dev = x.device
    nbr = blocks_per_row(cols)
    if packed is None:
        packed = torch.empty((rows, 8 * nbr), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, nbr), dtype=torch.uint8, device=dev)
    global_scale = _scalar(dev, global_scale, name="global_scale")
    if amax_out is not None:
        _scalar(dev, amax_out, name="amax_out")
    _bytes(packed, "packed", (rows, 8 * nbr), dev)
    _bytes(scales, "scales", (rows, nbr), dev)
    ws = _workspace(dev, workspace)
    _check(lib.nvfp4_quantize_pack_ws(_ptr(x), rows, cols, _ptr(amax_out), _ptr(packed), _ptr(scales),
                                      _ptr(global_scale), _ptr(ws), _stream(dev)), "nvfp4_quantize_pack_ws")
    return packed, scales, global_scale


# ---- the MXFP4 variant: 32-element blocks, one binary32 scale each, no global scale

def mx_blocks_per_row(cols: int) -> int:
    """32-element blocks per row; a ragged row is zero-padded to a whole block."""
    return -(-cols // MX_BLOCK)


def nvfp4_mx_fake_quant(x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [R, C] -> MXFP4 fake-quantized bf16 [R, C] (y may be x)."""
    rows, cols = _matrix(x, "x")
    if y is None:
        y = torch.empty_like(x)
    _matrix(y, "y", x.device, x.shape)
    _check(lib.nvfp4_mx_fake_quant(_ptr(x), _ptr(y), rows, cols, _stream(x.device)), "nvfp4_mx_fake_quant")
    return y


def nvfp4_mx_quantize_pack(x: torch.Tensor, packed: torch.Tensor | None = None,
                           scales: torch.Tensor | None = None):
    """bf16 [R, C] -> (packed uint8 [R, 16*nbr], float32 block scales [R, nbr]), nbr = ceil(C / 32)."""
    rows, cols = _matrix(x, "x")
    dev = x.device
    nbr = mx_blocks_per_row(cols)
    if packed is None:
        packed = torch.empty((rows, 16 * nbr), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, nbr), dtype=torch.float32, device=dev)
    _bytes(packed, "packed", (rows, 16 * nbr), dev)
    if scales.dtype != torch.float32 or tuple(scales.shape) != (rows, nbr) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous float32 tensor of shape %s" % ((rows, nbr),))
    _same_device(scales, dev, "scales")
    _check(lib.nvfp4_mx_quantize_pack(_ptr(x), rows, cols, _ptr(packed), _ptr(scales), _stream(dev)),
           "nvfp4_mx_quantize_pack")
    return packed, scales


def nvfp4_mx_dequant_unpack(packed: torch.Tensor, scales: torch.Tensor, y: torch.Tensor | None = None,
                            cols: int | None = None) -> torch.Tensor:
    """(packed [R, 16*nbr], float32 scales [R, nbr]) -> bf16 [R, cols]; cols defaults to 32*nbr."""
    if packed.dtype != torch.uint8 or packed.dim() != 2 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous 2-D uint8 CUDA tensor")
    _same_device(packed, None, "packed")
    if packed.shape[1] % 16:
        raise ValueError("packed rows hold 16 bytes per 32-element block")
    rows, nbr = packed.shape[0], packed.shape[1] // 16
    if cols is None:
        cols = MX_BLOCK * nbr
    if mx_blocks_per_row(cols) != nbr:
        raise ValueError("cols=%d does not match %d packed blocks per row" % (cols, nbr))
    if scales.dtype != torch.float32 or tuple(scales.shape) != (rows, nbr) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous float32 tensor of shape %s" % ((rows, nbr),))
    _same_device(scales, packed.device, "scales")
    if y is None:
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=packed.device)
    _matrix(y, "y", packed.device, (rows, cols))
    _check(lib.nvfp4_mx_dequant_unpack(_ptr(packed), _ptr(scales), rows, cols, _ptr(y), _stream(packed.device)),
           "nvfp4_mx_dequant_unpack")
    return y


class FakeQuantSTE(torch.autograd.Function):
    """Fake-quant forward through the library; identity backward (straight-through
    estimator, verl QATLinear page section 2)."""

    @staticmethod
    def forward(ctx, x, amax_in=None, workspace=None):
        # without amax_in, a workspace (when given) saves the clearing launch
        if amax_in is None and workspace is not None:
            return nvfp4_fake_quant_ws(x.contiguous(), workspace=workspace)
        return nvfp4_fake_quant(x.contiguous(), amax_in=amax_in)

    @staticmethod
    def backward(ctx, grad_out):
        return grad_out, None, None
