"""CPU oracle for NVFP4 two-level block quantization -- TEST INFRASTRUCTURE.

A ctypes front end over ``nvfp4_oracle.c``: plain scalar C in IEEE binary32,
written from the pages (see the header of the C file for sources, readings and
which tests pin each function).  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP
library never does, and this package never imports the HIP library.

All arrays are numpy: bf16 tensors travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")

OBS_STATIC_MINMAX = 0
OBS_EMA = 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        F = ctypes.c_float
        sig = {
            "nvo_bf16_to_f32": (F, [ctypes.c_uint16]),
            "nvo_f32_to_bf16": (ctypes.c_uint16, [F]),
            "nvo_e4m3_decode": (F, [ctypes.c_uint8]),
            "nvo_e4m3_encode": (ctypes.c_uint8, [F]),
            "nvo_e2m1_round": (ctypes.c_int, [F]),
            "nvo_amax": (F, [P, I64]),
            "nvo_amax_group": (F, [P, P, ctypes.c_int]),
            "nvo_observer": (F, [F, F, ctypes.c_int, F]),
            "nvo_global_scale": (F, [F]),
            "nvo_quantize": (None, [P, I64, I64, F, P, P, P]),
            "nvo_dequantize": (None, [P, P, F, I64, I64, P]),
            "nvo_fake_quant": (ctypes.c_int, [P, P, I64, I64, F]),
            "nvo_e4m3_encode_array": (None, [P, P, I64]),
            "nvo_e4m3_decode_array": (None, [P, P, I64]),
            "nvo_e2m1_round_array": (None, [P, P, I64]),
            "nvo_f32_to_bf16_array": (None, [P, P, I64]),
            "nvo_mx_quantize": (None, [P, I64, I64, P, P]),
            "nvo_mx_dequantize": (None, [P, P, I64, I64, P]),
            "nvo_mx_fake_quant": (ctypes.c_int, [P, P, I64, I64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ---- scalar pieces ----------------------------------------------------------

def bf16_to_f32(h: int) -> float:
    return _load().nvo_bf16_to_f32(h)


def e4m3_decode(b: int) -> float:
    return _load().nvo_e4m3_decode(b)


def e4m3_encode(v: float) -> int:
    return _load().nvo_e4m3_encode(v)


def e2m1_round(a: float) -> int:
    return _load().nvo_e2m1_round(a)


def global_scale(amax: float) -> float:
    return _load().nvo_global_scale(amax)


def observer(state: float, cur: float, mode: int, decay: float = 0.01) -> float:
    return _load().nvo_observer(state, cur, mode, decay)


# ---- array pieces -----------------------------------------------------------

def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32).reshape(-1)
    out = np.empty(v.size, np.uint8)
    _load().nvo_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_decode_array(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint8).reshape(-1)
    out = np.empty(b.size, np.float32)
    _load().nvo_e4m3_decode_array(_ptr(b), _ptr(out), b.size)
    return out


def e2m1_round_array(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32).reshape(-1)
    out = np.empty(a.size, np.uint8)
    _load().nvo_e2m1_round_array(_ptr(a), _ptr(out), a.size)
    return out


def f32_to_bf16_array(f: np.ndarray) -> np.ndarray:
    f = _c(f, np.float32).reshape(-1)
    out = np.empty(f.size, np.uint16)
    _load().nvo_f32_to_bf16_array(_ptr(f), _ptr(out), f.size)
    return out


# ---- the path ----------------------------------------------------------------

def amax(x: np.ndarray) -> float:
    x = _c(x, np.uint16)
    return _load().nvo_amax(_ptr(x), x.size)


def amax_group(xs) -> float:
    xs = [_c(x, np.uint16) for x in xs]
    ptrs = (ctypes.c_void_p * len(xs))(*[x.ctypes.data for x in xs])
    ns = (ctypes.c_int64 * len(xs))(*[x.size for x in xs])
    return _load().nvo_amax_group(ctypes.cast(ptrs, ctypes.c_void_p),
                                  ctypes.cast(ns, ctypes.c_void_p), len(xs))


def quantize(x: np.ndarray, amax_value: float | None = None):
    """bf16 [rows, cols] -> (packed uint8 [rows, padded/2], scales uint8 [rows, padded/16], gs float32)."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    padded = -(-cols // 16) * 16
    if amax_value is None:
        amax_value = amax(x)
    packed = np.empty((rows, padded // 2), np.uint8)
    scales = np.empty((rows, padded // 16), np.uint8)
    gs = np.empty(1, np.float32)
    _load().nvo_quantize(_ptr(x), rows, cols, amax_value, _ptr(packed), _ptr(scales), _ptr(gs))
    return packed, scales, np.float32(gs[0])


def dequantize(packed: np.ndarray, scales: np.ndarray, gs, cols: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows = packed.shape[0]
    y = np.empty((rows, cols), np.uint16)
    _load().nvo_dequantize(_ptr(packed), _ptr(scales), float(np.float32(gs)), rows, cols, _ptr(y))
    return y


def fake_quant(x: np.ndarray, amax_value: float | None = None) -> np.ndarray:
    x = _c(x, np.uint16)
    rows, cols = x.shape
    if amax_value is None:
        amax_value = amax(x)
    y = np.empty((rows, cols), np.uint16)
    rc = _load().nvo_fake_quant(_ptr(x), _ptr(y), rows, cols, amax_value)
    if rc != 0:
        raise MemoryError("oracle fake_quant: allocation failed")
    return y


# ---- the MXFP4 variant (block 32, one binary32 scale per block, no global scale) ---

MX_BLOCK = 32


def mx_quantize(x: np.ndarray):
    """bf16 [rows, cols] -> (packed uint8 [rows, padded/2], scales float32 [rows, padded/32]),
    padded = cols rounded up to a multiple of 32."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    padded = -(-cols // MX_BLOCK) * MX_BLOCK
    packed = np.empty((rows, padded // 2), np.uint8)
    scales = np.empty((rows, padded // MX_BLOCK), np.float32)
    _load().nvo_mx_quantize(_ptr(x), rows, cols, _ptr(packed), _ptr(scales))
    return packed, scales


def mx_dequantize(packed: np.ndarray, scales: np.ndarray, cols: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.float32)
    rows = packed.shape[0]
    y = np.empty((rows, cols), np.uint16)
    _load().nvo_mx_dequantize(_ptr(packed), _ptr(scales), rows, cols, _ptr(y))
    return y


def mx_fake_quant(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.uint16)
    if _load().nvo_mx_fake_quant(_ptr(x), _ptr(y), rows, cols) != 0:
        raise MemoryError("oracle mx_fake_quant: allocation failed")
    return y


# ---- the consumer: a linear layer over a packed weight ---------------------------

def bf16_array_to_f64(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (a bf16 is the upper half of a binary32)."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def linear(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, gs, k: int,
           bias: np.ndarray | None = None) -> np.ndarray:
    """y = x . dq(W)^T + b in float64: the VideoX-Fun page's per-forward reconstruction,
    which dequantizes the packed weight to its bf16 form (dequantize above) and runs the
    layer's linear on it.  x: bf16 bits [M, k]; packed, scales: as quantize() returns
    them for W [N, k]; bias: bf16 bits [N] or None.  The product is a float64 library
    matmul; a device result (binary32 sums, bf16 output) is compared with it under the
    error bound that linear_magnitude() scales."""
    w = bf16_array_to_f64(dequantize(packed, scales, gs, k))
    y = bf16_array_to_f64(x) @ w.T
    if bias is not None:
        y = y + bf16_array_to_f64(bias)[None, :]
    return y


def linear_magnitude(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, gs, k: int,
                     bias: np.ndarray | None = None) -> np.ndarray:
    """sum_k |x[m, k] w[n, k]| + |b[n]|, the scale of a rounding-error bound for y."""
    w = np.abs(bf16_array_to_f64(dequantize(packed, scales, gs, k)))
    s = np.abs(bf16_array_to_f64(x)) @ w.T
    if bias is not None:
        s = s + np.abs(bf16_array_to_f64(bias))[None, :]
    return s
