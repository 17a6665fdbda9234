"""Constructed test tensors shared by the oracle pins and the GPU parity tests.

These build inputs only (bf16 bit patterns and amax values); expected outputs
always come from the oracle or from the construction itself.
"""
import numpy as np
import torch

import synth


def torch_fp8_decode(b):
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()


def torch_fp8_encode(v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def log_uniform_bf16(seed, shape, lo=-133, hi=120):
    """Magnitudes spread log-uniformly over 2^lo .. 2^hi, with a per-block factor and random signs."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(lo, hi, shape))
    blockscale = np.exp2(rng.uniform(-20, 20, (shape[0], shape[1] // 16, 1)))
    v = (mag.reshape(shape[0], -1, 16) * blockscale).reshape(shape)
    v = np.minimum(v, 1e37) * np.where(rng.random(shape) < 0.5, -1, 1)
    return synth.to_bf16_bits(v.astype(np.float32))


def scale_straddle_cases(n=48):
    """(amax, block max) pairs where fl(bamax / 6) * gs and fl(bamax * fl(1/6)) * gs round
    to different E4M3 bytes: they tell an IEEE divide by 6 from a reciprocal multiply."""
    rng = np.random.default_rng(5)
    x = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    r, r2 = x / np.float32(6), x * (np.float32(1) / np.float32(6))
    keep = (r != r2) & (x > 1e-8) & (x < 1e8)
    x, r, r2 = x[keep], r[keep], r2[keep]
    vals = torch_fp8_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2)[8:120]
    cases = []
    with np.errstate(over="ignore", invalid="ignore"):
        for i in rng.permutation(len(x)):
            gs0 = np.float32(rng.choice(mids) / np.float64(r[i]))
            for k in range(-3, 4):
                gs = np.uint32(int(gs0.view(np.uint32)) + k).view(np.float32)
                e = torch_fp8_encode(np.float32([r[i] * gs, r2[i] * gs]))
                if e[0] == e[1]:
                    continue
                a0 = np.float32(2688.0 / np.float64(gs)).view(np.uint32).astype(np.int64)
                for j in range(-8, 9):
                    a = np.uint32(int(a0) + j).view(np.float32)
                    if np.float32(2688.0) / a == gs and 1e-11 < a < 1e30:   # above the 1e-12 clamp
                        cases.append((float(a), float(x[i])))
                        break
                break
            if len(cases) == n:
                return cases
    return cases


def straddle_block(bmax):
    """One 16-element block whose largest magnitude is bmax."""
    row = np.zeros((1, 16), np.float32)
    row[0, 0] = bmax
    row[0, 1:] = np.float32(bmax) * np.float32(0.3)
    return synth.to_bf16_bits(row)
