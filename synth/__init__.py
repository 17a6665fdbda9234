"""Seeded synthetic bf16 inputs for the NVFP4 quantization path.

This module only *draws* inputs.  It holds none of the quantizer's arithmetic:
no amax, no scales, no rounding onto the E2M1 grid.  Both sides of every parity
check -- the CPU oracle under ``oracle/`` and the HIP library -- receive the
same byte-identical arrays from here.

Every generator returns a C-contiguous ``numpy.uint16`` array holding bf16 bit
patterns.  Values are drawn in float32 with numpy's PCG64 ``default_rng`` and
rounded to bf16 by torch's CPU cast (round-to-nearest-even), so a seed fixes the
bytes exactly.

The workloads stand in for what the pages quantize: ``nn.Linear`` weights and
activations of LLMs under QAT (verl tutorial page on ``verl.utils.qat.linear``)
and diffusion-transformer ``nn.Linear`` weights packed to FP4 (VideoX-Fun
``fp4_optimization.py`` page).  No page uses a public dataset for this path.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

__all__ = [
    "to_bf16_bits", "bits_to_f32", "normal_bf16",
    "c1_weight", "c2_weight", "c2_tie_blocks", "c3_siblings",
    "c4_outlier_channels", "c4_activation", "c4_weight", "c5_weight",
    "CONFIGS",
]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), rounded to nearest-even by torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exact float32 values."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, shape, sigma: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(sigma)
    return to_bf16_bits(a)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

def c1_weight() -> np.ndarray:
    """Single weight [256, 1024], N(0, 0.02), seed 0."""
    return normal_bf16(0, (256, 1024), 0.02)


# Exponents of the tie-block scales: E4M3 normal exponents -6..8, written as the
# power of two that multiplies a (1 + m/8) significand.
_TIE_EXPONENTS = np.arange(-6, 9)
# Quarter-steps k/4 with k in 0..24 span [0, 6]; these k sit exactly on the seven
# mid-points between neighbouring E2M1 magnitudes.
_TIE_K = np.array([1, 3, 5, 7, 10, 14, 20])


def c2_tie_blocks(rng: np.random.Generator, nblocks: int, pow2: int):
    """Blocks whose elements are exact quarter multiples of a 3-bit scale.

    Each block gets a scale ``s = c * 2**e / 2**pow2`` where ``c`` is one of
    1, 1.25, 1.5, 1.75 (an even last significand bit of a 3-bit mantissa) or a
    subnormal-range 2/512, 4/512, 6/512.  Element 0 is the anchor ``+-6 s``; the
    other fifteen are ``+-(k/4) s`` with k in 0..24, at least half of them on a
    mid-point k in {1, 3, 5, 7, 10, 14, 20}.  All products fit in bf16 exactly.
    Returns (values float32 [nblocks, 16], scale float32 [nblocks]).
    """
    n_norm = len(_TIE_EXPONENTS) * 4
    choice = rng.integers(0, n_norm + 3, size=nblocks)
    sig = np.empty(nblocks, dtype=np.float64)
    norm = choice < n_norm
    e = _TIE_EXPONENTS[np.minimum(choice, n_norm - 1) // 4]
    sig[norm] = (1.0 + 2.0 * (choice[norm] % 4) / 8.0) * np.exp2(e[norm])
    sub = ~norm
    sig[sub] = (2.0 * (choice[sub] - n_norm + 1)) / 512.0
    s = sig / np.exp2(pow2)
    k = rng.integers(0, 25, size=(nblocks, 16))
    # force at least 8 of elements 1..15 onto a mid-point
    tie_pos = rng.random((nblocks, 16)) < 0.6
    tie_pos[:, 1:9] = True
    k = np.where(tie_pos, _TIE_K[rng.integers(0, 7, size=(nblocks, 16))], k)
    k[:, 0] = 24  # anchor 6 s
    sign = np.where(rng.random((nblocks, 16)) < 0.5, -1.0, 1.0)
    vals = sign * (k / 4.0) * s[:, None]
    return vals.astype(np.float32), s.astype(np.float32)


@functools.lru_cache(maxsize=1)
def _c2_parts():
    rows, cols = 4096, 4096
    n = rows * cols
    rng = np.random.default_rng(2)
    a = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    flat = a.reshape(-1)
    out_pos = rng.choice(n, 16777, replace=False)          # 0.1 % outliers
    flat[out_pos] *= np.float32(20.0)
    # Pin the largest magnitude to 2688 * 2**-k so that the per-tensor factor is an
    # exact power of two and the injected quarter-step values are exact ties.
    big = int(np.argmax(np.abs(flat)))
    amax0 = float(np.abs(flat[big]))
    pow2 = int(np.floor(np.log2(2688.0 / amax0)))
    flat[big] = np.float32(np.copysign(2688.0 * 2.0 ** -pow2, flat[big]))
    nblocks = n // 16
    candidates = np.setdiff1d(np.arange(nblocks), [big // 16])
    tie_blocks = np.sort(rng.choice(candidates, 10486, replace=False))  # 1 % of blocks
    vals, scale = c2_tie_blocks(rng, len(tie_blocks), pow2)
    blocks = flat.reshape(nblocks, 16)
    blocks[tie_blocks] = vals
    bits = to_bf16_bits(a)
    return bits, tie_blocks, scale, pow2


def c2_weight() -> np.ndarray:
    """Weight [4096, 4096], N(0, 0.02), 0.1 % outliers x20, exact ties in 1 % of blocks, seed 2."""
    return _c2_parts()[0]


def c2_tie_info():
    """(tie block indices, tie scale per block, k with the per-tensor factor 2**k)."""
    _, blocks, scale, pow2 = _c2_parts()
    return blocks, scale, pow2


def c3_siblings():
    """Fused QKV siblings: Q [4096,4096], K [1024,4096], V [1024,4096] with std 0.02 x (1.0, 1.5, 0.7)."""
    return (normal_bf16(30, (4096, 4096), 0.02 * 1.0),
            normal_bf16(31, (1024, 4096), 0.02 * 1.5),
            normal_bf16(32, (1024, 4096), 0.02 * 0.7))


def c4_outlier_channels() -> np.ndarray:
    return np.sort(np.random.default_rng(4).choice(4096, 8, replace=False))


def c4_activation(step: int, tokens: int = 8192) -> np.ndarray:
    """Activation [tokens, 4096] ~ N(0, 1) with 8 fixed outlier channels x50; step t uses seed 400 + t."""
    rng = np.random.default_rng(400 + step)
    a = rng.standard_normal((tokens, 4096), dtype=np.float32)
    a[:, c4_outlier_channels()] *= np.float32(50.0)
    return to_bf16_bits(a)


def c4_weight() -> np.ndarray:
    """MLP weight [14336, 4096], N(0, 0.02), seed 41."""
    return normal_bf16(41, (14336, 4096), 0.02)


def c5_weight(rows: int = 28672, cols: int = 8192) -> np.ndarray:
    """Large MLP weight [28672, 8192], N(0, 0.015), 0.01 % Laplace(0, 0.015) x30 outliers, seed 5.

    ``rows`` may be lowered to draw the same recipe at a smaller size (the first
    rows then differ from the full tensor's because the outlier positions move).
    """
    rng = np.random.default_rng(5)
    a = rng.standard_normal((rows, cols), dtype=np.float32)
    a *= np.float32(0.015)
    n = rows * cols
    pos = rng.choice(n, max(1, round(n * 1e-4)), replace=False)
    lap = rng.laplace(0.0, 0.015, size=pos.size).astype(np.float32)
    a.reshape(-1)[pos] = np.float32(30.0) * lap
    return to_bf16_bits(a)


CONFIGS = {
    "c1": "weight 256x1024 N(0,0.02) seed 0",
    "c2": "weight 4096x4096 N(0,0.02), 0.1% outliers x20, exact ties in 1% of blocks, seed 2",
    "c3": "QKV siblings 4096x4096 + 2x 1024x4096, std 0.02x(1.0,1.5,0.7), seeds 30-32",
    "c4": "activations 8192x4096 N(0,1) with 8 outlier channels x50 (10 steps, seeds 400+t); "
          "weight 14336x4096 N(0,0.02) seed 41",
    "c5": "MLP weight 28672x8192 N(0,0.015), 0.01% Laplace x30 outliers, seed 5",
}
