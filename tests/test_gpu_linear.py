"""GPU parity of nvfp4_linear, the linear layer over a packed NVFP4 weight (VideoX-Fun
page, the per-forward reconstruction: dequantize the packed weight to bf16, then the
layer's linear).

Expected values come from the oracle: its dequantize() gives the bf16 weight and a
float64 matmul gives y.  The device sums binary32 products of bf16 values (exact) in an
order of its own and rounds y to bf16 once, so

    |y_dev - y| <= 2^-9 |y| (final rounding) + (1 + 2^-9) * gamma * S,
    gamma = (k + 4) * 2^-24 * 1.01,  S = sum_k |x w| + |b|,

(k products and at most 4 more additions, the standard bound for any summation order).
The test uses 2^-8 |y| + 2 (k + 8) 2^-24 S + 2^-133, which is looser than that bound, and
also holds in the bf16 subnormal range.  One case is exact: one-hot rows of x with no bias
give y = w^T exactly (as values: -0 weights come out +0), which checks every decoded
weight element through the product.
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
from gpu_util import DEV, assert_same, dev, host, say  # noqa: E402


def weight(n, k, seed, sigma=0.02):
    rng = np.random.default_rng(seed)
    w = synth.to_bf16_bits((rng.standard_normal((n, k)) * sigma).astype(np.float32))
    return oracle.quantize(w)


def to_dev_packed(packed, scales, gs):
    return (torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
            torch.tensor([gs], dtype=torch.float32, device=DEV))


def check_bound(y_dev_bits, x, packed, scales, gs, k, bias, what):
    y = oracle.linear(x, packed, scales, gs, k, bias)
    s = oracle.linear_magnitude(x, packed, scales, gs, k, bias)
    got = oracle.bf16_array_to_f64(y_dev_bits)
    tol = 2.0 ** -8 * np.abs(y) + 2 * (k + 8) * 2.0 ** -24 * s + 2.0 ** -133
    err = np.abs(got - y)
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, "%s: %d outside the bound, first %s: got %r want %r (tol %r)" % (
        what, bad.size, np.unravel_index(bad[0], y.shape), got.flat[bad[0]], y.flat[bad[0]], tol.flat[bad[0]])
    return float((err / np.maximum(tol, 1e-300)).max())


@pytest.mark.parametrize("n,k", [(40, 256), (100, 96), (16, 32), (33, 160), (300, 512), (130, 192), (200, 384),
                                 (70, 128), (260, 320)])
def test_one_hot_rows_give_the_weight_exactly(n, k):
    packed, scales, gs = weight(n, k, n + k)
    eye = np.where(np.eye(k, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    say("linear one-hot n=%d k=%d" % (n, k))
    y = nv.nvfp4_linear(dev(eye), *to_dev_packed(packed, scales, gs))
    torch.cuda.synchronize()
    # values, not bit patterns: a code-8 weight is -0, and a sum that starts at +0 gives +0
    got = oracle.bf16_array_to_f64(host(y))
    want = oracle.bf16_array_to_f64(oracle.dequantize(packed, scales, gs, k).T)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "one-hot rows: %d mismatches, first at %d: got %r want %r" % (
        bad.size, bad[0], got.flat[bad[0]], want.flat[bad[0]])
    assert (got != 0).sum() > got.size // 2


@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (16, 48, 256), (17, 40, 4096), (64, 96, 352),
                                   (100, 130, 512), (3, 2048, 8192), (200, 64, 160), (65, 1, 32)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_linear_within_the_rounding_bound(m, n, k, with_bias):
    packed, scales, gs = weight(n, k, 7 * m + n + k)
    rng = np.random.default_rng(m + 3 * n + 5 * k)
    x = synth.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    bias = synth.to_bf16_bits(rng.standard_normal(n).astype(np.float32)) if with_bias else None
    say("linear m=%d n=%d k=%d bias=%s" % (m, n, k, with_bias))
    yt = nv.nvfp4_linear(dev(x), *to_dev_packed(packed, scales, gs),
                         bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    check_bound(host(yt), x, packed, scales, gs, k, bias, "m=%d n=%d k=%d" % (m, n, k))
    # deterministic: a second call gives the same bits
    y2 = nv.nvfp4_linear(dev(x), *to_dev_packed(packed, scales, gs),
                         bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    assert torch.equal(yt.view(torch.int16), y2.view(torch.int16))


# Launch shapes the tile choice reaches: 256-wide steps whose scale bytes are not 4-byte
# aligned (k % 64 == 32, up to 16 rows of x), one workgroup per CU for widths n = 4096 c
# (c tiles of 16 weight rows per workgroup, c = 1, 3, 5, 8), several 16-row tiles of x,
# the tiled kernel from 65 rows of x where K is not a multiple of 64 (64- and 128-row
# tiles, 32- and 64-wide K steps, ragged rows of x, many x tiles, and a width that is not
# a multiple of the 128-row weight tile), and from 65 rows of x with K a multiple of 64
# the kernel that decodes weight tiles into LDS, with 128 x 128 tiles up to 256 rows and
# 256 x 256 tiles from 257 (one to three K steps
# against its four-deep load ring, whole groups of four steps with and without a partial
# last group, ragged rows of x and of the weight, several x tiles, grids with the
# XCD-ordered tiles; 128 x 128 tiles in two K groups when K / 64 is even and the tiles
# fit one per CU, in one group otherwise, as for 100 x 33000 and 256 x 33000), and on
# 256 CUs 129-256 rows whose 128 x 128 tiles outnumber the CUs as one round of 256 x 128
# tiles (192 x 28672) and the partial last round of 256 x 256 tiles re-tiled into 192-,
# 128- and 64-row weight tiles (1024 x 28672, 2048 x 12288, 512 x 33000).
@pytest.mark.parametrize("m,n,k", [(5, 40, 288), (16, 130, 800), (4, 12288, 256), (2, 20480, 128),
                                   (64, 32768, 64), (33, 4096, 96), (48, 8192, 160),
                                   (129, 256, 1024), (300, 200, 2048), (1024, 520, 256), (128, 4096, 4096),
                                   (128, 96, 192), (600, 200, 512), (512, 130, 96), (1100, 1024, 2048),
                                   (200, 300, 64), (257, 129, 128), (300, 1000, 192), (512, 4096, 320),
                                   (1030, 2056, 576), (2048, 256, 256), (400, 300, 64), (512, 129, 128),
                                   (384, 520, 192), (769, 8192, 1024), (160, 1024, 64), (383, 4096, 256),
                                   (250, 130, 128), (100, 200, 224), (80, 4096, 96), (65, 300, 1088),
                                   (96, 2056, 512), (1024, 28672, 64), (2048, 12288, 64), (512, 33000, 64),
                                   (192, 28672, 128), (100, 33000, 64), (256, 33000, 128)])
def test_linear_launch_shapes(m, n, k):
    packed, scales, gs = weight(n, k, 11 * m + n + k)
    rng = np.random.default_rng(m * 5 + n + k)
    x = synth.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    bias = synth.to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    say("linear launch shape m=%d n=%d k=%d" % (m, n, k))
    yt = nv.nvfp4_linear(dev(x), *to_dev_packed(packed, scales, gs), bias=dev(bias))
    torch.cuda.synchronize()
    check_bound(host(yt), x, packed, scales, gs, k, bias, "m=%d n=%d k=%d" % (m, n, k))


# Up to 16 rows of x with wide K (1024 to 8192): every count of 16-row weight tiles per
# workgroup (1-8 for widths n = 4096 c; 4, 2 and 1 otherwise, with a ragged last
# workgroup), one to sixteen rows of x, 128- and 256-wide K steps over several rounds
# of the eight waves.
@pytest.mark.parametrize("m,n,k", [(1, 4096, 1024), (16, 12288, 2048), (5, 32768, 1024), (7, 16400, 1024),
                                   (2, 8200, 2048), (16, 20480, 3072), (9, 24576, 1024), (1, 33, 1024),
                                   (12, 8192, 8192), (3, 28672, 1024), (16, 16384, 1024)])
def test_small_m_wide_k(m, n, k):
    packed, scales, gs = weight(n, k, 13 * m + n + k)
    rng = np.random.default_rng(m * 7 + n + 3 * k)
    x = synth.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    bias = synth.to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    say("linear small m, wide k: m=%d n=%d k=%d" % (m, n, k))
    yt = nv.nvfp4_linear(dev(x), *to_dev_packed(packed, scales, gs), bias=dev(bias))
    torch.cuda.synchronize()
    check_bound(host(yt), x, packed, scales, gs, k, bias, "m=%d n=%d k=%d" % (m, n, k))


@pytest.mark.parametrize("n,k", [(40, 1024), (12288, 3072)])
def test_one_hot_rows_of_few_tokens_give_the_weight_exactly(n, k):
    """Sixteen one-hot rows of x (columns spread over every K step, wave and lane group)
    read back those columns of the decoded weight exactly."""
    packed, scales, gs = weight(n, k, 3 * n + k)
    rng = np.random.default_rng(n + k)
    cols = np.concatenate([[0, k - 1], rng.choice(np.arange(1, k - 1), 14, replace=False)])
    x = np.zeros((16, k), dtype=np.uint16)
    x[np.arange(16), cols] = 0x3F80
    say("linear one-hot, 16 rows, n=%d k=%d" % (n, k))
    y = nv.nvfp4_linear(dev(x), *to_dev_packed(packed, scales, gs))
    torch.cuda.synchronize()
    got = oracle.bf16_array_to_f64(host(y))
    want = oracle.bf16_array_to_f64(oracle.dequantize(packed, scales, gs, k)[:, cols].T)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "one-hot rows: %d mismatches, first at %d: got %r want %r" % (
        bad.size, bad[0], got.flat[bad[0]], want.flat[bad[0]])
    assert (got != 0).sum() > got.size // 2


def test_c5_weight_as_a_layer():
    """The c5 weight (28672 x 8192) quantized on the device, then used as a linear layer
    on 1, 16 and 64 tokens (the register-decode kernel) and 256, 1024 and 2048 tokens
    (the LDS-staged kernel; on 256 CUs 256 tokens take 256 x 128 tiles, and 1024 and
    2048 tokens re-tile the last round of tiles), shapes the bench times; sampled output
    columns, the last one among them, are checked against the oracle."""
    w = synth.c5_weight()
    say("linear on the c5 weight")
    packed, scales, gs = nv.nvfp4_quantize_pack(dev(w))
    rng = np.random.default_rng(55)
    cols = np.unique(np.concatenate([[0, w.shape[0] - 1], rng.choice(w.shape[0], 62, replace=False)]))
    p_rows, s_rows = packed.cpu().numpy()[cols], scales.cpu().numpy()[cols]
    g = float(gs.item())
    p_ref, s_ref, g_ref = oracle.quantize(w[cols], oracle.amax(w))
    assert_same(p_rows, p_ref, "c5 packed rows")
    assert_same(s_rows, s_ref, "c5 scale rows")
    for m in (1, 16, 64, 256, 1024, 2048):
        x = synth.to_bf16_bits(rng.standard_normal((m, w.shape[1])).astype(np.float32))
        y = nv.nvfp4_linear(dev(x), packed, scales, gs)
        torch.cuda.synchronize()
        check_bound(host(y)[:, cols], x, p_rows, s_rows, g, w.shape[1], None, "c5 sampled columns, m=%d" % m)


def test_empty_and_rejected_shapes():
    packed, scales, gs = to_dev_packed(*weight(8, 64, 1))
    y = nv.nvfp4_linear(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), packed, scales, gs)
    assert y.shape == (0, 8)
    with pytest.raises(nv.NVFP4Error):
        p2, s2, g2 = to_dev_packed(*weight(8, 48, 2))
        nv.nvfp4_linear(torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV), p2, s2, g2)
