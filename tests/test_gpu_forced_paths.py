"""Code paths that ordinary shapes rarely or never reach, forced on everything, against
the oracle bit for bit.  tests/libnvfp4_test_paths.so is libnvfp4's own source built
with three switches, and the binding is pointed at it for the duration of this module:

* every quantizing wave on the exact-quotient code path.  In the library a wave takes
  it only when one of its blocks has a scale byte whose multiplier is not certified
  (for example the c2 weight, whose global scale is a power of two and whose mantissa-7
  scale bytes meet exact ties).  Here it runs under every scale byte of every global
  scale the cases reach: the sweeps of every bf16 magnitude around every decision
  threshold and as a block maximum, every code times every scale, exact ties, underflow
  and -0, wide dynamic ranges, saturating and clamped amaxes, and whole c2 and c4-weight
  tensors;
* every ragged shape (rows not a multiple of the block) through the one-lane-per-block
  kernels, NVFP4 and MXFP4, which the library keeps for tensors of 2^31 (MXFP4: 2^30)
  blocks and more, and the workspace calls through their three-launch form (a
  one-workgroup reduction of the partial maxima between the passes): the ragged parity,
  workspace, observer and MXFP4 cases.
* the linear layer's tile rounds planned for 6 CUs instead of the device's, so that
  small layers reach each narrower tile of the re-tiled last round of 256 x 256 tiles
  (64, 128 and 192 weight rows) and the 256 x 128 tiles that 129-256 rows of x take
  when their 128 x 128 tiles outnumber the CUs: the oracle's rounding bound, and
  one-hot rows of x that read back every decoded weight exactly.

The parity helpers are those of test_gpu_parity.py, test_gpu_workspace.py,
test_gpu_observe.py and test_gpu_mx.py.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import fp4_block_fake_amd as nv  # noqa: E402
import test_gpu_mx as mx  # noqa: E402
import test_gpu_observe as observe  # noqa: E402
import test_gpu_parity as parity  # noqa: E402
import test_gpu_linear as linear  # noqa: E402
import test_gpu_workspace as workspace  # noqa: E402

EXACT_LIB = os.path.join(ROOT, "tests", "libnvfp4_test_paths.so")


@pytest.fixture(scope="module", autouse=True)
def exact_path_library():
    if not os.path.exists(EXACT_LIB):
        pytest.fail("tests/libnvfp4_test_paths.so is not built (run __graft_entry__.build())")
    saved = nv.lib
    nv.lib = nv._load(EXACT_LIB)
    yield
    nv.lib = saved


@pytest.mark.parametrize("amax_value", parity.SWEEP_AMAX)
def test_every_magnitude_around_every_threshold(amax_value):
    parity.test_every_magnitude_around_every_threshold(amax_value)


@pytest.mark.parametrize("amax_value", parity.SWEEP_AMAX)
def test_every_bf16_magnitude_as_a_block(amax_value):
    parity.test_every_bf16_magnitude_as_a_block(amax_value)


@pytest.mark.parametrize("k", [4, 10, 12])
def test_every_code_times_every_scale(k):
    parity.test_every_code_times_every_scale(k)


def test_exact_ties():
    parity.test_exact_ties()


def test_underflow_and_negative_zero_codes():
    parity.test_underflow_and_negative_zero_codes()


def test_zero_and_negative_zero_tensor():
    parity.test_zero_and_negative_zero_tensor()


@pytest.mark.parametrize("seed,lo,hi", [(1, -133, 120), (2, -140, -100), (3, 60, 127), (4, -30, 10)])
def test_wide_dynamic_range(seed, lo, hi):
    parity.test_wide_dynamic_range(seed, lo, hi)


@pytest.mark.parametrize("amax_in", [1e-20, 3e-12, 0.01, 0.37, 6.0, 12345.6, 5e20, 3.3e38])
def test_cached_amax_saturation_and_clamp(amax_in):
    parity.test_cached_amax_saturation_and_clamp(amax_in)


def test_block_scale_divide_by_six_straddles():
    parity.test_block_scale_divide_by_six_straddles()


def test_c2_whole():
    parity.check_all_ops(synth.c2_weight(), what="c2 (forced paths)")


def test_c4_weight_whole():
    w = synth.c4_weight()
    parity.say("c4 weight %s (forced paths)" % (w.shape,))
    amax = parity.scalar(0.0)
    y = nv.nvfp4_fake_quant(parity.dev(w), amax_out=amax)
    torch.cuda.synchronize()
    a = parity.oracle_amax(w)
    assert parity.fbits(amax.item()) == parity.fbits(a)
    parity.assert_same(parity.host(y), parity.oracle_fake_quant(w, a), "c4 weight fq (forced paths)")


def test_the_library_is_the_test_build():
    assert nv.lib._name == EXACT_LIB
    x = np.zeros((1, 16), np.uint16)
    parity.check_all_ops(x, amax_in=1.0, what="test build loaded")


RAGGED = [(1, 1), (3, 7), (5, 15), (4, 17), (33, 40), (9, 1000), (2, 4097), (130, 24), (1000, 33), (2, 2),
          (7, 18), (64, 4100), (1025, 30), (17, 1006), (300, 62), (513, 8)]


@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_columns_zero_padded(shape):
    parity.test_ragged_columns_zero_padded(shape)


@pytest.mark.parametrize("shape", [s for s in workspace.SHAPES if s[1] % 16])
@pytest.mark.parametrize("inplace", [False, True])
def test_ragged_fake_quant_ws(shape, inplace):
    workspace.test_fake_quant_ws(shape, inplace)


@pytest.mark.parametrize("shape", [s for s in workspace.SHAPES if s[1] % 16])
def test_ragged_quantize_pack_ws(shape):
    workspace.test_quantize_pack_ws(shape)


@pytest.mark.parametrize("shape", [s for s in observe.SHAPES if s[1] % 16])
@pytest.mark.parametrize("inplace", [None, 0, 1])
def test_ragged_observe_fake_quant(shape, inplace):
    observe.test_two_observers_shapes(shape, inplace)


@pytest.mark.parametrize("shape", mx.MX_RAGGED)
def test_mx_ragged_rows(shape):
    mx.test_ragged_rows_zero_padded(shape)


# (m, n, k) and the tile width of the re-tiled last round when 6 CUs are planned for:
# two 256-row tiles of x (the second ragged), three whole 256-wide tiles per x tile in
# the first launch, then the remaining 100, 232 and 450 weight rows as 64-, 128- and
# 192-row tiles (ragged at the end).
RETILE = [((400, 868, 128), 64), ((400, 1000, 128), 128), ((400, 1218, 192), 192)]


def retile_width(m, n, cus=6):
    """The host's plan, restated: the narrower tile width, or 256 when nothing is re-tiled."""
    mt = (m + 255) // 256
    tiles = mt * ((n + 255) // 256)
    whole = tiles // cus * cus
    if not (tiles > cus and whole < tiles and whole % mt == 0):
        return 256
    rest = n - whole // mt * 256
    for w in (64, 128, 192):
        if mt * ((rest + w - 1) // w) <= cus:
            return w
    return 256


@pytest.mark.parametrize("shape,width", RETILE)
def test_linear_retiled_last_round(shape, width):
    m, n, k = shape
    assert retile_width(m, n) == width
    linear.test_linear_launch_shapes(m, n, k)


# 129-256 rows of x whose 128 x 128 tiles outnumber the CUs run as one round of
# 256 x 128 tiles; with 6 CUs that is 385-768 weight rows.
NARROW = [(129, 390, 192), (200, 600, 128), (256, 768, 64)]


def narrow_tiles(m, n, cus=6):
    """The host's choice of 256 x 128 tiles, restated."""
    return 128 < m <= 256 and 2 * ((n + 127) // 128) > cus and (n + 127) // 128 <= cus


@pytest.mark.parametrize("shape", NARROW)
def test_linear_narrow_tiles(shape):
    m, n, k = shape
    assert narrow_tiles(m, n) and not narrow_tiles(m, 384) and not narrow_tiles(128, n)
    linear.test_linear_launch_shapes(m, n, k)


@pytest.mark.parametrize("shape,width", RETILE + [(shape, 128) for shape in NARROW])
def test_linear_retiled_one_hot(shape, width):
    m, n, k = shape
    packed, scales, gs = linear.weight(n, k, n + 3 * k)
    eye = np.where(np.eye(k, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    x = np.concatenate([eye] * ((m + k - 1) // k))[:m]
    parity.say("linear re-tiled one-hot m=%d n=%d k=%d" % (m, n, k))
    y = nv.nvfp4_linear(parity.dev(x), *linear.to_dev_packed(packed, scales, gs))
    torch.cuda.synchronize()
    got = oracle.bf16_array_to_f64(parity.host(y))
    w = oracle.bf16_array_to_f64(oracle.dequantize(packed, scales, gs, k).T)
    want = np.concatenate([w] * ((m + k - 1) // k))[:m]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "re-tiled one-hot rows: %d mismatches, first at %d" % (bad.size, bad[0])
