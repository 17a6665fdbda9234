"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

tests/oracle_sanitize_main.c links the oracle's C source with both sanitizers, gives
every buffer exactly the size the oracle's contract states, and runs amax, quantize,
dequantize, fake-quant, the group amax, the observer and the element-wise forms over
ragged, empty and special-value tensors, and the MXFP4 variant's quantize, dequantize and
fake-quant on the same tensors.  Any out-of-bounds access, use after free,
leak, signed overflow, bad shift or out-of-range float-to-int conversion aborts the
run.  Its outputs must also equal the normal (-O2) build's, byte for byte: the
sanitized build is compiled at -O1, so this also checks that the oracle's results do
not depend on the optimisation level.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "nvfp4_oracle.c")
MAIN_SRC = os.path.join(HERE, "oracle_sanitize_main.c")
SANITIZERS = "-fsanitize=address,undefined,float-cast-overflow"

# ragged rows, single elements, empty, a wide row, several blocks per row
SHAPES = [(0, 16), (1, 1), (1, 16), (3, 20), (7, 1), (5, 33), (17, 144), (2, 48), (4, 16), (9, 31), (3, 64),
          (2, 65)]


def special_tensor(shape, rng):
    """Normal values over a wide range, with +-0, bf16 subnormals, the largest finite
    bf16 and values on the E2M1 grid sprinkled in."""
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-6.0, 6.0, shape))
    bits = synth.to_bf16_bits(x.astype(np.float32)).reshape(-1)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x3F00, 0x40C0, 0xC0A0,
                         0x3E80], np.uint16)
    if bits.size:
        pick = rng.random(bits.size) < 0.2
        bits[pick] = rng.choice(specials, int(pick.sum()))
    return bits.reshape(shape)


def floats(rng):
    grid = np.arange(0, 7.0, 0.125, dtype=np.float32)
    e4m3 = oracle.e4m3_decode_array(np.arange(0x7F, dtype=np.uint8))
    mids = (e4m3[:-1] + e4m3[1:]) / np.float32(2)
    wide = (rng.standard_normal(300) * np.exp(rng.uniform(-30, 30, 300))).astype(np.float32)
    edge = np.array([0.0, -0.0, 448.0, 464.0, 1e30, -1e30, np.inf, -np.inf, np.nan, 1e-45, 3.4e38],
                    np.float32)
    return np.concatenate([grid, -grid, e4m3, mids, wide, edge]).astype(np.float32)


def expected(cases, fl):
    out = bytearray()
    for x in cases:
        rows, cols = x.shape
        a = oracle.amax(x) if x.size else 0.0
        p, s, g = oracle.quantize(x, a)
        out += struct.pack("<ff", a, float(g))
        out += p.tobytes() + s.tobytes()
        out += oracle.dequantize(p, s, g, cols).tobytes()
        out += oracle.fake_quant(x, a).tobytes()
        mp, ms = oracle.mx_quantize(x)
        out += mp.tobytes() + ms.tobytes()
        out += oracle.mx_dequantize(mp, ms, cols).tobytes()
        out += oracle.mx_fake_quant(x).tobytes()
    out += struct.pack("<f", oracle.amax_group(cases))
    mag = np.abs(fl)
    out += oracle.e4m3_encode_array(fl).tobytes()
    out += oracle.e2m1_round_array(mag).tobytes()
    out += oracle.f32_to_bf16_array(fl).tobytes()
    out += oracle.e4m3_decode_array(np.arange(256, dtype=np.uint8)).tobytes()
    for m in mag[:64]:
        m = float(m)
        vals = (oracle.observer(-1.0, m, 0), oracle.observer(m, float(np.float32(2.0 * m + 1.0)), 0),
                oracle.observer(m, 0.5, 1, float(np.float32(0.01))), oracle.global_scale(m))
        out += struct.pack("<ffff", *vals)
    return bytes(out)


@pytest.fixture(scope="module")
def sanitized_binary(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("sanitize") / "oracle_sanitized")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           SANITIZERS, "-fno-sanitize-recover=all", "-o", exe, ORACLE_SRC, MAIN_SRC, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return exe


def test_oracle_is_clean_under_sanitizers(sanitized_binary, tmp_path):
    rng = np.random.default_rng(404)
    cases = [special_tensor(shape, rng) for shape in SHAPES]
    cases.append(np.zeros((3, 40), np.uint16))                       # an all-zero tensor
    fl = floats(rng)
    blob = bytearray(struct.pack("<q", len(cases)))
    for x in cases:
        blob += struct.pack("<qq", *x.shape) + np.ascontiguousarray(x, np.uint16).tobytes()
    blob += struct.pack("<q", fl.size) + fl.tobytes()
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    src.write_bytes(bytes(blob))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized_binary, str(src), str(dst)], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-4000:]
    got = dst.read_bytes()
    want = expected(cases, fl)
    assert len(got) == len(want)
    assert got == want, "first difference at byte %d" % next(i for i, (a, b) in enumerate(zip(got, want)) if a != b)
