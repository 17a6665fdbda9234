"""C ABI checks that need no GPU: the library loads, exports what include/nvfp4.h
declares, and rejects bad arguments on the host before enqueuing anything.

The pointers below are never dereferenced: every call here fails validation,
which runs before any HIP call.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT

nv = pytest.importorskip("fp4_block_fake_amd")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_OVERLAP, ERR_ARG = 0, 1, 2, 3, 4, 5
A = 0x7F0000000000            # a 256-byte-aligned fake device address
N = None


def P(addr):
    return ctypes.c_void_p(addr)


def declared_functions():
    with open(os.path.join(ROOT, "include", "nvfp4.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_]+)\s*\(", text)))


def test_header_declares_every_call():
    names = declared_functions()
    for n in ("nvfp4_amax", "nvfp4_fake_quant", "nvfp4_fake_quant_group", "nvfp4_fake_quant_dual",
              "nvfp4_quantize_pack", "nvfp4_dequant_unpack", "nvfp4_linear", "nvfp4_observer_update",
              "nvfp4_observe_fake_quant", "nvfp4_fake_quant_ws", "nvfp4_quantize_pack_ws",
              "nvfp4_fake_quant_group_ws", "nvfp4_fake_quant_noalloc", "nvfp4_mx_fake_quant",
              "nvfp4_mx_quantize_pack", "nvfp4_mx_dequant_unpack", "nvfp4_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(nv.library_path)
    for name in declared_functions():
        assert hasattr(so, name), name


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "nvfp4.h"

int main(void)
{
    /* every call is reachable from C; the arguments below fail validation, which
       returns before any HIP call */
    const void* xs[1] = {0};
    int64_t numels[1] = {16};
    int bad = 0;
    bad |= nvfp4_amax(xs, numels, 1, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_fake_quant(0, 0, 4, 16, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_fake_quant_group(0, 0, 0, 0, 1, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_fake_quant_dual(0, 4, 0, 0, 0, 0, 0, 0) != NVFP4_ERR_SHAPE;
    bad |= nvfp4_quantize_pack(0, -1, 16, 0, 0, 0, 0, 0, 0) != NVFP4_ERR_SHAPE;
    bad |= nvfp4_dequant_unpack(0, 0, 0, 4, 16, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_linear(0, 4, 48, 0, 0, 0, 8, 0, 0, 0) != NVFP4_ERR_SHAPE;
    bad |= nvfp4_observer_update(0, 0, NVFP4_OBS_EMA, 0.5f, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_observe_fake_quant(0, 4, 16, 0, 0, 0, 0.0f, 0, 0, 0, 0.0f, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_fake_quant_ws(0, 0, 4, 16, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_quantize_pack_ws(0, 4, 0, 0, 0, 0, 0, 0, 0) != NVFP4_ERR_SHAPE;
    bad |= nvfp4_fake_quant_group_ws(0, 0, 0, 0, 1, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_fake_quant_noalloc(0, 0, 4, 16, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_mx_fake_quant(0, 0, 4, 0, 0) != NVFP4_ERR_SHAPE;
    bad |= nvfp4_mx_quantize_pack(0, 4, 32, 0, 0, 0) != NVFP4_ERR_NULL;
    bad |= nvfp4_mx_dequant_unpack(0, 0, 4, 32, 0, 0) != NVFP4_ERR_NULL;
    bad |= NVFP4_MX_BLOCK != 32;
    bad |= NVFP4_WORKSPACE_BYTES < 2304;
    bad |= strcmp(nvfp4_strerror(NVFP4_OK), "ok") != 0;
    printf("%s\n", bad ? "FAIL" : "OK");
    return bad;
}
"""


def test_header_is_c99_and_links(tmp_path):
    """include/nvfp4.h compiles as C99 and a C program links and calls the library."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(nv.library_path)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                           str(src), "-o", str(exe), "-L", libdir, "-lnvfp4", "-Wl,-rpath," + libdir])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout + out.stderr


def test_strerror_names_every_status():
    for s in range(7):
        assert nv.nvfp4_strerror(s) and nv.nvfp4_strerror(s) != "unknown status"
    assert nv.nvfp4_strerror(99) == "unknown status"


def fq(x, y, rows, cols, amax_in, amax_out):
    return nv.lib.nvfp4_fake_quant(P(x), P(y), rows, cols, P(amax_in), P(amax_out), None)


def test_fake_quant_validation():
    assert fq(A, A + (1 << 30), 4, 0, None, A + (2 << 30)) == ERR_SHAPE          # cols < 1
    assert fq(A, A + (1 << 30), 4, -16, None, A + (2 << 30)) == ERR_SHAPE
    assert fq(A, A + (1 << 30), -1, 16, None, A + (2 << 30)) == ERR_SHAPE
    assert fq(A, A + (1 << 30), 1 << 40, 1 << 40, None, A + (2 << 30)) == ERR_SHAPE  # overflow
    assert fq(None, A, 4, 16, None, A + (2 << 30)) == ERR_NULL
    assert fq(A, None, 4, 16, None, A + (2 << 30)) == ERR_NULL
    assert fq(A, A + (1 << 30), 4, 16, None, None) == ERR_NULL                   # amax needed
    assert fq(A + 2, A + (1 << 30), 4, 16, None, A + (2 << 30)) == ERR_ALIGN
    assert fq(A, A + (1 << 30) + 8, 4, 16, None, A + (2 << 30)) == ERR_ALIGN
    assert fq(A, A + (1 << 30), 4, 16, None, A + (2 << 30) + 1) == ERR_ALIGN
    assert fq(A, A + 16, 4, 16, None, A + (2 << 30)) == ERR_OVERLAP             # partial overlap
    assert fq(A, A + (1 << 30), 4, 16, None, A + 64) == ERR_OVERLAP             # amax inside x
    assert fq(A, A + (1 << 30), 4, 16, A + (1 << 30) + 4, None) == ERR_OVERLAP  # amax_in inside y


def test_fake_quant_group_validation():
    g = nv.lib.nvfp4_fake_quant_group
    G = 1 << 30

    def call(xs, ys, shapes, amax_in=None, amax_out=A + 9 * G, n=None):
        n = len(xs) if n is None else n
        k = max(len(xs), 1)
        xp = (ctypes.c_void_p * k)(*xs)
        yp = (ctypes.c_void_p * k)(*ys)
        rs = (ctypes.c_int64 * k)(*[r for r, _ in shapes])
        cs = (ctypes.c_int64 * k)(*[c for _, c in shapes])
        return g(xp, yp, rs, cs, n, P(amax_in), P(amax_out), None)

    x0, x1, y0, y1 = A, A + G, A + 2 * G, A + 3 * G
    sh = [(4, 16), (8, 32)]
    assert g(None, None, None, None, 1, None, P(A), None) == ERR_NULL
    assert call([x0], [y0], [(4, 16)], n=0) == ERR_ARG
    assert call([x0, x1], [y0, y1], [(4, 16), (4, 0)]) == ERR_SHAPE
    assert call([x0, None], [y0, y1], sh) == ERR_NULL
    assert call([x0, x1], [y0, y1], sh, amax_in=None, amax_out=None) == ERR_NULL
    assert call([x0, x1 + 8], [y0, y1], sh) == ERR_ALIGN
    assert call([x0, x1], [y0, y1 + 4], sh) == ERR_ALIGN
    assert call([x0, x1], [y0, y1], sh, amax_out=A + 9 * G + 2) == ERR_ALIGN
    assert call([x0, x1], [x1, y1], sh) == ERR_OVERLAP             # y0 is another member's input
    assert call([x0, x1], [y0, y0 + 64], sh) == ERR_OVERLAP        # two outputs overlap
    assert call([x0, x1], [x0 + 16, y1], sh) == ERR_OVERLAP        # partial overlap with its input
    assert call([x0, x1], [y0, y1], sh, amax_out=x1 + 4) == ERR_OVERLAP
    assert call([x0, x1], [y0, y1], sh, amax_in=y1 + 8) == ERR_OVERLAP


def test_fake_quant_dual_validation():
    d = nv.lib.nvfp4_fake_quant_dual
    G = 1 << 30
    x, y0, y1, a0, a1 = A, A + G, A + 2 * G, A + 3 * G, A + 3 * G + 4
    assert d(P(x), 4, 0, P(a0), P(y0), P(a1), P(y1), None) == ERR_SHAPE
    assert d(P(x), -1, 16, P(a0), P(y0), P(a1), P(y1), None) == ERR_SHAPE
    assert d(None, 4, 16, P(a0), P(y0), P(a1), P(y1), None) == ERR_NULL
    assert d(P(x), 4, 16, None, P(y0), P(a1), P(y1), None) == ERR_NULL
    assert d(P(x), 4, 16, P(a0), P(y0), None, P(y1), None) == ERR_NULL
    assert d(P(x), 4, 16, P(a0), P(y0), P(a1), None, None) == ERR_NULL
    assert d(P(x + 8), 4, 16, P(a0), P(y0), P(a1), P(y1), None) == ERR_ALIGN
    assert d(P(x), 4, 16, P(a0 + 1), P(y0), P(a1), P(y1), None) == ERR_ALIGN
    assert d(P(x), 4, 16, P(a0), P(y0), P(a1), P(y0), None) == ERR_OVERLAP     # y0 == y1
    assert d(P(x), 4, 16, P(a0), P(x), P(a1), P(x), None) == ERR_OVERLAP       # both in place
    assert d(P(x), 4, 16, P(a0), P(x + 32), P(a1), P(y1), None) == ERR_OVERLAP  # partial
    assert d(P(x), 4, 16, P(y1 + 4), P(y0), P(a1), P(y1), None) == ERR_OVERLAP  # amax in an output


def test_quantize_pack_validation():
    q = nv.lib.nvfp4_quantize_pack
    x, p, s, g, a = A, A + (1 << 30), A + (2 << 30), A + (3 << 30), A + (4 << 30)
    assert q(P(x), 4, 0, None, P(a), P(p), P(s), P(g), None) == ERR_SHAPE
    # a ragged row (cols 20) pads to 2 blocks: 16 packed bytes per row, so 64 overlap 48 past p
    assert q(P(x), 4, 20, None, P(a), P(p), P(p + 48), P(g), None) == ERR_OVERLAP
    assert q(P(x), 4, 16, None, None, P(p), P(s), P(g), None) == ERR_NULL
    assert q(P(x), 4, 16, None, P(a), None, P(s), P(g), None) == ERR_NULL
    assert q(P(x), 4, 16, None, P(a), P(p), P(s), None, None) == ERR_NULL
    assert q(P(x), 4, 16, None, P(a), P(p + 4), P(s), P(g), None) == ERR_ALIGN
    assert q(P(x), 4, 16, None, P(a), P(p), P(s), P(g + 2), None) == ERR_ALIGN
    assert q(P(x), 4, 16, None, P(a), P(x + 8), P(s), P(g), None) == ERR_OVERLAP   # packed in x
    assert q(P(x), 4, 16, None, P(a), P(p), P(p + 16), P(g), None) == ERR_OVERLAP  # scales in packed
    assert q(P(x), 4, 16, None, P(s), P(p), P(s), P(g), None) == ERR_OVERLAP       # amax_out on scales
    assert q(P(x), 4, 16, P(g), None, P(p), P(s), P(g), None) == ERR_OVERLAP       # gs on amax_in


def test_dequant_unpack_validation():
    d = nv.lib.nvfp4_dequant_unpack
    p, s, g, y = A, A + (1 << 30), A + (2 << 30), A + (3 << 30)
    assert d(P(p), P(s), P(g), 4, 0, P(y), None) == ERR_SHAPE
    assert d(P(p), P(s), P(g), 4, 17, P(p + 64 - 8), None) == ERR_ALIGN
    assert d(None, P(s), P(g), 4, 16, P(y), None) == ERR_NULL
    assert d(P(p), P(s), P(g), 4, 16, None, None) == ERR_NULL
    assert d(P(p + 1), P(s), P(g), 4, 16, P(y), None) == ERR_ALIGN
    assert d(P(p), P(s), P(g), 4, 16, P(y + 8), None) == ERR_ALIGN
    assert d(P(p), P(s), P(g), 4, 16, P(p), None) == ERR_OVERLAP
    assert d(P(p), P(s), P(g), 4, 16, P(g - 16), None) == ERR_OVERLAP


def test_linear_validation():
    li = nv.lib.nvfp4_linear
    G = 1 << 30
    x, p, sc, g, b, y = A, A + G, A + 2 * G, A + 3 * G, A + 3 * G + 256, A + 4 * G
    assert li(P(x), 4, 48, P(p), P(sc), P(g), 8, None, P(y), None) == ERR_SHAPE      # k % 32
    assert li(P(x), 4, 16, P(p), P(sc), P(g), 8, None, P(y), None) == ERR_SHAPE      # k < 32
    assert li(P(x), -1, 64, P(p), P(sc), P(g), 8, None, P(y), None) == ERR_SHAPE
    assert li(P(x), 4, 64, P(p), P(sc), P(g), -8, None, P(y), None) == ERR_SHAPE
    assert li(P(x), 64 * 65536, 64, P(p), P(sc), P(g), 8, None, P(y), None) == ERR_SHAPE  # grid rows
    assert li(None, 4, 64, P(p), P(sc), P(g), 8, None, P(y), None) == ERR_NULL
    assert li(P(x), 4, 64, None, P(sc), P(g), 8, None, P(y), None) == ERR_NULL
    assert li(P(x), 4, 64, P(p), None, P(g), 8, None, P(y), None) == ERR_NULL
    assert li(P(x), 4, 64, P(p), P(sc), None, 8, None, P(y), None) == ERR_NULL
    assert li(P(x), 4, 64, P(p), P(sc), P(g), 8, None, None, None) == ERR_NULL
    assert li(P(x + 8), 4, 64, P(p), P(sc), P(g), 8, None, P(y), None) == ERR_ALIGN
    assert li(P(x), 4, 64, P(p + 8), P(sc), P(g), 8, None, P(y), None) == ERR_ALIGN
    assert li(P(x), 4, 64, P(p), P(sc + 1), P(g), 8, None, P(y), None) == ERR_ALIGN
    assert li(P(x), 4, 64, P(p), P(sc), P(g), 8, P(b + 1), P(y), None) == ERR_ALIGN
    assert li(P(x), 4, 64, P(p), P(sc), P(g), 8, None, P(y + 1), None) == ERR_ALIGN
    assert li(P(x), 4, 64, P(p), P(sc), P(g), 8, None, P(x + 64), None) == ERR_OVERLAP
    assert li(P(x), 4, 64, P(p), P(sc), P(g), 8, None, P(p + 32), None) == ERR_OVERLAP
    assert li(P(x), 4, 64, P(p), P(sc), P(g), 8, P(b), P(b - 2), None) == ERR_OVERLAP


def test_amax_validation():
    am = nv.lib.nvfp4_amax
    ptrs = (ctypes.c_void_p * 2)(A, A + (1 << 30))
    ns = (ctypes.c_int64 * 2)(64, 64)
    assert am(None, ns, 2, P(A + (2 << 30)), 0, None) == ERR_NULL
    assert am(ptrs, ns, 2, None, 0, None) == ERR_NULL
    assert am(ptrs, ns, 0, P(A + (2 << 30)), 0, None) == ERR_ARG
    bad_n = (ctypes.c_int64 * 2)(64, -1)
    assert am(ptrs, bad_n, 2, P(A + (2 << 30)), 0, None) == ERR_SHAPE
    nul = (ctypes.c_void_p * 2)(A, None)
    assert am(nul, ns, 2, P(A + (2 << 30)), 0, None) == ERR_NULL
    mis = (ctypes.c_void_p * 2)(A, A + 2)
    assert am(mis, ns, 2, P(A + (2 << 30)), 0, None) == ERR_ALIGN
    assert am(ptrs, ns, 2, P(A + 8), 0, None) == ERR_OVERLAP
    assert am(ptrs, ns, 2, P(A + (2 << 30) + 2), 0, None) == ERR_ALIGN


def test_observer_validation():
    ob = nv.lib.nvfp4_observer_update
    s, c = P(A), P(A + 256)
    assert ob(None, c, 0, 0.01, None) == ERR_NULL
    assert ob(s, None, 0, 0.01, None) == ERR_NULL
    assert ob(P(A + 2), c, 0, 0.01, None) == ERR_ALIGN
    assert ob(s, c, 2, 0.01, None) == ERR_ARG
    assert ob(s, c, -1, 0.01, None) == ERR_ARG
    for bad in (0.0, -0.5, 1.5, float("nan")):
        assert ob(s, c, 1, bad, None) == ERR_ARG


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv.nvfp4_fake_quant(x)
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_pack(x)
    with pytest.raises(ValueError):
        nv.nvfp4_amax([x])


def test_observe_fake_quant_validation():
    f = nv.lib.nvfp4_observe_fake_quant
    G = 1 << 30
    x, y0, y1, s0, s1, c, w = A, A + G, A + 2 * G, A + 3 * G, A + 4 * G, A + 5 * G, A + 6 * G
    S, E = nv.OBS_STATIC_MINMAX, nv.OBS_EMA

    def call(x=x, rows=4, cols=16, cur=c, st0=s0, m0=S, d0=0.0, out0=y0, st1=s1, m1=E, d1=0.01, out1=y1, ws=w):
        return f(P(x), rows, cols, P(cur), P(st0), m0, d0, P(out0), P(st1), m1, d1, P(out1), P(ws), None)

    assert call(cols=0) == ERR_SHAPE
    assert call(rows=-2) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(cur=None) == ERR_NULL                           # the step amax goes somewhere
    assert call(st0=None) == ERR_NULL
    assert call(out0=None) == ERR_NULL
    assert call(out1=None) == ERR_NULL                          # two observers need two outputs
    assert call(rows=0, x=None, out0=None, out1=None, cur=None) == ERR_NULL
    assert call(st1=None) == ERR_ARG                            # y1 without a second observer
    assert call(m0=2) == ERR_ARG
    assert call(m1=-1) == ERR_ARG
    assert call(m1=E, d1=0.0) == ERR_ARG
    assert call(m1=E, d1=1.5) == ERR_ARG
    assert call(m0=E, d0=float("nan")) == ERR_ARG
    assert call(out0=y0 + 8) == ERR_ALIGN
    assert call(x=x + 2) == ERR_ALIGN
    assert call(st1=s1 + 2) == ERR_ALIGN
    assert call(cur=c + 1) == ERR_ALIGN
    assert call(out0=x + 32) == ERR_OVERLAP                     # partial overlap with x
    assert call(out0=x, out1=x) == ERR_OVERLAP                  # both outputs in place
    assert call(out1=y0 + 64) == ERR_OVERLAP
    assert call(st1=s0) == ERR_OVERLAP                          # one state for both observers
    assert call(cur=s0) == ERR_OVERLAP
    assert call(cur=s1) == ERR_OVERLAP
    assert call(st0=x + 4) == ERR_OVERLAP
    assert call(cur=y1 + 8) == ERR_OVERLAP
    assert call(ws=None) == ERR_NULL
    assert call(ws=w + 64) == ERR_ALIGN
    assert call(ws=y0) == ERR_OVERLAP
    assert call(cur=w + 8) == ERR_OVERLAP                       # cur inside the workspace


def test_workspace_size_matches_binding():
    with open(os.path.join(ROOT, "include", "nvfp4.h")) as f:
        m = re.search(r"#define NVFP4_WORKSPACE_BYTES (\d+)", f.read())
    assert m and int(m.group(1)) == nv.WORKSPACE_BYTES


def test_fake_quant_ws_validation():
    f = nv.lib.nvfp4_fake_quant_ws
    G = 1 << 30
    x, y, a, w = A, A + G, A + 2 * G, A + 3 * G

    def call(x=x, y=y, rows=4, cols=16, amax=a, ws=w):
        return f(P(x), P(y), rows, cols, P(amax), P(ws), None)

    assert call(cols=0) == ERR_SHAPE
    assert call(rows=-1) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(y=None) == ERR_NULL
    assert call(ws=None) == ERR_NULL                            # the workspace is required
    assert call(rows=0, x=None, y=None, ws=None) == ERR_NULL
    assert call(x=x + 8) == ERR_ALIGN
    assert call(ws=w + 128) == ERR_ALIGN                        # 256-byte aligned
    assert call(amax=a + 2) == ERR_ALIGN
    assert call(y=x + 16) == ERR_OVERLAP
    assert call(amax=x + 64) == ERR_OVERLAP
    assert call(amax=w + 4) == ERR_OVERLAP                      # amax inside the workspace
    assert call(ws=x) == ERR_OVERLAP
    assert call(ws=y - 256) == ERR_OVERLAP                      # the workspace runs into y


def test_fake_quant_noalloc_validation():
    """Every check runs before the scratch lookup, so none of these touches HIP."""
    f = nv.lib.nvfp4_fake_quant_noalloc
    G = 1 << 30
    x, y, a = A, A + G, A + 2 * G

    def call(x=x, y=y, rows=4, cols=16, amax=a):
        return f(P(x), P(y), rows, cols, P(amax), None)

    assert call(cols=0) == ERR_SHAPE
    assert call(rows=-1) == ERR_SHAPE
    assert call(rows=1 << 62, cols=1 << 20) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(y=None) == ERR_NULL
    assert call(x=x + 8) == ERR_ALIGN
    assert call(y=y + 2) == ERR_ALIGN
    assert call(amax=a + 2) == ERR_ALIGN
    assert call(y=x + 16) == ERR_OVERLAP
    assert call(amax=x + 64) == ERR_OVERLAP
    assert call(amax=y + 4) == ERR_OVERLAP


def test_mx_validation():
    G = 1 << 30
    x, y, p, sc = A, A + G, A + 2 * G, A + 3 * G
    fq = nv.lib.nvfp4_mx_fake_quant
    assert fq(P(x), P(y), 4, 0, None) == ERR_SHAPE
    assert fq(P(x), P(y), -1, 32, None) == ERR_SHAPE
    assert fq(None, P(y), 4, 32, None) == ERR_NULL
    assert fq(P(x + 8), P(y), 4, 32, None) == ERR_ALIGN
    assert fq(P(x), P(x + 16), 4, 32, None) == ERR_OVERLAP
    qp = nv.lib.nvfp4_mx_quantize_pack
    assert qp(P(x), 4, 32, None, P(sc), None) == ERR_NULL
    assert qp(P(x), 4, 32, P(p + 8), P(sc), None) == ERR_ALIGN       # packed 16-byte aligned
    assert qp(P(x), 4, 32, P(p), P(sc + 2), None) == ERR_ALIGN
    assert qp(P(x), 4, 32, P(x + 64), P(sc), None) == ERR_OVERLAP
    assert qp(P(x), 4, 32, P(p), P(p + 16), None) == ERR_OVERLAP     # scales inside the codes
    dq = nv.lib.nvfp4_mx_dequant_unpack
    assert dq(P(p), None, 4, 32, P(y), None) == ERR_NULL
    assert dq(P(p), P(sc), 4, 32, P(y + 2), None) == ERR_ALIGN
    assert dq(P(p), P(sc), 4, 32, P(p), None) == ERR_OVERLAP
    assert dq(P(p), P(sc), 0, 32, None, None) == OK                  # empty: nothing to do


def test_quantize_pack_ws_validation():
    f = nv.lib.nvfp4_quantize_pack_ws
    G = 1 << 30
    x, pk, sc, gs, a, w = A, A + G, A + 2 * G, A + 3 * G, A + 4 * G, A + 5 * G

    def call(x=x, rows=4, cols=32, amax=a, packed=pk, scales=sc, g=gs, ws=w):
        return f(P(x), rows, cols, P(amax), P(packed), P(scales), P(g), P(ws), None)

    assert call(cols=-3) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(packed=None) == ERR_NULL
    assert call(g=None) == ERR_NULL
    assert call(ws=None) == ERR_NULL
    assert call(packed=pk + 4) == ERR_ALIGN
    assert call(ws=w + 64) == ERR_ALIGN
    assert call(amax=a + 1) == ERR_ALIGN
    assert call(g=gs + 2) == ERR_ALIGN
    assert call(packed=x + 32) == ERR_OVERLAP
    assert call(scales=pk + 8) == ERR_OVERLAP
    assert call(g=w + 8) == ERR_OVERLAP                         # gs inside the workspace
    assert call(amax=gs) == ERR_OVERLAP
    assert call(ws=sc) == ERR_OVERLAP


def test_fake_quant_group_ws_validation():
    g = nv.lib.nvfp4_fake_quant_group_ws
    G = 1 << 30
    x0, x1, y0, y1, a, w = A, A + G, A + 2 * G, A + 3 * G, A + 4 * G, A + 5 * G

    def call(xs, ys, shapes, amax=a, ws=w, n=None):
        n = len(xs) if n is None else n
        k = max(len(xs), 1)
        xp = (ctypes.c_void_p * k)(*xs)
        yp = (ctypes.c_void_p * k)(*ys)
        rs = (ctypes.c_int64 * k)(*[r for r, _ in shapes])
        cs = (ctypes.c_int64 * k)(*[c for _, c in shapes])
        return g(xp, yp, rs, cs, n, P(amax), P(ws), None)

    sh = [(4, 16), (8, 32)]
    assert g(None, None, None, None, 1, None, P(w), None) == ERR_NULL
    assert call([x0, x1], [y0, y1], sh, ws=None) == ERR_NULL
    assert call([x0], [y0], [(4, 16)], n=0) == ERR_ARG
    assert call([A + i * G for i in range(9)], [A + (10 + i) * G for i in range(9)], [(1, 16)] * 9) == ERR_ARG
    assert call([x0, x1], [y0, y1], [(4, 16), (4, 0)]) == ERR_SHAPE
    assert call([x0, None], [y0, y1], sh) == ERR_NULL
    assert call([x0, x1 + 8], [y0, y1], sh) == ERR_ALIGN
    assert call([x0, x1], [y0, y1], sh, ws=w + 128) == ERR_ALIGN
    assert call([x0, x1], [y0, y1], sh, amax=a + 2) == ERR_ALIGN
    assert call([x0, x1], [x1, y1], sh) == ERR_OVERLAP                 # y0 is another member's input
    assert call([x0, x1], [y0, y1], sh, amax=x0 + 4) == ERR_OVERLAP
    assert call([x0, x1], [y0, y1], sh, ws=y1) == ERR_OVERLAP
    assert call([x0, x1], [y0, y1], sh, amax=w + 4) == ERR_OVERLAP    # amax inside the workspace


def test_a_missing_library_fails_loudly(tmp_path):
    # the binding has no fallback: without the built library there is nothing to call
    with pytest.raises(ImportError, match="is not built"):
        nv._load(str(tmp_path / "libnvfp4.so"))


def test_product_code_never_reaches_the_oracle():
    # the package (binding, QAT glue, build script) neither imports nor loads the oracle
    pkg = os.path.join(ROOT, "fp4_block_fake_amd")
    for name in sorted(os.listdir(pkg)):
        if name.endswith(".py"):
            with open(os.path.join(pkg, name)) as f:
                src = f.read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), name
            assert "nvfp4_oracle" not in src, name
    csrc = os.path.join(pkg, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            assert "oracle" not in f.read().lower(), name


def test_oracle_never_reaches_the_product_code():
    # and the other way round: the oracle shares no source, header or import with the library
    odir = os.path.join(ROOT, "oracle")
    for name in sorted(os.listdir(odir)):
        if name.endswith((".py", ".c", ".h")):
            with open(os.path.join(odir, name)) as f:
                src = f.read()
            assert "fp4_block_fake_amd" not in src and "csrc" not in src and "nvfp4.h" not in src, name
