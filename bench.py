"""Throughput of the NVFP4 path on one MI355X.

One step is the whole path over the large MLP weight (bf16 28672 x 8192, the
largest workload): fused amax + fake-quant, fused amax + quantize-pack, and
dequant-unpack of the packed result.  Inputs are resident in HBM before the
timed region.  The step is issued as the library calls

    nvfp4_amax(x)                    -> a1        \\ = nvfp4_fake_quant(x, amax_in=NULL)
    nvfp4_fake_quant(x, amax_in=a1)  -> y         /
    nvfp4_amax(x)                    -> a2        \\ = nvfp4_quantize_pack(x, amax_in=NULL)
    nvfp4_quantize_pack(x, amax_in=a2)            /
    nvfp4_dequant_unpack(...)        -> y2

which enqueue exactly the kernels of the two fused calls.  Inside the timed
region, HIP events on the launch stream (created without the system-scope fence
of a default event) bracket the fake-quant kernel (the dominant launch) in every
step; a diagnostic pass afterwards records events between all calls for the
per-op times.

Prints one JSON line on stdout (logs go to stderr):
  value         algorithmic GB/s of the whole step (13.125 bytes per element)
  roofline      the dominant kernel's algorithmic GB/s against 8 TB/s HBM
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  ops           per-op times of the diagnostic pass
  secondary     per-call-sequence times on the other workloads (fused siblings,
                the activation step with its observers, the mid-size weight)
                and the packed c5 weight used as a linear layer; --no-secondary
                skips them, --secondary-only NAME runs only the matching ones
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# bytes per element each op must move (read + write), from the method itself
BYTES_PER_ELEM = {
    "amax": 2.0,                 # read x
    "fake_quant": 4.0,           # read x, write y (amax given)
    "quantize_pack": 2.5625,     # read x, write 1/2 byte code + 1/16 byte scale
    "dequant_unpack": 2.5625,    # read codes + scales, write y
}
STEP_BYTES_PER_ELEM = (2 * BYTES_PER_ELEM["amax"] + BYTES_PER_ELEM["fake_quant"]
                       + BYTES_PER_ELEM["quantize_pack"] + BYTES_PER_ELEM["dequant_unpack"])
KERNEL_NAMES = {
    "amax": "k_amax",
    "fake_quant": "k_fake_quant",
    "quantize_pack": "k_quantize_pack",
    "dequant_unpack": "k_dequant_unpack",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PROBE_SOURCE = "stream_probe.hip"     # the benchmark's own stream probes, not a library kernel

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class KernelEvent:
    """A HIP timing event created with hipEventDisableSystemFence, recorded on a stream.

    A default event record also performs a system-scope release, which writes back the
    caches and holds the next kernel until it is done: a pair of torch events around one
    kernel of the step costs the step about 8 us, a pair of these about 4 us.  The
    timestamps are the same kind either way (the fake-quant kernel measured 132.3 us
    between these and 133.7 us between torch's in one process)."""
    _hip = None

    def __init__(self):
        import ctypes
        if KernelEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")       # the HIP runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            KernelEvent._hip = hip
        self._ct = ctypes
        self.e = ctypes.c_void_p()
        if self._hip.hipEventCreateWithFlags(ctypes.byref(self.e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._hip.hipEventRecord(self.e, self._ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        if self._hip.hipEventElapsedTime(self._ct.byref(ms), self.e, end.e) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.e:
            self._hip.hipEventDestroy(self.e)


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash():
    """SHA-256 (first 16 hex digits) over the library's kernel sources, file names included.
    Comments, blank lines and spacing are left out, so that only a change of code changes
    it (no string literal in these sources holds a comment marker)."""
    csrc = os.path.join(ROOT, "fp4_block_fake_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")) and name != PROBE_SOURCE:
            h.update(name.encode())
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                text = _COMMENT.sub(" ", f.read())
            code = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
            h.update(code.encode())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """Bytes per launch that crossed the L2's memory-side interface (rocprofv3 FETCH_SIZE +
    WRITE_SIZE, scaled by a copy of known size), if taken on the current source.  These
    requests go on to the Infinity Cache, so its hits count too: an upper bound on HBM
    bytes, not a DRAM-only figure (no per-kernel counter on gfx950 separates the two)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["bytes_past_l2_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(x, rows):
    import numpy as np

    import oracle
    sample = np.ascontiguousarray(x[:rows])
    n = sample.size
    t0 = time.perf_counter()
    a = oracle.amax(sample)
    oracle.fake_quant(sample, a)
    a = oracle.amax(sample)
    packed, scales, gs = oracle.quantize(sample, a)
    oracle.dequantize(packed, scales, gs, sample.shape[1])
    dt = time.perf_counter() - t0
    return {
        "value": round(STEP_BYTES_PER_ELEM * n / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "first %d of %d rows (%d elements), one step: amax+fake-quant, "
                  "amax+quantize-pack, dequant-unpack; %.1f s single-threaded" % (rows, x.shape[0], n, dt),
        "elements_per_s": round(n / dt, 1),
        "host": host_info(),
    }


def cpu_baseline_threads(x, rows, threads):
    """The same oracle step over row shards on `threads` host threads (the oracle's C
    calls release the GIL): the amax of the shards, reduced, then each shard quantized
    with it.  Rows are independent, so the bytes equal the single-threaded run's."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    sample = np.ascontiguousarray(x[:rows])
    n = sample.size
    shards = [s for s in np.array_split(sample, threads) if s.size]
    cols = sample.shape[1]
    with ThreadPoolExecutor(threads) as pool:
        t0 = time.perf_counter()
        a = max(pool.map(oracle.amax, shards))
        list(pool.map(lambda s: oracle.fake_quant(s, a), shards))
        a = max(pool.map(oracle.amax, shards))
        packs = list(pool.map(lambda s: oracle.quantize(s, a), shards))
        list(pool.map(lambda p: oracle.dequantize(p[0], p[1], p[2], cols), packs))
        dt = time.perf_counter() - t0
    return {
        "value": round(STEP_BYTES_PER_ELEM * n / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "first %d of %d rows (%d elements) in %d row shards, one step; %.2f s" % (
            rows, x.shape[0], n, len(shards), dt),
        "elements_per_s": round(n / dt, 1),
        "host": host_info(),
    }


def cold_times(torch, stream, flush, fn, reps):
    """GPU times of single calls of fn, each started with no data of its own in the caches:
    a 1 GiB read (outside the events) evicts the Infinity Cache and the L2s first.  The
    events and the calls are enqueued behind the flush without waiting for it, so the
    host's submission of fn overlaps the flush and is not counted as GPU time."""
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush.sum()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return sorted(ts)


def median(ts):
    return ts[len(ts) // 2]


def secondary(nv, synth, np, torch, dev, reps=20, only=None):
    """Per-call throughput on the other workloads (not part of the headline step).

    only: run just the lines whose name contains this string (and set up just their
    workloads), for profiling one workload's calls."""
    stream = torch.cuda.current_stream(dev)
    out = {}

    def timed(fn, nbytes, elems=None):
        # warm up for at least 10 ms of calls, so each line is timed after the clock
        # transient that a change of load starts
        t_end = time.perf_counter() + 0.010
        calls = 0
        while calls < 3 or time.perf_counter() < t_end:
            fn()
            calls += 1
            if calls % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        r = {"us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
             "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
        if elems:
            r["elements_per_s"] = round(elems / (us * 1e-6), 1)
        return r

    # float32, so that sum() is one read-only reduction over 1 GiB (an int32 tensor would
    # first be widened to int64, a 2 GB write stream that then overlaps the timed call)
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)

    def cold_us(fn, reps=9):
        """Median GPU time of single calls, each after a 1 GiB read has evicted the
        Infinity Cache and the L2s."""
        return round(median(cold_times(torch, stream, flush, fn, reps)), 2)

    def line(name, fn, nbytes, cold=False, elems=None):
        if only is None or only in name:
            out[name] = timed(fn, nbytes, elems)
            if cold:
                c = cold_us(fn)
                out[name]["cold_us"] = c
                out[name]["cold_pct_of_hbm_peak"] = round(100 * nbytes / (c * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)
                if elems:
                    out[name]["cold_elements_per_s"] = round(elems / (c * 1e-6), 1)

    def group(prefix):
        return only is None or only.startswith(prefix) or prefix.startswith(only)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    ws = nv.new_workspace(dev)

    if group("c1_"):
        # c1: one small weight, fused amax + fake-quant (launch-bound: no bandwidth target)
        x = to_dev(synth.c1_weight())
        n1 = x.numel()
        y = torch.empty_like(x)
        a = torch.empty(1, dtype=torch.float32, device=dev)
        line("c1_fused_amax_fake_quant_256x1024", lambda: nv.nvfp4_fake_quant(x, y=y, amax_out=a), 6.0 * n1,
             cold=True, elems=n1)
        line("c1_fused_amax_fake_quant_ws", lambda: nv.nvfp4_fake_quant_ws(x, y=y, amax_out=a, workspace=ws),
             6.0 * n1, cold=True, elems=n1)
        line("c1_fused_amax_fake_quant_noalloc", lambda: nv.nvfp4_fake_quant_noalloc(x, y=y, amax_out=a),
             6.0 * n1, cold=True, elems=n1)
        del x, y

    if group("c2_"):
        # c2: 4096 x 4096 with outliers and exact ties; a power-of-two global scale, so
        # 14 of the 126 scale bytes take the integer-threshold code path
        x = to_dev(synth.c2_weight())
        n2 = x.numel()
        y = torch.empty_like(x)
        a = torch.empty(1, dtype=torch.float32, device=dev)
        p2 = torch.empty((x.shape[0], x.shape[1] // 2), dtype=torch.uint8, device=dev)
        s2 = torch.empty((x.shape[0], x.shape[1] // 16), dtype=torch.uint8, device=dev)
        g2 = torch.empty(1, dtype=torch.float32, device=dev)
        line("c2_fused_amax_fake_quant_4096x4096", lambda: nv.nvfp4_fake_quant(x, y=y, amax_out=a), 6.0 * n2,
             cold=True, elems=n2)
        line("c2_fused_amax_fake_quant_ws", lambda: nv.nvfp4_fake_quant_ws(x, y=y, amax_out=a, workspace=ws),
             6.0 * n2, cold=True, elems=n2)
        line("c2_fused_amax_quantize_pack",
             lambda: nv.nvfp4_quantize_pack(x, amax_out=a, packed=p2, scales=s2, global_scale=g2), 4.5625 * n2,
             cold=True, elems=n2)
        line("c2_fused_amax_quantize_pack_ws",
             lambda: nv.nvfp4_quantize_pack_ws(x, amax_out=a, packed=p2, scales=s2, global_scale=g2,
                                               workspace=ws), 4.5625 * n2, cold=True, elems=n2)
        line("c2_dequant_unpack", lambda: nv.nvfp4_dequant_unpack(p2, s2, g2, y=y), 2.5625 * n2, cold=True,
             elems=n2)
        del x, y, p2, s2

    if group("ragged_"):
        # rows whose length is not a multiple of 16 (zero-padded last block of each row):
        # the half-block kernels, with dword accesses for even lengths and element-wise
        # ones for odd lengths
        for cols in (4100, 4097):
            xr = to_dev(synth.normal_bf16(9, (4096, cols), 0.02))
            nr = xr.numel()
            yr = torch.empty_like(xr)
            nbr = (cols + 15) // 16
            pr = torch.empty((xr.shape[0], 8 * nbr), dtype=torch.uint8, device=dev)
            sr = torch.empty((xr.shape[0], nbr), dtype=torch.uint8, device=dev)
            gr = torch.empty(1, dtype=torch.float32, device=dev)
            ar = torch.empty(1, dtype=torch.float32, device=dev)
            tag = "ragged_4096x%d" % cols
            line(tag + "_fused_amax_fake_quant_ws",
                 lambda: nv.nvfp4_fake_quant_ws(xr, y=yr, amax_out=ar, workspace=ws), 6.0 * nr, cold=True,
                 elems=nr)
            line(tag + "_fused_amax_quantize_pack_ws",
                 lambda: nv.nvfp4_quantize_pack_ws(xr, amax_out=ar, packed=pr, scales=sr, global_scale=gr,
                                                   workspace=ws), 4.5625 * nr, cold=True, elems=nr)
            line(tag + "_dequant_unpack", lambda: nv.nvfp4_dequant_unpack(pr, sr, gr, y=yr, cols=cols),
                 2.5625 * nr, cold=True, elems=nr)
            del xr, yr, pr, sr

    if group("c3_"):
        # c3: shared amax of fused QKV siblings in one launch, then a fake-quant of each
        sibs = [to_dev(a) for a in synth.c3_siblings()]
        ys = [torch.empty_like(t) for t in sibs]
        shared = torch.empty(1, dtype=torch.float32, device=dev)
        n3 = sum(t.numel() for t in sibs)

        def c3():
            nv.nvfp4_amax(sibs, amax=shared)
            for t, y in zip(sibs, ys):
                nv.nvfp4_fake_quant(t, y=y, amax_in=shared)
        line("c3_qkv_shared_amax_fake_quant", c3, 6.0 * n3, cold=True, elems=n3)
        line("c3_qkv_group_fake_quant_one_launch",
             lambda: nv.nvfp4_fake_quant_group(sibs, ys=ys, amax_out=shared), 6.0 * n3, cold=True, elems=n3)
        line("c3_qkv_group_fake_quant_ws",
             lambda: nv.nvfp4_fake_quant_group_ws(sibs, ys=ys, amax_out=shared, workspace=ws), 6.0 * n3,
             cold=True, elems=n3)
        del sibs, ys

    if group("c4_activation"):
        # c4 activation step: amax, both observers, a fake-quant with each observer's amax
        x = to_dev(synth.c4_activation(0))
        n4 = x.numel()
        y1, y2 = torch.empty_like(x), torch.empty_like(x)
        cur = torch.empty(1, dtype=torch.float32, device=dev)
        st_s = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
        st_e = torch.full((1,), -1.0, dtype=torch.float32, device=dev)

        def c4act():
            nv.nvfp4_amax(x, amax=cur)
            nv.nvfp4_observer_update(st_s, cur, nv.OBS_STATIC_MINMAX)
            nv.nvfp4_observer_update(st_e, cur, nv.OBS_EMA, 0.01)
            nv.nvfp4_fake_quant(x, y=y1, amax_in=st_s)
            nv.nvfp4_fake_quant(x, y=y2, amax_in=st_e)
        line("c4_activation_step_8192x4096", c4act, 10.0 * n4, cold=True, elems=n4)

        def c4act_dual():
            nv.nvfp4_amax(x, amax=cur)
            nv.nvfp4_observer_update(st_s, cur, nv.OBS_STATIC_MINMAX)
            nv.nvfp4_observer_update(st_e, cur, nv.OBS_EMA, 0.01)
            nv.nvfp4_fake_quant_dual(x, st_s, st_e, y0=y1, y1=y2)
        # same outputs from one read of x: 8 bytes per element of traffic instead of 10
        line("c4_activation_step_dual_fake_quant", c4act_dual, 8.0 * n4, cold=True, elems=n4)
        # the same step as one call: 3 launches (amax to partial maxima, their reduction
        # with both observer steps, dual fake-quant) instead of 5
        line("c4_activation_step_observe_fake_quant",
             lambda: nv.nvfp4_observe_fake_quant(x, st_s, nv.OBS_STATIC_MINMAX, 0.0, st_e, nv.OBS_EMA, 0.01,
                                                 y0=y1, y1=y2, cur=cur, workspace=ws), 8.0 * n4,
             cold=True, elems=n4)
        line("c4_activation_cached_fake_quant", lambda: nv.nvfp4_fake_quant(x, y=y1, amax_in=st_s), 4.0 * n4,
             cold=True, elems=n4)
        line("c4_activation_fused_amax_fake_quant", lambda: nv.nvfp4_fake_quant(x, y=y1, amax_out=cur), 6.0 * n4,
             cold=True, elems=n4)
        pa = torch.empty((x.shape[0], x.shape[1] // 2), dtype=torch.uint8, device=dev)
        sa = torch.empty((x.shape[0], x.shape[1] // 16), dtype=torch.uint8, device=dev)
        ga = torch.empty(1, dtype=torch.float32, device=dev)
        line("c4_activation_fused_amax_quantize_pack",
             lambda: nv.nvfp4_quantize_pack(x, amax_out=cur, packed=pa, scales=sa, global_scale=ga), 4.5625 * n4,
             cold=True, elems=n4)
        # the fused calls through a workspace: no clearing launch, no atomics
        line("c4_activation_fused_amax_fake_quant_ws",
             lambda: nv.nvfp4_fake_quant_ws(x, y=y1, amax_out=cur, workspace=ws), 6.0 * n4, cold=True, elems=n4)
        line("c4_activation_fused_amax_quantize_pack_ws",
             lambda: nv.nvfp4_quantize_pack_ws(x, amax_out=cur, packed=pa, scales=sa, global_scale=ga,
                                               workspace=ws), 4.5625 * n4, cold=True, elems=n4)
        del pa, sa, x, y1, y2

    if group("c4_weight"):
        w = to_dev(synth.c4_weight())
        nw = w.numel()
        yw = torch.empty_like(w)
        aw = torch.empty(1, dtype=torch.float32, device=dev)
        pk = torch.empty((w.shape[0], w.shape[1] // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((w.shape[0], w.shape[1] // 16), dtype=torch.uint8, device=dev)
        gsw = torch.empty(1, dtype=torch.float32, device=dev)
        line("c4_weight_fused_amax_fake_quant_14336x4096",
             lambda: nv.nvfp4_fake_quant(w, y=yw, amax_out=aw), 6.0 * nw, cold=True, elems=nw)
        line("c4_weight_fused_amax_quantize_pack_14336x4096",
             lambda: nv.nvfp4_quantize_pack(w, amax_out=aw, packed=pk, scales=sc, global_scale=gsw), 4.5625 * nw,
             cold=True, elems=nw)
        line("c4_weight_fused_amax_fake_quant_ws",
             lambda: nv.nvfp4_fake_quant_ws(w, y=yw, amax_out=aw, workspace=ws), 6.0 * nw, cold=True, elems=nw)
        line("c4_weight_fused_amax_quantize_pack_ws",
             lambda: nv.nvfp4_quantize_pack_ws(w, amax_out=aw, packed=pk, scales=sc, global_scale=gsw,
                                               workspace=ws), 4.5625 * nw, cold=True, elems=nw)
        del w, yw, pk, sc

    if group("mx_"):
        # the MXFP4 variant (32-element blocks, binary32 block scales, no amax pass): one
        # launch per call; bytes per element 2 + 2 (fake-quant), 2 + 0.5 + 4 / 32 (pack)
        for tag, arr in (("c4_weight_14336x4096", synth.c4_weight()), ("c5_weight_28672x8192", synth.c5_weight())):
            xm = to_dev(arr)
            del arr
            nm = xm.numel()
            ym = torch.empty_like(xm)
            pm = torch.empty((xm.shape[0], xm.shape[1] // 2), dtype=torch.uint8, device=dev)
            sm = torch.empty((xm.shape[0], xm.shape[1] // 32), dtype=torch.float32, device=dev)
            line("mx_%s_fake_quant" % tag, lambda: nv.nvfp4_mx_fake_quant(xm, y=ym), 4.0 * nm, cold=True, elems=nm)
            line("mx_%s_quantize_pack" % tag, lambda: nv.nvfp4_mx_quantize_pack(xm, packed=pm, scales=sm),
                 2.625 * nm, cold=True, elems=nm)
            line("mx_%s_dequant_unpack" % tag, lambda: nv.nvfp4_mx_dequant_unpack(pm, sm, y=ym), 2.625 * nm,
                 cold=True, elems=nm)
            del xm, ym, pm, sm
        # ragged rows (4100 = 128 blocks of 32 and 4 elements): the quarter-block row kernels
        xm = to_dev(synth.normal_bf16(9, (4096, 4100), 0.02))
        nm = xm.numel()
        ym = torch.empty_like(xm)
        pm, sm = nv.nvfp4_mx_quantize_pack(xm)
        line("mx_ragged_4096x4100_fake_quant", lambda: nv.nvfp4_mx_fake_quant(xm, y=ym), 4.0 * nm, cold=True,
             elems=nm)
        line("mx_ragged_4096x4100_quantize_pack", lambda: nv.nvfp4_mx_quantize_pack(xm, packed=pm, scales=sm),
             2.625 * nm, cold=True, elems=nm)
        line("mx_ragged_4096x4100_dequant_unpack",
             lambda: nv.nvfp4_mx_dequant_unpack(pm, sm, y=ym, cols=4100), 2.625 * nm, cold=True, elems=nm)
        del xm, ym, pm, sm

    if group("c5_"):
        wc = to_dev(synth.c5_weight())
        n, k = wc.shape
        # one rank's shard of the c5 weight under 8-way row sharding: with the all-reduced
        # amax given, the shard runs the cached-amax calls (the exchange itself is one fp32)
        sh = wc[: n // 8]
        amax_all = nv.nvfp4_amax(wc)
        ysh = torch.empty_like(sh)
        psh = torch.empty((sh.shape[0], k // 2), dtype=torch.uint8, device=dev)
        ssh = torch.empty((sh.shape[0], k // 16), dtype=torch.uint8, device=dev)
        gsh = torch.empty(1, dtype=torch.float32, device=dev)
        ns = sh.numel()
        line("c5_row_shard_3584x8192_cached_fake_quant",
             lambda: nv.nvfp4_fake_quant(sh, y=ysh, amax_in=amax_all), 4.0 * ns, cold=True, elems=ns)
        line("c5_row_shard_3584x8192_cached_quantize_pack",
             lambda: nv.nvfp4_quantize_pack(sh, amax_in=amax_all, packed=psh, scales=ssh, global_scale=gsh),
             2.5625 * ns, cold=True, elems=ns)
        line("c5_row_shard_3584x8192_dequant_unpack",
             lambda: nv.nvfp4_dequant_unpack(psh, ssh, gsh, y=ysh), 2.5625 * ns, cold=True, elems=ns)
        del sh, ysh, psh, ssh
        # the fused calls on the c5 weight through the workspace (the step uses the
        # three-launch form, whose quantizing kernel the roofline times alone)
        yc = torch.empty_like(wc)
        pc = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        scc = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        ac, gc = torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev)
        line("c5_weight_fused_amax_fake_quant_ws",
             lambda: nv.nvfp4_fake_quant_ws(wc, y=yc, amax_out=ac, workspace=ws), 6.0 * wc.numel(), cold=True,
             elems=wc.numel())
        line("c5_weight_fused_amax_quantize_pack_ws",
             lambda: nv.nvfp4_quantize_pack_ws(wc, amax_out=ac, packed=pc, scales=scc, global_scale=gc,
                                               workspace=ws), 4.5625 * wc.numel(), cold=True, elems=wc.numel())
        del yc, pc, scc
        # the c5 weight used as a linear layer (packed once), against unpack + torch's bf16
        # GEMM and torch's bf16 GEMM on an already unpacked weight (context only).  Calls
        # on one weight find its 132 MB of codes and scales in the 256 MB Infinity Cache;
        # the "rotated" figures cycle through three copies of it (396 MB), so every call
        # reads its weight from HBM, as the layers of a model forward do.
        if only is None or only in "c5_weight_linear":
            packed, scales, gsc = nv.nvfp4_quantize_pack(wc)
            wdq = nv.nvfp4_dequant_unpack(packed, scales, gsc)
            del wc
            copies = [(packed, scales), (packed.clone(), scales.clone()), (packed.clone(), scales.clone())]
            turn = [0]

            def rotated(f):
                def call():
                    p_, s_ = copies[turn[0] % 3]
                    turn[0] += 1
                    f(p_, s_)
                return call
            gen = torch.Generator(device="cpu").manual_seed(7)
            for m in (1, 16, 64, 128, 256, 512, 1024, 2048):
                xm = torch.randn(m, k, generator=gen).to(torch.bfloat16).to(dev)
                ym = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
                res = timed(lambda: nv.nvfp4_linear(xm, packed, scales, gsc, y=ym),
                            n * k * 0.5625 + 2.0 * m * (k + n))
                res["unpack_plus_torch_gemm_us"] = timed(
                    lambda: torch.nn.functional.linear(xm, nv.nvfp4_dequant_unpack(packed, scales, gsc, y=wdq)),
                    1.0)["us"]
                res["torch_bf16_gemm_us"] = timed(lambda: torch.nn.functional.linear(xm, wdq), 1.0)["us"]
                if m <= 64:
                    res["rotated_us"] = timed(rotated(lambda p_, s_: nv.nvfp4_linear(xm, p_, s_, gsc, y=ym)),
                                              1.0)["us"]
                    res["rotated_pct_of_hbm_peak"] = round(
                        100 * (n * k * 0.5625 + 2.0 * m * (k + n)) / (res["rotated_us"] * 1e3) / HBM_PEAK_GBS, 1)
                    res["unpack_plus_torch_gemm_rotated_us"] = timed(rotated(
                        lambda p_, s_: torch.nn.functional.linear(xm, nv.nvfp4_dequant_unpack(p_, s_, gsc, y=wdq))),
                        1.0)["us"]
                out["c5_weight_linear_%dx8192_by_28672x8192" % m] = res
            del copies
    return out


def stream_ceilings(torch, stream, flush, x, y, n):
    """Read-only, write-only and copy streams over the c5 tensor (2n bytes each way) by
    the probe kernels of libnvfp4_probe.so: the best of a few launch shapes, warm (a loop)
    and cold (median of single runs after the flush)."""
    import ctypes
    path = os.path.join(ROOT, "fp4_block_fake_amd", "libnvfp4_probe.so")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.nvfp4_probe_read.argtypes = [P, I64, P, I, P]
    lib.nvfp4_probe_write.argtypes = [P, I64, I, P]
    lib.nvfp4_probe_copy.argtypes = [P, P, I64, I, P]
    sink = torch.zeros(256, dtype=torch.int32, device=x.device)
    sp = P(stream.cuda_stream)
    nbytes = 2 * n
    kinds = {
        "read": (lambda w: lib.nvfp4_probe_read(P(x.data_ptr()), nbytes, P(sink.data_ptr()), w, sp), nbytes),
        "write": (lambda w: lib.nvfp4_probe_write(P(y.data_ptr()), nbytes, w, sp), nbytes),
        "copy": (lambda w: lib.nvfp4_probe_copy(P(x.data_ptr()), P(y.data_ptr()), nbytes, w, sp), 2 * nbytes),
    }
    out = {}
    for kind, (call, moved) in kinds.items():
        best = None
        for w in (2, 8, 32, 64):
            for _ in range(20):
                assert call(w) == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                call(w)
            e1.record(stream)
            torch.cuda.synchronize()
            warm = e0.elapsed_time(e1) / 20 * 1e3
            cold = median(cold_times(torch, stream, flush, lambda: call(w), 5))
            if best is None or cold < best[2]:
                best = (w, warm, cold)
        w, warm, cold = best
        out[kind] = {"wg_per_cu": w, "warm_us": round(warm, 2), "cold_us": round(cold, 2),
                     "warm_gbs": round(moved / (warm * 1e-6) / 1e9, 1),
                     "cold_gbs": round(moved / (cold * 1e-6) / 1e9, 1)}
    return out


def host_info():
    """The host's CPUs as the CPU-baseline figures ran on them."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


class OracleRunner:
    """The oracle's calls on `threads` host threads over row shards (1: the plain calls).
    Rows are independent and the amax of shards reduces exactly, so the bytes do not depend
    on the thread count; the oracle's C calls release the GIL."""

    def __init__(self, threads):
        from concurrent.futures import ThreadPoolExecutor

        import numpy as np

        import oracle
        self.o, self.np, self.threads = oracle, np, threads
        self.pool = ThreadPoolExecutor(threads) if threads > 1 else None

    def _map(self, fn, items):
        return list(self.pool.map(fn, items)) if self.pool else [fn(i) for i in items]

    def _shards(self, x):
        if not self.pool:
            return [x]
        return [s for s in self.np.array_split(x, self.threads) if s.shape[0]]

    def amax(self, *xs):
        if not self.pool:
            return self.o.amax_group(list(xs)) if len(xs) > 1 else self.o.amax(xs[0])
        return max(max(self._map(self.o.amax, self._shards(x))) for x in xs)

    def fake_quant(self, x, a):
        self._map(lambda s: self.o.fake_quant(s, a), self._shards(x))

    def quantize(self, x, a):
        return self._map(lambda s: self.o.quantize(s, a), self._shards(x))

    def dequantize(self, parts, cols):
        self._map(lambda p: self.o.dequantize(p[0], p[1], p[2], cols), parts)


def cpu_table(synth):
    """The oracle timed per configuration on the host: each configuration's op sequence
    (the calls a step of that workload makes), on 1 thread and on all usable host threads (at most 16),
    median of 3 runs for c4 and c5 and of 10 for the others; generation is not timed."""
    import numpy as np

    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    acts = [synth.c4_activation(t) for t in range(10)]
    w4 = synth.c4_weight()

    def c1(r, x=synth.c1_weight()):
        r.fake_quant(x, r.amax(x))

    def c2(r, x=synth.c2_weight()):
        r.fake_quant(x, r.amax(x))
        r.dequantize(r.quantize(x, r.amax(x)), x.shape[1])

    def c3(r, sibs=synth.c3_siblings()):
        a = r.amax(*sibs)
        for t in sibs:
            r.fake_quant(t, a)

    def c4(r):
        st = em = -1.0
        for x in acts:
            a = r.amax(x)
            st = oracle.observer(st, a, oracle.OBS_STATIC_MINMAX)
            em = oracle.observer(em, a, oracle.OBS_EMA, float(np.float32(0.01)))
            r.fake_quant(x, st)
            r.fake_quant(x, em)
        r.fake_quant(w4, r.amax(w4))

    x5 = synth.c5_weight()

    def c5(r):
        r.dequantize(r.quantize(x5, r.amax(x5)), x5.shape[1])
        r.fake_quant(x5, r.amax(x5))

    n1, n2, n3 = 256 * 1024, 4096 * 4096, sum(t.size for t in synth.c3_siblings())
    n4a, n4w, n5 = acts[0].size, w4.size, x5.size
    configs = {   # name: (run, elements, algorithmic bytes, repetitions)
        "c1": (c1, n1, 6.0 * n1, 10),
        "c2": (c2, n2, STEP_BYTES_PER_ELEM * n2, 10),
        "c3": (c3, n3, 6.0 * n3, 10),
        "c4": (c4, 10 * n4a + n4w, 10 * 10.0 * n4a + 6.0 * n4w, 3),
        "c5": (c5, n5, STEP_BYTES_PER_ELEM * n5, 3),
    }
    out = {"host": host_info(), "threads": threads}
    for name, (run, elems, nbytes, reps) in configs.items():
        row = {"elements": elems, "bytes": nbytes, "reps": reps}
        for t in (1, threads):
            r = OracleRunner(t)
            ts = []
            for k in range(reps):
                t0 = time.perf_counter()
                run(r)
                ts.append(time.perf_counter() - t0)
                log("cpu table %s, %d thread(s), run %d: %.3f s" % (name, t, k, ts[-1]))
            ts.sort()
            med = ts[len(ts) // 2]
            row["threads_%d" % t] = {"median_s": round(med, 4), "gbs": round(nbytes / med / 1e9, 4),
                                     "elements_per_s": round(elems / med, 1)}
            log("cpu table %s, %d thread(s): median %.3f s" % (name, t, med))
        out[name] = row
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 50 untimed steps (~25 ms): under a new sustained load the GPU's clock manager
    # lowers and then settles the engine clock over the first ~10 ms, and a 5-step
    # warm-up left part of that transient inside the timed steps (+2.4% per step)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--rows", type=int, default=28672)
    ap.add_argument("--cols", type=int, default=8192)
    ap.add_argument("--cpu-rows", type=int, default=28672,
                    help="rows of the oracle's CPU sample (default: the whole c5 weight, ~13 s; 0: skip)")
    ap.add_argument("--no-secondary", action="store_true", help="skip the c3/c4 per-call lines")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the CPU oracle per configuration (1 thread and all host threads; no GPU) "
                         "and print that JSON instead of the bench line")
    ap.add_argument("--secondary-only", metavar="NAME", default=None,
                    help="diagnostic mode: skip the step and run only the secondary lines whose name "
                         "contains NAME (prints their JSON, not the bench line); for profiling")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only; the library has no multi-GPU path. Sharded "
              "tensors would need one 4-byte max all-reduce of the amax per tensor.", file=sys.stderr)
        sys.exit(2)

    if args.cpu_table:
        import synth
        print(json.dumps({"cpu_table": cpu_table(synth)}), flush=True)
        return

    import numpy as np
    import torch

    import fp4_block_fake_amd as nv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.secondary_only is not None:
        print(json.dumps({"secondary": secondary(nv, synth, np, torch, dev, only=args.secondary_only)}),
              flush=True)
        return
    log("generating c5 weight %dx%d" % (args.rows, args.cols))
    x_host = synth.c5_weight(rows=args.rows, cols=args.cols)
    rows, cols = x_host.shape
    n = rows * cols
    x = torch.from_numpy(x_host.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty_like(x)
    y2 = torch.empty_like(x)
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    gs = torch.empty(1, dtype=torch.float32, device=dev)
    a1 = torch.empty(1, dtype=torch.float32, device=dev)
    a2 = torch.empty(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    ops = ["amax", "fake_quant", "amax", "quantize_pack", "dequant_unpack"]

    def step(events=None, fq_events=None):
        calls = [
            lambda: nv.nvfp4_amax(x, amax=a1),
            lambda: nv.nvfp4_fake_quant(x, y=y, amax_in=a1),
            lambda: nv.nvfp4_amax(x, amax=a2),
            lambda: nv.nvfp4_quantize_pack(x, amax_in=a2, packed=packed, scales=scales, global_scale=gs),
            lambda: nv.nvfp4_dequant_unpack(packed, scales, gs, y=y2),
        ]
        for i, c in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            if fq_events is not None and i == 1:
                fq_events[0].record(stream)
            c()
            if fq_events is not None and i == 1:
                fq_events[1].record(stream)
        if events is not None:
            events[len(calls)].record(stream)

    # The box's stream ceilings come first, from probe kernels with the kernels' access
    # pattern and none of their arithmetic (best launch shape of a few; median of cold
    # runs).  Under a new sustained load the engine clock dips for roughly the first
    # 10 ms; measured first, the probes take that transient, and the timed steps (after
    # the W warm-up steps) run at the steady clock however small W is.
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)     # sum(): a pure read
    log("stream ceilings")
    streams = stream_ceilings(torch, stream, flush, x, y, n)

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps.  The only events inside it bracket the
    # fake-quant kernel (the dominant launch) in every step, for the roofline
    # figure; they are fence-free HIP events, which perturb the step least.
    fq_ev = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(fq_events=fq_ev[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    fq_ms = sum(a.elapsed_time(b) for a, b in fq_ev) / args.steps

    # Diagnostic pass (not timed as a step): events between every call.
    diag = max(5, args.steps // 5)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(diag)]
    for k in range(diag):
        step(events=ev[k])
    torch.cuda.synchronize()
    per_op_ms = {}
    for i, name in enumerate(ops):
        key = name if name not in per_op_ms else name + "_2"
        per_op_ms[key] = sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(diag)) / diag
    per_op_ms["fake_quant"] = fq_ms
    op_report = {}
    for key, ms in per_op_ms.items():
        base = key.replace("_2", "")
        op_report[key] = {"us": round(ms * 1e3, 2),
                          "gbs": round(BYTES_PER_ELEM[base] * n / (ms * 1e-3) / 1e9, 1)}
    fused_fq_ms = per_op_ms["amax"] + per_op_ms["fake_quant"]
    fused_qp_ms = per_op_ms["amax_2"] + per_op_ms["quantize_pack"]
    op_report["fused_amax_fake_quant"] = {"us": round(fused_fq_ms * 1e3, 2),
                                          "gbs": round(6.0 * n / (fused_fq_ms * 1e-3) / 1e9, 1)}
    op_report["fused_amax_quantize_pack"] = {"us": round(fused_qp_ms * 1e3, 2),
                                             "gbs": round(4.5625 * n / (fused_qp_ms * 1e-3) / 1e9, 1)}

    # roofline of the dominant kernel, timed live in the timed region
    dom = "fake_quant"
    dom_bytes = BYTES_PER_ELEM[dom] * n
    achieved = dom_bytes / (fq_ms * 1e-3) / 1e9
    traffic = read_traffic(KERNEL_NAMES[dom], "c5")

    # Cold figures: before each run, 1 GiB is read to evict the Infinity Cache (256 MB)
    # and the L2s (a read leaves clean lines, so no write-back overlaps what follows);
    # the events and calls queue behind it, so host submission is not timed.
    cold_runs = max(5, args.steps // 10)
    cold_med = median(cold_times(torch, stream, flush, step, cold_runs)) * 1e-3
    # the dominant kernel alone, cold: k_fake_quant with the amax given reads all of x
    # from HBM (none of it in the Infinity Cache) and writes y
    hbm_only_us = median(cold_times(torch, stream, flush, lambda: nv.nvfp4_fake_quant(x, y=y, amax_in=a1), 9))
    del flush

    value = STEP_BYTES_PER_ELEM * n / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": "NVFP4 fake-quant / quantize-pack GB/s and % of HBM peak on 1 MI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.015) with 0.01% Laplace x30 outliers)",
        "config": {
            "workload": "c5: bf16 MLP weight %dx%d, one step = amax+fake-quant, amax+quantize-pack, "
                        "dequant-unpack" % (rows, cols),
            "rows": rows, "cols": cols, "block": 16, "io": "bf16 in/out, uint8 nibbles + E4M3 scales",
            "bytes_per_element_step": STEP_BYTES_PER_ELEM,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "elements_per_s": round(n / (ms_per_step * 1e-3), 1),
        "ops": op_report,
        "stream_ceilings": streams,
        "cold_step": {"ms": round(cold_med, 4),
                      "gbs": round(STEP_BYTES_PER_ELEM * n / (cold_med * 1e-3) / 1e9, 1),
                      "runs": cold_runs,
                      "note": "median step after reading 1 GiB (caches evicted); value is the warm rate"},
        "roofline": {
            "kernel": KERNEL_NAMES[dom],
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_note": "FETCH_SIZE + WRITE_SIZE: bytes past the L2, Infinity-Cache hits included",
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": round(fq_ms * 1e3, 2),
            "note": "in the step the amax pass before it leaves the last 192 MB of x in the "
                    "Infinity Cache; hbm_only is the same kernel alone with nothing cached",
            "hbm_only": {"us": round(hbm_only_us, 2),
                         "achieved": round(dom_bytes / (hbm_only_us * 1e-6) / 1e9, 1),
                         "frac": round(dom_bytes / (hbm_only_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "frac_of_copy_stream": round(dom_bytes / (hbm_only_us * 1e-6) / 1e9
                                                      / streams["copy"]["cold_gbs"], 4)},
        },
        "cpu_baseline": None,
    }
    if not args.no_secondary:
        log("secondary workloads")
        result["secondary"] = secondary(nv, synth, np, torch, dev)
    if args.cpu_rows > 0:
        log("cpu baseline: oracle on %d rows" % args.cpu_rows)
        result["cpu_baseline"] = cpu_baseline(x_host, min(args.cpu_rows, rows))
        # the same oracle on the host's cores (at most 16: the machine's CPU share per GPU)
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        result["cpu_baseline_threads"] = cpu_baseline_threads(x_host, min(args.cpu_rows, rows), threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
