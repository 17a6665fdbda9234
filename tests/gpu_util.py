"""Helpers shared by the GPU parity tests (imported only by modules that need a GPU)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def say(msg):
    print("[gpu-parity] " + msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def fbits(v):
    return int(np.float32(v).view(np.uint32))


def scalar(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def assert_same(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, "%s: shape %s vs %s" % (what, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, "%s: %d mismatches, first at %d: got %r want %r" % (
        what, bad.size, bad[0], got.reshape(-1)[bad[0]], want.reshape(-1)[bad[0]])


# ---------------------------------------------------------------- the oracle on many host threads
#
# Whole-tensor comparisons at the configurations' full sizes run the unchanged oracle
# calls over row shards on the host's cores (at most 16, the usual host share per GPU): blocks
# never cross rows, so each shard's bytes are the rows of the whole tensor's result,
# and the amax is the maximum of the shards' maxima, which is exact.  The oracle's C
# calls release the GIL.

ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _row_shards(x):
    x = np.ascontiguousarray(x)
    return [s for s in np.array_split(x, min(ORACLE_THREADS, max(1, x.shape[0]))) if s.shape[0]]


def _map(fn, items):
    with ThreadPoolExecutor(ORACLE_THREADS) as pool:
        return list(pool.map(fn, items))


def oracle_amax(x):
    return max(_map(oracle.amax, _row_shards(x)))


def oracle_fake_quant(x, amax_value=None):
    if amax_value is None:
        amax_value = oracle_amax(x)
    return np.concatenate(_map(lambda s: oracle.fake_quant(s, amax_value), _row_shards(x)))


def oracle_quantize(x, amax_value=None):
    """-> (packed, scales, gs), as oracle.quantize."""
    if amax_value is None:
        amax_value = oracle_amax(x)
    parts = _map(lambda s: oracle.quantize(s, amax_value), _row_shards(x))
    return (np.concatenate([p for p, _, _ in parts]), np.concatenate([q for _, q, _ in parts]), parts[0][2])


def oracle_dequantize(packed, scales, gs, cols):
    rows = np.array_split(np.arange(packed.shape[0]), min(ORACLE_THREADS, max(1, packed.shape[0])))
    return np.concatenate(_map(lambda r: oracle.dequantize(packed[r[0]:r[-1] + 1], scales[r[0]:r[-1] + 1], gs, cols),
                               [r for r in rows if r.size]))


def oracle_mx_fake_quant(x):
    return np.concatenate(_map(oracle.mx_fake_quant, _row_shards(x)))


def oracle_mx_quantize(x):
    """-> (packed, scales), as oracle.mx_quantize."""
    parts = _map(oracle.mx_quantize, _row_shards(x))
    return np.concatenate([p for p, _ in parts]), np.concatenate([s for _, s in parts])
