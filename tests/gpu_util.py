"""Helpers shared by the GPU parity tests (imported only by modules that need a GPU)."""
import numpy as np
import torch

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


def sample_rows(rows, seed, k=62):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, k, replace=False)]))
