"""How the path shards, checked on the CPU with two gloo ranks (no GPU).

The only coupling in the method is the per-tensor amax (verl QATLinear page, section 5
all-reduces the step amax across ranks; section 4's siblings share one).  So a rank
quantizes its shard of a weight with the all-reduced (MAX) amax and gets exactly the
bytes of the single-tensor result, as long as shards hold whole 16-element blocks of a
row.  The first test checks that protocol with the oracle; the second checks that the
QAT glue's observer all-reduces the step amax, so every rank keeps the same state (the
device calls are replaced by CPU stand-ins there: only the host logic is under test).
"""
import os
import socket

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import torch.distributed as dist  # noqa: E402
import torch.multiprocessing as mp  # noqa: E402


def free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def init(rank, world, port):
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)


def shard_worker(rank, world, port, results):
    import oracle
    import synth
    init(rank, world, port)
    try:
        w = synth.c1_weight()                              # [256, 1024]
        out = {}
        # row shards, column shards (64 columns = 4 whole blocks per row), and column
        # shards that split blocks (24 columns)
        for kind, part in (("rows", np.array_split(w, world, axis=0)[rank]),
                           ("cols", np.hsplit(w, world)[rank]),
                           ("ragged_cols", (w[:, :24] if rank == 0 else w[:, 24:48]))):
            part = np.ascontiguousarray(part)
            local = torch.tensor([oracle.amax(part)], dtype=torch.float32)
            dist.all_reduce(local, op=dist.ReduceOp.MAX)
            out[kind] = (oracle.quantize(part, float(local.item())), float(local.item()))
        results[rank] = out
    finally:
        dist.destroy_process_group()


def test_sharded_quantize_equals_single_tensor():
    import oracle
    import synth
    world = 2
    with mp.Manager() as manager:
        results = manager.dict()
        mp.spawn(shard_worker, args=(world, free_port(), results), nprocs=world, join=True)
        results = dict(results)
    w = synth.c1_weight()
    a = oracle.amax(w)
    p_ref, s_ref, g_ref = oracle.quantize(w, a)
    for rank in range(world):
        (p, s, g), amax = results[rank]["rows"]
        assert amax == a
        rows = np.array_split(np.arange(w.shape[0]), world)[rank]
        assert np.array_equal(p, p_ref[rows]) and np.array_equal(s, s_ref[rows]) and g == g_ref
        (p, s, g), amax = results[rank]["cols"]
        c0 = rank * w.shape[1] // world
        c1 = (rank + 1) * w.shape[1] // world
        assert np.array_equal(p, p_ref[:, c0 // 2:c1 // 2]) and np.array_equal(s, s_ref[:, c0 // 16:c1 // 16])
    # a shard of 24 columns ends in a block padded with zeros (columns 16..23 and 8 zeros),
    # where the whole row has columns 16..31: its first block matches, its second does not
    # (the reason shards must hold whole blocks)
    (p0, s0, _), amax = results[0]["ragged_cols"]
    _, s_whole, _ = oracle.quantize(np.ascontiguousarray(w[:, :48]), amax)
    assert np.array_equal(s0[:, 0], s_whole[:, 0])
    assert not np.array_equal(s0[:, 1], s_whole[:, 1])


def observer_worker(rank, world, port, results):
    init(rank, world, port)
    try:
        from fp4_block_fake_amd import qat
        import oracle

        # CPU stand-ins for the two device calls the observer makes
        def amax_cpu(t, amax=None, accumulate=False):
            return t.abs().max().float().reshape(1)

        def observe_cpu(state, cur, mode, decay=0.01):
            state.fill_(oracle.observer(float(state.item()), float(cur.item()), mode, decay))
            return state

        qat.nvfp4_amax = amax_cpu
        qat.nvfp4_observer_update = observe_cpu
        lin = qat.QATLinear(32, 8, mode="w4a4", activation_observer="minmax", ema_decay=0.25)
        lin.train()
        gen = torch.Generator().manual_seed(100 + rank)
        states = []
        for step in range(3):
            x = (torch.randn(4, 32, generator=gen) * (1 + rank + step)).to(torch.bfloat16)
            states.append(float(lin.observe(x).item()))
        results[rank] = states
    finally:
        dist.destroy_process_group()


def test_qat_observer_all_reduces_the_step_amax():
    import oracle
    world = 2
    pytest.importorskip("fp4_block_fake_amd")
    with mp.Manager() as manager:
        results = manager.dict()
        mp.spawn(observer_worker, args=(world, free_port(), results), nprocs=world, join=True)
        results = dict(results)
    assert results[0] == results[1]                        # every rank holds the same state
    # and that state follows the observer over the global step maxima
    state = -1.0
    for step in range(3):
        maxima = []
        for rank in range(world):
            gen = torch.Generator().manual_seed(100 + rank)
            for s in range(step + 1):
                x = (torch.randn(4, 32, generator=gen) * (1 + rank + s)).to(torch.bfloat16)
            maxima.append(float(x.abs().max()))
        state = oracle.observer(state, max(maxima), oracle.OBS_EMA, float(np.float32(0.25)))
        assert results[0][step] == np.float32(state)
