"""Draft-row KV append (the step before verify in the extend layout): the
NumPy definition in oracle/ pinned on the CPU, the HIP kernel checked against
it bit for bit on the GPU, and append + verify captured in one HIP graph."""
import numpy as np
import pytest

import oracle
from synthetic import inputs

from helpers import parity_gate


def small_workload(seed=11):
    return inputs.make_workload("append_small", B=3, H=2, T=5, prefixes=[7, 0, 33],
                                pool_slots=200, seed=seed)


def node_slots(wl):
    """Slots of the tree nodes, [B, T]: the last T entries of each segment."""
    out = np.empty((wl.B, wl.T), dtype=np.int64)
    seg = 0
    for b in range(wl.B):
        n = int(wl.seq_lens[b])
        out[b] = wl.slot_idx[seg + n - wl.T: seg + n]
        seg += n
    return out


def test_append_oracle_restores_cleared_tree_rows():
    """Pin: the generator stores every tree node's row at its slot; clearing
    those rows and appending them back must restore the pool exactly."""
    wl = small_workload()
    slots = node_slots(wl)
    kv_new = wl.kv_pool[slots]                     # [B, T, 576]
    cleared = wl.kv_pool.copy()
    cleared[slots.reshape(-1)] = 0
    assert not np.array_equal(cleared, wl.kv_pool)
    restored = oracle.append_kv(cleared, kv_new, wl.slot_idx, wl.seq_lens)
    assert np.array_equal(restored, wl.kv_pool)


def test_append_oracle_writes_only_tree_slots_and_skips_out_of_range():
    wl = small_workload(seed=12)
    rng = np.random.default_rng(0)
    kv_new = rng.integers(0, 1 << 16, size=(wl.B, wl.T, 576), dtype=np.uint16)
    slots = node_slots(wl)
    slot_idx = wl.slot_idx.copy()
    # node (1, 2) points outside the pool: nothing may be written for it
    slot_idx[int(wl.seq_lens[0]) + int(wl.seq_lens[1]) - wl.T + 2] = wl.pool_slots
    got = oracle.append_kv(wl.kv_pool, kv_new, slot_idx, wl.seq_lens)
    for b in range(wl.B):
        for t in range(wl.T):
            want = wl.kv_pool[slots[b, t]] if (b, t) == (1, 2) else kv_new[b, t]
            assert np.array_equal(got[slots[b, t]], want), (b, t)
    others = np.setdiff1d(np.arange(wl.pool_slots), slots.reshape(-1))
    assert np.array_equal(got[others], wl.kv_pool[others])


def _device(wl):
    import torch
    from synthetic.device import to_device
    return to_device(wl)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [
    dict(B=3, H=2, T=5, prefixes=[7, 0, 33], pool_slots=200),
    dict(B=4, H=8, T=64, prefixes=[100, 0, 4096, 31], pool_slots=20000),
])
def test_append_kernel_matches_oracle_bitwise(shape):
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import params_of
    wl = inputs.make_workload("append_gpu", seed=21, **shape)
    rng = np.random.default_rng(1)
    kv_new = rng.integers(0, 1 << 16, size=(wl.B, wl.T, 576), dtype=np.uint16)
    slot_idx = wl.slot_idx.copy()
    slot_idx[int(wl.seq_lens[0]) - 1] = -3  # last node of sequence 0: outside the pool, skipped
    expect = oracle.append_kv(wl.kv_pool, kv_new, slot_idx, wl.seq_lens)
    pool = torch.from_numpy(wl.kv_pool.view(np.int16)).cuda().view(torch.bfloat16)
    new = torch.from_numpy(kv_new.view(np.int16)).cuda().view(torch.bfloat16)
    sl = torch.from_numpy(slot_idx).cuda()
    lens = torch.from_numpy(wl.seq_lens).cuda()
    mtv.verify_attn_append_kv(new, sl, lens, pool, params_of(wl))
    torch.cuda.synchronize()
    got = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, expect)


@pytest.mark.gpu
def test_append_then_verify_in_one_graph():
    """Clear the tree rows, then (append, verify) recorded in one HIP graph:
    every replay reproduces the oracle's output for the original workload."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import params_of
    orc = oracle.load()
    wl = inputs.make_workload("append_graph", B=2, H=8, T=16, prefixes=[300, 1000],
                              pool_slots=4096, seed=31)
    ref = orc.run(wl)
    slots = node_slots(wl)
    dev = _device(wl)
    kv_new = dev["kv_pool"][torch.from_numpy(slots.reshape(-1)).cuda()].reshape(wl.B, wl.T, 576).clone()
    prm = params_of(wl)
    op = mtv.VerifyAttention(prm)
    out = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mtv.verify_attn_append_kv(kv_new, dev["slot_idx"], dev["seq_lens"], dev["kv_pool"], prm, stream=s)
            op(**dev, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    idx = torch.from_numpy(slots.reshape(-1)).cuda()
    for rep in range(3):
        dev["kv_pool"].index_fill_(0, idx, 0)  # eager work between replays: clear the tree rows
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        ok, worst, row = parity_gate(got, ref)
        assert ok, f"replay {rep}: worst row {row} at {worst:.2f} bf16 ulp"
