"""KV defragmentation (each sequence's rows gathered into one contiguous run):
the NumPy definition in oracle/ pinned on the CPU, the HIP kernel checked
against it bit for bit on the GPU, and verify on the compacted rows checked to
give exactly the result of verify on the scattered pool."""
import numpy as np
import pytest

import oracle
from synthetic import inputs

from helpers import parity_gate

SMALL = dict(B=3, H=2, T=5, prefixes=[7, 0, 33], pool_slots=200)


def test_compact_oracle_reproduces_generator_defragmented_layout():
    """Pin: the generator's contiguous layout stores logical row i of the slot
    list at slot i; compacting the scattered pool of the same seed must give
    exactly those rows."""
    scat = inputs.make_workload("compact_pin", seed=41, **SMALL)
    cont = inputs.make_workload("compact_pin", seed=41, layout="contiguous", **SMALL)
    assert not np.array_equal(scat.slot_idx, np.arange(scat.total_kv))
    got = oracle.compact_kv(scat.kv_pool, scat.slot_idx)
    assert got.shape == (scat.total_kv, 576)
    assert np.array_equal(got, cont.kv_pool[:scat.total_kv])


def test_compact_oracle_identity_and_out_of_range():
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 1 << 16, size=(50, 576), dtype=np.uint16)
    assert np.array_equal(oracle.compact_kv(pool, np.arange(50, dtype=np.int32)), pool)
    slots = np.array([4, -1, 50, 4, 49], dtype=np.int32)
    got = oracle.compact_kv(pool, slots)
    assert np.array_equal(got[[0, 3]], pool[[4, 4]]) and np.array_equal(got[4], pool[49])
    assert not got[[1, 2]].any()
    assert oracle.compact_kv(pool, np.zeros(0, dtype=np.int32)).shape == (0, 576)


def test_oracle_verify_is_layout_independent():
    """Attention reads rows only through the slot list: the oracle on the
    compacted rows with slot list 0, 1, 2, ... equals the oracle on the
    scattered pool exactly (same fp64 operations in the same order)."""
    orc = oracle.load()
    scat = inputs.make_workload("compact_verify", seed=42, **SMALL)
    cont = inputs.make_workload("compact_verify", seed=42, layout="contiguous", **SMALL)
    assert np.array_equal(orc.run(scat), orc.run(cont))


def test_paged64_layout_holds_the_same_rows():
    """The 64-row paged layout: logical row i of the slot list holds the row it
    holds in the scattered layout of the same seed, every run of 64 entries is
    one page of 64 consecutive slots starting at a multiple of 64, the pool is a
    permutation of the scattered pool's rows, and the oracle's result is the
    same in every layout."""
    small = dict(B=3, H=2, T=5, prefixes=[130, 0, 333], pool_slots=1024)
    scat = inputs.make_workload("paged", seed=43, **small)
    paged = inputs.make_workload("paged", seed=43, layout="paged64", **small)
    assert np.array_equal(paged.kv_pool[paged.slot_idx], scat.kv_pool[scat.slot_idx])
    s = paged.slot_idx.astype(np.int64)
    i = np.arange(s.size)
    assert np.all(s % 64 == i % 64)
    assert np.all(s - i % 64 == np.repeat(s[::64], 64)[:s.size])
    assert len(np.unique(s[::64])) == len(s[::64])
    key = lambda pool: sorted(r.tobytes() for r in pool)
    assert key(paged.kv_pool) == key(scat.kv_pool)
    orc = oracle.load()
    assert np.array_equal(orc.run(paged), orc.run(scat))


def _bf16_dev(a):
    import torch
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [
    SMALL,
    dict(B=4, H=8, T=64, prefixes=[100, 0, 4096, 31], pool_slots=20000),
])
def test_compact_kernel_matches_oracle_bitwise(shape):
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import params_of
    wl = inputs.make_workload("compact_gpu", seed=43, **shape)
    slot_idx = wl.slot_idx.copy()
    slot_idx[1] = -1                # outside the pool: a row of zeros
    slot_idx[-1] = wl.pool_slots    # likewise
    expect = oracle.compact_kv(wl.kv_pool, slot_idx)
    dst = torch.full((wl.total_kv, 576), 7.0, dtype=torch.bfloat16, device="cuda")
    mtv.verify_attn_compact_kv(_bf16_dev(wl.kv_pool), torch.from_numpy(slot_idx).cuda(), dst, params_of(wl))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dst), expect)


def _compact_then_verify_matches(wl, sample_rows=None):
    """Verify on the scattered pool, and verify on compacted rows with slot
    list 0, 1, 2, ... (page_size 64): identical bits; both against the oracle."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import to_device, params_of
    dev = to_device(wl)
    prm = params_of(wl)
    out_a = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.bfloat16, device="cuda")
    mtv.VerifyAttention(prm)(**dev, out=out_a)
    dst = torch.empty((wl.total_kv, 576), dtype=torch.bfloat16, device="cuda")
    mtv.verify_attn_compact_kv(dev["kv_pool"], dev["slot_idx"], dst, prm)
    prm_c = mtv.make_params(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T, max_seq_len=wl.max_seq_len,
                            total_kv=wl.total_kv, pool_slots=wl.total_kv, sm_scale=wl.sm_scale,
                            page_size=64)
    ident = torch.arange(wl.total_kv, dtype=torch.int32, device="cuda")
    out_b = torch.empty_like(out_a)
    mtv.VerifyAttention(prm_c)(q=dev["q"], kv_pool=dst, slot_idx=ident, seq_lens=dev["seq_lens"],
                               tree_parent=dev["tree_parent"], out=out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    return out_a


@pytest.mark.gpu
def test_compact_then_verify_equals_scattered_verify():
    wl = inputs.make_workload("compact_verify_gpu", B=3, H=8, T=16, prefixes=[300, 0, 1500],
                              pool_slots=8192, seed=44)
    out = _compact_then_verify_matches(wl)
    ok, worst, row = parity_gate(out.float().cpu().numpy(), oracle.load().run(wl))
    assert ok, f"worst row {row} at {worst:.2f} bf16 ulp"


@pytest.mark.gpu
def test_compact_then_verify_long_context_scattered():
    """The 64k-token scattered workload: verify after compaction gives the
    same bits as verify on the scattered pool."""
    _compact_then_verify_matches(inputs.config("c4a_long_scattered"))


@pytest.mark.gpu
def test_compact_then_verify_in_one_graph():
    """Compaction and verify on the compacted rows recorded in one HIP graph:
    every replay gives the bits of verify on the scattered pool."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import to_device, params_of
    wl = inputs.make_workload("compact_graph", B=2, H=8, T=16, prefixes=[900, 2100], pool_slots=8192,
                              seed=45)
    dev = to_device(wl)
    prm = params_of(wl)
    ref = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.bfloat16, device="cuda")
    mtv.VerifyAttention(prm)(**dev, out=ref)
    prm_c = mtv.make_params(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T, max_seq_len=wl.max_seq_len,
                            total_kv=wl.total_kv, pool_slots=wl.total_kv, sm_scale=wl.sm_scale,
                            page_size=64)
    dst = torch.empty((wl.total_kv, 576), dtype=torch.bfloat16, device="cuda")
    ident = torch.arange(wl.total_kv, dtype=torch.int32, device="cuda")
    op = mtv.VerifyAttention(prm_c)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mtv.verify_attn_compact_kv(dev["kv_pool"], dev["slot_idx"], dst, prm, stream=s)
            op(q=dev["q"], kv_pool=dst, slot_idx=ident, seq_lens=dev["seq_lens"],
               tree_parent=dev["tree_parent"], out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        dst.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"


@pytest.mark.gpu
@pytest.mark.parametrize("shape", ["small", "e2_h8_t9_65k"])
def test_layouts_give_identical_output(shape):
    """Verify reads KV rows only through the slot list: scattered, contiguous
    and 64-row paged layouts of the same rows give the same bits."""
    from helpers import run_gpu
    outs = []
    for layout in ("scattered", "contiguous", "paged64"):
        if shape == "small":
            wl = inputs.make_workload("layouts", B=2, H=8, T=9, prefixes=[3000, 1000], pool_slots=8192,
                                      seed=44, layout=layout)
        else:
            wl = inputs.make_workload(shape, **{**inputs.CONFIGS[shape], "layout": layout})
        outs.append(run_gpu(wl))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
