"""Addressing and concurrency (needs a gfx950 GPU).

- A KV pool larger than 4 GiB: the rows a call references sit at slots whose byte
  offsets are past 2^32; the result is bit-identical to the same call on a compact pool
  holding the same rows (the computation depends only on the logical key order).
- Two calls with distinct workspaces on two streams at once give the same bits as the
  calls run one after the other.
"""
import numpy as np
import pytest

import oracle
from helpers import parity_gate, bf16_out_to_f32
from synthetic import inputs
from synthetic.device import params_of, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_tree_verify_latent_amd as mtv
    mtv.load_library()


def _params(wl, **kw):
    import mla_tree_verify_latent_amd as mtv
    d = dict(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T, max_seq_len=wl.max_seq_len,
             total_kv=wl.total_kv, pool_slots=wl.pool_slots, sm_scale=wl.sm_scale, nsplit=0,
             page_size=wl.page_size)
    d.update(kw)
    return mtv.make_params(**d)


def test_pool_beyond_4gib():
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = inputs.make_workload("pool4g", B=2, H=8, T=16, prefixes=[700, 300], pool_slots=2000, seed=77)
    dev = to_device(wl)
    ref = mtv.VerifyAttention(params_of(wl))(**dev)
    big_slots = 4_000_000                         # 4.6 GB of rows; 2^32 bytes = 3,728,270 rows
    assert (big_slots - 1) * 576 * 2 > 2 ** 32
    used = np.unique(wl.slot_idx)
    top = big_slots - 1 - np.arange(used.size)    # every referenced row past the 4 GiB mark
    assert top.min() * 576 * 2 >= 2 ** 32
    remap = np.full(wl.pool_slots, -1, dtype=np.int64)
    remap[used] = top
    slot_big = torch.from_numpy(remap[wl.slot_idx].astype(np.int32)).cuda()
    pool = torch.zeros((big_slots, 576), dtype=torch.bfloat16, device="cuda")
    pool[torch.from_numpy(top).cuda()] = dev["kv_pool"][torch.from_numpy(used).cuda()]
    out = mtv.VerifyAttention(_params(wl, pool_slots=big_slots))(
        dev["q"], pool, slot_big, dev["seq_lens"], dev["tree_parent"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    ok, worst, row = parity_gate(bf16_out_to_f32(out), oracle.load().run(wl))
    assert ok, f"row {row} at {worst:.2f} bf16 ulp"
    del pool
    torch.cuda.empty_cache()


def test_two_streams_concurrently():
    import torch
    import mla_tree_verify_latent_amd as mtv
    wls = [inputs.make_workload("s1", B=1, H=8, T=64, prefixes=[20000], pool_slots=30000, seed=81),
           inputs.make_workload("s2", B=3, H=16, T=9, prefixes=[5000, 9000, 64], pool_slots=20000, seed=82)]
    devs = [to_device(w) for w in wls]
    ops = [mtv.VerifyAttention(params_of(w)) for w in wls]
    refs = [op(**d) for op, d in zip(ops, devs)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(r) for r in refs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(5):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for s, op, d, o in zip(streams, ops, devs, outs):
            with torch.cuda.stream(s):
                for _ in range(3):
                    op(**d, out=o)
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16))
