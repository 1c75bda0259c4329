"""verify_attn_noalloc, the entry point without a workspace argument (its split-K
partials live in the library's per-GPU scratch array), against verify_attn on the
same inputs, through the C ABI. It runs the same plan and kernels, so the outputs
must be equal bit for bit, on consecutive calls that share the one scratch array
(a large call, then smaller ones that must not see the earlier partials)."""
import numpy as np
import pytest

import oracle
from helpers import bf16_out_to_f32, parity_gate, params_of, to_device
from synthetic import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_tree_verify_latent_amd as mtv
    mtv.load_library()


def _both(wl):
    import torch
    import mla_tree_verify_latent_amd as mtv
    dev = to_device(wl)
    prm = params_of(wl)
    assert mtv.verify_attn_workspace_size(prm) <= mtv.NOALLOC_SCRATCH_BYTES
    ref = mtv.VerifyAttention(prm)(**dev)
    out = torch.full_like(ref, float("nan"))
    mtv.verify_attn_noalloc(**dev, out=out, params=prm)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_matches_verify_attn_on_consecutive_calls():
    import torch
    big = inputs.config("c4a_long_scattered")  # 32.25 MiB of partials
    small = inputs.make_workload("small", B=3, H=8, T=9, prefixes=[700, 0, 2048], pool_slots=4096,
                                 seed=77)
    # then fewer rows still: 16 rows per sequence, the small-row kernel
    smaller = inputs.make_workload("smaller", B=2, H=8, T=2, prefixes=[1500, 60], pool_slots=2048, seed=78)
    orc = oracle.load()
    for wl in (big, small, smaller):
        out, ref = _both(wl)
        assert torch.equal(out, ref), wl.name
        if wl is not big:  # each later call's output passes the oracle gate on its own
            ok, worst, idx = parity_gate(bf16_out_to_f32(out), orc.run(wl))
            assert ok, f"{wl.name}: worst row {idx} at {worst:.2f} bf16 ulp"


def test_noalloc_refuses_more_than_its_scratch():
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = inputs.make_workload("tiny", B=1, H=8, T=8, prefixes=[256], pool_slots=1024, seed=5)
    dev = to_device(wl)
    # a shape whose partials need more than the scratch (5 split rounds of 64 heads)
    prm = mtv.make_params(num_seqs=4, num_heads=64, tree_size=64, max_seq_len=200768,
                          total_kv=294400, pool_slots=300000, sm_scale=wl.sm_scale)
    assert mtv.verify_attn_workspace_size(prm) > mtv.NOALLOC_SCRATCH_BYTES
    lib = mtv.load_library()
    import ctypes
    out = torch.empty((4, 64, 64, 512), dtype=torch.bfloat16, device="cuda")
    rc = lib.verify_attn_noalloc(ctypes.byref(prm), dev["q"].data_ptr(), dev["kv_pool"].data_ptr(),
                                 dev["slot_idx"].data_ptr(), dev["seq_lens"].data_ptr(),
                                 dev["tree_parent"].data_ptr(), out.data_ptr(), None)
    assert rc == -10 and "scratch" in mtv.verify_attn_strerror(rc)
