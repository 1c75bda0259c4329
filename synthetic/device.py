"""Moving a synthetic workload to the device and describing it to the library
(marshalling only; no arithmetic of the method)."""
from __future__ import annotations

import numpy as np


def to_device(wl, device="cuda"):
    """torch tensors on `device`: bf16 q / kv_pool (from their bit patterns) or
    float32 ones for an fp32 workload, int32 rest."""
    import torch
    if wl.q.dtype == np.float32:
        q = torch.from_numpy(wl.q).to(device)
        kv = torch.from_numpy(wl.kv_pool).to(device)
    else:
        q = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).to(device)
        kv = torch.from_numpy(wl.kv_pool.view(np.int16)).view(torch.bfloat16).to(device)
    return dict(
        q=q,
        kv_pool=kv,
        slot_idx=torch.from_numpy(wl.slot_idx).to(device),
        seq_lens=torch.from_numpy(wl.seq_lens).to(device),
        tree_parent=torch.from_numpy(wl.tree_parent).to(device),
    )


def params_of(wl, nsplit: int = 0):
    """verify_attn_params of a call on this workload."""
    import mla_tree_verify_latent_amd as mtv
    return mtv.make_params(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T,
                           max_seq_len=wl.max_seq_len, total_kv=wl.total_kv,
                           pool_slots=wl.pool_slots, sm_scale=wl.sm_scale, nsplit=nsplit,
                           page_size=wl.page_size)
