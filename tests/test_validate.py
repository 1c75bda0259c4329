"""The debug validator of the device-resident inputs (slot_idx, seq_lens,
tree_parent): a valid workload gives 0, each planted defect its own bit."""
import numpy as np
import pytest

from synthetic import inputs

pytestmark = pytest.mark.gpu


def _run(wl, slot_idx=None, seq_lens=None, tree_parent=None, **param_kw):
    import torch
    import mla_tree_verify_latent_amd as mtv
    d = dict(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T, max_seq_len=wl.max_seq_len,
             total_kv=wl.total_kv, pool_slots=wl.pool_slots, sm_scale=wl.sm_scale)
    d.update(param_kw)
    prm = mtv.make_params(**d)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    return mtv.verify_attn_debug_validate(
        dev(wl.slot_idx if slot_idx is None else slot_idx),
        dev(wl.seq_lens if seq_lens is None else seq_lens),
        dev(wl.tree_parent if tree_parent is None else tree_parent), prm)


@pytest.fixture(scope="module")
def wl():
    return inputs.make_workload("validate", B=3, H=2, T=8, prefixes=[100, 0, 2000], pool_slots=4096,
                                seed=51)


def test_valid_inputs(wl):
    assert _run(wl) == 0


def test_each_defect_sets_its_bit(wl):
    import mla_tree_verify_latent_amd as mtv
    lens = wl.seq_lens.copy()
    lens[1] = wl.T - 1                                   # shorter than the tree
    assert _run(wl, seq_lens=lens) == mtv.BAD_LENGTH
    lens = wl.seq_lens.copy()
    lens[0] += 5                                         # the lengths overrun slot_idx
    assert _run(wl, seq_lens=lens) == mtv.BAD_TOTAL
    par = wl.tree_parent.copy()
    par[2, 5] = 5                                        # a node as its own parent
    assert _run(wl, tree_parent=par) == mtv.BAD_PARENT
    slots = wl.slot_idx.copy()
    slots[-1] = wl.pool_slots                            # past the pool
    assert _run(wl, slot_idx=slots) == mtv.BAD_SLOT
    slots[3] = -1
    par[0, 0] = -2
    assert _run(wl, slot_idx=slots, tree_parent=par) == mtv.BAD_SLOT | mtv.BAD_PARENT


def test_large_slot_table():
    """More entries than one pass of the grid covers."""
    import mla_tree_verify_latent_amd as mtv
    big = inputs.make_workload("validate_big", B=1, H=1, T=4, prefixes=[400000], pool_slots=500000, seed=52)
    assert _run(big) == 0
    slots = big.slot_idx.copy()
    slots[399999] = 500000
    assert _run(big, slot_idx=slots) == mtv.BAD_SLOT
