"""Seeded random sweep over valid shapes: the HIP path against the oracle on every
(batch size, heads, tree size, prefixes, split count, tree shape) drawn, through the
bf16 entry point and the fp32-input one, with the gates of test_parity_gpu.py (2 bf16
ULP of each row's largest value) and test_f32.py (2^-16 of it).

Shapes: 1-5 sequences, H in {1, 2, 3, 4, 8, 16, 32, 64}, T in 1..64, prefixes in
0..2999 (a zero prefix one time in five), split count automatic or forced to 1..19,
random, chain or flat trees; drawn again when the oracle's work would exceed about
1.5e7 (query row, key) pairs so the sweep stays within seconds.
"""
import numpy as np
import pytest

import oracle
from helpers import parity_gate, run_gpu
from synthetic import inputs
from test_f32 import rel_gate, run_gpu_f32

pytestmark = pytest.mark.gpu

MAX_PAIRS = 15_000_000


def draw_shapes(n, seed):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        B = int(rng.integers(1, 6))
        H = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
        T = int(rng.integers(1, 65))
        prefixes = [int(x) for x in rng.integers(0, 3000, size=B)]
        if rng.random() < 0.2:
            prefixes[int(rng.integers(B))] = 0
        nsplit = 0 if rng.random() < 0.5 else int(rng.integers(1, 20))
        tree = str(rng.choice(["random", "random", "chain", "flat"]))
        if H * T * sum(p + T for p in prefixes) > MAX_PAIRS:
            continue
        shapes.append(dict(B=B, H=H, T=T, prefixes=prefixes, nsplit=nsplit, tree=tree,
                           seed=7000 + len(shapes)))
    return shapes


SHAPES = draw_shapes(24, 2024)
SHAPES_F32 = draw_shapes(8, 4048)


def _id(c):
    return "B{B}_H{H}_T{T}_P{p}_n{nsplit}_{tree}".format(p="-".join(map(str, c["prefixes"])), **c)


def _workload(c, dtype="bf16"):
    pool = sum(c["prefixes"]) + c["B"] * c["T"] + 57
    return inputs.make_workload("random", B=c["B"], H=c["H"], T=c["T"], prefixes=c["prefixes"],
                                pool_slots=pool, seed=c["seed"], tree=c["tree"], dtype=dtype)


@pytest.fixture(scope="module")
def orc():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_tree_verify_latent_amd as mtv
    mtv.load_library()
    return oracle.load()


@pytest.mark.parametrize("case", SHAPES, ids=_id)
def test_random_shape_bf16(orc, case):
    wl = _workload(case)
    ok, worst, row = parity_gate(run_gpu(wl, case["nsplit"]), orc.run(wl))
    assert ok, f"row {row} at {worst:.2f} bf16 ulp"


@pytest.mark.parametrize("case", SHAPES_F32, ids=_id)
def test_random_shape_f32(orc, case):
    wl = _workload(case, dtype="f32")
    ok, worst, row = rel_gate(run_gpu_f32(wl, case["nsplit"]), orc.run(wl))
    assert ok, f"row {row} at {worst:.2e} of the row scale"


def draw_loose(n, seed):
    """Shapes whose host-side bounds run past the data: max_seq_len above every
    length and the slot table longer than the sequences, its extra entries
    naming pool rows of NaNs."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B = int(rng.choice([1, 1, 2, 3]))
        H = int(rng.choice([1, 2, 4, 8, 16, 64]))
        T = int(rng.integers(1, 65))
        prefixes = [int(x) for x in rng.integers(0, 3000, size=B)]
        if H * T * sum(p + T for p in prefixes) > MAX_PAIRS:
            continue
        bound = int(rng.integers(1, 4000))
        out.append(dict(B=B, H=H, T=T, prefixes=prefixes, nsplit=int(rng.choice([0, 0, 3, 11])),
                        tree="random", seed=9000 + len(out), bound=bound,
                        extra=min(int(rng.integers(1, 600)), bound)))  # total_kv <= B * max_seq_len
    return out


SHAPES_LOOSE = draw_loose(16, 77)


@pytest.mark.parametrize("case", SHAPES_LOOSE, ids=lambda c: _id(c) + "_b{bound}_x{extra}".format(**c))
def test_random_loose_bounds(orc, case):
    """Every kernel path (one or several sequences, small-row and 128-row
    kernels, idle waves, the sliced combine) with a loose max_seq_len and
    slot-table entries past the sequences that point at NaN rows: the output
    stays finite and within the gate of the unextended inputs."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    from helpers import bf16_out_to_f32, to_device
    wl = _workload(case)
    dev = to_device(wl)
    x = case["extra"]
    dev["kv_pool"] = torch.cat([dev["kv_pool"], torch.full((x, 576), float("nan"), dtype=torch.bfloat16,
                                                           device="cuda")])
    dev["slot_idx"] = torch.cat([dev["slot_idx"], torch.arange(wl.pool_slots, wl.pool_slots + x,
                                                               dtype=torch.int32, device="cuda")])
    prm = mtv.make_params(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T,
                          max_seq_len=wl.max_seq_len + case["bound"], total_kv=wl.total_kv + x,
                          pool_slots=wl.pool_slots + x, sm_scale=wl.sm_scale, nsplit=case["nsplit"])
    out = mtv.VerifyAttention(prm)(**dev)
    torch.cuda.synchronize()
    got = bf16_out_to_f32(out)
    assert np.isfinite(got).all()
    ok, worst, row = parity_gate(got, orc.run(wl))
    assert ok, f"row {row} at {worst:.2f} bf16 ulp"
