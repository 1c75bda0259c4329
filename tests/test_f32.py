"""fp32-input variant (binary32 q and KV, fp32 output) against the oracle's
binary32 entry points on identical seeded inputs.

Gate (per output row): max_d |gpu - oracle| <= REL_TOL * max_d |oracle|, with
REL_TOL = 2^-16 (about 256 fp32 units of the row's largest value). The GPU
computes in fp32 throughout (products, sums, the softmax weights), so its error
is a few fp32 roundings of the 576-term dot products, of the exponent and of
the weighted sums over a split's keys and then over the splits; the worst row
measured on these workloads is about 7e-7 (roughly 12 fp32 units), twenty
times inside the gate, which is itself 1,000 times tighter than the bf16
path's 2 bf16 ULP.
"""
import numpy as np
import pytest

import oracle
from synthetic import inputs

REL_TOL = 2.0 ** -16


def rel_gate(got, ref, tol=REL_TOL):
    got = np.asarray(got, dtype=np.float64).reshape(-1, 512)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 512)
    err = np.abs(got - ref).max(axis=1)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    ratio = err / scale
    worst = int(np.argmax(ratio))
    return bool((ratio <= tol).all()), float(ratio[worst]), worst


def test_rel_gate_catches_a_wrong_row():
    ref = np.ones((3, 512))
    got = ref.copy()
    assert rel_gate(got, ref)[0]
    got[1, 7] += 2 * REL_TOL
    ok, worst, row = rel_gate(got, ref)
    assert not ok and row == 1


def run_gpu_f32(wl, nsplit=0, dev=None):
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import params_of, to_device
    if dev is None:
        dev = to_device(wl)
    prm = params_of(wl, nsplit)
    ws = torch.empty(mtv.verify_attn_f32_workspace_size(prm), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.float32, device="cuda")
    mtv.verify_attn_f32(dev["q"], dev["kv_pool"], dev["slot_idx"], dev["seq_lens"], dev["tree_parent"],
                        out, ws, prm)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def f32_workload(name="f32", B=1, H=8, T=8, prefixes=(256,), pool=None, seed=21, **kw):
    prefixes = list(prefixes)
    if pool is None:
        pool = sum(prefixes) + B * T + 101
    return inputs.make_workload(name, B=B, H=H, T=T, prefixes=prefixes, pool_slots=pool, seed=seed,
                                dtype="f32", **kw)


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.gpu
@pytest.mark.parametrize("case", [
    dict(B=1, H=8, T=8, prefixes=[256]),
    dict(B=1, H=1, T=1, prefixes=[0]),                 # single key
    dict(B=3, H=2, T=7, prefixes=[0, 33, 95]),         # ragged batch, P=0
    dict(B=2, H=8, T=64, prefixes=[31, 64]),           # full tree, 8 row tiles of 64
    dict(B=1, H=64, T=3, prefixes=[1000]),             # 192 rows
    dict(B=1, H=16, T=9, prefixes=[4097]),             # ragged tail tile
    dict(B=1, H=8, T=32, prefixes=[4096], max_depth=8),
], ids=lambda c: "B{B}_H{H}_T{T}_P{prefixes}".format(**c))
def test_f32_matches_oracle(orc, case):
    wl = f32_workload(**case)
    got = run_gpu_f32(wl)
    ref = orc.run(wl)
    ok, worst, row = rel_gate(got, ref)
    print(f"f32 {case}: worst row {row} rel err {worst:.3e}")
    assert ok, f"row {row}: relative error {worst:.3e} > {REL_TOL:.3e}"


@pytest.mark.gpu
@pytest.mark.parametrize("nsplit", [1, 7])
def test_f32_nsplit_independent(orc, nsplit):
    wl = f32_workload(B=2, H=4, T=16, prefixes=[3000, 700], seed=23)
    ok, worst, row = rel_gate(run_gpu_f32(wl, nsplit), orc.run(wl))
    assert ok, f"nsplit {nsplit}: row {row} relative error {worst:.3e}"


@pytest.mark.gpu
def test_f32_on_bf16_values_matches_bf16_path_gate():
    """fp32 arrays holding bf16 values: the fp32 path meets the fp32 gate
    against the oracle's bf16 result (the same mathematical input)."""
    import dataclasses
    orc_ = oracle.load()
    wl = inputs.make_workload("f32b", B=1, H=8, T=16, prefixes=[2000], pool_slots=4096, seed=24)
    ref = orc_.run(wl)
    wl32 = dataclasses.replace(wl, q=inputs.bf16_bits_to_f32(wl.q), kv_pool=inputs.bf16_bits_to_f32(wl.kv_pool))
    ok, worst, row = rel_gate(run_gpu_f32(wl32), ref)
    assert ok, f"row {row}: relative error {worst:.3e}"


@pytest.mark.gpu
def test_f32_long_context_sampled(orc):
    """The 64k-token H=8, T=64 workload in fp32: sampled rows against the oracle."""
    wl = inputs.config("f4_long_f32")
    got = run_gpu_f32(wl)
    rng = np.random.default_rng(5)
    rows = np.array([(0, int(t), int(h)) for t, h in zip(rng.integers(0, wl.T, 24), rng.integers(0, wl.H, 24))])
    ref = orc.run_rows(wl, rows)
    g = np.stack([got[b, t, h] for b, t, h in rows])
    ok, worst, idx = rel_gate(g, ref)
    print(f"f32 long: worst sampled row {tuple(rows[idx])} rel err {worst:.3e}")
    assert ok, f"row {tuple(rows[idx])}: relative error {worst:.3e}"


@pytest.mark.gpu
def test_f32_graph_capture_replay():
    """The fp32 call captured in a HIP graph: every replay (with eager work in
    between) gives the eager call's bits."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    from synthetic.device import params_of, to_device
    wl = f32_workload(B=2, H=8, T=16, prefixes=[1500, 300], seed=25)
    dev = to_device(wl)
    prm = params_of(wl)
    ws = torch.empty(mtv.verify_attn_f32_workspace_size(prm), dtype=torch.uint8, device="cuda")
    eager = run_gpu_f32(wl, dev=dev)
    out = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mtv.verify_attn_f32(dev["q"], dev["kv_pool"], dev["slot_idx"], dev["seq_lens"],
                                dev["tree_parent"], out, ws, prm, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {rep}"
