"""HIP path vs the CPU oracle on identical seeded inputs (needs a gfx950 GPU).

Gate (per output row (b, t, h)): max_d |gpu - oracle| <= 2 bf16 ULP of
max_d |oracle|. The oracle is fp64; the GPU output is bf16 (RNE) of an fp32
online softmax with bf16 MFMA operands (q, K, V exact; P rounded to bf16).
"""
import numpy as np
import pytest

import oracle
from helpers import parity_gate, run_gpu, sample_rows, to_device, params_of, bf16_out_to_f32
from synthetic import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_tree_verify_latent_amd as mtv
    mtv.load_library()
    return torch.device("cuda")


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def check_full(orc, wl, nsplit=0, ulps=2.0):
    got = run_gpu(wl, nsplit)
    ref = orc.run(wl)
    ok, worst, idx = parity_gate(got, ref, ulps)
    assert ok, f"{wl.name}: worst row {idx} at {worst:.2f} bf16 ulp"
    return got, ref


def check_sampled(orc, wl, n_per_seq=24, nsplit=0, dev=None):
    got = run_gpu(wl, nsplit, dev)
    rows = sample_rows(wl, n_per_seq)
    ref = orc.run_rows(wl, rows)
    g = np.stack([got[b, t, h] for b, t, h in rows])
    ok, worst, idx = parity_gate(g, ref)
    assert ok, f"{wl.name}: row {tuple(rows[idx])} at {worst:.2f} bf16 ulp"
    return got


def small(name="small", B=1, H=8, T=8, prefixes=(256,), pool=None, seed=11, **kw):
    prefixes = list(prefixes)
    if pool is None:
        pool = sum(prefixes) + B * T + 101
    return inputs.make_workload(name, B=B, H=H, T=T, prefixes=prefixes, pool_slots=pool,
                                seed=seed, **kw)


# ------------------------------------------------------------ configurations

def test_c1_tiny_full(orc):
    check_full(orc, inputs.config("c1_tiny"))


def test_c2_tp_share_full(orc):
    check_full(orc, inputs.config("c2_tp_share"))


def test_c3_full_head_full(orc):
    check_full(orc, inputs.config("c3_full_head"))


def test_c4_long_both_layouts(orc):
    a = inputs.config("c4a_long_scattered")
    got_a = check_full(orc, a)[0]
    b = inputs.config("c4b_long_contiguous")
    got_b = run_gpu(b)
    assert np.array_equal(got_a, got_b), "layouts (a) and (b) hold the same values"


def test_c5_ragged_sampled(orc):
    check_sampled(orc, inputs.config("c5_ragged"), n_per_seq=16)


def test_e2_production_shape_full(orc):
    check_full(orc, inputs.config("e2_h8_t9_65k"))


def test_e1_full_head_65k_sampled(orc):
    # the H=64 point at 65k context that bench.py times beside the headline
    check_sampled(orc, inputs.config("e1_h64_65k"), n_per_seq=32)


def test_million_key_context_sampled(orc):
    """One sequence of a million cached keys (H=8, T=64, scattered over a 1.1M-slot
    pool): 64 splits of 15,648 keys (489 tiles each), so the running maximum and the
    fp32 sums carry over long runs of tiles. (These draws never raise a running
    maximum past its lazy threshold; test_rescale_gpu.py covers the rescale.)"""
    wl = inputs.make_workload("long_1m", B=1, H=8, T=64, prefixes=[1_000_000],
                              pool_slots=1_100_000, seed=61)
    check_sampled(orc, wl, n_per_seq=24)


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("case", [
    dict(B=1, H=1, T=1, prefixes=[0]),                 # single key: out == own V row
    dict(B=1, H=3, T=5, prefixes=[7]),                 # M=15 rows, ragged everything
    dict(B=3, H=2, T=7, prefixes=[0, 33, 95]),         # ragged batch, P=0 included
    dict(B=2, H=8, T=64, prefixes=[31, 64]),           # full tree size
    dict(B=1, H=64, T=3, prefixes=[1000]),             # 192 rows, 3 row tiles
    dict(B=1, H=16, T=9, prefixes=[4097]),             # tail tile of 1 key + tree
    dict(B=4, H=8, T=16, prefixes=[5000, 1, 32, 2047]),
    dict(B=1, H=128, T=64, prefixes=[2000]),           # 8,192 rows: 64 row tiles, T at its maximum
], ids=lambda c: "B{B}_H{H}_T{T}_P{prefixes}".format(**c))
def test_edge_shapes(orc, case):
    check_full(orc, small(**case))


@pytest.mark.parametrize("T", [1, 5, 9, 12])
@pytest.mark.parametrize("H", [8, 16])
def test_production_row_counts_full(orc, H, T):
    """One TP rank's heads verifying a few draft tokens at a 65k-token prefix: the
    row counts (H*T = 8 .. 192) on both sides of the small-row kernel's limit,
    every output row compared."""
    import mla_tree_verify_latent_amd as mtv
    wl = inputs.make_workload(f"h{H}_t{T}_65k", B=1, H=H, T=T, prefixes=[65536], pool_slots=131072,
                              seed=900 + 10 * H + T)
    plan = mtv.verify_attn_plan(params_of(wl))
    assert (plan["rows_per_tile"] <= 32) == (H * T <= 32), plan
    check_full(orc, wl)


@pytest.mark.parametrize("case", [
    dict(B=3, H=8, T=9, prefixes=[0, 4095, 70], nsplit=0),     # ragged, P = 0, a 4,104-key sequence
    dict(B=1, H=4, T=8, prefixes=[1000], nsplit=7),            # 32 rows: two row blocks, forced splits
    dict(B=2, H=1, T=32, prefixes=[129, 64], nsplit=0),        # 32 rows, the tree spans half a tile
    dict(B=1, H=8, T=3, prefixes=[63], nsplit=1),              # one split, the tree crosses the first tile
    dict(B=1, H=2, T=40, prefixes=[5000], nsplit=3, tree="chain"),
    dict(B=1, H=16, T=2, prefixes=[200000], nsplit=0),         # 32 rows in one row tile, 200k keys
], ids=lambda c: "B{B}_H{H}_T{T}_P{prefixes}_n{nsplit}".format(**c))
def test_small_row_kernel_shapes(orc, case):
    case = dict(case)
    nsplit = case.pop("nsplit")
    wl = small(**case, seed=40 + case["T"])
    check_full(orc, wl, nsplit=nsplit)


@pytest.mark.parametrize("B", [70, 130, 1000])
def test_many_sequences(orc, B):
    """More sequences than one 64-lane scan covers: the split location and the
    combine's sequence lookup take their multi-pass path."""
    rng = np.random.default_rng(B)
    prefixes = [int(p) for p in rng.integers(0, 400, size=B)]
    prefixes[B // 2] = 0
    check_full(orc, small(B=B, H=2, T=4, prefixes=prefixes, seed=B))


@pytest.mark.parametrize("extra", [1, 700, 5000])
def test_length_bound_above_actual(orc, extra):
    """One sequence whose host-side bound max_seq_len exceeds its actual length:
    the work items are dealt from the bound, splits past the end do nothing,
    and the last split (40 keys here) re-reads its slot entries. The partial
    results match those of the exact bound bit for bit (the combine's wave
    count follows the bound, so only its merge order may differ), and the
    output passes the oracle gate."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = small(B=1, H=8, T=16, prefixes=[2072], seed=31)
    dev = to_device(wl)
    def partials(prm):
        ws = torch.zeros(mtv.verify_attn_workspace_size(prm), dtype=torch.uint8, device="cuda")
        mtv.verify_attn_partial(dev["q"], dev["kv_pool"], dev["slot_idx"], dev["seq_lens"],
                                dev["tree_parent"], ws, prm)
        torch.cuda.synchronize()
        return ws.cpu().numpy()
    prm = mtv.make_params(num_seqs=1, num_heads=wl.H, tree_size=wl.T, max_seq_len=wl.max_seq_len + extra,
                          total_kv=wl.total_kv, pool_slots=wl.pool_slots, sm_scale=wl.sm_scale)
    assert np.array_equal(partials(prm), partials(params_of(wl)))
    out = mtv.VerifyAttention(prm)(**dev)
    torch.cuda.synchronize()
    got = bf16_out_to_f32(out)
    ok, worst, idx = parity_gate(got, orc.run(wl))
    assert ok, f"worst row {idx} at {worst:.2f} bf16 ulp"


@pytest.mark.parametrize("H,T,prefix", [(8, 16, 2072), (8, 4, 2072), (4, 3, 1000)])
@pytest.mark.parametrize("extra", [40, 3000])
def test_rows_past_the_end_are_never_read(orc, H, T, prefix, extra):
    """One sequence whose slot table and length bound run `extra` entries past
    its length, every one of them naming a pool row of bf16 NaNs: a split that
    starts before the end reads no KV row past it (its last tiles are masked,
    and a masked NaN row would still turn the weighted V sum into NaN), and the
    splits dealt past the end do nothing. Covers the 128-row kernel and the
    small-row kernel with one and two 16-row blocks; the output passes the
    oracle gate of the unextended inputs."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = small(B=1, H=H, T=T, prefixes=[prefix], seed=37)
    dev = to_device(wl)
    nan_rows = torch.full((extra, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    dev["kv_pool"] = torch.cat([dev["kv_pool"], nan_rows])
    past = torch.arange(wl.pool_slots, wl.pool_slots + extra, dtype=torch.int32, device="cuda")
    dev["slot_idx"] = torch.cat([dev["slot_idx"], past])
    prm = mtv.make_params(num_seqs=1, num_heads=H, tree_size=T, max_seq_len=wl.max_seq_len + extra,
                          total_kv=wl.total_kv + extra, pool_slots=wl.pool_slots + extra,
                          sm_scale=wl.sm_scale)
    out = mtv.VerifyAttention(prm)(**dev)
    torch.cuda.synchronize()
    got = bf16_out_to_f32(out)
    assert np.isfinite(got).all()
    ok, worst, idx = parity_gate(got, orc.run(wl))
    assert ok, f"worst row {idx} at {worst:.2f} bf16 ulp"


@pytest.mark.parametrize("tree", ["flat", "chain"])
def test_tree_shapes(orc, tree):
    check_full(orc, small(H=4, T=64, prefixes=[300], tree=tree, seed=5))


def _relabel_trees(wl):
    """Renumber every sequence's tree nodes in another topological order (always
    take the highest-numbered node whose parent is already numbered), moving the
    query rows and the tree slots with them. Returns the new workload and, per
    sequence, the map old label -> new label."""
    import copy
    new = copy.deepcopy(wl)
    sigmas = []
    seg = 0
    for b in range(wl.B):
        parent = wl.tree_parent[b]
        order, done = [], set()
        while len(order) < wl.T:
            ready = [u for u in range(wl.T) if u not in done and (parent[u] < 0 or parent[u] in done)]
            order.append(max(ready))
            done.add(order[-1])
        sigma = np.empty(wl.T, dtype=np.int64)
        sigma[order] = np.arange(wl.T)
        for u in range(wl.T):
            new.tree_parent[b, sigma[u]] = -1 if parent[u] < 0 else sigma[parent[u]]
        N = int(wl.seq_lens[b])
        base = seg + N - wl.T
        new.slot_idx[base + sigma] = wl.slot_idx[base:base + wl.T]
        new.q[b, sigma] = wl.q[b]
        sigmas.append(sigma)
        seg += N
    return new, sigmas


def test_tree_relabel_permutes_outputs(orc):
    # trees deep enough to cross the 32-key tile boundary, two sequences
    wl = small(B=2, H=8, T=40, prefixes=[1000, 77], seed=29)
    got = check_full(orc, wl)[0]
    wl2, sigmas = _relabel_trees(wl)
    assert not np.array_equal(wl2.tree_parent, wl.tree_parent)
    got2 = check_full(orc, wl2)[0]
    for b, sigma in enumerate(sigmas):
        ok, worst, idx = parity_gate(got2[b, sigma], got[b])
        assert ok, f"sequence {b}: relabelled row {idx} differs by {worst:.2f} bf16 ulp"


def test_single_key_exact():
    wl = small(B=2, H=4, T=1, prefixes=[0, 0], seed=3)
    got = run_gpu(wl)
    v = inputs.bf16_bits_to_f32(wl.kv_pool[wl.slot_idx])[:, :512]
    for b in range(2):
        for h in range(4):
            assert np.array_equal(got[b, 0, h], v[b])


@pytest.mark.parametrize("nsplit", [1, 2, 7, 64, 0])
def test_nsplit_independent(orc, nsplit):
    wl = inputs.config("c2_tp_share")
    check_full(orc, wl, nsplit=nsplit)


@pytest.mark.parametrize("case", [
    dict(B=1, H=64, T=64, prefixes=[6000], nsplit=40),           # 4096 rows, one wave per row
    dict(B=3, H=64, T=16, prefixes=[3000, 0, 5000], nsplit=48),  # rows of sequences 1 and 2 locate their splits
    dict(B=1, H=8, T=1, prefixes=[60000], nsplit=600),           # 8 rows: the sliced combine
    dict(B=2, H=8, T=2, prefixes=[30000, 20000], nsplit=800),
    dict(B=1, H=8, T=9, prefixes=[60000], nsplit=600),           # 72 rows: half rows, 16 waves per row
], ids=lambda c: "B{B}_H{H}_T{T}_n{nsplit}".format(**c))
def test_combine_batches(orc, case):
    """Splits enough that every combine wave takes several batches of loads
    (at most 16 partials per batch, at most 16 waves per row)."""
    import mla_tree_verify_latent_amd as mtv
    case = dict(case)
    nsplit = case.pop("nsplit")
    wl = small("combine", pool=sum(case["prefixes"]) + case["B"] * case["T"] + 300, seed=21, **case)
    plan = mtv.verify_attn_plan(params_of(wl, nsplit))
    c = plan["keys_per_split"]
    per_seq = [-(-(p + wl.T) // c) for p in case["prefixes"]]
    assert max(per_seq) > 16 * 16 or (wl.H * wl.T * case["B"] > 2048 and max(per_seq) > 12), per_seq
    check_full(orc, wl, nsplit=nsplit)


@pytest.mark.parametrize("case", [
    dict(B=1, H=8, T=1, prefixes=[140000], nsplit=2200),                # 16 waves, three batches each
    dict(B=4, H=2, T=4, prefixes=[9000, 0, 3000, 20000], nsplit=300),   # sequences 1-3 locate their splits
    dict(B=1, H=4, T=2, prefixes=[700], nsplit=0),                      # one wave per workgroup
    dict(B=2, H=16, T=1, prefixes=[40000, 1], nsplit=0),                # 32 rows, one sequence of one split
], ids=lambda c: "B{B}_H{H}_T{T}_n{nsplit}".format(**c))
def test_sliced_combine(orc, case):
    """Calls of at most 32 rows take the sliced combine (a workgroup per row
    and 64 features, four splits per load instruction): full-output parity
    with one to sixteen waves per workgroup, several batches per wave, and
    rows of later sequences that locate their splits."""
    import mla_tree_verify_latent_amd as mtv
    case = dict(case)
    nsplit = case.pop("nsplit")
    wl = small("sliced", pool=sum(case["prefixes"]) + case["B"] * case["T"] + 300, seed=23, **case)
    assert wl.B * wl.H * wl.T <= 32
    plan = mtv.verify_attn_plan(params_of(wl, nsplit))
    assert plan["combine_blocks"] == 8 * wl.B * wl.H * wl.T
    check_full(orc, wl, nsplit=nsplit)


def test_zero_query_is_mean(orc):
    wl = small(H=2, T=12, prefixes=[500], seed=8)
    wl.q[:] = 0
    check_full(orc, wl)


@pytest.mark.parametrize("H,T,prefix,nsplit", [
    (4, 8, 777, 0),       # small-row kernel
    (4, 8, 5000, 9),      # small-row kernel, nine splits merged by the combine
    (8, 16, 3000, 0),     # 128-row kernel
    (8, 16, 20000, 40),   # 128-row kernel, forty splits
])
def test_constant_column(H, T, prefix, nsplit):
    """Softmax weights sum to one, so a feature that is the same in every KV row
    comes out as exactly that value, whatever the splits and their merge."""
    wl = small(H=H, T=T, prefixes=[prefix], seed=9)
    for f, v in ((100, 0.375), (511, -3.0e-3), (7, 1.5e4)):
        wl.kv_pool[:, f] = inputs.f32_to_bf16_bits(np.array([v], np.float32))[0]
    got = run_gpu(wl, nsplit)
    for f, v in ((100, 0.375), (511, -3.0e-3), (7, 1.5e4)):
        want = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.array([v], np.float32)))[0]
        assert np.all(got[..., f] == want), (f, np.unique(got[..., f]))


def test_slot_permutation_bitwise():
    wl = small(B=2, H=8, T=8, prefixes=[900, 300], pool=4096, seed=12)
    got = run_gpu(wl)
    rng = np.random.default_rng(1)
    pi = rng.permutation(wl.pool_slots)
    pool = np.empty_like(wl.kv_pool)
    pool[pi] = wl.kv_pool
    wl.kv_pool = pool
    wl.slot_idx = pi[wl.slot_idx].astype(np.int32)
    assert np.array_equal(run_gpu(wl), got)


def test_head_subset_bitwise():
    wl64 = small(H=64, T=8, prefixes=[2000], seed=13)
    got64 = run_gpu(wl64, nsplit=4)
    wl8 = small(H=64, T=8, prefixes=[2000], seed=13)
    wl8.H = 8
    wl8.q = np.ascontiguousarray(wl64.q[:, :, :8])
    got8 = run_gpu(wl8, nsplit=4)
    assert np.array_equal(got8, got64[:, :, :8])


def test_deterministic():
    wl = inputs.config("c2_tp_share")
    dev = to_device(wl)
    a = run_gpu(wl, dev=dev)
    b = run_gpu(wl, dev=dev)
    assert np.array_equal(a, b)


def test_graph_capture_replay():
    """The call records into a HIP graph; replays match eager, with inputs changed between."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = small(B=2, H=8, T=16, prefixes=[3000, 1200], seed=14)
    dev = to_device(wl)
    op = mtv.VerifyAttention(params_of(wl))
    out = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.bfloat16, device="cuda")
    op(**dev, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        op(**dev, out=out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(**dev, out=out)
    q0 = dev["q"].clone()
    for rep in range(4):
        out.zero_()
        if rep % 2:
            dev["q"].copy_(torch.flip(q0, dims=[1]))
        else:
            dev["q"].copy_(q0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if rep % 2:
            ref = torch.empty_like(out)
            op(**dev, out=ref)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), rep
        else:
            assert torch.equal(out, eager), rep


def test_stage_entry_points_match_full_call():
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = small(B=2, H=8, T=8, prefixes=[1500, 700], seed=15)
    dev = to_device(wl)
    prm = params_of(wl)
    op = mtv.VerifyAttention(prm)
    full = op(**dev)
    out = torch.empty_like(full)
    mtv.verify_attn_partial(dev["q"], dev["kv_pool"], dev["slot_idx"], dev["seq_lens"],
                            dev["tree_parent"], op.workspace, prm)
    mtv.verify_attn_combine(dev["seq_lens"], out, op.workspace, prm)
    torch.cuda.synchronize()
    assert torch.equal(out, full)


def test_host_errors_raise_without_launch():
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = small(seed=16)
    dev = to_device(wl)
    prm = params_of(wl)
    ws = torch.empty(mtv.verify_attn_workspace_size(prm) - 16, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 8, 8, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mtv.VerifyAttnError) as e:
        mtv.verify_attn(**dev, out=out, workspace=ws, params=prm)
    assert e.value.status == -5


def test_binding_refuses_tensors_smaller_than_params():
    # the kernels index by the params' sizes: the binding checks the tensors hold them
    import torch
    import mla_tree_verify_latent_amd as mtv
    wl = small(seed=17)
    dev = to_device(wl)
    prm = params_of(wl)
    ws = torch.empty(mtv.verify_attn_workspace_size(prm), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.B, wl.T, wl.H, 512), dtype=torch.bfloat16, device="cuda")
    def with_(**kw):
        p = mtv.make_params(num_seqs=wl.B, num_heads=wl.H, tree_size=wl.T, max_seq_len=wl.max_seq_len,
                            total_kv=wl.total_kv, pool_slots=wl.pool_slots, sm_scale=wl.sm_scale)
        for k, v in kw.items():
            setattr(p, k, v)
        return p
    for p in (with_(pool_slots=wl.pool_slots + 1), with_(total_kv=wl.total_kv + 1),
              with_(num_heads=wl.H * 2), with_(tree_size=wl.T - 1), with_(num_seqs=wl.B + 1)):
        with pytest.raises(ValueError):
            mtv.verify_attn(**dev, out=out, workspace=ws, params=p)
        with pytest.raises(ValueError):
            mtv.verify_attn_partial(**dev, workspace=ws, params=p)
    with pytest.raises(ValueError):
        mtv.verify_attn_combine(dev["seq_lens"], out[:, :-1], ws, prm)
    with pytest.raises(ValueError):
        mtv.verify_attn_combine(dev["seq_lens"], out.float(), ws, prm)
    with pytest.raises(ValueError):
        mtv.verify_attn_debug_validate(dev["slot_idx"][:-1], dev["seq_lens"], dev["tree_parent"], prm)
    with pytest.raises(ValueError):
        mtv.verify_attn_debug_validate(dev["slot_idx"], dev["seq_lens"], dev["tree_parent"], prm,
                                       flags=torch.zeros(1, dtype=torch.float32, device="cuda"))
    # the matching call still runs
    mtv.verify_attn(**dev, out=out, workspace=ws, params=prm)
    torch.cuda.synchronize()
