"""Pins for the CPU oracle: facts fixed by the mathematics, not by the oracle.

Each ``pin_*`` takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with the fact it checks. The same
functions are run against deliberately broken copies of the oracle
(test_oracle_mutations.py) to show that a plausible mistake fails at least one.

The method (verify attention of a draft tree against the full latent KV cache,
prefix slots first and draft-token slots after them, mask stride prefix +
q_len) is described in "The Milestone Commit" (Input Knowledge) and "The
Checkpoint Report" (Mistakes and Incorrect Assumptions).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from synthetic import inputs

KV, DV = 576, 512


def _f64(x):
    """fp64 values of bf16 bit patterns (uint16) or of binary32 values."""
    if x.dtype == np.float32:
        return x.astype(np.float64)
    return inputs.bf16_bits_to_f32(x).astype(np.float64)


def ancestor_closure(parent: np.ndarray) -> np.ndarray:
    """Boolean [T, T] matrix R with R[t, u] = u is t or an ancestor of t.

    Computed as the reflexive-transitive closure of the child->parent relation by
    repeated boolean squaring, independently of any parent-chain walk.
    """
    T = parent.shape[0]
    A = np.zeros((T, T), dtype=bool)
    for t in range(T):
        if parent[t] >= 0:
            A[t, parent[t]] = True
    R = A | np.eye(T, dtype=bool)
    for _ in range(max(1, int(math.ceil(math.log2(T + 1))))):
        R = R | ((R.astype(np.int64) @ R.astype(np.int64)) > 0)
    return R


def library_attention(wl) -> np.ndarray:
    """Reference via torch.nn.functional.scaled_dot_product_attention (fp64, CPU).

    For each sequence: dense K = gathered rows [N, 576], V = K[:, :512], and an
    explicit boolean mask [T, N] = [all prefix columns | ancestor closure].
    """
    out = np.empty((wl.B, wl.T, wl.H, DV), dtype=np.float64)
    seg = 0
    for b in range(wl.B):
        N = int(wl.seq_lens[b])
        P = N - wl.T
        rows = wl.slot_idx[seg:seg + N]
        K = torch.from_numpy(_f64(wl.kv_pool[rows]))          # [N, 576]
        V = K[:, :DV].contiguous()
        mask = np.zeros((wl.T, N), dtype=bool)
        mask[:, :P] = True
        mask[:, P:] = ancestor_closure(wl.tree_parent[b])
        Q = torch.from_numpy(_f64(wl.q[b])).permute(1, 0, 2).contiguous()  # [H, T, 576]
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K.expand(wl.H, N, KV), V.expand(wl.H, N, DV),
            attn_mask=torch.from_numpy(mask), scale=wl.sm_scale)
        out[b] = o.permute(1, 0, 2).numpy()
        seg += N
    return out


def plain_decode_attention(qv: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Unmasked single-query attention: softmax(K q * scale) weighted mean of K[:, :512]."""
    s = (K @ qv) * scale
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ K[:, :DV]


def tiny(B=1, H=2, T=4, prefixes=(5,), pool=None, seed=1, tree="random", **kw):
    prefixes = list(prefixes)
    if pool is None:
        pool = sum(prefixes) + B * T + 7
    return inputs.make_workload("tiny", B=B, H=H, T=T, prefixes=prefixes, pool_slots=pool,
                                seed=seed, tree=tree, **kw)


def numpy_bruteforce(wl) -> np.ndarray:
    """Dense fp64 brute force in NumPy, independent of the oracle and of torch:
    per sequence, gather K [N, 576] through the slot list, build the mask matrix
    M [T, N] (stride N = prefix + T: every prefix column, then the ancestor-or-self
    closure of the tree), and compute softmax(Q K^T * scale + log M) V with
    V = K[:, :512]; log 0 = -inf removes the masked keys."""
    out = np.empty((wl.B, wl.T, wl.H, DV), dtype=np.float64)
    seg = 0
    for b in range(wl.B):
        N = int(wl.seq_lens[b])
        P = N - wl.T
        K = _f64(wl.kv_pool[wl.slot_idx[seg:seg + N]])
        M = np.zeros((wl.T, N), dtype=bool)
        M[:, :P] = True
        M[:, P:] = ancestor_closure(wl.tree_parent[b])
        with np.errstate(divide="ignore"):
            log_m = np.log(M.astype(np.float64))                      # 0 or -inf
        S = np.einsum("thd,nd->thn", _f64(wl.q[b]), K) * wl.sm_scale + log_m[:, None, :]
        S -= S.max(axis=2, keepdims=True)
        W = np.exp(S)
        W /= W.sum(axis=2, keepdims=True)
        out[b] = np.einsum("thn,nv->thv", W, K[:, :DV])
        seg += N
    return out


def run(orc, wl):
    return orc.run(wl)


# ---------------------------------------------------------------- pins

def pin_library_attention(orc):
    """Random small shapes: oracle == library attention with an explicit mask."""
    cases = [
        dict(B=1, H=1, T=1, prefixes=[0]), dict(B=1, H=2, T=1, prefixes=[1]),
        dict(B=1, H=2, T=3, prefixes=[5]), dict(B=1, H=8, T=8, prefixes=[17]),
        dict(B=2, H=2, T=8, prefixes=[0, 64]), dict(B=3, H=1, T=3, prefixes=[1, 5, 17]),
        dict(B=1, H=2, T=64, prefixes=[64]), dict(B=2, H=8, T=2, prefixes=[17, 5]),
    ]
    for i, c in enumerate(cases):
        wl = tiny(seed=100 + i, **c)
        got = run(orc, wl)
        ref = library_attention(wl)
        err = np.abs(got - ref).max()
        assert err <= 1e-13, f"case {c}: max |oracle - library| = {err}"


def pin_flat_tree_is_decode(orc):
    """Depth-0 tree: each node is plain decode attention over [prefix; own row]."""
    wl = tiny(B=1, H=3, T=6, prefixes=[23], seed=7, tree="flat")
    got = run(orc, wl)
    P = 23
    rows = wl.slot_idx
    K_all = _f64(wl.kv_pool[rows])
    for t in range(wl.T):
        K = np.concatenate([K_all[:P], K_all[P + t:P + t + 1]])
        for h in range(wl.H):
            ref = plain_decode_attention(_f64(wl.q[0, t, h]), K, wl.sm_scale)
            assert np.abs(got[0, t, h] - ref).max() <= 1e-13, (t, h)


def pin_chain_tree_is_causal(orc):
    """Chain tree: node t sees prefix + nodes 0..t, i.e. causal attention."""
    wl = tiny(B=1, H=2, T=7, prefixes=[11], seed=8, tree="chain")
    got = run(orc, wl)
    P = 11
    K_all = _f64(wl.kv_pool[wl.slot_idx])
    for t in range(wl.T):
        for h in range(wl.H):
            ref = plain_decode_attention(_f64(wl.q[0, t, h]), K_all[:P + t + 1], wl.sm_scale)
            assert np.abs(got[0, t, h] - ref).max() <= 1e-13, (t, h)


def pin_zero_query_is_mean(orc):
    """q = 0: all visible scores equal, so out = mean of the visible V rows."""
    wl = tiny(B=2, H=2, T=9, prefixes=[6, 0], seed=9)
    wl.q[:] = 0
    got = run(orc, wl)
    seg = 0
    for b in range(wl.B):
        N = int(wl.seq_lens[b]); P = N - wl.T
        V = _f64(wl.kv_pool[wl.slot_idx[seg:seg + N]])[:, :DV]
        R = ancestor_closure(wl.tree_parent[b])
        for t in range(wl.T):
            vis = np.concatenate([np.ones(P, bool), R[t]])
            assert vis.sum() == P + 1 + _depth(wl.tree_parent[b], t)
            ref = V[vis].mean(axis=0)
            for h in range(wl.H):
                assert np.abs(got[b, t, h] - ref).max() <= 1e-14, (b, t, h)
        seg += N


def _depth(parent, t):
    d = 0
    while parent[t] >= 0:
        t = parent[t]
        d += 1
    return d


def pin_single_key(orc):
    """P = 0, T = 1: the only visible key is the node's own row; out = its V exactly."""
    wl = tiny(B=2, H=4, T=1, prefixes=[0, 0], seed=10)
    got = run(orc, wl)
    for b in range(2):
        v = _f64(wl.kv_pool[wl.slot_idx[b]])[:DV]
        for h in range(4):
            assert np.array_equal(got[b, 0, h], v), (b, h)


def pin_weights(orc):
    """Softmax weights: >= 0, sum to 1, exactly 0 outside the visible set, equal to
    the library softmax of the masked scores."""
    wl = tiny(B=2, H=2, T=8, prefixes=[13, 4], seed=11)
    seg = 0
    for b in range(wl.B):
        N = int(wl.seq_lens[b]); P = N - wl.T
        K = _f64(wl.kv_pool[wl.slot_idx[seg:seg + N]])
        R = ancestor_closure(wl.tree_parent[b])
        for t in range(wl.T):
            vis = np.concatenate([np.ones(P, bool), R[t]])
            for h in range(wl.H):
                w, o = orc.row_weights(wl.q, wl.kv_pool, wl.slot_idx, wl.seq_lens,
                                       wl.tree_parent, wl.sm_scale, b, t, h)
                assert (w >= 0).all()
                assert abs(w.sum() - 1.0) <= 1e-12
                assert (w[~vis] == 0).all()
                s = torch.from_numpy(K @ _f64(wl.q[b, t, h]) * wl.sm_scale)
                s[torch.from_numpy(~vis)] = -math.inf
                ref = torch.softmax(s, dim=0).numpy()
                assert np.abs(w - ref).max() <= 1e-14
                assert np.abs(o - ref @ K[:, :DV]).max() <= 1e-13
        seg += N


def pin_slot_permutation(orc):
    """Moving pool rows and remapping slot_idx leaves the output bit-identical."""
    wl = tiny(B=2, H=2, T=5, prefixes=[9, 3], seed=12, pool=64)
    got = run(orc, wl)
    rng = np.random.default_rng(5)
    pi = rng.permutation(wl.pool_slots)
    new_pool = np.empty_like(wl.kv_pool)
    new_pool[pi] = wl.kv_pool
    wl.kv_pool = new_pool
    wl.slot_idx = pi[wl.slot_idx].astype(np.int32)
    assert np.array_equal(run(orc, wl), got)


def pin_tree_relabel(orc):
    """Renumbering tree nodes in another topological order permutes the outputs."""
    wl = tiny(B=1, H=2, T=10, prefixes=[7], seed=13)
    got = run(orc, wl)
    parent = wl.tree_parent[0]
    # A different topological order: repeatedly take the highest-numbered ready node.
    order, done = [], set()
    while len(order) < wl.T:
        ready = [u for u in range(wl.T) if u not in done and (parent[u] < 0 or parent[u] in done)]
        u = max(ready)
        order.append(u)
        done.add(u)
    sigma = np.empty(wl.T, dtype=np.int64)
    sigma[order] = np.arange(wl.T)            # old label -> new label
    new_parent = np.empty(wl.T, dtype=np.int32)
    for u in range(wl.T):
        new_parent[sigma[u]] = -1 if parent[u] < 0 else sigma[parent[u]]
    P = 7
    tree_slots = wl.slot_idx[P:].copy()
    new_slots = wl.slot_idx.copy()
    new_slots[P + sigma] = tree_slots
    new_q = np.empty_like(wl.q)
    new_q[0, sigma] = wl.q[0]
    wl.tree_parent = new_parent[None]
    wl.slot_idx = new_slots
    wl.q = new_q
    got2 = run(orc, wl)
    assert np.abs(got2[0, sigma] - got[0]).max() <= 1e-14


def pin_head_subset(orc):
    """Heads are independent: H=2 output equals heads 0..1 of an H=5 run with the same q rows."""
    wl5 = tiny(B=2, H=5, T=4, prefixes=[6, 2], seed=14)
    got5 = run(orc, wl5)
    wl2 = tiny(B=2, H=5, T=4, prefixes=[6, 2], seed=14)
    wl2.H = 2
    wl2.q = np.ascontiguousarray(wl5.q[:, :, :2])
    assert np.array_equal(run(orc, wl2), got5[:, :, :2])


def pin_sequences_independent(orc):
    """Batching is segment-wise: each sequence's rows equal a run of that sequence alone."""
    wl = tiny(B=3, H=2, T=4, prefixes=[5, 0, 12], seed=15)
    got = run(orc, wl)
    seg = 0
    for b in range(3):
        N = int(wl.seq_lens[b])
        one = tiny(B=1, H=2, T=4, prefixes=[N - 4], seed=15)
        one.kv_pool = wl.kv_pool
        one.pool_slots = wl.pool_slots
        one.slot_idx = wl.slot_idx[seg:seg + N].copy()
        one.q = np.ascontiguousarray(wl.q[b:b + 1])
        one.tree_parent = np.ascontiguousarray(wl.tree_parent[b:b + 1])
        assert np.array_equal(run(orc, one)[0], got[b]), b
        seg += N


def pin_constant_column(orc):
    """If column d of every row is the constant c, then out[..., d] == c (weights sum to 1)."""
    wl = tiny(B=1, H=3, T=6, prefixes=[20], seed=16)
    c = inputs.f32_to_bf16_bits(np.array([0.375], np.float32))[0]
    for d in (0, 200, 511):
        wl.kv_pool[:, d] = c
    got = run(orc, wl)
    for d in (0, 200, 511):
        assert np.abs(got[..., d] - 0.375).max() <= 1e-15, d


def pin_scale_linear(orc):
    """Scaling q by 2 (exact in bf16) equals doubling sm_scale, bit for bit."""
    wl = tiny(B=1, H=2, T=5, prefixes=[8], seed=17)
    a = orc.verify_attn(wl.q, wl.kv_pool, wl.slot_idx, wl.seq_lens, wl.tree_parent,
                        2.0 * wl.sm_scale)
    q2 = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(wl.q) * 2.0)
    b = orc.verify_attn(q2, wl.kv_pool, wl.slot_idx, wl.seq_lens, wl.tree_parent, wl.sm_scale)
    assert np.array_equal(a, b)


def pin_worked_example(orc):
    """Hand-built example with a closed form (tests/golden/worked_example.txt).

    One head, P = 2 prefix rows, T = 2 nodes (node 1's parent is node 0). Only
    columns 0 (latent), 1 (latent) and 512 (rope) are non-zero. Node 0 sees keys
    {p0, p1, n0}; node 1 sees {p0, p1, n0, n1}. With q = (x at col 0, y at col 512),
    s_j = scale * (x * a_j + y * r_j), out[0] = sum w_j a_j, out[1] = sum w_j c_j,
    and every other output column is 0.
    """
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")
    spec = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=")
            spec[k.strip()] = [float(x) for x in v.split(",")]
    a, c, r = spec["a"], spec["c"], spec["r"]
    x, y, scale = spec["x"][0], spec["y"][0], spec["scale"][0]
    kv = np.zeros((4, KV), np.float32)
    kv[:, 0], kv[:, 1], kv[:, 512] = a, c, r
    q = np.zeros((1, 2, 1, KV), np.float32)
    q[..., 0], q[..., 512] = x, y
    kvb, qb = inputs.f32_to_bf16_bits(kv), inputs.f32_to_bf16_bits(q)
    assert np.array_equal(inputs.bf16_bits_to_f32(kvb), kv), "fixture values must be exact in bf16"
    out = orc.verify_attn(qb, kvb, np.array([3, 1, 0, 2], np.int32), np.array([4], np.int32),
                          np.array([[-1, 0]], np.int32), scale)
    # slot list is (p0 -> row 3, p1 -> row 1, n0 -> row 0, n1 -> row 2)
    rows = [3, 1, 0, 2]
    for t, visible in ((0, [0, 1, 2]), (1, [0, 1, 2, 3])):
        s = [scale * (x * a[rows[j]] + y * r[rows[j]]) for j in visible]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        w = [v / sum(e) for v in e]
        o0 = sum(wj * a[rows[j]] for wj, j in zip(w, visible))
        o1 = sum(wj * c[rows[j]] for wj, j in zip(w, visible))
        assert abs(out[0, t, 0, 0] - o0) <= 1e-15 and abs(out[0, t, 0, 1] - o1) <= 1e-15, t
        assert not np.any(out[0, t, 0, 2:]), t


def pin_f32_library_attention(orc):
    """fp32 inputs (the binary32 entry points): oracle == library attention with
    an explicit mask, on the same draws kept unrounded."""
    cases = [
        dict(B=1, H=1, T=1, prefixes=[0]), dict(B=1, H=2, T=3, prefixes=[5]),
        dict(B=2, H=2, T=8, prefixes=[0, 64]), dict(B=1, H=2, T=64, prefixes=[64]),
        dict(B=3, H=1, T=3, prefixes=[1, 5, 17]),
    ]
    for i, c in enumerate(cases):
        wl = tiny(seed=300 + i, dtype="f32", **c)
        assert wl.q.dtype == np.float32
        got = run(orc, wl)
        ref = library_attention(wl)
        err = np.abs(got - ref).max()
        assert err <= 1e-13, f"f32 case {c}: max |oracle - library| = {err}"


def pin_f32_on_bf16_values(orc):
    """binary32 arrays that hold bf16 values give exactly the bf16 result."""
    import dataclasses
    wl = tiny(B=2, H=2, T=8, prefixes=[17, 3], seed=7)
    wl32 = dataclasses.replace(wl, q=inputs.bf16_bits_to_f32(wl.q),
                               kv_pool=inputs.bf16_bits_to_f32(wl.kv_pool))
    assert wl32.q.dtype == np.float32
    assert np.array_equal(run(orc, wl), run(orc, wl32))


def pin_bruteforce_grid(orc):
    """Oracle == NumPy dense brute force with an explicit log-mask, over every
    combination of prefix P in {0, 1, 5, 17, 64}, tree size T in {1, 2, 3, 8, 64}
    and heads H in {1, 2, 8} (random trees, two seeds each, the second as one
    sequence of a two-sequence batch), and on the 1,024-slot, 256-token, H=8, T=8
    configuration itself."""
    n = 0
    for P in (0, 1, 5, 17, 64):
        for T in (1, 2, 3, 8, 64):
            for H in (1, 2, 8):
                for rep in range(2):
                    seed = 500 + 100 * rep + 10 * P + 3 * T + H
                    if rep == 0:
                        wl = tiny(B=1, H=H, T=T, prefixes=[P], seed=seed)
                    else:
                        wl = tiny(B=2, H=H, T=T, prefixes=[P, (P * 7 + 3) % 19], seed=seed)
                    err = np.abs(run(orc, wl) - numpy_bruteforce(wl)).max()
                    assert err <= 1e-12, f"P={P} T={T} H={H} rep={rep}: max |oracle - brute force| = {err}"
                    n += 1
    wl = inputs.config("c1_tiny")
    err = np.abs(run(orc, wl) - numpy_bruteforce(wl)).max()
    assert err <= 1e-12, f"c1_tiny: max |oracle - brute force| = {err}"
    assert n == 150


ALL_PINS = [
    pin_library_attention, pin_flat_tree_is_decode, pin_chain_tree_is_causal,
    pin_zero_query_is_mean, pin_single_key, pin_weights, pin_slot_permutation,
    pin_tree_relabel, pin_head_subset, pin_sequences_independent, pin_constant_column,
    pin_scale_linear, pin_worked_example, pin_f32_library_attention, pin_f32_on_bf16_values,
    pin_bruteforce_grid,
]
