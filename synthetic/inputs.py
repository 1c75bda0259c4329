"""Seeded synthetic inputs for MLA tree-verify attention.

This module only draws and lays out inputs; it computes nothing of the attention
itself. Both the HIP path (through its tests and benchmark) and the CPU oracle
consume what it returns.

Shapes follow the workloads the pages describe: a latent KV pool of bf16 rows of
576 values (512 latent + 64 rope; V is the first 512), scattered page_size=1
placement of each sequence's rows ("The Milestone Commit", Context: page_size=1
scattered access), a draft tree of T nodes per sequence whose KV rows follow the
prefix in the same slot list ("The Checkpoint Report", Mistakes: prefix slots,
then the draft tokens, mask stride prefix + q_len), and query rows [B, T, H, 576].

Draw order for one workload (one ``numpy.random.SeedSequence(seed)`` spawned into
four independent streams, used in this order):
  1. pool values ~ N(0, 1) * 0.1 for every pool row,
  2. the slot permutation,
  3. the draft trees (node i's parent uniform in [-1, i-1], redrawn while a
     depth cap is exceeded),
  4. q ~ N(0, 1), shape [B, T, H, 576].
Values are drawn in float32 and rounded to nearest-even bfloat16 (torch's CPU
conversion). bf16 arrays are returned as their raw uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

KV_DIM = 576
V_DIM = 512
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_tree(rng: np.random.Generator, T: int, max_depth: Optional[int] = None) -> np.ndarray:
    """Parent pointers of a random draft tree: parent[i] uniform in [-1, i-1].

    -1 means the node hangs directly off the prefix. With ``max_depth`` the draw
    for node i is repeated until its depth (0 for a root) is <= max_depth.
    """
    parent = np.empty(T, dtype=np.int32)
    depth = np.empty(T, dtype=np.int64)
    for i in range(T):
        while True:
            p = int(rng.integers(-1, i)) if i > 0 else -1
            d = 0 if p < 0 else int(depth[p]) + 1
            if max_depth is None or d <= max_depth:
                break
        parent[i] = p
        depth[i] = d
    return parent


def chain_tree(T: int) -> np.ndarray:
    """Every node's parent is the node before it (a single draft sequence)."""
    return np.arange(-1, T - 1, dtype=np.int32)


def flat_tree(T: int) -> np.ndarray:
    """Depth-0 tree: every node hangs directly off the prefix."""
    return np.full(T, -1, dtype=np.int32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    T: int
    prefixes: list
    pool_slots: int
    q: np.ndarray            # uint16 [B, T, H, 576] (bf16 bits), or float32 values
    kv_pool: np.ndarray      # uint16 [pool_slots, 576] (bf16 bits), or float32 values
    slot_idx: np.ndarray     # int32 [sum_b (P_b + T)]
    seq_lens: np.ndarray     # int32 [B] = P_b + T
    tree_parent: np.ndarray  # int32 [B, T]
    sm_scale: float = DEFAULT_SCALE
    page_size: int = 1
    seed: int = 0

    @property
    def M(self) -> int:
        return self.H * self.T

    @property
    def total_kv(self) -> int:
        return int(self.slot_idx.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def f32(self) -> bool:
        """True for fp32 q / kv_pool (values), False for bf16 (bit patterns)."""
        return self.q.dtype == np.float32

    def kv_bytes(self) -> int:
        """Bytes of KV rows one call touches (each referenced row once)."""
        return self.total_kv * KV_DIM * self.kv_pool.itemsize


def make_workload(
    name: str,
    *,
    B: int,
    H: int,
    T: int,
    prefixes: Sequence[int],
    pool_slots: int,
    seed: int,
    max_depth: Optional[int] = None,
    tree: str = "random",
    q_std: float = 1.0,
    kv_std: float = 0.1,
    sm_scale: float = DEFAULT_SCALE,
    layout: str = "scattered",
    dtype: str = "bf16",
) -> Workload:
    """Build one seeded workload.

    ``tree``: "random" (uniform parents, optional depth cap), "chain" or "flat".
    ``layout``: "scattered" (page_size=1, one seeded permutation of all pool
    slots, sequences take consecutive slices of it: prefix rows then tree rows),
    "contiguous" (the same row values moved so that the slot list of all
    sequences is 0, 1, 2, ...; page_size=64), or "paged64" (the same row values
    moved so that every run of 64 consecutive slot-list entries fills one page
    of 64 consecutive slots, the pages in seeded random order over the pool;
    page_size=64).
    ``dtype``: "bf16" (values rounded to nearest even, stored as bit patterns)
    or "f32" (the same draws kept as binary32 values).
    """
    prefixes = [int(p) for p in prefixes]
    assert len(prefixes) == B and T >= 1
    lens = [p + T for p in prefixes]
    total = sum(lens)
    assert total <= pool_slots, "pool too small for prefixes + trees"
    ss = np.random.SeedSequence(seed)
    s_pool, s_perm, s_tree, s_q = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]

    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    pool32 = s_pool.standard_normal((pool_slots, KV_DIM), dtype=np.float32)
    pool32 *= np.float32(kv_std)
    kv_pool = pool32 if dtype == "f32" else f32_to_bf16_bits(pool32)
    del pool32

    perm = s_perm.permutation(pool_slots).astype(np.int64)
    slot_idx = perm[:total].astype(np.int32)

    parents = []
    for _ in range(B):
        if tree == "random":
            parents.append(random_tree(s_tree, T, max_depth))
        elif tree == "chain":
            parents.append(chain_tree(T))
        elif tree == "flat":
            parents.append(flat_tree(T))
        else:
            raise ValueError(tree)
    tree_parent = np.stack(parents).astype(np.int32)

    q32 = s_q.standard_normal((B, T, H, KV_DIM), dtype=np.float32)
    if q_std != 1.0:
        q32 *= np.float32(q_std)
    q = q32 if dtype == "f32" else f32_to_bf16_bits(q32)

    page_size = 1
    if layout == "contiguous":
        # Same values, defragmented: logical row i of the slot list moves to slot i.
        rest = perm[total:]
        order = np.concatenate([slot_idx.astype(np.int64), rest])
        kv_pool = np.ascontiguousarray(kv_pool[order])
        slot_idx = np.arange(total, dtype=np.int32)
        page_size = 64
    elif layout == "paged64":
        # Logical row i of the slot list goes to slot 64 * page[i // 64] + i % 64.
        n_pages = pool_slots // 64
        assert -(-total // 64) <= n_pages, "pool too small for 64-row pages"
        page = np.random.Generator(np.random.PCG64(seed + 1)).permutation(n_pages)
        i = np.arange(total, dtype=np.int64)
        new_slot = 64 * page[i // 64] + i % 64
        moved = np.zeros(pool_slots, dtype=bool)
        moved[new_slot] = True
        rest_slots = np.flatnonzero(~moved)
        rest_rows = perm[total:][:rest_slots.size]
        pool = np.empty_like(kv_pool)
        pool[new_slot] = kv_pool[slot_idx]
        pool[rest_slots] = kv_pool[rest_rows]
        kv_pool = pool
        slot_idx = new_slot.astype(np.int32)
        page_size = 64
    elif layout != "scattered":
        raise ValueError(layout)

    return Workload(
        name=name, B=B, H=H, T=T, prefixes=prefixes, pool_slots=pool_slots,
        q=q, kv_pool=kv_pool, slot_idx=slot_idx,
        seq_lens=np.asarray(lens, dtype=np.int32), tree_parent=tree_parent,
        sm_scale=sm_scale, page_size=page_size, seed=seed,
    )


# The named workloads: the five configurations the benchmark is specified on
# (tiny smoke case, TP-share decode verify, full-head verify, long-context
# verify in two layouts, ragged batch) plus two extra points at 65k context
# (the production H=8, T=9 shape also in two more layouts).
CONFIGS = {
    "c1_tiny": dict(B=1, H=8, T=8, prefixes=[256], pool_slots=1024, seed=1000),
    "c2_tp_share": dict(B=1, H=8, T=32, prefixes=[4096], pool_slots=65536, seed=2000, max_depth=8),
    "c3_full_head": dict(B=1, H=64, T=32, prefixes=[16384], pool_slots=131072, seed=3000),
    "c4a_long_scattered": dict(B=1, H=8, T=64, prefixes=[65536], pool_slots=131072, seed=4000),
    "c4b_long_contiguous": dict(B=1, H=8, T=64, prefixes=[65536], pool_slots=131072, seed=4000,
                                layout="contiguous"),
    "c5_ragged": dict(B=4, H=64, T=64, prefixes=[4096, 23552, 65536, 200704], pool_slots=300000,
                      seed=5000),
    "e1_h64_65k": dict(B=1, H=64, T=64, prefixes=[65536], pool_slots=131072, seed=6000),
    "e2_h8_t9_65k": dict(B=1, H=8, T=9, prefixes=[65536], pool_slots=131072, seed=7000),
    # the same production shape with its KV rows defragmented, and in 64-row pages
    "e2_h8_t9_65k_contiguous": dict(B=1, H=8, T=9, prefixes=[65536], pool_slots=131072, seed=7000,
                                    layout="contiguous"),
    "e2_h8_t9_65k_paged64": dict(B=1, H=8, T=9, prefixes=[65536], pool_slots=131072, seed=7000,
                                 layout="paged64"),
    # fp32 inputs (binary32 q and KV pool) at the 64k-token H=8 shape
    "f4_long_f32": dict(B=1, H=8, T=64, prefixes=[65536], pool_slots=131072, seed=4000,
                        dtype="f32"),
}


def config(name: str) -> Workload:
    return make_workload(name, **CONFIGS[name])
