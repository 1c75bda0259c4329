"""CPU oracle for MLA tree-verify attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP product path does not use it
and shares no code with it.

The oracle itself is ``verify_attn_oracle.c`` (plain C, fp64, OpenMP over
output rows); this module compiles it with gcc and calls it through ctypes.

Parity status of each oracle function (pins live in tests/test_oracle_pins.py):
  oracle_verify_attn / oracle_verify_attn_rows: pinned (library attention with
      an explicit mask, a NumPy dense brute force with a log-mask over 150
      random small shapes and the tiny configuration, closed forms, invariants,
      planted-mistake checks).
  oracle_verify_attn_f32 / oracle_verify_attn_rows_f32 (binary32 q and KV):
      pinned (library attention with an explicit mask on fp32 data; bit-equal
      to the bf16 entry points when the fp32 values are bf16 values).
  oracle_row_weights: pinned (weights sum to 1, zero outside the visible set,
      match the library routine's attention probabilities).
  append_kv (NumPy, below): pinned (re-appending a workload's own tree rows
      into a pool where they were cleared restores the pool exactly).
  compact_kv (NumPy, below): pinned (compacting the scattered long-context
      workload reproduces the generator's defragmented pool rows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "verify_attn_oracle.c")
LIB = os.path.join(HERE, "libverify_attn_oracle.so")

V_DIM = 512
ERRORS = {0: "ok", -1: "bad argument", -2: "bad tree_parent", -3: "slot index out of range",
          -4: "out of memory"}


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle C source into a shared library (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror",
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_verify_attn.argtypes = [i32, i32, i32, vp, vp, i64, vp, vp, vp, dbl, vp, i32]
        lib.oracle_verify_attn.restype = i32
        lib.oracle_verify_attn_rows.argtypes = [i32, i32, i32, vp, vp, i64, vp, vp, vp, dbl, i64, vp,
                                                vp, i32]
        lib.oracle_verify_attn_rows.restype = i32
        lib.oracle_row_weights.argtypes = [i32, i32, i32, vp, vp, i64, vp, vp, vp, dbl, i32, i32, i32,
                                           vp, vp]
        lib.oracle_row_weights.restype = i32
        lib.oracle_verify_attn_f32.argtypes = lib.oracle_verify_attn.argtypes
        lib.oracle_verify_attn_f32.restype = i32
        lib.oracle_verify_attn_rows_f32.argtypes = lib.oracle_verify_attn_rows.argtypes
        lib.oracle_verify_attn_rows_f32.restype = i32
        lib.oracle_num_threads.restype = i32
        self.lib = lib

    @staticmethod
    def _prep(q, kv_pool, slot_idx, seq_lens, tree_parent):
        # bf16 bit patterns (uint16), or binary32 values for the fp32 entry points
        dt = np.float32 if np.asarray(q).dtype == np.float32 else np.uint16
        q = np.ascontiguousarray(q, dtype=dt)
        kv_pool = np.ascontiguousarray(kv_pool, dtype=dt)
        slot_idx = np.ascontiguousarray(slot_idx, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        tree_parent = np.ascontiguousarray(tree_parent, dtype=np.int32)
        B, T, H, D = q.shape
        assert D == 576 and kv_pool.ndim == 2 and kv_pool.shape[1] == 576
        assert seq_lens.shape == (B,) and tree_parent.shape == (B, T)
        return q, kv_pool, slot_idx, seq_lens, tree_parent, B, T, H

    @staticmethod
    def _check(rc: int):
        if rc != 0:
            raise ValueError(f"oracle: {ERRORS.get(rc, rc)}")

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def verify_attn(self, q, kv_pool, slot_idx, seq_lens, tree_parent, sm_scale: float,
                    nthreads: int = 0) -> np.ndarray:
        """Full output, fp64 [B, T, H, 512]."""
        q, kv_pool, slot_idx, seq_lens, tree_parent, B, T, H = self._prep(
            q, kv_pool, slot_idx, seq_lens, tree_parent)
        out = np.empty((B, T, H, V_DIM), dtype=np.float64)
        fn = self.lib.oracle_verify_attn_f32 if q.dtype == np.float32 else self.lib.oracle_verify_attn
        rc = fn(B, H, T, q.ctypes.data, kv_pool.ctypes.data,
                                         kv_pool.shape[0], slot_idx.ctypes.data,
                                         seq_lens.ctypes.data, tree_parent.ctypes.data,
                                         float(sm_scale), out.ctypes.data, int(nthreads))
        self._check(rc)
        return out

    def verify_attn_rows(self, q, kv_pool, slot_idx, seq_lens, tree_parent, sm_scale: float,
                         rows_bth, nthreads: int = 0) -> np.ndarray:
        """Selected output rows; rows_bth is int [n, 3] of (b, t, h). Returns fp64 [n, 512]."""
        q, kv_pool, slot_idx, seq_lens, tree_parent, B, T, H = self._prep(
            q, kv_pool, slot_idx, seq_lens, tree_parent)
        rows = np.ascontiguousarray(rows_bth, dtype=np.int32).reshape(-1, 3)
        out = np.empty((rows.shape[0], V_DIM), dtype=np.float64)
        fn = self.lib.oracle_verify_attn_rows_f32 if q.dtype == np.float32 else self.lib.oracle_verify_attn_rows
        rc = fn(B, H, T, q.ctypes.data, kv_pool.ctypes.data,
                                              kv_pool.shape[0], slot_idx.ctypes.data,
                                              seq_lens.ctypes.data, tree_parent.ctypes.data,
                                              float(sm_scale), rows.shape[0], rows.ctypes.data,
                                              out.ctypes.data, int(nthreads))
        self._check(rc)
        return out

    def row_weights(self, q, kv_pool, slot_idx, seq_lens, tree_parent, sm_scale: float,
                    b: int, t: int, h: int):
        """(weights over the sequence's seq_lens[b] keys, output row) for one (b, t, h)."""
        q, kv_pool, slot_idx, seq_lens, tree_parent, B, T, H = self._prep(
            q, kv_pool, slot_idx, seq_lens, tree_parent)
        if q.dtype != np.uint16:
            raise ValueError("row_weights takes bf16 inputs")
        w = np.empty(int(seq_lens[b]), dtype=np.float64)
        o = np.empty(V_DIM, dtype=np.float64)
        rc = self.lib.oracle_row_weights(B, H, T, q.ctypes.data, kv_pool.ctypes.data,
                                         kv_pool.shape[0], slot_idx.ctypes.data,
                                         seq_lens.ctypes.data, tree_parent.ctypes.data,
                                         float(sm_scale), int(b), int(t), int(h), w.ctypes.data,
                                         o.ctypes.data)
        self._check(rc)
        return w, o

    # Convenience wrappers taking a synthetic.inputs.Workload
    def run(self, wl, nthreads: int = 0) -> np.ndarray:
        return self.verify_attn(wl.q, wl.kv_pool, wl.slot_idx, wl.seq_lens, wl.tree_parent,
                                wl.sm_scale, nthreads)

    def run_rows(self, wl, rows_bth, nthreads: int = 0) -> np.ndarray:
        return self.verify_attn_rows(wl.q, wl.kv_pool, wl.slot_idx, wl.seq_lens, wl.tree_parent,
                                     wl.sm_scale, rows_bth, nthreads)


_default: Optional[Oracle] = None


def append_kv(kv_pool: np.ndarray, kv_new: np.ndarray, slot_idx: np.ndarray,
              seq_lens: np.ndarray) -> np.ndarray:
    """Draft-row KV append, written out: returns a copy of kv_pool ([slots, 576]
    bf16 bits) with row (b, t) of kv_new ([B, T, 576]) stored at the slot of
    tree node t of sequence b, slot_idx[seg_b + seq_lens[b] - T + t], where
    seg_b is the sum of the earlier sequences' lengths (the extend layout: a
    sequence's prefix slots, then its draft tokens' slots in node order).
    Slots outside the pool are skipped."""
    out = np.array(kv_pool, copy=True)
    B, T, _ = kv_new.shape
    seg = 0
    for b in range(B):
        n = int(seq_lens[b])
        for t in range(T):
            slot = int(slot_idx[seg + n - T + t])
            if 0 <= slot < out.shape[0]:
                out[slot] = kv_new[b, t]
        seg += n
    return out


def compact_kv(kv_pool: np.ndarray, slot_idx: np.ndarray) -> np.ndarray:
    """KV defragmentation, written out: row i of the result is pool row
    slot_idx[i] (a row of zeros for a slot outside the pool)."""
    out = np.zeros((slot_idx.shape[0], kv_pool.shape[1]), dtype=kv_pool.dtype)
    for i, slot in enumerate(slot_idx.tolist()):
        if 0 <= slot < kv_pool.shape[0]:
            out[i] = kv_pool[slot]
    return out


def load(path: Optional[str] = None) -> Oracle:
    """Load the oracle library, compiling it first if it is missing or stale."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default
