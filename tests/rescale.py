"""Inputs that make the online softmax rescale its running sums, and a host-side
count of where it does.

The partial kernels keep, per query row and split, a running reference maximum
of the base-2 scores (sm_scale * log2(e) * q.K) over the split's key tiles. It
is raised only when a tile's maximum exceeds it by more than 8; when a row that
already holds weights has its maximum raised, the kernel multiplies the row's
accumulated V sum by 2^(old - new) (the "online" part of the online softmax).
Scores drawn like the benchmark's inputs (q ~ N(0,1), K ~ N(0,1)*0.1) have a
base-2 spread of about 0.25, so the raise never happens there; the inputs
below make it happen, and `rescale_events` shows from the inputs alone how
often (it is told the split and tile lengths by the library's published plan).
"""
from __future__ import annotations

import numpy as np

from synthetic import inputs

LOG2E = 1.4426950408889634
RAISE_LOG2 = 8.0
ROPE = slice(512, 576)  # the 64 rope dimensions: part of the scores, not of V


def _widen(wl, a):
    return np.asarray(a, dtype=np.float32) if wl.f32 else inputs.bf16_bits_to_f32(a)


def _narrow(wl, x):
    x = np.asarray(x, dtype=np.float32)
    return x if wl.f32 else inputs.f32_to_bf16_bits(x)


def plant_score_ramp(wl, amplitude_log2: float, period: int, offset: int = 0, c: float = 1.0):
    """Add a sawtooth ramp to every sequence's scores, in place.

    The query's rope dimensions are set to c and the rope dimensions of the KV
    row at position j of a sequence get r_j added, so that every score of that
    key changes by -amplitude_log2 * (1 - ((j + offset) % period) / period) in
    base-2 units: from -amplitude up to 0 over each period. Within a period the
    scores climb steadily, so a split that spans part of it sees its running
    maximum overtaken again and again; the keys that dominate keep scores of
    the unramped size, and keys far below them (amplitude > 126) carry weights
    that underflow binary32."""
    wl.q[..., ROPE] = _narrow(wl, np.full(wl.q[..., ROPE].shape, c, np.float32))
    per_unit = wl.sm_scale * LOG2E * 64 * c  # base-2 score rise per unit added to each rope value
    seg = 0
    for b in range(wl.B):
        n = int(wl.seq_lens[b])
        slots = wl.slot_idx[seg:seg + n]
        frac = ((np.arange(n) + offset) % period) / period
        r = (amplitude_log2 * (frac - 1.0) / per_unit).astype(np.float32)
        rows = _widen(wl, wl.kv_pool[slots][:, ROPE]) + r[:, None]
        wl.kv_pool[slots[:, None], np.arange(512, 576)[None, :]] = _narrow(wl, rows)
        seg += n
    return wl


def underflowing_keys(wl, b=0):
    """Visible (row, key) pairs of sequence b whose exact softmax weight is below
    2^-126 of the row's largest (binary32 underflow)."""
    S = base2_scores(wl, b)
    return int(((S < S.max(axis=1, keepdims=True) - 126) & np.isfinite(S)).sum())


def visible_tree(parent):
    """vis[t, u]: node u is t or an ancestor of t (parent pointers, -1 = root)."""
    T = len(parent)
    vis = np.zeros((T, T), dtype=bool)
    for t in range(T):
        u = t
        while u >= 0:
            vis[t, u] = True
            u = int(parent[u])
    return vis


def base2_scores(wl, b):
    """sm_scale * log2(e) * q.K of sequence b, rows r = t*H + h, masked keys -inf
    (float32 [T*H, seq_len]; the row's visible set is the prefix plus the node's
    ancestors-or-self)."""
    seg = int(wl.seq_lens[:b].sum())
    n = int(wl.seq_lens[b])
    P = n - wl.T
    K = _widen(wl, wl.kv_pool[wl.slot_idx[seg:seg + n]])
    Q = _widen(wl, wl.q[b]).reshape(wl.T * wl.H, 576)
    S = (Q @ K.T) * np.float32(wl.sm_scale * LOG2E)
    vis = visible_tree(wl.tree_parent[b])
    node = np.arange(wl.T * wl.H) // wl.H
    S[:, P:] = np.where(vis[node], S[:, P:], -np.inf)
    return S


def rescale_events(wl, keys_per_split: int, keys_per_tile: int):
    """Count, over every sequence, split and query row, the tiles at which the
    running maximum of a row that already holds weights is raised (tile maximum
    above the running maximum + 8). Returns (events, splits with at least one,
    most events in one (row, split))."""
    events = splits_hit = most = 0
    for b in range(wl.B):
        S = base2_scores(wl, b)
        n = S.shape[1]
        for k0 in range(0, n, keys_per_split):
            k1 = min(k0 + keys_per_split, n)
            nt = -(-(k1 - k0) // keys_per_tile)
            pad = np.full((S.shape[0], nt * keys_per_tile), -np.inf, dtype=np.float32)
            pad[:, :k1 - k0] = S[:, k0:k1]
            tmax = pad.reshape(S.shape[0], nt, keys_per_tile).max(axis=2)
            m = np.full(S.shape[0], -np.inf, dtype=np.float32)
            count = np.zeros(S.shape[0], dtype=np.int64)
            for i in range(nt):
                raise_ = tmax[:, i] > m + RAISE_LOG2
                count += raise_ & np.isfinite(m)
                m = np.where(raise_, tmax[:, i], m)
            events += int(count.sum())
            splits_hit += int(count.sum() > 0)
            most = max(most, int(count.max()))
    return events, splits_hit, most
