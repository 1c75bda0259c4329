"""Shared test helpers: moving synthetic workloads to the device, the parity gate."""
from __future__ import annotations

import numpy as np

from synthetic import inputs


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits); tiny values use
    the smallest normal's spacing."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def parity_gate(got: np.ndarray, ref: np.ndarray, ulps: float = 2.0):
    """Row-wise gate: max_d |got - ref| <= ulps * ulp_bf16(max_d |ref|) for every
    output row (last axis = the 512 features). Returns (ok, worst ratio, row index)."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, 512)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 512)
    err = np.abs(got - ref).max(axis=1)
    tol = ulps * bf16_ulp(np.abs(ref).max(axis=1))
    ratio = err / tol
    worst = int(np.argmax(ratio))
    return bool((ratio <= 1.0).all()), float(ratio[worst] * ulps), worst


from synthetic.device import params_of, to_device  # noqa: E402,F401


def run_gpu(wl, nsplit: int = 0, dev=None) -> np.ndarray:
    """One verify_attn call; returns the bf16 output widened to float32 on the host."""
    import torch
    import mla_tree_verify_latent_amd as mtv
    if dev is None:
        dev = to_device(wl)
    prm = params_of(wl, nsplit)
    op = mtv.VerifyAttention(prm)
    out = op(**dev)
    torch.cuda.synchronize()
    return bf16_out_to_f32(out)


def bf16_out_to_f32(out) -> np.ndarray:
    import torch
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.bf16_bits_to_f32(bits)


def sample_rows(wl, n_per_seq: int, seed: int = 0) -> np.ndarray:
    """(b, t, h) triples: corners of every sequence plus seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(wl.B):
        for t in (0, wl.T - 1):
            for h in (0, wl.H - 1):
                rows.add((b, t, h))
        while len([r for r in rows if r[0] == b]) < n_per_seq:
            rows.add((b, int(rng.integers(wl.T)), int(rng.integers(wl.H))))
    return np.array(sorted(rows), dtype=np.int32)
