"""Host logic of the rescale inputs (tests/rescale.py), no GPU: the planted ramp
moves the scores exactly as stated and leaves V untouched, the host-side count
of running-maximum raises agrees with a direct per-row walk, and the
benchmark-like draws never raise a running maximum (which is why the peaked
cases exist)."""
import numpy as np

import rescale
from synthetic import inputs


def _tiny(**kw):
    return inputs.make_workload("t", B=2, H=3, T=5, prefixes=[200, 77], pool_slots=400, seed=3, **kw)


def test_ramp_moves_scores_as_stated():
    """After planting, score(r, j) = score with the same queries and the unramped
    keys, minus amp * (1 - ((j + offset) % period) / period), up to the rounding of
    the ramped rope values (bf16: 64 values of spacing <= 2^-5 at these sizes)."""
    import copy
    for dtype, tol in (("bf16", 0.15), ("f32", 1e-4)):
        wl = _tiny(dtype=dtype)
        v_before = wl.kv_pool[:, :512].copy()
        period, amp, offset = 50, 30.0, 7
        planted = rescale.plant_score_ramp(copy.deepcopy(wl), amp, period, offset=offset)
        assert np.array_equal(planted.kv_pool[:, :512], v_before), "V (the first 512 values) is unchanged"
        unramped = copy.deepcopy(wl)
        unramped.q = planted.q  # same queries, keys as drawn
        for b in range(wl.B):
            S0, S1 = rescale.base2_scores(unramped, b), rescale.base2_scores(planted, b)
            n = S0.shape[1]
            want = -amp * (1 - ((np.arange(n) + offset) % period) / period)
            fin = np.isfinite(S0)
            assert np.array_equal(fin, np.isfinite(S1))
            err = np.abs(np.where(fin, S1 - S0 - want[None, :], 0.0))
            assert err.max() < tol, (dtype, err.max())


def test_rescale_count_matches_direct_walk():
    wl = _tiny(q_std=40.0)
    chunk, tile = 64, 16
    events, splits, most = rescale.rescale_events(wl, chunk, tile)
    direct = 0
    for b in range(wl.B):
        S = rescale.base2_scores(wl, b)
        for r in range(S.shape[0]):
            for k0 in range(0, S.shape[1], chunk):
                m = -np.inf
                for t0 in range(k0, min(k0 + chunk, S.shape[1]), tile):
                    mx = S[r, t0:min(t0 + tile, k0 + chunk, S.shape[1])].max()
                    if mx > m + 8:
                        direct += np.isfinite(m)
                        m = mx
    assert events == direct > 0


def test_benchmark_draws_never_rescale():
    wl = inputs.config("c2_tp_share")
    assert rescale.rescale_events(wl, 256, 32)[0] == 0


def test_masked_keys_are_minus_infinity():
    wl = _tiny(tree="chain")
    S = rescale.base2_scores(wl, 0)
    P = int(wl.seq_lens[0]) - wl.T
    for t in range(wl.T):
        row = S[t * wl.H]
        assert np.all(np.isfinite(row[:P + t + 1])) and np.all(np.isneginf(row[P + t + 1:]))
