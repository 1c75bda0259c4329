"""Online-softmax rescale under peaked scores, GPU vs the oracle (needs a gfx950 GPU).

Each case first shows on the host, from its inputs and the library's published
plan (split and tile lengths), that some split's running maximum is raised
after its first tile in rows that already hold weights, so that the kernels'
rescale of the accumulated V sums runs; then the whole output is compared with
the oracle at the usual gates (bf16: 2 bf16 ULP of the row's largest value;
fp32 inputs: 2^-16 of it). The scores are made peaked by scaling the queries
(q ~ N(0, q_std^2)) or by a planted sawtooth ramp in the rope dimensions
(tests/rescale.py), with amplitudes up to 300 in base 2, far past the
binary32 range of the weights.
"""
import numpy as np
import pytest

import oracle
import rescale
from helpers import parity_gate, params_of, run_gpu
from synthetic import inputs
from test_f32 import rel_gate, run_gpu_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_tree_verify_latent_amd as mtv
    mtv.load_library()


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


# The synthetic shapes hold a few thousand keys per sequence, where the
# library's own plan takes splits of one or two tiles: too short for a running
# maximum to rise within a split. Four splits per sequence make them hundreds
# of keys (several tiles) long.
FORCED_SPLITS = {"small": 4, "ragged": 4, "few_rows": 4, "decode": 4}


def _plan(wl, nsplit=0):
    import mla_tree_verify_latent_amd as mtv
    return mtv.verify_attn_plan_for(params_of(wl, nsplit), wl.f32)


def _workload(shape, seed, dtype="bf16", **kw):
    if shape in inputs.CONFIGS:
        cfg = {**inputs.CONFIGS[shape], "dtype": dtype, **kw}
        return inputs.make_workload(shape, **cfg)
    B, H, T, prefixes = dict(small=(2, 8, 16, [3000, 1200]), ragged=(3, 4, 24, [0, 2500, 700]),
                             few_rows=(2, 8, 4, [3000, 1200]), decode=(3, 8, 1, [4000, 0, 777]))[shape]
    return inputs.make_workload(shape, B=B, H=H, T=T, prefixes=prefixes,
                                pool_slots=sum(prefixes) + B * T + 101, seed=seed, dtype=dtype, **kw)


def _show_rescale(wl, nsplit=0, at_least=1):
    pl = _plan(wl, nsplit)
    events, splits, most = rescale.rescale_events(wl, pl["keys_per_split"], pl["keys_per_tile"])
    print(f"{wl.name}: {events} rescales of running sums in {splits} splits "
          f"(up to {most} in one row and split; {pl['keys_per_split']}-key splits, "
          f"{pl['keys_per_tile']}-key tiles)")
    assert events >= at_least, "these inputs must raise some split's running maximum past +8"
    return events


def _check_bf16(orc, wl, nsplit=0):
    got = run_gpu(wl, nsplit)
    ref = orc.run(wl)
    ok, worst, idx = parity_gate(got, ref)
    print(f"{wl.name}: worst row {idx} at {worst:.3f} bf16 ulp")
    assert ok, f"{wl.name}: worst row {idx} at {worst:.2f} bf16 ulp"


def _check_f32(orc, wl, nsplit=0):
    got = run_gpu_f32(wl, nsplit)
    ref = orc.run(wl)
    ok, worst, idx = rel_gate(got, ref)
    print(f"{wl.name}: worst row {idx} at {worst:.3g} of the row scale")
    assert ok, f"{wl.name}: worst row {idx} at {worst:.3g} of the row scale"


# ------------------------------------------------------------ bf16 entry point

@pytest.mark.parametrize("q_std", [16, 64])
@pytest.mark.parametrize("shape", ["small", "ragged", "few_rows", "decode", "e2_h8_t9_65k"])
def test_peaked_queries(orc, shape, q_std):
    if shape == "decode" and q_std == 16:
        q_std = 32  # 8 query rows at spread 16 never overtake a running maximum by 8
    wl = _workload(shape, seed=50 + q_std, q_std=float(q_std))
    nsplit = FORCED_SPLITS.get(shape, 0)
    _show_rescale(wl, nsplit)
    _check_bf16(orc, wl, nsplit)


@pytest.mark.parametrize("shape,amp,period,offset,nsplit", [
    ("c2_tp_share", 40.0, None, 0, 0),     # one ramp per split, aligned with the splits
    ("c2_tp_share", 300.0, 700, 123, 0),   # unaligned, early keys' weights underflow
    ("c2_tp_share", 200.0, None, 0, 1),    # one split of the whole sequence, one long ramp
    ("ragged", 60.0, 333, 5, 0),
    ("e2_h8_t9_65k", 40.0, None, 0, 0),
    ("c4a_long_scattered", 80.0, None, 0, 0),
    ("few_rows", 60.0, None, 0, 0),        # 32 rows: the small-row kernel, one ramp per split
    ("few_rows", 300.0, 700, 123, 0),
    ("decode", 200.0, None, 0, 1),         # T = 1, one split of each whole sequence
], ids=lambda v: str(v))
def test_score_ramp(orc, shape, amp, period, offset, nsplit):
    wl = _workload(shape, seed=70)
    nsplit = nsplit or FORCED_SPLITS.get(shape, 0)
    if period is None:  # aligned with the splits, or the whole sequence for one split
        period = _plan(wl, nsplit)["keys_per_split"] if nsplit != 1 else int(wl.seq_lens.max())
    rescale.plant_score_ramp(wl, amp, period, offset)
    _show_rescale(wl, nsplit)
    if amp > 126:
        assert rescale.underflowing_keys(wl) > 0
    _check_bf16(orc, wl, nsplit)


# ------------------------------------------------------------ fp32 entry point

@pytest.mark.parametrize("q_std", [16, 32])
@pytest.mark.parametrize("shape", ["small", "ragged"])
def test_peaked_queries_f32(orc, shape, q_std):
    wl = _workload(shape, seed=90 + q_std, dtype="f32", q_std=float(q_std))
    nsplit = FORCED_SPLITS.get(shape, 0)
    _show_rescale(wl, nsplit)
    _check_f32(orc, wl, nsplit)


@pytest.mark.parametrize("shape,amp,period,offset,nsplit", [
    ("small", 40.0, None, 0, 0),
    ("small", 300.0, 700, 123, 0),   # early keys' weights underflow
    ("ragged", 30.0, 333, 5, 0),
    ("c2_tp_share", 200.0, None, 0, 1),
], ids=lambda v: str(v))
def test_score_ramp_f32(orc, shape, amp, period, offset, nsplit):
    wl = _workload(shape, seed=110, dtype="f32")
    nsplit = nsplit or FORCED_SPLITS.get(shape, 0)
    if period is None:
        period = _plan(wl, nsplit)["keys_per_split"] if nsplit != 1 else int(wl.seq_lens.max())
    rescale.plant_score_ramp(wl, amp, period, offset)
    _show_rescale(wl, nsplit)
    if amp > 126:
        assert rescale.underflowing_keys(wl) > 0
    _check_f32(orc, wl, nsplit)
