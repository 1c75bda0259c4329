"""The CPU oracle against facts fixed by the mathematics (see tests/pins.py)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_tree(orc):
    wl = pins.tiny(B=1, H=1, T=3, prefixes=[2], seed=3)
    wl.tree_parent[0, 1] = 1  # a node cannot be its own parent
    with pytest.raises(ValueError):
        orc.run(wl)


def test_rejects_bad_slot(orc):
    wl = pins.tiny(B=1, H=1, T=3, prefixes=[2], seed=3)
    wl.slot_idx[0] = wl.pool_slots
    with pytest.raises(ValueError):
        orc.run(wl)


def test_rows_match_full(orc):
    import numpy as np
    wl = pins.tiny(B=2, H=3, T=5, prefixes=[9, 4], seed=21)
    full = orc.run(wl)
    rows = np.array([[1, 4, 2], [0, 0, 0], [1, 0, 1]], dtype=np.int32)
    got = orc.run_rows(wl, rows)
    for i, (b, t, h) in enumerate(rows):
        assert np.array_equal(got[i], full[b, t, h])
