"""The library's host prefix scheduler against the oracle (CPU only: the
scheduler is host code; DSpark tutorial, "hardware-aware prefix scheduler")."""
import numpy as np
import pytest

import block_drafting_amd as bd
from oracle import schedule as osch


@pytest.fixture(scope="module", autouse=True)
def built():
    import os
    if not os.path.exists(bd.lib_path()):
        from block_drafting_amd import build
        build.build()


def _case(rng, R, Lmax):
    surv = [rng.uniform(0.0, 1.0, rng.integers(0, Lmax + 1)).astype(np.float32) for _ in range(R)]
    # a measured-looking curve: flat, then falling (steps/s drop as the batch grows)
    tb = np.array([1, 64, 128, 256, 512, 1024, 4096], dtype=np.float32)
    tv = np.array([1400, 1390, 1300, 1100, 800, 450, 120], dtype=np.float32)
    return surv, tb, tv


@pytest.mark.parametrize("seed", range(12))
def test_library_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    surv, tb, tv = _case(rng, int(rng.integers(1, 200)), 16)
    ell, theta = bd.prefix_schedule(surv, tb, tv)
    oe, ot = osch.prefix_schedule([np.asarray(c, np.float64) for c in surv], tb.astype(np.float64),
                                  tv.astype(np.float64))
    assert ell == [int(x) for x in oe]
    assert theta == pytest.approx(ot, rel=1e-12)


def test_ties_and_unsorted_table():
    surv = [np.array([1.0, 1.0, 0.5], np.float32), np.array([1.0, 0.5], np.float32)]
    tb = np.array([10, 1, 5], np.float32)        # any order
    tv = np.array([1.0, 1.0, 1.0], np.float32)
    ell, theta = bd.prefix_schedule(surv, tb, tv)
    oe, ot = osch.prefix_schedule(surv, np.sort(tb), tv)
    assert ell == list(oe) == [3, 2] and theta == pytest.approx(ot)


def test_empty_pool():
    assert bd.prefix_schedule([], [1.0], [1.0]) == ([], 0.0)
