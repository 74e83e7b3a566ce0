"""Pins of the prefix-scheduler oracle (CPU only; DSpark tutorial,
"hardware-aware prefix scheduler"): closed forms for a flat throughput curve,
a hard batch limit and the tokens-per-verified-token objective, the last
checked against brute force over every prefix-consistent choice."""
import itertools

import numpy as np
import pytest

from oracle import schedule as osch


def test_interpolation_is_linear_and_clamped():
    tb, tv = [1, 3, 7], [10.0, 6.0, 2.0]
    assert osch.sps_interp(2, tb, tv) == pytest.approx(8.0)
    assert osch.sps_interp(5, tb, tv) == pytest.approx(4.0)
    assert osch.sps_interp(0, tb, tv) == 10.0 and osch.sps_interp(100, tb, tv) == 2.0


def test_flat_curve_verifies_every_token_with_positive_survival():
    surv = [np.array([0.9, 0.5, 0.0, 0.7]), np.array([0.3]), np.array([])]
    ell, theta = osch.prefix_schedule(surv, [1, 100], [5.0, 5.0])
    # cumulative survival of the third token of request 0 is 0: it never raises Theta
    assert list(ell) == [2, 1, 0]
    assert theta == pytest.approx(5.0 * (3 + 0.9 + 0.45 + 0.3))


def test_hard_batch_limit_takes_the_best_tokens_that_fit():
    rng = np.random.default_rng(3)
    surv = [rng.uniform(0.5, 1.0, 6) for _ in range(4)]
    R, B0 = 4, 13
    ell, _ = osch.prefix_schedule(surv, [1, B0, B0 + 1, 1000], [1.0, 1.0, 0.5, 0.5])
    assert ell.sum() + R == B0
    cum = sorted((float(v) for c in surv for v in np.cumprod(c)), reverse=True)
    chosen = sorted((float(np.cumprod(surv[r])[k]) for r in range(R) for k in range(ell[r])), reverse=True)
    np.testing.assert_allclose(chosen, cum[:B0 - R])


def _theta(surv, ell, tb, tv):
    tau = sum(1 + float(np.cumprod(c)[:l].sum()) for c, l in zip(surv, ell))
    B = sum(l + 1 for l in ell)
    return tau * osch.sps_interp(B, tb, tv)


@pytest.mark.parametrize("seed", range(5))
def test_tokens_per_verified_token_matches_brute_force(seed):
    # SPS(B) = 1 / B makes Theta the mean tokens per verified token; the best
    # set of n tokens is the n largest cumulative survivals and the mean is
    # unimodal in n, so the greedy with early stop is optimal here
    rng = np.random.default_rng(seed)
    surv = [rng.uniform(0.0, 1.0, rng.integers(0, 4)) for _ in range(3)]
    tb = np.arange(1, 20)
    tv = 1.0 / tb
    ell, theta = osch.prefix_schedule(surv, tb, tv)
    best = max(_theta(surv, e, tb, tv) for e in itertools.product(*[range(len(c) + 1) for c in surv]))
    assert theta == pytest.approx(best, rel=1e-12)
    assert _theta(surv, ell, tb, tv) == pytest.approx(theta, rel=1e-12)


def test_no_requests():
    ell, theta = osch.prefix_schedule([], [1, 2], [1.0, 1.0])
    assert len(ell) == 0 and theta == 0.0
