"""Pins of the round-commit oracle (CPU only): a hand-worked example and the
token count invariant (DSpark tutorial, basics: tau + 1 tokens per round)."""
import numpy as np

from oracle import commit as oc


def test_hand_worked_example():
    # tau 2 -> +3; tau 0 -> +1 and 1 + 16 > 16 slots: done; tau -1: unchanged, done;
    # tau 15 -> +16 and 4016 + 16 > 4030: done
    ctx, pos, done = oc.commit_round([2, 0, -1, 15], [100, 0, 50, 4000], 16, cap=[200, 16, 100, 4030])
    assert list(ctx) == [103, 1, 50, 4016]
    assert list(pos) == [100, 0, 50, 4000]      # the verified block's first position
    assert list(done) == [0, 1, 1, 1]


def test_committed_tokens_are_tau_plus_one():
    rng = np.random.default_rng(0)
    tau = rng.integers(0, 16, 500)
    ctx0 = rng.integers(0, 5000, 500)
    ctx, _, done = oc.commit_round(tau, ctx0, 16)
    assert (ctx - ctx0).sum() == (tau + 1).sum()
    assert not done.any()
