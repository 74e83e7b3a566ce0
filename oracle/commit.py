"""Oracle of the round commit (test infrastructure only).

DFlash/Spec V2 blog, A7: between two rounds each request's metadata is
updated (the page's host clean-up); here the update is the plain definition:
tau + 1 tokens are committed (DSpark tutorial, basics: the accepted drafts
plus one target token per round), so the context grows by tau + 1.  A7,
immediate materialization: before the next draft forward the drafter's KV of
the target's hidden states is written; those are the K rows this round
verified, at the block's positions, so the next injected rows start at the
context length before this commit.

Readings: tau < 0 (a request the verify flagged invalid) leaves the request
unchanged and marks it done; a request is also done when its next K rows
would pass its slot capacity (ctx + K > cap).
"""
import numpy as np


def commit_round(tau, ctx_len, K: int, cap=None):
    """Returns (ctx_next int32 [B], row_pos0 int32 [B] (the context length
    before this commit), done int32 [B])."""
    tau = np.asarray(tau, dtype=np.int64)
    ctx0 = np.asarray(ctx_len, dtype=np.int64)
    ctx = ctx0.copy()
    done = np.zeros(len(ctx), dtype=np.int32)
    for b in range(len(ctx)):
        if tau[b] >= 0:
            ctx[b] += tau[b] + 1
        else:
            done[b] = 1
        if cap is not None and ctx[b] + K > int(cap[b]):
            done[b] = 1
    return ctx.astype(np.int32), ctx0.astype(np.int32), done
