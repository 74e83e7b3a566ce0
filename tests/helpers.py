"""Shared helpers of the test suite (no method arithmetic here)."""
import sys

import numpy as np


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x: np.ndarray, y: np.ndarray) -> float:
    """max |x - y| / max |y| over one slice (relative to the slice's scale)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.abs(y).max()
    if den == 0:
        return float(np.abs(x - y).max())
    return float(np.abs(x - y).max() / den)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def cuda_bits(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def host_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def f32(x: float) -> float:
    """The value a float argument has after crossing the C ABI as fp32 (the
    oracle is given the same temperature and top-p the kernels see)."""
    return float(np.float32(x))


def check_request(label, b, greedy, tau_o, tau_g, tok_o, tok_g, ratio_o, ratio_g, u_acc, u_draw, weights,
                  near=1e-6):
    """Compare one request's verification on the two sides, decision by decision.

    Returns None when tau and every emitted token agree.  Otherwise only the
    first decision at which the two paths part may differ, and only as a near
    tie; everything after it follows from that decision:
      * tau differs: the accept test at position t = min(tau) must have
        |u_t - ratio_t| < near on the oracle's or the kernel's ratio;
      * tau agrees, the drawn token differs: the kernel's token must be the
        positive-weight index next to the oracle's token (below or above it)
        and u' * Z must lie within `near` of that token's CDF interval, on the
        oracle's fp64 weights (``weights(t)``).
    Greedy decisions compare raw logits and must agree exactly.  Returns
    "accept" or "draw" for an excused near tie; raises AssertionError else."""
    from oracle import verify as ov
    tok_o = np.asarray(tok_o)
    tok_g = np.asarray(tok_g)
    if tau_o == tau_g and (tok_o == tok_g).all():
        return None
    head = f"{label}: request {b}: oracle tau={tau_o} {tok_o.tolist()} / kernel tau={tau_g} {tok_g.tolist()}"
    assert not greedy, head + " (greedy decisions must agree exactly)"
    assert tau_g >= 0, head
    t = int(min(tau_o, tau_g))
    assert (tok_o[:t] == tok_g[:t]).all(), head + " (accepted prefixes differ)"
    if tau_o != tau_g:
        u = float(u_acc[t])
        d = min(abs(u - float(ratio_o[t])), abs(u - float(ratio_g[t])))
        assert d < near, head + (f" (accept test {t}: u={u!r} oracle ratio {float(ratio_o[t])!r} kernel ratio "
                                 f"{float(ratio_g[t])!r}, not within {near})")
        return "accept"
    assert (tok_o[t + 1:] == tok_g[t + 1:]).all(), head + " (tokens after the draw differ)"
    x_o, x_g = int(tok_o[t]), int(tok_g[t])
    w = weights(t)
    pos = np.nonzero(w > 0)[0]
    below = pos[pos < x_o]
    above = pos[pos > x_o]
    adjacent = {int(below[-1])} if len(below) else set()
    adjacent |= {int(above[0])} if len(above) else set()
    assert x_g in adjacent, head + f" (drawn token {x_g} is not a positive-weight neighbour of {x_o})"
    dist = ov.cdf_distance(w, float(u_draw[t]), x_g)
    assert dist < near, head + f" (draw at {t}: u'Z lies {dist:.3e} from token {x_g}'s interval)"
    return "draw"
