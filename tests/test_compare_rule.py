"""The decision-exact comparison rule of the GPU parity tests, checked on the
CPU with planted disagreements (a copy of the oracle's result with one
decision changed): only the first diverging decision may differ, and only as
a near tie on that decision."""
import numpy as np
import pytest

from oracle import verify as ov
from tests.helpers import check_request

NEAR = 1e-6


def case():
    rng = np.random.default_rng(3)
    V, G = 8, 3
    zt = rng.standard_normal((1, G + 1, V)).astype(np.float32)
    zd = rng.standard_normal((1, G, V)).astype(np.float32)
    d = np.array([[int(np.argmax(zd[0, i])) for i in range(G)]], np.int32)
    return zt, zd, d, V, G


def weights_fn(zt, zd, G):
    def w(t):
        P = ov.filtered_probs(zt[0, t], 1.0)
        Q = ov.filtered_probs(zd[0, t], 1.0) if t < G else None
        return ov.draw_weights(P, Q)
    return w


def run(zt, zd, d, u):
    return ov.verify(zt, zd, d, u, 1.0)


def check(o, g_tau, g_tok, g_ratio, u, zt, zd, G):
    return check_request("planted", 0, False, int(o["tau"][0]), g_tau, o["out_tokens"][0], g_tok,
                         o["accept_ratio"][0], g_ratio, u[0, :G, 0], u[0, :, 1], weights_fn(zt, zd, G), NEAR)


def test_identical_results_pass():
    zt, zd, d, V, G = case()
    u = np.full((1, G + 1, 2), 0.5, np.float32)
    o = run(zt, zd, d, u)
    assert check(o, int(o["tau"][0]), o["out_tokens"][0].copy(), o["accept_ratio"][0], u, zt, zd, G) is None


def _draw_near_boundary(offset):
    """u' of the first position placed `offset` below a CDF boundary of its
    draw (first test rejected with u = 1 - 2^-24)."""
    zt, zd, d, V, G = case()
    u = np.zeros((1, G + 1, 2), np.float32)
    u[0, :, 0] = np.float32(1 - 2 ** -24)
    w = weights_fn(zt, zd, G)(0)
    c = np.cumsum(w)
    x = int(np.nonzero(w > 0)[0][1])                    # a token with a positive-weight neighbour above it
    nxt = int(np.nonzero(w > 0)[0][2])
    target = (c[x] - offset) / c[-1]
    u[0, 0, 1] = np.float32(target)
    return zt, zd, d, u, G, x, nxt, w


def test_draw_flip_to_neighbour_within_band_is_excused():
    zt, zd, d, u, G, x, nxt, w = _draw_near_boundary(3e-7)
    o = run(zt, zd, d, u)
    assert o["tau"][0] == 0
    dist = ov.cdf_distance(w, float(u[0, 0, 1]), nxt)
    if not (o["out_tokens"][0, 0] == x and dist < NEAR):
        pytest.skip("fp32 rounding of u' moved the planted boundary")
    g_tok = o["out_tokens"][0].copy()
    g_tok[0] = nxt
    assert check(o, 0, g_tok, o["accept_ratio"][0], u, zt, zd, G) == "draw"


def test_draw_flip_outside_band_fails():
    zt, zd, d, u, G, x, nxt, w = _draw_near_boundary(0.05)
    o = run(zt, zd, d, u)
    g_tok = o["out_tokens"][0].copy()
    g_tok[0] = nxt if g_tok[0] != nxt else x
    with pytest.raises(AssertionError):
        check(o, 0, g_tok, o["accept_ratio"][0], u, zt, zd, G)


def test_draw_flip_to_non_neighbour_fails():
    zt, zd, d, u, G, x, nxt, w = _draw_near_boundary(3e-7)
    o = run(zt, zd, d, u)
    g_tok = o["out_tokens"][0].copy()
    far = [i for i in np.nonzero(w > 0)[0] if abs(int(i) - int(g_tok[0])) > 1 and i != nxt]
    g_tok[0] = int(far[-1])
    with pytest.raises(AssertionError):
        check(o, 0, g_tok, o["accept_ratio"][0], u, zt, zd, G)


def _accept_case(delta):
    zt, zd, d, V, G = case()
    o0 = run(zt, zd, d, np.full((1, G + 1, 2), 0.5, np.float32))
    r0 = float(o0["accept_ratio"][0, 0])
    assert 0 < r0 < 1
    u = np.full((1, G + 1, 2), 0.5, np.float32)
    u[0, 0, 0] = np.float32(r0 + delta)                  # u just above the ratio: the oracle rejects
    return zt, zd, d, u, G


def test_accept_flip_within_band_is_excused():
    zt, zd, d, u, G = _accept_case(2e-7)
    o = run(zt, zd, d, u)
    assert o["tau"][0] == 0
    # the kernel accepted the first draft (and went on): tau differs at position 0
    g_tok = np.array([d[0, 0], 5, -1, -1], np.int32)
    assert check(o, 1, g_tok, o["accept_ratio"][0], u, zt, zd, G) == "accept"


def test_accept_flip_outside_band_fails():
    zt, zd, d, u, G = _accept_case(1e-3)
    o = run(zt, zd, d, u)
    g_tok = np.array([d[0, 0], 5, -1, -1], np.int32)
    with pytest.raises(AssertionError):
        check(o, 1, g_tok, o["accept_ratio"][0], u, zt, zd, G)


def test_difference_after_an_agreed_decision_fails():
    zt, zd, d, V, G = case()
    u = np.zeros((1, G + 1, 2), np.float32)            # u = 0 accepts every draft with P(d) > 0
    o = run(zt, zd, d, u)
    t = int(o["tau"][0])
    g_tok = o["out_tokens"][0].copy()
    g_tok[t] = (g_tok[t] + 3) % V                      # a different extra token with no near tie
    with pytest.raises(AssertionError):
        check(o, t, g_tok, o["accept_ratio"][0], u, zt, zd, G)


def test_greedy_difference_always_fails():
    zt, zd, d, V, G = case()
    o = ov.verify(zt, None, d, None, 0.0)
    g_tok = o["out_tokens"][0].copy()
    g_tok[int(o["tau"][0])] += 1
    with pytest.raises(AssertionError):
        check_request("greedy", 0, True, int(o["tau"][0]), int(o["tau"][0]), o["out_tokens"][0], g_tok,
                      o["accept_ratio"][0], o["accept_ratio"][0], np.zeros(G), np.zeros(G + 1), None, NEAR)
