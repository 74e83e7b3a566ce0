"""Pins of the verification oracle (CPU only).

Each test fixes the oracle to something other than itself: hand-derived
worked examples (tests/golden), a library routine (scipy softmax, stable
argsort), brute force, the closed form of the acceptance probability
(DSpark tutorial, confidence-scheduled verification: 1 - 1/2 |p_d - p_t|_1),
and statistical tests of losslessness (DSpark tutorial, basics and FAQ).
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

from oracle import verify as ov

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "verify_worked_examples.json")))


def logits_of(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32)


def pad_rows(rows, V):
    return np.stack([np.asarray(r, dtype=np.float32) for r in rows])


# ---------------------------------------------------------------- golden cases
@pytest.mark.parametrize("case", GOLD["sampling_cases"], ids=lambda c: c["name"])
def test_golden_sampling(case):
    zt = logits_of(case["P"])[None]
    zd = logits_of(case["Q"])[None]
    d = np.array([case["draft"]], dtype=np.int32)
    u = np.array([case["u"]], dtype=np.float32)
    r = ov.verify(zt, zd, d, u, temperature=1.0)
    assert int(r["tau"][0]) == case["tau"]
    assert r["out_tokens"][0].tolist() == case["out"]


@pytest.mark.parametrize("case", GOLD["greedy_cases"], ids=lambda c: c["name"])
def test_golden_greedy(case):
    zt = np.array([case["Zt"]], dtype=np.float32)
    d = np.array([case["draft"]], dtype=np.int32)
    u = np.zeros((1, zt.shape[1], 2), np.float32)
    r = ov.verify(zt, None, d, u, temperature=0.0)
    assert int(r["tau"][0]) == case["tau"]
    assert r["out_tokens"][0].tolist() == case["out"]


@pytest.mark.parametrize("case", GOLD["filter_cases"], ids=lambda c: c["name"])
def test_golden_filters(case):
    p = ov.filtered_probs(np.array(case["z"], np.float32), case["temperature"], case["top_k"], case["top_p"])
    np.testing.assert_allclose(p, case["P"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- filters
def test_softmax_matches_scipy_and_temperature():
    rng = np.random.default_rng(1)
    for T in (1.0, 0.7, 2.5):
        z = rng.standard_normal(1000).astype(np.float32) * 3
        p = ov.filtered_probs(z, T)
        np.testing.assert_allclose(p, special.softmax(z.astype(np.float64) / T), rtol=1e-12, atol=0)
        assert abs(p.sum() - 1) < 1e-12


def brute_filter(z, T, k, top_p):
    """Full stable sort, then the first n with cumulative mass >= top_p."""
    z = np.asarray(z)
    V = len(z)
    order = np.argsort(-z.astype(np.float64), kind="stable")   # value desc, index asc
    kept = order[:k] if 0 < k < V else order
    w = np.exp(z[kept].astype(np.float64) / T - (z[kept].astype(np.float64) / T).max())
    w = w / w.sum()
    if top_p < 1.0:
        n = len(kept)
        for m in range(1, len(kept) + 1):
            if w[:m].sum() >= top_p:
                n = m
                break
        kept, w = kept[:n], w[:n] / w[:n].sum()
    p = np.zeros(V)
    p[kept] = w
    return p


@pytest.mark.parametrize("k,top_p", [(20, 1.0), (20, 0.95), (0, 0.5), (5, 0.3), (1, 0.9), (64, 0.99)])
def test_filters_match_brute_force(k, top_p):
    rng = np.random.default_rng(k * 100 + int(top_p * 100))
    for _ in range(5):
        z = rng.standard_normal(3000).astype(np.float32)
        z[rng.integers(0, 3000, 50)] = z[rng.integers(0, 3000, 50)]   # plant ties
        p = ov.filtered_probs(z, 1.0, k, top_p)
        np.testing.assert_allclose(p, brute_filter(z, 1.0, k, top_p), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- closed forms
def test_acceptance_identity_tv_distance():
    rng = np.random.default_rng(2)
    for V in (2, 8, 1000):
        for _ in range(20):
            p = rng.dirichlet(np.ones(V) * 0.3)
            q = rng.dirichlet(np.ones(V) * 0.3)
            beta = ov.acceptance_probability(p, q)
            assert abs(beta - (1 - 0.5 * np.abs(p - q).sum())) < 1e-12


def test_inverse_cdf_against_linear_scan():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 40))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if w.sum() == 0:
            w[0] = 1.0
        u = float(rng.random())
        x, _ = ov.inverse_cdf(w, u)
        t = u * w.sum()
        run, scan = 0.0, None
        for i, wi in enumerate(w):
            run += wi
            if run > t:
                scan = i
                break
        if scan is None:
            scan = int(np.nonzero(w > 0)[0][-1])
        assert x == scan


def test_greedy_tau_brute_force():
    rng = np.random.default_rng(4)
    B, G, V = 64, 7, 6
    zt = rng.integers(0, 4, (B, G + 1, V)).astype(np.float32)   # many ties
    choice = np.argmax(zt, axis=-1)
    d = np.where(rng.random((B, G)) < 0.7, choice[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
    r = ov.verify(zt, None, d, np.zeros((B, G + 1, 2), np.float32), 0.0)
    for b in range(B):
        t = max(t for t in range(G + 1) if all(d[b, j] == choice[b, j] for j in range(t)))
        assert r["tau"][b] == t
        assert r["out_tokens"][b, :t].tolist() == d[b, :t].tolist()
        assert r["out_tokens"][b, t] == choice[b, t]
        assert (r["out_tokens"][b, t + 1:] == -1).all()


def test_one_hot_sampling_reduces_to_greedy():
    rng = np.random.default_rng(5)
    B, G, V = 32, 5, 7
    choice_t = rng.integers(0, V, (B, G + 1))
    d = np.where(rng.random((B, G)) < 0.6, choice_t[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
    zt = np.full((B, G + 1, V), -np.inf, np.float32)
    zd = np.full((B, G, V), -np.inf, np.float32)
    for b in range(B):
        for i in range(G + 1):
            zt[b, i, choice_t[b, i]] = 0.0
        for i in range(G):
            zd[b, i, d[b, i]] = 0.0
    zg = np.where(np.isinf(zt), 0.0, 1.0).astype(np.float32)
    u = rng.random((B, G + 1, 2), dtype=np.float32)
    rs = ov.verify(zt, zd, d, u, 1.0)
    rg = ov.verify(zg, None, d, u, 0.0)
    assert (rs["tau"] == rg["tau"]).all()
    assert (rs["out_tokens"] == rg["out_tokens"]).all()


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(6)
    B, G, V = 16, 6, 50
    zd = rng.standard_normal((B, G, V)).astype(np.float32)
    zt = np.concatenate([zd, rng.standard_normal((B, 1, V)).astype(np.float32)], axis=1)
    d = rng.integers(0, V, (B, G)).astype(np.int32)
    u = rng.random((B, G + 1, 2), dtype=np.float32)
    r = ov.verify(zt, zd, d, u, 1.0)
    assert (r["tau"] == G).all()
    np.testing.assert_array_equal(r["accept_ratio"], np.ones((B, G), np.float32))


def test_disjoint_supports_reject_first():
    B, G, V = 8, 4, 6
    zt = np.full((B, G + 1, V), -np.inf, np.float32)
    zd = np.full((B, G, V), -np.inf, np.float32)
    zt[..., :3] = 0.0
    zd[..., 3:] = 0.0
    rng = np.random.default_rng(7)
    d = rng.integers(3, 6, (B, G)).astype(np.int32)
    u = rng.random((B, G + 1, 2), dtype=np.float32)
    r = ov.verify(zt, zd, d, u, 1.0)
    assert (r["tau"] == 0).all()
    assert (r["out_tokens"][:, 0] < 3).all()


# ---------------------------------------------------------------- statistics
def _draw(q, rng, n):
    return rng.choice(len(q), size=n, p=q)


@pytest.mark.slow
@pytest.mark.parametrize("V,top_k,top_p", [(8, 0, 1.0), (32, 0, 1.0), (32, 6, 0.9)])
def test_lossless_chi_square(V, top_k, top_p):
    """The first emitted token is distributed as the (filtered) target P_1; given
    d_1 accepted, the second emitted token follows P_2."""
    rng = np.random.default_rng(100 + V + top_k)
    N = 200_000
    zt = (rng.standard_normal((1, 3, V)) * 1.2).astype(np.float32)
    zd = (rng.standard_normal((1, 2, V)) * 1.2).astype(np.float32)
    P = [ov.filtered_probs(zt[0, i], 1.0, top_k, top_p) for i in range(3)]
    Q = [ov.filtered_probs(zd[0, i], 1.0, top_k, top_p) for i in range(2)]
    d = np.stack([_draw(Q[0], rng, N), _draw(Q[1], rng, N)], axis=1).astype(np.int32)
    u = rng.random((N, 3, 2), dtype=np.float32)
    r = ov.verify(np.broadcast_to(zt, (N, 3, V)), np.broadcast_to(zd, (N, 2, V)), d, u, 1.0, top_k, top_p)
    first = r["out_tokens"][:, 0]
    sup = P[0] > 0
    obs = np.bincount(first, minlength=V)
    assert obs[~sup].sum() == 0
    p1 = stats.chisquare(obs[sup], N * P[0][sup]).pvalue
    assert p1 > 0.01, p1
    sel = r["tau"] >= 1
    second = r["out_tokens"][sel, 1]
    sup2 = P[1] > 0
    obs2 = np.bincount(second, minlength=V)
    assert obs2[~sup2].sum() == 0
    p2 = stats.chisquare(obs2[sup2], sel.sum() * P[1][sup2]).pvalue
    assert p2 > 0.01, p2


@pytest.mark.slow
def test_acceptance_frequency_and_tau_law():
    """Per-position acceptance frequency matches sum min(P, Q) within 4 binomial
    sigma, and the mean accepted length matches sum_i prod_{j<=i} beta_j."""
    rng = np.random.default_rng(11)
    V, G, N = 16, 3, 100_000
    zt = (rng.standard_normal((1, G + 1, V)) * 0.8).astype(np.float32)
    zd = (rng.standard_normal((1, G, V)) * 0.8).astype(np.float32)
    P = [ov.filtered_probs(zt[0, i], 1.0) for i in range(G + 1)]
    Q = [ov.filtered_probs(zd[0, i], 1.0) for i in range(G)]
    beta = np.array([ov.acceptance_probability(P[i], Q[i]) for i in range(G)])
    d = np.stack([_draw(Q[i], rng, N) for i in range(G)], axis=1).astype(np.int32)
    u = rng.random((N, G + 1, 2), dtype=np.float32)
    r = ov.verify(np.broadcast_to(zt, (N, G + 1, V)), np.broadcast_to(zd, (N, G, V)), d, u, 1.0)
    acc1 = (r["tau"] >= 1).mean()
    assert abs(acc1 - beta[0]) < 4 * np.sqrt(beta[0] * (1 - beta[0]) / N)
    expect = sum(np.prod(beta[: i + 1]) for i in range(G))
    sd = r["tau"].std() / np.sqrt(N)
    assert abs(r["tau"].mean() - expect) < 4 * sd


def test_ratio_is_fp32_division():
    rng = np.random.default_rng(12)
    B, G, V = 4, 3, 20
    zt = rng.standard_normal((B, G + 1, V)).astype(np.float32)
    zd = rng.standard_normal((B, G, V)).astype(np.float32)
    d = rng.integers(0, V, (B, G)).astype(np.int32)
    r = ov.verify(zt, zd, d, rng.random((B, G + 1, 2), dtype=np.float32), 1.0)
    for b in range(B):
        for i in range(G):
            p = special.softmax(zt[b, i].astype(np.float64))[d[b, i]]
            q = special.softmax(zd[b, i].astype(np.float64))[d[b, i]]
            assert r["accept_ratio"][b, i] == np.float32(np.float32(p) / np.float32(q))


# ---- per-request verify lengths and the confidence label (DSpark tutorial,
# confidence-scheduled verification)

def _ragged_case(rng, G_list, V, T):
    row_cu = np.concatenate([[0], np.cumsum(np.asarray(G_list) + 1)])
    N, B = int(row_cu[-1]), len(G_list)
    zt = rng.standard_normal((N, V)).astype(np.float32)
    zd = rng.standard_normal((N - B, V)).astype(np.float32)
    d = rng.integers(0, V, N - B).astype(np.int32)
    u = rng.uniform(0, 1, (N, 2)).astype(np.float32)
    return zt, zd, d, u, row_cu


@pytest.mark.parametrize("T,k,p", [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.7, 5, 0.9)])
def test_ragged_with_equal_lengths_is_the_batched_form(T, k, p):
    rng = np.random.default_rng(40)
    B, G, V = 3, 4, 50
    zt, zd, d, u, row_cu = _ragged_case(rng, [G] * B, V, T)
    a = ov.verify_ragged(zt, zd, d, u, row_cu, T, k, p)
    b = ov.verify(zt.reshape(B, G + 1, V), zd.reshape(B, G, V), d.reshape(B, G), u.reshape(B, G + 1, 2), T, k, p)
    np.testing.assert_array_equal(a["tau"], b["tau"])
    np.testing.assert_array_equal(a["out_tokens"], b["out_tokens"].reshape(-1))
    np.testing.assert_array_equal(a["accept_ratio"], b["accept_ratio"].reshape(-1))


def test_ragged_request_without_drafts_emits_one_target_token():
    rng = np.random.default_rng(41)
    zt, zd, d, u, row_cu = _ragged_case(rng, [2, 0, 3], 30, 1.0)
    g = ov.verify_ragged(zt, zd, d, u, row_cu, 0.0)
    assert g["tau"][1] == 0 and g["out_tokens"][3] == int(np.argmax(zt[3]))
    s = ov.verify_ragged(zt, zd, d, u, row_cu, 1.0)
    p = special.softmax(zt[3].astype(np.float64))
    c = np.cumsum(p)
    assert s["tau"][1] == 0 and s["out_tokens"][3] == int(np.searchsorted(c, u[3, 1] * c[-1], side="right"))


def test_confidence_label_closed_forms():
    rng = np.random.default_rng(42)
    p = rng.dirichlet(np.ones(20))
    q = rng.dirichlet(np.ones(20))
    assert ov.confidence_label(p, p) == pytest.approx(1.0)
    assert ov.confidence_label(p, q) == pytest.approx(1.0 - 0.5 * np.abs(p - q).sum())
    a = np.zeros(20); a[:10] = 0.1
    b = np.zeros(20); b[10:] = 0.1
    assert ov.confidence_label(a, b) == 0.0


def test_ragged_beta_is_the_label_of_each_drafted_position():
    rng = np.random.default_rng(43)
    zt, zd, d, u, row_cu = _ragged_case(rng, [3, 1, 0, 2], 40, 0.8)
    r = ov.verify_ragged(zt, zd, d, u, row_cu, 0.8, want_beta=True)
    for b in range(4):
        t0, t1 = row_cu[b], row_cu[b + 1]
        for i in range(t1 - t0 - 1):
            p = special.softmax(zt[t0 + i].astype(np.float64) / 0.8)
            q = special.softmax(zd[t0 - b + i].astype(np.float64) / 0.8)
            assert r["beta"][t0 - b + i] == pytest.approx(1.0 - 0.5 * np.abs(p - q).sum(), rel=1e-12)
    # greedy: the point masses at the two lowest-index maxima
    zt2 = zt.copy(); zd2 = zd.copy()
    zd2[0] = zt2[0]                       # same argmax -> 1
    zd2[1] = -zt2[1]                      # argmax differs (almost surely) -> 0
    g = ov.verify_ragged(zt2, zd2, d, u, row_cu, 0.0, want_beta=True)
    assert g["beta"][0] == 1.0 and g["beta"][1] == 0.0
