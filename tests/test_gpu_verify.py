"""GPU parity of verify_block against the oracle (called through the C ABI).

Bar: tau, accepted tokens and the replacement / extra token bit-exact, except
for decisions the oracle or the kernel takes within 1e-6 of the boundary
(counted and reported); probabilities within 1e-5 absolute; ratios within a
few fp32 ulps.  Greedy decisions compare raw fp32 logits on both sides, so
they must match exactly.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import verify as ov
from tests.helpers import check_request, f32, say

pytestmark = pytest.mark.gpu

NEAR = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import block_drafting_amd as bd
    bd.load()
    return bd


def run_gpu(zt, zd, dt, u, T, k=0, p=1.0, probs=False):
    import block_drafting_amd as bd
    B, G1, V = zt.shape
    G = G1 - 1
    dev = "cuda"
    zt_d = torch.from_numpy(np.ascontiguousarray(zt)).to(dev)
    zd_d = torch.from_numpy(np.ascontiguousarray(zd)).to(dev) if zd is not None else None
    dt_d = torch.from_numpy(np.ascontiguousarray(dt, dtype=np.int32)).to(dev)
    u_d = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).to(dev) if u is not None else None
    ratio = torch.full((B, max(G, 1)), -7.0, dtype=torch.float32, device=dev)
    margin = torch.full((B,), -7.0, dtype=torch.float32, device=dev)
    tp = torch.full((B, G + 1, V), -1.0, device=dev) if probs else None
    dp = torch.full((B, G, V), -1.0, device=dev) if (probs and zd is not None) else None
    tau, out = bd.verify_block(zt_d, zd_d, dt_d, u_d, T, k, p, target_probs=tp, draft_probs=dp,
                               accept_ratio=ratio, sample_margin=margin)
    torch.cuda.synchronize()
    res = dict(tau=tau.cpu().numpy(), out_tokens=out.cpu().numpy(), accept_ratio=ratio.cpu().numpy()[:, :G],
               sample_margin=margin.cpu().numpy())
    if probs:
        res["target_probs"] = tp.cpu().numpy()
        res["draft_probs"] = dp.cpu().numpy() if dp is not None else None
    return res


def oracle_verify(zt, zd, dt, u, T, k=0, p=1.0, **kw):
    """The oracle with the temperature and top-p the kernel receives (fp32)."""
    return ov.verify(zt, zd, dt, u, f32(T), k, f32(p), **kw)


def compare(o, g, u, greedy, label="", zt=None, zd=None, T=1.0, k=0, p=1.0):
    """Decision-exact agreement per request (tests.helpers.check_request):
    only the first decision where the paths part may differ, and only as a
    near tie on that very decision.  Prints and checks the excused count."""
    B = len(o["tau"])
    G = o["out_tokens"].shape[1] - 1
    kinds = []
    for b in range(B):
        def weights(t, b=b):
            P = ov.filtered_probs(zt[b, t], f32(T), k, f32(p))
            Q = ov.filtered_probs(zd[b, t], f32(T), k, f32(p)) if t < G else None
            return ov.draw_weights(P, Q)
        uu = u[b] if u is not None else np.zeros((G + 1, 2), np.float32)
        kind = check_request(label, b, greedy, int(o["tau"][b]), int(g["tau"][b]), o["out_tokens"][b],
                             g["out_tokens"][b], o["accept_ratio"][b], g["accept_ratio"][b], uu[:G, 0], uu[:, 1],
                             weights, NEAR)
        if kind is not None:
            kinds.append((b, kind))
    oracle_near = set(np.nonzero(o["near_ties"] > 0)[0].tolist())
    for b, kind in kinds:
        # a draw flip lies within 1e-6 of the oracle's own boundary, so the
        # oracle counted it; an accept flip may be near only on the kernel's ratio
        if kind == "draw":
            assert b in oracle_near, f"{label}: excused draw of request {b} not among the oracle's near ties"
    say(f"{label}: {B} requests, {len(kinds)} excused near-tie differences {kinds}, "
        f"oracle near-tie requests {len(oracle_near)}")
    return len(kinds)


def check_ratios(o, g):
    ro, rg = o["accept_ratio"], g["accept_ratio"]
    fin = np.isfinite(ro) & np.isfinite(rg)
    assert (np.isfinite(ro) == np.isfinite(rg)).all()
    np.testing.assert_allclose(rg[fin], ro[fin], rtol=4e-6, atol=1e-30)


def check_probs(o, g):
    assert np.abs(g["target_probs"] - o["target_probs"]).max() <= 1e-5
    if o.get("draft_probs") is not None and g.get("draft_probs") is not None:
        assert np.abs(g["draft_probs"] - o["draft_probs"]).max() <= 1e-5


def synth(B, G, V, sigma, seed, T=1.0, top_k=0):
    cfg = wl.Config("t", B=B, K=G + 1, L=1, n_q=1, n_kv=1, hd=64, d_in=64, V=V, ctx_kind="fixed", ctx_a=1,
                    temperature=T, top_k=top_k, sigma=sigma)
    st = wl.streams(seed)
    zt, zd = wl.logits(cfg, st)
    dt = wl.draft_tokens(cfg, zd, st)
    u = wl.uniforms(cfg, st)
    return zt, zd, dt, u


# ------------------------------------------------------------------ greedy
@pytest.mark.parametrize("B,G,V,sigma,seed", [(1, 7, 4096, 0.5, 0), (16, 15, 151936, wl.SIGMA_TAU5, 1),
                                              (3, 5, 1003, 0.3, 2), (2, 0, 5000, 0.3, 3), (4, 15, 8192, 0.2, 4),
                                              (5, 3, 8193, 0.2, 5)])
def test_greedy_parity(B, G, V, sigma, seed):
    say(f"greedy B={B} G={G} V={V}")
    zt, zd, dt, u = synth(B, G, V, sigma, seed, T=0.0)
    o = ov.verify(zt, None, dt, u, 0.0)
    g = run_gpu(zt, None, dt, None, 0.0)
    compare(o, g, u, greedy=True, label="greedy")


def test_greedy_ties_lowest_index():
    say("greedy ties")
    rng = np.random.default_rng(7)
    B, G, V = 32, 7, 9000
    zt = rng.integers(0, 3, (B, G + 1, V)).astype(np.float32)     # many exact ties at the maximum
    choice = np.argmax(zt, axis=-1)
    dt = np.where(rng.random((B, G)) < 0.8, choice[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
    # a few ties where the draft picks a later tied maximum
    dt[0, 0] = np.nonzero(zt[0, 0] == zt[0, 0].max())[0][1]
    o = ov.verify(zt, None, dt, np.zeros((B, G + 1, 2), np.float32), 0.0)
    g = run_gpu(zt, None, dt, None, 0.0)
    compare(o, g, None, greedy=True, label="ties")
    assert g["tau"][0] == 0


def test_greedy_config_tiny_inputs():
    say("greedy tiny config")
    r = wl.make_round(wl.CONFIGS["tiny"], parts=("verify",))
    o = ov.verify(r.z_target, None, r.draft_tokens, r.uniforms, 0.0)
    g = run_gpu(r.z_target, None, r.draft_tokens, None, 0.0)
    compare(o, g, r.uniforms, greedy=True, label="tiny")


# ------------------------------------------------------------------ sampling
@pytest.mark.parametrize("B,G,V,sigma,T,seed", [(8, 15, 20000, 1.0, 1.0, 10), (4, 3, 151936, 0.5, 0.7, 11),
                                                (6, 4, 999, 0.4, 1.3, 12), (3, 0, 3000, 0.4, 1.0, 13),
                                                (64, 2, 24, 0.6, 1.0, 14)])
def test_sampling_parity(B, G, V, sigma, T, seed):
    say(f"sampling B={B} G={G} V={V} T={T}")
    zt, zd, dt, u = synth(B, G, V, sigma, seed, T=T)
    o = oracle_verify(zt, zd, dt, u, T)
    g = run_gpu(zt, zd, dt, u, T)
    compare(o, g, u, greedy=False, label="sampling", zt=zt, zd=zd, T=T)
    check_ratios(o, g)


@pytest.mark.parametrize("B,G,V,k,p,seed", [(8, 15, 30000, 20, 0.95, 20), (4, 7, 151936, 64, 1.0, 21),
                                            (4, 7, 5000, 1, 0.9, 22), (6, 5, 12345, 20, 0.5, 23),
                                            (3, 2, 10, 5, 0.8, 24), (4, 7, 151936, 40, 0.9, 25),
                                            (2, 5, 151936, 50, 1.0, 26)])
def test_topk_topp_parity(B, G, V, k, p, seed):
    say(f"top-k B={B} G={G} V={V} k={k} p={p}")
    zt, zd, dt, u = synth(B, G, V, 0.3, seed, T=1.0, top_k=k)
    o = oracle_verify(zt, zd, dt, u, 1.0, k, p)
    g = run_gpu(zt, zd, dt, u, 1.0, k, p)
    compare(o, g, u, greedy=False, label="topk", zt=zt, zd=zd, T=1.0, k=k, p=p)
    check_ratios(o, g)


def test_topk_with_tied_logits():
    say("top-k ties")
    rng = np.random.default_rng(30)
    B, G, V = 6, 4, 20000
    zt = np.round(rng.standard_normal((B, G + 1, V)) * 2).astype(np.float32)   # heavy ties
    zd = np.round(rng.standard_normal((B, G, V)) * 2).astype(np.float32)
    dt = rng.integers(0, 40, (B, G)).astype(np.int32)
    u = rng.random((B, G + 1, 2), dtype=np.float32)
    for k, p in ((20, 0.95), (64, 1.0)):
        o = oracle_verify(zt, zd, dt, u, 1.0, k, p)
        g = run_gpu(zt, zd, dt, u, 1.0, k, p)
        compare(o, g, u, greedy=False, label=f"topk ties k={k}", zt=zt, zd=zd, T=1.0, k=k, p=p)


def structured_rows(kind, n, V, rng):
    """n rows of one kind: 0 ascending, 1 constant, 2 finite at 7 places only
    (-inf elsewhere), 3 descending."""
    if kind == 0:
        z = np.tile(np.linspace(-3.0, 3.0, V, dtype=np.float32), (n, 1))
    elif kind == 1:
        z = np.full((n, V), 0.25, np.float32)
    elif kind == 2:
        z = np.full((n, V), -np.inf, np.float32)
        for r in range(n):
            z[r, rng.choice(V, 7, replace=False)] = rng.standard_normal(7).astype(np.float32)
    else:
        z = np.tile(np.linspace(3.0, -3.0, V, dtype=np.float32), (n, 1))
    return z + (rng.standard_normal((n, V)).astype(np.float32) * 1e-3 if kind in (0, 3) else 0)


def test_topk_structured_rows_every_path():
    """Rows that drive the streaming top-k statistics through its rare paths,
    at a size where each workgroup walks several chunks: ascending logits (every
    half chunk beats the bound: list trims, undone half chunks and the k-round
    fallback), constant logits (every logit ties with the bound: the lowest
    indices are kept), fewer finite logits than k (-inf elsewhere), and
    descending logits (nothing after the first chunk)."""
    rng = np.random.default_rng(31)
    B, G, V = 32, 3, 151936
    zt = np.empty((B, G + 1, V), np.float32)
    zd = np.empty((B, G, V), np.float32)
    for b in range(B):
        zt[b] = structured_rows(b % 4, G + 1, V, rng)
        zd[b] = structured_rows(b % 4, G, V, rng)
    u = rng.random((B, G + 1, 2), dtype=np.float32)
    for k, p in ((20, 0.95), (64, 1.0)):
        # drafted tokens the drafter could draw: among its own k best
        dt = np.empty((B, G), np.int32)
        for b in range(B):
            for i in range(G):
                dt[b, i] = ov.row_order(zd[b, i])[rng.integers(0, min(k, 7))]
        say(f"top-k structured rows k={k} p={p}")
        o = oracle_verify(zt, zd, dt, u, 1.0, k, p)
        g = run_gpu(zt, zd, dt, u, 1.0, k, p)
        compare(o, g, u, greedy=False, label=f"topk structured k={k}", zt=zt, zd=zd, T=1.0, k=k, p=p)


@pytest.mark.parametrize("T,k,p", [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.8, 20, 0.95)])
def test_probabilities_within_1e5(T, k, p):
    say(f"probs T={T} k={k}")
    zt, zd, dt, u = synth(2, 3, 20000, 0.5, 40, T=max(T, 1.0), top_k=k)
    o = oracle_verify(zt, zd, dt, u, T, k, p, want_probs=True)
    if T == 0.0:
        # greedy: plain softmax of the raw logits for both rows
        o["draft_probs"] = np.stack([np.stack([ov.softmax(zd[b, i]) for i in range(3)]) for b in range(2)])
    g = run_gpu(zt, zd, dt, u, T, k, p, probs=True)
    check_probs(o, g)


def test_draft_token_out_of_range_is_rejected():
    say("out-of-range draft tokens")
    zt, zd, dt, u = synth(4, 3, 1000, 0.3, 50)
    dt[:, 0] = np.array([-1, 1000, 5000, 2 ** 30])
    g = run_gpu(zt, zd, dt, u, 1.0)
    assert (g["tau"] == 0).all()
    g2 = run_gpu(zt, None, dt, None, 0.0)
    assert (g2["tau"] == 0).all()


def test_deterministic_run_to_run():
    say("determinism")
    zt, zd, dt, u = synth(8, 15, 151936, 1.0, 60)
    a = run_gpu(zt, zd, dt, u, 1.0)
    b = run_gpu(zt, zd, dt, u, 1.0)
    for key in ("tau", "out_tokens", "accept_ratio", "sample_margin"):
        np.testing.assert_array_equal(a[key], b[key])


# ------------------------------------------------------------------ statistics on the GPU
@pytest.mark.parametrize("V,k,p", [(8, 0, 1.0), (32, 6, 0.9)])
def test_gpu_lossless_chi_square(V, k, p):
    """Many requests with the same logits and fresh (d ~ Q, u): the first
    emitted token follows the (filtered) target distribution."""
    from scipy import stats
    say(f"chi-square V={V} k={k}")
    rng = np.random.default_rng(70 + V)
    N = 200_000
    zt1 = (rng.standard_normal((2, V)) * 1.2).astype(np.float32)
    zd1 = (rng.standard_normal((1, V)) * 1.2).astype(np.float32)
    P = ov.filtered_probs(zt1[0], 1.0, k, f32(p))
    Q = ov.filtered_probs(zd1[0], 1.0, k, f32(p))
    dt = rng.choice(V, size=(N, 1), p=Q).astype(np.int32)
    u = rng.random((N, 2, 2), dtype=np.float32)
    zt = np.broadcast_to(zt1, (N, 2, V)).copy()
    zd = np.broadcast_to(zd1, (N, 1, V)).copy()
    g = run_gpu(zt, zd, dt, u, 1.0, k, p)
    first = g["out_tokens"][:, 0]
    obs = np.bincount(first, minlength=V)
    sup = P > 0
    assert obs[~sup].sum() == 0
    pv = stats.chisquare(obs[sup], N * P[sup]).pvalue
    say(f"chi-square p = {pv:.4f}")
    assert pv > 0.01
    beta = ov.acceptance_probability(P, Q)
    acc = (g["tau"] == 1).mean()
    assert abs(acc - beta) < 4 * np.sqrt(beta * (1 - beta) / N)


# ------------------------------------------------------------------ full-size workloads
def test_full_size_8b_sampling():
    """The batch-32 temperature-1 workload at full size (every request)."""
    say("full-size qwen3-8b verify")
    r = wl.make_round(wl.CONFIGS["qwen3-8b"], parts=("verify",))
    o = oracle_verify(r.z_target, r.z_draft, r.draft_tokens, r.uniforms, 1.0)
    g = run_gpu(r.z_target, r.z_draft, r.draft_tokens, r.uniforms, 1.0)
    compare(o, g, r.uniforms, greedy=False, label="qwen3-8b", zt=r.z_target, zd=r.z_draft, T=1.0)
    check_ratios(o, g)
    say(f"tau mean {g['tau'].mean():.3f}")


def test_full_size_sweep_topk_subset():
    """The batch-128 top-k/top-p workload at full size on the GPU; the oracle
    checks every 8th request (requests are independent)."""
    say("full-size sweep verify")
    r = wl.make_round(wl.CONFIGS["sweep-b128"], parts=("verify",))
    g = run_gpu(r.z_target, r.z_draft, r.draft_tokens, r.uniforms, 1.0, 20, 0.95)
    sel = np.arange(0, 128, 8)
    o = oracle_verify(r.z_target[sel], r.z_draft[sel], r.draft_tokens[sel], r.uniforms[sel], 1.0, 20, 0.95)
    gs = {k: v[sel] for k, v in g.items() if v is not None}
    compare(o, gs, r.uniforms[sel], greedy=False, label="sweep-b128", zt=r.z_target[sel], zd=r.z_draft[sel],
            T=1.0, k=20, p=0.95)
    check_ratios(o, gs)


def test_full_size_greedy_27b():
    say("full-size 27b verify")
    r = wl.make_round(wl.CONFIGS["27b-long"], parts=("verify",))
    o = ov.verify(r.z_target, None, r.draft_tokens, r.uniforms, 0.0)
    g = run_gpu(r.z_target, None, r.draft_tokens, None, 0.0)
    compare(o, g, r.uniforms, greedy=True, label="27b-long")


def test_full_size_greedy_4b():
    """Batch 1, 15 drafted tokens over the full vocabulary, greedy."""
    say("full-size 4b verify")
    r = wl.make_round(wl.CONFIGS["qwen3-4b"], parts=("verify",))
    o = ov.verify(r.z_target, None, r.draft_tokens, r.uniforms, 0.0)
    g = run_gpu(r.z_target, None, r.draft_tokens, None, 0.0)
    compare(o, g, r.uniforms, greedy=True, label="qwen3-4b")
    say(f"tau {g['tau']}")
