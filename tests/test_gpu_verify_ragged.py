"""GPU parity of verify_block_ragged (per-request drafted lengths, packed
rows, confidence labels) against the oracle, through the C ABI.

Bar: as verify_block (tau and tokens bit-exact except decisions within 1e-6
of a boundary); labels within 2e-5 absolute for the full-vocabulary sums
(fp32 probabilities, fp64 sums), 1e-6 with top-k (fp64 kept probabilities),
exact for greedy.
"""
import numpy as np
import pytest
import torch

from oracle import verify as ov
from tests.helpers import check_request, f32, say
from tests.test_gpu_verify import NEAR, synth

pytestmark = pytest.mark.gpu


def pack(zt, zd, dt, u, G_list):
    """Cut request b of a [B, G_max + 1, ...] case to its own G_b and pack."""
    zt_p = np.concatenate([zt[b, :g + 1] for b, g in enumerate(G_list)])
    zd_p = np.concatenate([zd[b, :g] for b, g in enumerate(G_list)]) if zd is not None else None
    dt_p = np.concatenate([dt[b, :g] for b, g in enumerate(G_list)]).astype(np.int32)
    u_p = np.concatenate([u[b, :g + 1] for b, g in enumerate(G_list)]).astype(np.float32)
    row_cu = np.concatenate([[0], np.cumsum(np.asarray(G_list) + 1)]).astype(np.int32)
    return zt_p, zd_p, dt_p, u_p, row_cu


def run_ragged(zt, zd, dt, u, row_cu, G_max, T, k=0, p=1.0, want_beta=True, row_cu_dev=None):
    import block_drafting_amd as bd
    dev = "cuda"
    N, V = zt.shape
    B = len(row_cu) - 1
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    beta = torch.full((max(N - B, 1),), -7.0, dtype=torch.float32, device=dev) if want_beta else None
    ratio = torch.full((max(N - B, 1),), -7.0, dtype=torch.float32, device=dev)
    margin = torch.full((B,), -7.0, dtype=torch.float32, device=dev)
    cu = t(row_cu if row_cu_dev is None else row_cu_dev)
    tau, out = bd.verify_block_ragged(t(zt), t(zd) if zd is not None else None, t(dt), t(u), cu, G_max, T, k, p,
                                      accept_ratio=ratio, sample_margin=margin, beta=beta)
    torch.cuda.synchronize()
    return dict(tau=tau.cpu().numpy(), out_tokens=out.cpu().numpy(), accept_ratio=ratio.cpu().numpy()[:N - B],
                sample_margin=margin.cpu().numpy(), beta=beta.cpu().numpy()[:N - B] if want_beta else None)


def compare(o, g, u, row_cu, greedy, label, zt=None, zd=None, T=1.0, k=0, p=1.0):
    """Decision-exact agreement per request (tests.helpers.check_request)."""
    B = len(row_cu) - 1
    kinds = []
    for b in range(B):
        t0, t1 = int(row_cu[b]), int(row_cu[b + 1])
        d0 = t0 - b
        G = t1 - t0 - 1

        def weights(t, t0=t0, d0=d0, G=G):
            P = ov.filtered_probs(zt[t0 + t], f32(T), k, f32(p))
            Q = ov.filtered_probs(zd[d0 + t], f32(T), k, f32(p)) if t < G else None
            return ov.draw_weights(P, Q)
        kind = check_request(label, b, greedy, int(o["tau"][b]), int(g["tau"][b]), o["out_tokens"][t0:t1],
                             g["out_tokens"][t0:t1], o["accept_ratio"][d0:d0 + G], g["accept_ratio"][d0:d0 + G],
                             u[t0:t0 + G, 0], u[t0:t1, 1], weights, NEAR)
        if kind is not None:
            kinds.append((b, kind))
            if kind == "draw":
                assert o["near_ties"][b] > 0, f"{label}: excused draw of request {b} not an oracle near tie"
    say(f"{label}: {B} requests, {len(kinds)} excused near-tie differences {kinds}, "
        f"oracle near-tie requests {int((o['near_ties'] > 0).sum())}")


CASES = [
    # B, G_list, V, sigma, T, top_k, top_p, seed
    (6, [0, 3, 15, 7, 1, 15], 151936, 0.5, 1.0, 0, 1.0, 70),
    (5, [2, 0, 0, 9, 4], 50000, 0.4, 0.0, 0, 1.0, 71),
    (4, [5, 1, 0, 7], 32003, 0.3, 0.7, 20, 0.9, 72),
    (7, [3, 3, 0, 1, 2, 6, 4], 8193, 0.6, 1.3, 0, 1.0, 73),
]


@pytest.mark.parametrize("B,G_list,V,sigma,T,k,p,seed", CASES)
def test_ragged_parity_and_labels(B, G_list, V, sigma, T, k, p, seed):
    say(f"ragged B={B} G={G_list} V={V} T={T} k={k}")
    G_max = max(G_list)
    zt, zd, dt, u = synth(B, G_max, V, sigma, seed, T=max(T, 1.0), top_k=k)
    zt_p, zd_p, dt_p, u_p, row_cu = pack(zt, zd, dt, u, G_list)
    o = ov.verify_ragged(zt_p, zd_p, dt_p, u_p, row_cu, f32(T), k, f32(p), want_beta=True)
    g = run_ragged(zt_p, zd_p, dt_p, u_p, row_cu, G_max, T, k, p)
    compare(o, g, u_p, row_cu, greedy=(T == 0.0), label="ragged", zt=zt_p, zd=zd_p, T=T, k=k, p=p)
    tol = 0.0 if T == 0.0 else (1e-6 if k else 2e-5)
    err = np.abs(g["beta"] - o["beta"]).max() if len(o["beta"]) else 0.0
    say(f"  label max abs err {err:.2e}")
    assert err <= tol


def test_equal_lengths_match_the_batched_entry_point():
    import block_drafting_amd as bd
    say("ragged == uniform")
    B, G, V = 8, 15, 151936
    zt, zd, dt, u = synth(B, G, V, 0.5, 74)
    zt_p, zd_p, dt_p, u_p, row_cu = pack(zt, zd, dt, u, [G] * B)
    g = run_ragged(zt_p, zd_p, dt_p, u_p, row_cu, G, 1.0, want_beta=False)
    dev = "cuda"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    tau, out = bd.verify_block(t(zt), t(zd), t(dt.astype(np.int32)), t(u.astype(np.float32)), 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g["tau"], tau.cpu().numpy())
    np.testing.assert_array_equal(g["out_tokens"], out.cpu().numpy().reshape(-1))


def test_benchmark_shape_ragged_mix():
    say("ragged B=32, G_b in 0..15, V=151936")
    rng = np.random.default_rng(75)
    G_list = [int(x) for x in rng.integers(0, 16, 32)]
    zt, zd, dt, u = synth(32, 15, 151936, 0.5, 75)
    zt_p, zd_p, dt_p, u_p, row_cu = pack(zt, zd, dt, u, G_list)
    o = ov.verify_ragged(zt_p, zd_p, dt_p, u_p, row_cu, 1.0, want_beta=True)
    g = run_ragged(zt_p, zd_p, dt_p, u_p, row_cu, 15, 1.0)
    compare(o, g, u_p, row_cu, greedy=False, label="bench mix", zt=zt_p, zd=zd_p, T=1.0)
    assert np.abs(g["beta"] - o["beta"]).max() <= 2e-5


def test_inconsistent_row_map_flags_only_that_request():
    say("invalid row map entry")
    B, G_list, V = 4, [2, 3, 1, 2], 5000
    zt, zd, dt, u = synth(B, 3, V, 0.4, 76)
    zt_p, zd_p, dt_p, u_p, row_cu = pack(zt, zd, dt, u, G_list)
    o = ov.verify_ragged(zt_p, zd_p, dt_p, u_p, row_cu, 1.0)
    bad = row_cu.copy()
    # G_max = 2 makes request 1 (G = 3) invalid; the others keep their rows
    g = run_ragged(zt_p, zd_p, dt_p, u_p, row_cu, 2, 1.0, want_beta=False, row_cu_dev=bad)
    assert g["tau"][1] == -1
    for b in (0, 2, 3):
        t0, t1 = row_cu[b], row_cu[b + 1]
        assert g["tau"][b] == o["tau"][b]
        np.testing.assert_array_equal(g["out_tokens"][t0:t1], o["out_tokens"][t0:t1])
