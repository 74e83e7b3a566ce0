"""GPU parity of select_block (transition-cache selection) against the oracle,
through the C ABI.

Candidates are integer work on the same fp32 logits: bit-exact.  The tables
add bf16 products in fp32 on the GPU and in float64 in the oracle.  A bf16 x
bf16 product is exact in fp32, so an entry z + sum_k e_k f_k differs from its
exact value only by the rounding of the r - 1 additions of the products in some
order and of the addition of z: at most (r - 1) u sum_k |e_k f_k| + u |entry|
with u = 2^-24 (the standard bound for a sum in any order).  The walk is
compared with that bound, per row: the tokens must equal the oracle's unless
the oracle's own path meets a near tie (two entries of a visited row within
twice the row's bound); in every case each step the GPU took must be within
twice the bound of the best entry of its row (recomputed in float64), and the
reported score must be within the entry's own bound of it.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import select as osel
from tests.helpers import bits_to_f64, cuda_bits, say

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def entry_bounds(E, F, a, cands, entries):
    """Rounding bound of each fp32 table entry z + E[a] . F[c] (c in cands)."""
    r = E.shape[1]
    sabs = np.abs(F[np.asarray(cands)]) @ np.abs(E[int(a)])
    return (r - 1) * U32 * sabs + U32 * np.abs(entries)


def run_gpu(z, anchor, Eb, Fb):
    import block_drafting_amd as bd
    B, G, V = z.shape
    zt = torch.from_numpy(np.ascontiguousarray(z, np.float32)).cuda()
    an = torch.from_numpy(np.asarray(anchor, np.int32)).cuda()
    sc = torch.full((B, G), -7.0, dtype=torch.float32, device="cuda")
    cd = torch.full((B, G, 16), -7, dtype=torch.int32, device="cuda")
    tok = bd.select_block(zt, an, cuda_bits(Eb), cuda_bits(Fb), scores=sc, candidates=cd)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), sc.cpu().numpy(), cd.cpu().numpy()


def check(z, anchor, Eb, Fb, label="", reqs=None):
    """GPU on the whole batch; the oracle on the requests `reqs` (all by
    default): selection is independent per request."""
    B, G, V = z.shape
    say(f"select_block {label} B={B} G={G} V={V} r={Eb.shape[1]}")
    gt, gs, gc = run_gpu(z, anchor, Eb, Fb)
    anchor = np.asarray(anchor)
    if reqs is not None:
        z, anchor, gt, gs, gc = z[reqs], anchor[reqs], gt[reqs], gs[reqs], gc[reqs]
        B = len(reqs)
    E, F = bits_to_f64(Eb), bits_to_f64(Fb)
    z64 = np.asarray(z, np.float32).astype(np.float64)
    # the oracle defines valid anchors only; an invalid one is checked for its flag
    ot, osc, oc, otab = osel.select_block(z64, np.where((anchor >= 0) & (anchor < V), anchor, 0), E, F)
    np.testing.assert_array_equal(gc, oc)
    n_diff = 0
    for b in range(B):
        valid = 0 <= anchor[b] < V
        if not valid:
            assert (gt[b] == -1).all() and np.isnan(gs[b]).all()
            continue
        # the oracle's path has a near tie?
        tie = False
        jp = 0
        for t in range(G):
            row = otab[b, t, 0] if t == 0 else otab[b, t, jp]
            prev_tok = anchor[b] if t == 0 else oc[b, t - 1, jp]
            band = 2 * entry_bounds(E, F, prev_tok, oc[b, t], row).max()
            srt = np.sort(row)[::-1]
            tie |= srt[0] - srt[1] < band
            jp = int(np.argmax(row))
        if not tie:
            np.testing.assert_array_equal(gt[b], ot[b])
        n_diff += int((gt[b] != ot[b]).any())
        # each GPU step is a best entry of its row, and its score is that entry
        prev = np.array([anchor[b]])
        for t in range(G):
            T = osel.transition_table(z64[b, t], E, F, prev, oc[b, t])
            jp_gpu = 0 if t == 0 else int(np.where(oc[b, t - 1] == gt[b, t - 1])[0][0])
            row = T[0] if t == 0 else T[jp_gpu]
            j = int(np.where(oc[b, t] == gt[b, t])[0][0])
            prev_tok = anchor[b] if t == 0 else gt[b, t - 1]
            bnd = entry_bounds(E, F, prev_tok, oc[b, t], row)
            assert row[j] >= row.max() - 2 * bnd.max(), (b, t)
            assert abs(gs[b, t] - row[j]) <= bnd[j], (b, t, gs[b, t], row[j], bnd[j])
            prev = oc[b, t]
    say(f"  requests whose path differs from the oracle's (near ties only): {n_diff}")


def tables(rng, V, r, std):
    Eb, _ = wl.bf16_normal(rng, (V, r), std=std)
    Fb, _ = wl.bf16_normal(rng, (V, r), std=std)
    return Eb, Fb


@pytest.mark.parametrize("B,G,V,r,seed", [
    (3, 5, 100, 8, 0),          # scalar rows, one chunk
    (2, 7, 1000, 64, 1),
    (4, 15, 20000, 256, 2),     # several chunks, a ragged last one
    (2, 3, 40001, 32, 3),       # V % 4 != 0: scalar loads
    (3, 6, 9000, 40, 11),       # ranks that are no multiple of the 32-element k step
    (2, 5, 17000, 200, 12),
    (1, 1, 5000, 16, 15),       # one request, one drafted position: only the anchor row
])
def test_random_parity(B, G, V, r, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, G, V)).astype(np.float32)
    Eb, Fb = tables(rng, V, r, 0.15)
    check(z, rng.integers(0, V, B), Eb, Fb, label="random")


def test_equal_logits_resolve_to_the_lower_index():
    """Integer logits: many equal values among the best; candidates are
    ordered by index among equals on both sides."""
    rng = np.random.default_rng(4)
    B, G, V, r = 2, 4, 30000, 16
    z = rng.integers(-2, 3, (B, G, V)).astype(np.float32)
    Eb, Fb = tables(rng, V, r, 0.05)
    check(z, rng.integers(0, V, B), Eb, Fb, label="ties")


def test_concentrated_maxima_take_the_exact_path():
    """The two first threads of every chunk hold its 64 largest logits: the
    first wave then keeps more threshold candidates than it has room for, and
    the chunk goes through the exact one-element-per-round selection."""
    rng = np.random.default_rng(9)
    B, G, V, r = 2, 3, 3 * 8192, 32
    z = rng.standard_normal((B, G, V)).astype(np.float32)
    e = np.arange(V)
    hot = ((e % 8192) // 4) % 256 < 2  # slots of threads 0 and 1 (vector layout)
    z[:, :, hot] += 10.0
    Eb, Fb = tables(rng, V, r, 0.15)
    check(z, rng.integers(0, V, B), Eb, Fb, label="concentrated maxima")


def test_no_transition_is_the_base_argmax():
    rng = np.random.default_rng(5)
    B, G, V, r = 3, 6, 5000, 16
    z = rng.standard_normal((B, G, V)).astype(np.float32)
    Eb = np.zeros((V, r), np.uint16)
    _, Fb = tables(rng, V, r, 0.3)
    gt, gs, _ = run_gpu(z, rng.integers(0, V, B), Eb, Fb)
    np.testing.assert_array_equal(gt, np.argmax(z, axis=2))
    np.testing.assert_array_equal(gs, np.max(z, axis=2))


def test_invalid_anchor_flags_only_that_request():
    rng = np.random.default_rng(6)
    B, G, V, r = 3, 4, 2000, 8
    z = rng.standard_normal((B, G, V)).astype(np.float32)
    Eb, Fb = tables(rng, V, r, 0.15)
    check(z, np.array([5, V + 3, -1]), Eb, Fb, label="invalid anchors")


def test_full_size_8b_draft_logits():
    """The batch-32 workload's draft logits (G = 15, V = 151936) with rank-256
    tables; every request is checked."""
    cfg = wl.CONFIGS["qwen3-8b"]
    r = wl.make_round(cfg, parts=("verify",))
    rng = np.random.default_rng(7)
    Eb, Fb = tables(rng, cfg.V, 256, 0.1)
    anchor = rng.integers(0, cfg.V, cfg.B)
    check(r.z_draft, anchor, Eb, Fb, label="8B draft logits")


def test_full_size_batch_128_sampled_requests():
    """The batch-128 workload's draft logits (lognormal contexts, G = 15,
    V = 151936), rank-256 tables: the whole batch on the GPU, every 8th
    request and the last against the oracle."""
    cfg = wl.CONFIGS["sweep-b128"]
    z_draft = wl.streams(0)["z_draft"].standard_normal((cfg.B, cfg.G, cfg.V), dtype=np.float32)
    rng = np.random.default_rng(10)
    Eb, Fb = tables(rng, cfg.V, 256, 0.1)
    anchor = rng.integers(0, cfg.V, cfg.B)
    reqs = np.unique(np.r_[np.arange(0, cfg.B, 8), cfg.B - 1])
    check(z_draft, anchor, Eb, Fb, label="batch-128 draft logits", reqs=reqs)


def test_largest_vocabulary_merges_64_chunk_lists():
    """V = 524288, the largest supported vocabulary: 64 chunk lists per
    position, one per lane of the merging wave."""
    rng = np.random.default_rng(13)
    B, G, V, r = 2, 3, 524288, 64
    z = rng.standard_normal((B, G, V)).astype(np.float32)
    Eb, Fb = tables(rng, V, r, 0.15)
    check(z, rng.integers(0, V, B), Eb, Fb, label="largest vocabulary")


@pytest.mark.parametrize("B,G", [(0, 5), (3, 0)])
def test_empty_batch_is_a_no_op(B, G):
    """No request or no drafted position: nothing is launched and the
    caller's buffers are untouched."""
    import block_drafting_amd as bd
    V, r = 1000, 8
    rng = np.random.default_rng(14)
    Eb, Fb = tables(rng, V, r, 0.15)
    z = torch.zeros((B, G, V), dtype=torch.float32, device="cuda")
    tok = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    bd.select_block(z, torch.zeros(B, dtype=torch.int32, device="cuda"), cuda_bits(Eb), cuda_bits(Fb), tokens=tok)
    torch.cuda.synchronize()
    assert (tok.cpu().numpy() == -7).all()


def test_deterministic_run_to_run():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((4, 9, 30000)).astype(np.float32)
    Eb, Fb = tables(rng, 30000, 64, 0.15)
    an = rng.integers(0, 30000, 4)
    a, b = run_gpu(z, an, Eb, Fb), run_gpu(z, an, Eb, Fb)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
