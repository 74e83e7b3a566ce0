"""GPU parity of draft_block_attn against the oracle (called through the C ABI).

Bar: per (request, layer) slice, max |gpu - oracle| / max |oracle| <= 2e-2 for
the bf16 output (bf16 inputs, fp32 accumulation); lse within 1e-3 absolute.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oa
from tests.helpers import bits_to_f64, cuda_bits, host_bits, rel_err, say

pytestmark = pytest.mark.gpu

TOL = 2e-2


def case(B, K, n_q, n_kv, hd, ctx, seed, extra_slots=0):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    base, T = wl.cache_layout(ctx, K)
    T += extra_slots
    q, _ = wl.bf16_normal(rng, (B, K, n_q, hd))
    kb, _ = wl.bf16_normal(rng, (B, K, n_kv, hd))
    vb, _ = wl.bf16_normal(rng, (B, K, n_kv, hd))
    kc, _ = wl.bf16_normal(rng, (T, n_kv, hd))
    vc, _ = wl.bf16_normal(rng, (T, n_kv, hd))
    return q, kb, vb, kc, vc, base, ctx, T


def run_gpu(q, kb, vb, kc, vc, base, ctx, window, scale=0.0, max_ctx=None, with_lse=True, flags=0):
    import block_drafting_amd as bd
    B, K, n_q, hd = q.shape
    max_ctx = int(ctx.max()) if max_ctx is None else max_ctx
    lse = torch.full((B, K, n_q), -7.0, dtype=torch.float32, device="cuda") if with_lse else None
    out, lse = bd.draft_block_attn(cuda_bits(q), cuda_bits(kb), cuda_bits(vb), cuda_bits(kc), cuda_bits(vc),
                                   torch.from_numpy(base).cuda(), torch.from_numpy(ctx).cuda(), max_ctx,
                                   window, flags=flags, scale=scale, lse=lse)
    torch.cuda.synchronize()
    return bits_to_f64(host_bits(out)), (lse.cpu().numpy() if with_lse else None)


def check(q, kb, vb, kc, vc, base, ctx, window, scale=0.0, label="", flags=0, **kw):
    say(f"attention {label} q={q.shape} ctx={list(ctx)[:6]} window={window} flags={flags}")
    go, gl = run_gpu(q, kb, vb, kc, vc, base, ctx, window, scale, flags=flags, **kw)
    oo, ol = oa.block_attn(bits_to_f64(q), bits_to_f64(kb), bits_to_f64(vb), bits_to_f64(kc), bits_to_f64(vc),
                           base, ctx, window, scale, causal=bool(flags & 1), per_query_window=bool(flags & 2))
    worst = max(rel_err(go[b], oo[b]) for b in range(q.shape[0]))
    say(f"  worst relative error {worst:.2e}, lse max abs err {np.abs(gl - ol).max():.2e}")
    assert worst <= TOL
    assert np.abs(gl - ol).max() <= 1e-3
    return worst


@pytest.mark.parametrize("window", [0, 100])
def test_tiny_config_shape(window):
    cfg = wl.CONFIGS["tiny"]
    check(*case(1, cfg.K, cfg.n_q, cfg.n_kv, cfg.hd, [512], 0)[:7], window, label="tiny")


@pytest.mark.parametrize("window", [0, 100, 64])
def test_ragged_contexts(window):
    check(*case(6, 16, 32, 8, 128, [0, 1, 63, 64, 1000, 130], 1)[:7], window, label="ragged")


def test_group5_two_row_blocks():
    # 40 query heads over 8 KV heads, K = 16: 80 query rows per item
    check(*case(2, 16, 40, 8, 128, [3000, 17], 2)[:7], 1024, label="group5")


def test_hd64_128_rows():
    check(*case(3, 64, 4, 2, 64, [700, 5, 129], 3)[:7], 0, label="hd64 K64")


def test_custom_scale_and_no_lse():
    q, kb, vb, kc, vc, base, ctx, _ = case(2, 8, 8, 2, 128, [300, 40], 4)
    check(q, kb, vb, kc, vc, base, ctx, 0, scale=0.05, label="scale")
    go, _ = run_gpu(q, kb, vb, kc, vc, base, ctx, 0, with_lse=False)
    oo, _ = oa.block_attn(bits_to_f64(q), bits_to_f64(kb), bits_to_f64(vb), bits_to_f64(kc), bits_to_f64(vc),
                          base, ctx, 0)
    assert max(rel_err(go[b], oo[b]) for b in range(2)) <= TOL


def test_max_ctx_larger_than_needed():
    q, kb, vb, kc, vc, base, ctx, _ = case(2, 16, 32, 8, 128, [200, 900], 5)
    check(q, kb, vb, kc, vc, base, ctx, 0, label="max_ctx slack", max_ctx=5000)


def test_window_never_reads_outside():
    """Slots outside the window hold NaN: any read of them would poison the output."""
    q, kb, vb, kc, vc, base, ctx, _ = case(3, 16, 32, 8, 128, [5000, 2100, 300], 6)
    W = 2048
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(3):
        lo = max(0, ctx[b] - W)
        kc2[base[b]: base[b] + lo] = 0x7FC0
        vc2[base[b]: base[b] + lo] = 0x7FC0
    go, gl = run_gpu(q, kb, vb, kc2, vc2, base, ctx, W)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    check(q, kb, vb, kc, vc, base, ctx, W, label="window")


@pytest.mark.parametrize("B,n_q,n_kv", [(3, 32, 8), (80, 16, 4)])
def test_invalid_request_metadata_gives_nan_not_fault(B, n_q, n_kv):
    """A request whose context length lies beyond max_ctx and the cache gets
    NaN outputs and lse; the others are finite.  Few (item, row block) pairs
    take the merge split over dimension groups (3 requests x 8 heads x 2 row
    blocks), many the one workgroup per pair merge (80 x 4 x 2 = 640)."""
    rng = np.random.default_rng(7)
    ctx0 = rng.integers(50, 350, B)
    q, kb, vb, kc, vc, base, ctx, T = case(B, 16, n_q, n_kv, 128, ctx0, 7)
    bad = ctx.copy()
    bad[1] = 10_000  # beyond max_ctx and beyond the cache
    go, gl = run_gpu(q, kb, vb, kc, vc, base, bad, 0, max_ctx=400)
    assert np.isnan(go[1]).all() and np.isnan(gl[1]).all()
    keep = np.arange(B) != 1
    assert np.isfinite(go[keep]).all() and np.isfinite(gl[keep]).all()


def test_deterministic_run_to_run():
    args = case(4, 16, 32, 8, 128, [1500, 77, 3000, 640], 8)[:7]
    a = run_gpu(*args, 0)
    b = run_gpu(*args, 0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_full_size_8b_layer_sampled_requests():
    """The batch-32 ragged workload (U[512, 4096] contexts) at full size on the
    GPU; the oracle checks four requests."""
    cfg = wl.CONFIGS["qwen3-8b"]
    r = wl.make_round(cfg, parts=("attn",))
    rng = np.random.default_rng(9)
    kc, _ = wl.bf16_normal(rng, (r.T_cap, cfg.n_kv, cfg.hd))
    vc, _ = wl.bf16_normal(rng, (r.T_cap, cfg.n_kv, cfg.hd))
    q, kb, vb = r.q_bits[0], r.k_blk_bits[0], r.v_blk_bits[0]
    say(f"full-size qwen3-8b layer, T_cap={r.T_cap}")
    go, gl = run_gpu(q, kb, vb, kc, vc, r.cache_base, r.ctx_len, 0, max_ctx=cfg.ctx_b)
    for b in (0, 7, 19, 31):
        sub = slice(b, b + 1)
        s0, s1 = int(r.cache_base[b]), int(r.cache_base[b] + r.ctx_len[b])
        oo, ol = oa.block_attn(bits_to_f64(q[sub]), bits_to_f64(kb[sub]), bits_to_f64(vb[sub]),
                               bits_to_f64(kc[s0:s1]), bits_to_f64(vc[s0:s1]), np.array([0]), r.ctx_len[sub], 0)
        e = rel_err(go[b], oo[0])
        say(f"  request {b} ctx={r.ctx_len[b]} rel err {e:.2e}")
        assert e <= TOL
        assert np.abs(gl[b] - ol[0]).max() <= 1e-3


def test_full_size_27b_window_sampled_requests():
    """Batch 8, 32768-token contexts, 8192-token window, 40 query heads."""
    cfg = wl.CONFIGS["27b-long"]
    r = wl.make_round(cfg, parts=("attn",))
    rng = np.random.default_rng(10)
    n_kv, hd = cfg.n_kv, cfg.hd
    # only the window (plus a NaN guard just below it) is materialised
    kc = np.full((r.T_cap, n_kv, hd), 0x7FC0, np.uint16)
    vc = np.full((r.T_cap, n_kv, hd), 0x7FC0, np.uint16)
    for b in range(cfg.B):
        lo = r.cache_base[b] + r.ctx_len[b] - cfg.window
        kc[lo: lo + cfg.window], _ = wl.bf16_normal(rng, (cfg.window, n_kv, hd))
        vc[lo: lo + cfg.window], _ = wl.bf16_normal(rng, (cfg.window, n_kv, hd))
    q, kb, vb = r.q_bits[0], r.k_blk_bits[0], r.v_blk_bits[0]
    say("full-size 27b-long layer")
    go, gl = run_gpu(q, kb, vb, kc, vc, r.cache_base, r.ctx_len, cfg.window, max_ctx=cfg.ctx_a)
    assert np.isfinite(go).all()
    for b in (0, 5):
        sub = slice(b, b + 1)
        lo = r.cache_base[b] + r.ctx_len[b] - cfg.window
        # the oracle sees a compact cache holding only the window
        oo, ol = oa.block_attn(bits_to_f64(q[sub]), bits_to_f64(kb[sub]), bits_to_f64(vb[sub]),
                               bits_to_f64(kc[lo: lo + cfg.window]), bits_to_f64(vc[lo: lo + cfg.window]),
                               np.array([0]), np.array([cfg.window]), 0)
        e = rel_err(go[b], oo[0])
        say(f"  request {b} rel err {e:.2e}")
        assert e <= TOL
        assert np.abs(gl[b] - ol[0]).max() <= 1e-3


def test_full_size_sweep_layer_sampled_requests():
    """Batch 128 with lognormal contexts (median 2048, clipped to [256, 16384]):
    short and long items share the schedule, the longest spanning many
    workgroups; the oracle checks the shortest, the longest and two others."""
    import block_drafting_amd as bd
    cfg = wl.CONFIGS["sweep-b128"]
    r = wl.make_round(cfg, parts=("attn",))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    shape = (r.T_cap, cfg.n_kv, cfg.hd)
    kc = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    vc = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    q, kb, vb = r.q_bits[0], r.k_blk_bits[0], r.v_blk_bits[0]
    max_ctx = int(r.ctx_len.max())
    say(f"full-size sweep-b128 layer, T_cap={r.T_cap} max ctx={max_ctx}")
    lse = torch.full((cfg.B, cfg.K, cfg.n_q), -7.0, dtype=torch.float32, device="cuda")
    out, lse = bd.draft_block_attn(cuda_bits(q), cuda_bits(kb), cuda_bits(vb), kc, vc,
                                   torch.from_numpy(r.cache_base).cuda(), torch.from_numpy(r.ctx_len).cuda(),
                                   max_ctx, 0, lse=lse)
    torch.cuda.synchronize()
    go, gl = bits_to_f64(host_bits(out)), lse.cpu().numpy()
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    for b in sorted({int(np.argmin(r.ctx_len)), int(np.argmax(r.ctx_len)), 17, 90}):
        sub = slice(b, b + 1)
        s0, s1 = int(r.cache_base[b]), int(r.cache_base[b] + r.ctx_len[b])
        oo, ol = oa.block_attn(bits_to_f64(q[sub]), bits_to_f64(kb[sub]), bits_to_f64(vb[sub]),
                               bits_to_f64(host_bits(kc[s0:s1])), bits_to_f64(host_bits(vc[s0:s1])),
                               np.array([0]), r.ctx_len[sub], 0)
        e = rel_err(go[b], oo[0])
        say(f"  request {b} ctx={r.ctx_len[b]} rel err {e:.2e}")
        assert e <= TOL
        assert np.abs(gl[b] - ol[0]).max() <= 1e-3


def test_one_long_item_many_partials():
    """One request, one KV head, 20000-token context: the item spans many
    workgroups, so the merge combines many partial records."""
    check(*case(1, 16, 4, 1, 64, [20000], 11)[:7], 0, label="long item")


def test_batch1_4b_shape():
    cfg = wl.CONFIGS["qwen3-4b"]
    check(*case(1, cfg.K, cfg.n_q, cfg.n_kv, cfg.hd, [cfg.ctx_a], 12)[:7], 0, label="qwen3-4b")


# ---- causal in-block mask and per-query window

CAUSAL, PER_QUERY = 1, 2


def _segment_starts_at_last_tile(ctx, K, n_kv, window=0, per_query=False):
    """Requests b (every KV head alike) one of whose partial segments holds only
    the item's last tile, under the kernel's head-synchronous schedule (each
    head's items form one sequence of tiles, cut into equal group shares of at
    least 2 tiles, at most 64 groups per item, grid at most 768 and at least
    n_kv): there a causal block gives rows that see no key of the segment."""
    TK = 32
    vis = window if (window > 0 and max(ctx) > window) else max(ctx)
    nt_max = (vis + TK - 1) // TK + 2
    tmin = max(2, (nt_max + 61) // 62)
    grid = max(n_kv, min(768, -(-len(ctx) * n_kv * nt_max // tmin)), 1)
    nts = []
    for c in ctx:
        w_lo = c + 1 - window if per_query else c - window
        lo = w_lo if (window > 0 and w_lo > 0) else 0
        nts.append((c - lo + TK - 1) // TK + (K + TK - 1) // TK)
    pref = np.concatenate([[0], np.cumsum(nts)])
    total = int(pref[-1])
    gmax = grid // n_kv
    groups = gmax if total >= gmax * tmin else max(1, total // tmin)
    starts = {total * j // groups for j in range(groups)}
    return [b for b, nt in enumerate(nts) if nt > 1 and int(pref[b]) + nt - 1 in starts]


@pytest.mark.parametrize("flags", [CAUSAL, PER_QUERY, CAUSAL | PER_QUERY])
def test_flags_ragged_contexts(flags):
    check(*case(6, 16, 32, 8, 128, [0, 1, 63, 64, 1000, 130], 31)[:7], 100, label="ragged", flags=flags)


def test_causal_no_window():
    check(*case(4, 16, 32, 8, 128, [0, 5, 700, 33], 32)[:7], 0, label="causal", flags=CAUSAL)


def test_causal_two_block_tiles_hd64():
    # K = 64: the block spans two key tiles, rows of position < 32 see none of the second
    check(*case(3, 64, 4, 2, 64, [700, 0, 129], 33)[:7], 0, label="causal K64", flags=CAUSAL)


def test_per_query_window_shorter_than_block():
    # W = 10 < K: block keys j <= i - 10 drop out as well
    check(*case(4, 16, 32, 8, 128, [0, 3, 9, 2000], 34)[:7], 10, label="W<K", flags=PER_QUERY)
    check(*case(4, 16, 32, 8, 128, [0, 3, 9, 2000], 35)[:7], 10, label="W<K causal", flags=CAUSAL | PER_QUERY)


def test_flags_group5_padding_rows():
    check(*case(2, 16, 40, 8, 128, [3000, 17], 36)[:7], 1024, label="group5", flags=CAUSAL | PER_QUERY)


def test_flags_causal_window_of_one():
    # W = 1 and causal: every query sees only its own key, so out = its value
    q, kb, vb, kc, vc, base, ctx, _ = case(2, 16, 32, 8, 128, [50, 0], 37)
    go, _ = run_gpu(q, kb, vb, kc, vc, base, ctx, 1, flags=CAUSAL | PER_QUERY)
    vbf = bits_to_f64(vb)
    for b in range(2):
        for h in range(32):
            np.testing.assert_array_equal(go[b, :, h], vbf[b, :, h // 4])
    check(q, kb, vb, kc, vc, base, ctx, 1, label="W=1 causal", flags=CAUSAL | PER_QUERY)
    check(q, kb, vb, kc, vc, base, ctx, 1, label="W=1", flags=PER_QUERY)


def test_causal_segments_that_see_no_key():
    # many partial segments; some hold only an item's last block tile, which
    # the rows of positions below 32 do not see: their records carry l = 0
    args = case(8, 64, 2, 1, 64, [2551, 1910, 1533, 809, 923, 122, 225, 49], 38)[:7]
    assert _segment_starts_at_last_tile(list(args[6]), 64, 1)
    check(*args, 0, label="empty segments", flags=CAUSAL)


def test_flags_rejects_unknown_bits():
    import block_drafting_amd as bd
    q, kb, vb, kc, vc, base, ctx, _ = case(1, 16, 32, 8, 128, [5], 39)
    with pytest.raises(RuntimeError, match="flags"):
        run_gpu(q, kb, vb, kc, vc, base, ctx, 0, flags=4)
    assert bd.BD_ATTN_CAUSAL == CAUSAL and bd.BD_ATTN_QUERY_WINDOW == PER_QUERY
