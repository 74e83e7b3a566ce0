"""Pins of the block-attention oracle (CPU only): special cases with closed
forms (zero query, dominant key, GQA head mapping, window), the LSE merge of a
key partition (Didi EAGLE-3 article, 5.3), permutation invariance, and scipy's
softmax / logsumexp on random inputs."""
import math

import numpy as np
import pytest
from scipy import special

from oracle import attention as oa
from oracle.bf16 import round_to_bf16


def make(B=2, K=4, n_q=4, n_kv=2, hd=16, ctx=(7, 12), seed=0, window=0):
    rng = np.random.default_rng(seed)
    ctx = np.array(ctx)
    base = np.concatenate([[0], np.cumsum(ctx + K)[:-1]])
    T = int((ctx + K).sum())
    q = rng.standard_normal((B, K, n_q, hd))
    kb = rng.standard_normal((B, K, n_kv, hd))
    vb = rng.standard_normal((B, K, n_kv, hd))
    kc = rng.standard_normal((T, n_kv, hd))
    vc = rng.standard_normal((T, n_kv, hd))
    return q, kb, vb, kc, vc, base, ctx


def test_zero_query_gives_mean_of_visible_values():
    q, kb, vb, kc, vc, base, ctx = make()
    q[:] = 0
    for window in (0, 5):
        out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, window)
        for b in range(2):
            lo = max(0, ctx[b] - window) if window else 0
            for h in range(4):
                g = h // 2
                vis = np.concatenate([vc[base[b] + lo: base[b] + ctx[b], g], vb[b, :, g]])
                np.testing.assert_allclose(out[b, :, h], np.broadcast_to(round_to_bf16(vis.mean(0)), (4, 16)))
                np.testing.assert_allclose(lse[b, :, h], math.log(len(vis)), rtol=1e-12)


def test_dominant_key_selects_its_value():
    q, kb, vb, kc, vc, base, ctx = make(seed=1)
    b, h, g, i = 1, 3, 1, 2
    star = base[b] + 4
    kc[star, g] = q[b, i, h] * 100.0
    out, _ = oa.block_attn(q, kb, vb, kc, vc, base, ctx)
    np.testing.assert_allclose(out[b, i, h], round_to_bf16(vc[star, g]), rtol=1e-6, atol=1e-6)
    # and a dominant in-block key
    kb[b, 3, g] = q[b, i, h] * 100.0
    kc[star, g] = 0.0
    out, _ = oa.block_attn(q, kb, vb, kc, vc, base, ctx)
    np.testing.assert_allclose(out[b, i, h], round_to_bf16(vb[b, 3, g]), rtol=1e-6, atol=1e-6)


def test_gqa_head_mapping():
    q, kb, vb, kc, vc, base, ctx = make(n_q=6, n_kv=3, seed=2)
    for g in range(3):
        kc[:, g] = 0.0
        vc[:, g] = g + 1.0
        vb[:, :, g] = g + 1.0
    out, _ = oa.block_attn(q, kb, vb, kc, vc, base, ctx)
    for h in range(6):
        np.testing.assert_allclose(out[:, :, h], h // 2 + 1.0)


def test_window_equals_full_attention_on_truncated_context():
    q, kb, vb, kc, vc, base, ctx = make(ctx=(30, 9), seed=3)
    W = 10
    out_w, lse_w = oa.block_attn(q, kb, vb, kc, vc, base, ctx, window=W)
    # rebuild a cache holding only the last W context tokens of each request
    kc2 = np.concatenate([kc[base[0] + 20: base[0] + 30], kc[base[1]: base[1] + 9]])
    vc2 = np.concatenate([vc[base[0] + 20: base[0] + 30], vc[base[1]: base[1] + 9]])
    out_f, lse_f = oa.block_attn(q, kb, vb, kc2, vc2, np.array([0, 10]), np.array([10, 9]), window=0)
    np.testing.assert_array_equal(out_w, out_f)
    np.testing.assert_allclose(lse_w, lse_f, rtol=1e-13)


def test_lse_merge_of_key_partition_equals_whole():
    q, kb, vb, kc, vc, base, ctx = make(B=1, ctx=(20,), seed=4)
    scale = 1 / 4.0
    s = q[0, :, 0] @ np.concatenate([kc[:20, 0], kb[0, :, 0]]).T * scale
    vals = np.concatenate([vc[:20, 0], vb[0, :, 0]])
    parts = []
    for sl in (slice(0, 7), slice(7, 20), slice(20, 24)):
        ss = s[:, sl]
        w = special.softmax(ss, axis=1)
        parts.append((w @ vals[sl], special.logsumexp(ss, axis=1)))
    o, l = oa.merge_lse(parts)
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx)
    np.testing.assert_allclose(round_to_bf16(o), out[0, :, 0], rtol=1e-12)
    np.testing.assert_allclose(l, lse[0, :, 0], rtol=1e-12)
    o1, l1 = oa.merge_lse(parts[:1])
    np.testing.assert_allclose(o1, parts[0][0])


def test_permuting_context_keys_changes_nothing():
    q, kb, vb, kc, vc, base, ctx = make(B=1, ctx=(25,), seed=5)
    perm = np.random.default_rng(0).permutation(25)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:25], vc2[:25] = kc[perm], vc[perm]
    a = oa.block_attn(q, kb, vb, kc, vc, base, ctx)
    b = oa.block_attn(q, kb, vb, kc2, vc2, base, ctx)
    np.testing.assert_allclose(a[0], b[0], rtol=2 ** -7)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)


def test_random_case_against_scipy():
    q, kb, vb, kc, vc, base, ctx = make(B=2, K=5, n_q=8, n_kv=2, hd=32, ctx=(0, 40), seed=6)
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, window=0, scale=0.3)
    for b in range(2):
        for h in range(8):
            g = h // 4
            keys = np.concatenate([kc[base[b]: base[b] + ctx[b], g], kb[b, :, g]])
            vals = np.concatenate([vc[base[b]: base[b] + ctx[b], g], vb[b, :, g]])
            s = q[b, :, h] @ keys.T * 0.3
            np.testing.assert_allclose(out[b, :, h], round_to_bf16(special.softmax(s, axis=1) @ vals), rtol=1e-12)
            np.testing.assert_allclose(lse[b, :, h], special.logsumexp(s, axis=1), rtol=1e-12)


def test_default_scale_is_inverse_sqrt_hd():
    q, kb, vb, kc, vc, base, ctx = make(seed=7)
    a = oa.block_attn(q, kb, vb, kc, vc, base, ctx, scale=0.0)
    b = oa.block_attn(q, kb, vb, kc, vc, base, ctx, scale=1 / 4.0)
    np.testing.assert_array_equal(a[0], b[0])


# ---- causal in-block mask and per-query window (DSpine article, "principle";
# "what these weights are" for the window)

def _attn_abs_positions(q, kb, vb, kc, vc, base, ctx, window, causal, per_query, b, h, i, scale):
    """One query by brute force over absolute positions: the context token p
    sits at position p, block key j at ctx + j, the query at ctx + i."""
    n_q, n_kv = q.shape[2], kb.shape[2]
    g = h // (n_q // n_kv)
    c = int(ctx[b])
    keys, vals = [], []
    for p in range(c + q.shape[1]):
        is_block = p >= c
        if causal and is_block and p > c + i:
            continue
        if window > 0:
            if per_query and (c + i) - p >= window:
                continue
            if not per_query and not is_block and p < c - window:
                continue
        if is_block:
            keys.append(kb[b, p - c, g]); vals.append(vb[b, p - c, g])
        else:
            keys.append(kc[base[b] + p, g]); vals.append(vc[base[b] + p, g])
    s = np.array(keys) @ q[b, i, h] * scale
    return round_to_bf16(special.softmax(s) @ np.array(vals)), special.logsumexp(s)


@pytest.mark.parametrize("window,causal,per_query", [(0, True, False), (5, True, False), (5, False, True),
                                                     (3, True, True), (30, False, True), (2, False, True)])
def test_masks_match_absolute_position_brute_force(window, causal, per_query):
    q, kb, vb, kc, vc, base, ctx = make(B=3, K=6, ctx=(0, 4, 13), seed=21)
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, window, causal=causal, per_query_window=per_query)
    for b in range(3):
        for h in range(4):
            for i in range(6):
                o, l = _attn_abs_positions(q, kb, vb, kc, vc, base, ctx, window, causal, per_query, b, h, i,
                                           1 / 4.0)
                np.testing.assert_allclose(out[b, i, h], o, rtol=0, atol=1e-12)
                assert abs(lse[b, i, h] - l) < 1e-10


def test_causal_with_one_position_equals_bidirectional():
    q, kb, vb, kc, vc, base, ctx = make(K=1, seed=22)
    a = oa.block_attn(q, kb, vb, kc, vc, base, ctx)
    c = oa.block_attn(q, kb, vb, kc, vc, base, ctx, causal=True)
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1], c[1])


def test_causal_first_position_without_context_returns_its_own_value():
    q, kb, vb, kc, vc, base, ctx = make(ctx=(0, 0), seed=23)
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, causal=True)
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(out[b, 0, h], round_to_bf16(vb[b, 0, g]))
            assert abs(lse[b, 0, h] - q[b, 0, h] @ kb[b, 0, g] / 4.0) < 1e-12


def test_causal_position_t_equals_bidirectional_block_cut_after_t():
    q, kb, vb, kc, vc, base, ctx = make(K=5, seed=24)
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, window=6, causal=True)
    for t in range(5):
        o2, l2 = oa.block_attn(q[:, :t + 1], kb[:, :t + 1], vb[:, :t + 1], kc, vc, base, ctx, window=6)
        np.testing.assert_allclose(out[:, t], o2[:, t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, t], l2[:, t], rtol=0, atol=1e-12)


def test_per_query_window_row_equals_block_uniform_window_shrunk_by_position():
    # query i sees context [ctx + i + 1 - W, ctx): the block-uniform window W - i - 1
    q, kb, vb, kc, vc, base, ctx = make(K=4, ctx=(9, 12), seed=25)
    W = 8
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, W, per_query_window=True)
    for i in range(4):
        o2, l2 = oa.block_attn(q, kb, vb, kc, vc, base, ctx, W - i - 1)
        np.testing.assert_allclose(out[:, i], o2[:, i], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, i], l2[:, i], rtol=0, atol=1e-12)


def test_per_query_window_wider_than_everything_is_no_window():
    q, kb, vb, kc, vc, base, ctx = make(K=4, seed=26)
    a = oa.block_attn(q, kb, vb, kc, vc, base, ctx, 0, causal=True)
    c = oa.block_attn(q, kb, vb, kc, vc, base, ctx, int(ctx.max()) + 4, causal=True, per_query_window=True)
    np.testing.assert_allclose(a[0], c[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[1], c[1], rtol=0, atol=1e-12)


def test_causal_sliding_window_without_context_is_banded_attention():
    # ctx = 0: block position i sees block keys max(0, i - W + 1) .. i (a band)
    K, W = 7, 3
    q, kb, vb, kc, vc, base, ctx = make(B=1, K=K, n_q=2, n_kv=2, ctx=(0,), seed=27)
    out, lse = oa.block_attn(q, kb, vb, kc, vc, base, ctx, W, causal=True, per_query_window=True)
    band = np.tril(np.ones((K, K), bool)) & ~np.tril(np.ones((K, K), bool), -W)
    for h in range(2):
        s = q[0, :, h] @ kb[0, :, h].T / 4.0
        s = np.where(band, s, -np.inf)
        np.testing.assert_allclose(out[0, :, h], round_to_bf16(special.softmax(s, axis=1) @ vb[0, :, h]),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, :, h], special.logsumexp(s, axis=1), rtol=0, atol=1e-12)
