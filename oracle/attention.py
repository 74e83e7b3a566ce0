"""Oracle of the block-draft attention (test infrastructure only).

DFlash/Spec V2 blog, A2: the drafter attends, in every layer, to the context
K/V injected from the target, and one forward produces the whole block.
DSpine article, "principle": in DFlash the positions inside a block see each
other in both directions (DSpine restricts this to earlier positions; that
variant is not this function).  DSpine article, "what these weights are": the
drafter's attention uses an 8192-token sliding window.  DSpine article,
"principle": DSpine's own drafter keeps the block causal (a position sees only
the earlier positions of its block); ``causal=True`` gives that variant.

Readings taken where the pages leave a step open:
  * by default every query of a block sees the same keys: the last ``window``
    context positions [max(0, ctx - window), ctx) (all of them when
    window == 0), followed by the K in-block keys; no mask;
  * ``per_query_window=True`` reads the window per query instead, as a
    sliding window over absolute positions: block position i sits at position
    ctx + i, and sees a key at position p only when ctx + i - p < window;
  * ``causal=True`` hides block key j from block position i when j > i;
  * grouped-query attention: query head h reads KV head h // (n_q / n_kv);
  * scores are q.k * scale with scale = 1/sqrt(hd) unless given;
  * the output is rounded to bf16; lse is the natural log of the sum of
    exp(score).
The definition is the plain softmax(q K^T * scale) V, in float64.
"""
import numpy as np

from .bf16 import round_to_bf16


def visible_range(ctx: int, window: int):
    lo = max(0, ctx - window) if window > 0 else 0
    return lo, ctx


def key_mask(ctx: int, K: int, window: int, causal: bool = False, per_query_window: bool = False):
    """Which keys each block position sees.  Returns (lo, hi, mask) where the
    candidate keys are the context positions [lo, hi) followed by the K block
    keys, and mask[i, k] says whether block position i sees candidate k."""
    if per_query_window and window > 0:
        lo, hi = max(0, ctx + 1 - window), ctx   # the widest query: position 0
    else:
        lo, hi = visible_range(ctx, window)
    n = hi - lo
    mask = np.ones((K, n + K), dtype=bool)
    for i in range(K):
        if per_query_window and window > 0:
            for c in range(n):
                mask[i, c] = (ctx + i) - (lo + c) < window
            for j in range(K):
                mask[i, n + j] = i - j < window
        if causal:
            for j in range(i + 1, K):
                mask[i, n + j] = False
    return lo, hi, mask


def block_attn(q, k_blk, v_blk, k_cache, v_cache, cache_base, ctx_len, window: int = 0,
               scale: float = 0.0, causal: bool = False, per_query_window: bool = False):
    """q [B, K, n_q, hd]; k_blk, v_blk [B, K, n_kv, hd]; k_cache, v_cache
    [T_cap, n_kv, hd] (one layer); cache_base int [B]; ctx_len int [B].
    Returns (out [B, K, n_q, hd] float64 with bf16 values, lse [B, K, n_q])."""
    q = np.asarray(q, dtype=np.float64)
    B, K, n_q, hd = q.shape
    n_kv = k_blk.shape[2]
    group = n_q // n_kv
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(hd)
    out = np.zeros((B, K, n_q, hd))
    lse = np.zeros((B, K, n_q))
    for b in range(B):
        lo, hi, mask = key_mask(int(ctx_len[b]), K, window, causal, per_query_window)
        base = int(cache_base[b])
        for g in range(n_kv):
            keys = np.concatenate([np.asarray(k_cache[base + lo: base + hi, g], dtype=np.float64),
                                   np.asarray(k_blk[b, :, g], dtype=np.float64)], axis=0)
            vals = np.concatenate([np.asarray(v_cache[base + lo: base + hi, g], dtype=np.float64),
                                   np.asarray(v_blk[b, :, g], dtype=np.float64)], axis=0)
            for h in range(g * group, (g + 1) * group):
                s = q[b, :, h, :] @ keys.T * scale          # [K, n_keys]
                s = np.where(mask, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                out[b, :, h, :] = (e / z) @ vals
                lse[b, :, h] = (m + np.log(z))[:, 0]
    return round_to_bf16(out), lse


def merge_lse(parts):
    """Merge partial results [(o_i, lse_i)] of one query over disjoint key sets,
    each o_i already normalised over its own keys (Didi EAGLE-3 article, 5.3:
    the streaming-softmax fusion of main and branch parts).  Returns (o, lse)."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    o = sum(wi[..., None] * np.asarray(p[0], dtype=np.float64) for wi, p in zip(w, parts)) / tot[..., None]
    return o, m + np.log(tot)
