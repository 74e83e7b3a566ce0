"""Oracle of one drafter forward over a block (test infrastructure only).

DFlash/Spec V2 blog, A2: the drafter's layers attend to the target's
injected context K/V plus the block's own K/V, and a single forward yields
every position of the block.  Readings where the pages leave the layer open
(the drafters they describe are built on Qwen3 layers):
  * pre-norm RMSNorm (gain, eps) before attention and before the MLP, and a
    final RMSNorm before the LM head;
  * Q, K, V from one projection of the normed rows (weight rows: Q heads,
    then K heads, then V heads); every Q and K head RMS-normed over hd with
    its own gain vector (one for Q, one for K); RoPE (the inject step's
    half-split rotation) at the absolute position ctx + i of block position i;
  * attention = the block attention of this package's oracle (context window
    plus the K block keys, no mask), 1/sqrt(hd) scale;
  * residual adds after the output projection and after the MLP;
  * MLP: SiLU(gate) * up then the down projection (gate rows, then up rows);
  * logits = final-normed rows times the LM head, kept in float64;
  * every intermediate the kernels store in bf16 is rounded to bf16 here at
    the same point (normed rows, projections, rotated heads, attention
    output, residual stream, MLP hidden).
"""
import numpy as np

from .attention import block_attn
from .bf16 import round_to_bf16
from .inject import rms_norm_heads, rope_neox


def rms_norm_rows(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gain, dtype=np.float64)


def silu(x):
    return x / (1.0 + np.exp(-x))


def draft_forward(x_in, layers, final_norm, lm_head, k_cache, v_cache, cache_base, ctx_len, B, K, n_q, n_kv, hd,
                  window=0, rope_theta=1e6, eps=1e-6):
    """x_in [B*K, d]; layers: list of dicts with g_attn [d], w_qkv [(n_q+2n_kv)hd, d], g_q [hd], g_k [hd],
    w_o [d, n_q hd], g_mlp [d], w_gu [2F, d], w_down [d, F]; k_cache / v_cache [L, T_cap, n_kv, hd].
    Returns logits [B*K, V] float64."""
    x = np.asarray(x_in, dtype=np.float64)
    pos = (np.asarray(ctx_len, dtype=np.int64)[:, None] + np.arange(K)[None, :]).reshape(-1)
    for l, w in enumerate(layers):
        xn = round_to_bf16(rms_norm_rows(x, w["g_attn"], eps))
        qkv = round_to_bf16(xn @ np.asarray(w["w_qkv"], np.float64).T)
        q = qkv[:, :n_q * hd].reshape(-1, n_q, hd)
        k = qkv[:, n_q * hd:(n_q + n_kv) * hd].reshape(-1, n_kv, hd)
        v = qkv[:, (n_q + n_kv) * hd:].reshape(-1, n_kv, hd)
        q = round_to_bf16(rope_neox(rms_norm_heads(q, w["g_q"], eps), pos, rope_theta))
        k = round_to_bf16(rope_neox(rms_norm_heads(k, w["g_k"], eps), pos, rope_theta))
        att, _ = block_attn(q.reshape(B, K, n_q, hd), k.reshape(B, K, n_kv, hd), v.reshape(B, K, n_kv, hd),
                            k_cache[l], v_cache[l], cache_base, ctx_len, window)
        x = round_to_bf16(x + att.reshape(B * K, n_q * hd) @ np.asarray(w["w_o"], np.float64).T)
        xn = round_to_bf16(rms_norm_rows(x, w["g_mlp"], eps))
        gu = round_to_bf16(xn @ np.asarray(w["w_gu"], np.float64).T)
        F = gu.shape[1] // 2
        h = round_to_bf16(silu(gu[:, :F]) * gu[:, F:])
        x = round_to_bf16(x + h @ np.asarray(w["w_down"], np.float64).T)
    xn = round_to_bf16(rms_norm_rows(x, final_norm, eps))
    return xn @ np.asarray(lm_head, np.float64).T
