"""Oracle of the KV-injection step (test infrastructure only).

DFlash/Spec V2 blog, summary and A2: every draft layer l gets its K/V from a
projection of the target's context hidden states,
KV_draft^(l) = Projection^(l)(H_target).  A7: the projection of all layers is
one layer-batched linear map, followed by fused Norm + RoPE post-processing,
and the result is written straight into the draft KV cache before the draft
forward (immediate materialization).

Readings taken where the pages leave a step open (listed in the design notes):
  * Projection^(l) is a bias-free linear map d_in -> 2 * n_kv * hd; the weight
    rows are ordered [layer][K, V][head][dim].
  * "Norm" is an RMSNorm of each K head over its hd dims with a learned gain
    g_l (eps an argument); V gets neither norm nor RoPE.
  * RoPE is the half-split (NeoX) rotation: dim i pairs with dim i + hd/2 and
    turns by angle pos * theta^(-2i/hd), at the token's 0-based absolute
    position.
  * K and V are stored as bf16 (round to nearest even).
"""
import numpy as np

from .bf16 import round_to_bf16


def projection(h: np.ndarray, w_kv: np.ndarray) -> np.ndarray:
    """Y = H W^T in float64: one row per token, all layers' K and V columns."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(w_kv, dtype=np.float64).T


def rms_norm_heads(k: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """k: [..., hd]; each head vector is divided by sqrt(mean(k^2) + eps) and
    multiplied elementwise by the gain."""
    k = np.asarray(k, dtype=np.float64)
    ms = np.mean(k * k, axis=-1, keepdims=True)
    return k / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope_inv_freq(hd: int, theta: float) -> np.ndarray:
    """theta^(-2i/hd) for i = 0 .. hd/2 - 1."""
    i = np.arange(hd // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / hd)


def rope_neox(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate x [..., n, hd] at positions pos [...] (one per leading index):
    (x_i, x_{i+hd/2}) -> (x_i cos a - x_{i+hd/2} sin a, x_{i+hd/2} cos a + x_i sin a),
    a = pos * theta^(-2i/hd)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(hd, theta)  # [..., half]
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def inject_kv(h, w_kv, k_norm_w, row_cu, row_pos0, cache_base, k_cache, v_cache,
              L: int, n_kv: int, hd: int, rope_theta: float, rms_eps: float):
    """Project rows of H into every layer's K/V and write them into the caches.

    h          [M, d_in]   bf16-valued hidden states (concatenated target layers)
    w_kv       [L*2*n_kv*hd, d_in] bf16-valued weights, rows [l][K|V][head][dim]
    k_norm_w   [L, hd] gains, or None for ones
    row_cu     [B+1]  rows of request b are row_cu[b] .. row_cu[b+1]-1
    row_pos0   [B]    absolute position of request b's first row
    cache_base [B]    cache slot of position 0 of request b
    k_cache, v_cache  [L, T_cap, n_kv, hd] float64 arrays, updated in place with
               bf16-valued results at slot cache_base[b] + row_pos0[b] + j.
    Returns (k_cache, v_cache).
    """
    y = projection(h, w_kv)                      # [M, L*2*n_kv*hd]
    y = y.reshape(y.shape[0], L, 2, n_kv, hd)
    gains = np.ones((L, hd)) if k_norm_w is None else np.asarray(k_norm_w, dtype=np.float64)
    B = len(row_pos0)
    for b in range(B):
        r0, r1 = int(row_cu[b]), int(row_cu[b + 1])
        if r1 <= r0:
            continue
        pos = int(row_pos0[b]) + np.arange(r1 - r0)
        slots = int(cache_base[b]) + pos
        for l in range(L):
            k = y[r0:r1, l, 0]                      # [rows, n_kv, hd]
            v = y[r0:r1, l, 1]
            k = rms_norm_heads(k, gains[l], rms_eps)
            k = rope_neox(k, pos, rope_theta)
            k_cache[l, slots] = round_to_bf16(k)
            v_cache[l, slots] = round_to_bf16(v)
    return k_cache, v_cache
