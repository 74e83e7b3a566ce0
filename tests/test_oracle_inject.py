"""Pins of the KV-injection oracle (CPU only): bf16 rounding against torch's
conversion, the projection against brute-force dot products, RMSNorm and RoPE
against their invariants and closed forms, and the layer/head/slot layout
against constructed one-hot cases."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16 as ob
from oracle import inject as oi


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100_000),
                        np.array([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.4e38, -3.4e38, 1e-40],
                                 dtype=np.float32)]).astype(np.float32)
    ours = ob.round_f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_ties_to_even_by_hand():
    # 1 + 2^-8 is exactly half-way between 1 and 1 + 2^-7: ties go to the even 1.0
    assert ob.round_f32_to_bf16(np.array([1 + 2 ** -8], np.float32))[0] == 1.0
    # 1 + 3*2^-8 is half-way between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert ob.round_f32_to_bf16(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 1 + 2 ** -6
    assert ob.round_f32_to_bf16(np.array([1 + 2 ** -8 + 2 ** -20], np.float32))[0] == 1 + 2 ** -7


def test_projection_brute_force():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = oi.projection(h, w)
    for m in range(3):
        for n in range(4):
            assert abs(y[m, n] - sum(h[m, k] * w[n, k] for k in range(5))) < 1e-12


def test_rmsnorm_invariants():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 4, 128)) * 3.0
    y = oi.rms_norm_heads(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(oi.rms_norm_heads(7.5 * x, np.ones(128), 0.0), y, rtol=1e-12)
    g = rng.standard_normal(128)
    np.testing.assert_allclose(oi.rms_norm_heads(x, g, 0.0), y * g, rtol=1e-12)
    # eps enters under the square root: a constant head c gives c / sqrt(c^2 + eps)
    c = np.full((1, 1, 8), 0.01)
    np.testing.assert_allclose(oi.rms_norm_heads(c, np.ones(8), 1e-4), 0.01 / math.sqrt(1e-4 + 1e-4), rtol=1e-12)


def test_rope_closed_form_pairing_and_sign():
    hd, theta = 128, 1e6
    for i in (0, 1, 17, 63):
        for pos in (0, 1, 5, 32767):
            e = np.zeros((1, 1, hd))
            e[0, 0, i] = 1.0
            r = oi.rope_neox(e, np.array([pos]), theta)[0, 0]
            a = pos * theta ** (-2.0 * i / hd)
            expect = np.zeros(hd)
            expect[i] = math.cos(a)
            expect[i + hd // 2] = math.sin(a)
            np.testing.assert_allclose(r, expect, atol=1e-12)
            # the partner dimension rotates the other way
            e2 = np.zeros((1, 1, hd))
            e2[0, 0, i + hd // 2] = 1.0
            r2 = oi.rope_neox(e2, np.array([pos]), theta)[0, 0]
            expect2 = np.zeros(hd)
            expect2[i] = -math.sin(a)
            expect2[i + hd // 2] = math.cos(a)
            np.testing.assert_allclose(r2, expect2, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    hd, theta = 64, 10000.0
    x = rng.standard_normal((5, 3, hd))
    np.testing.assert_allclose(oi.rope_neox(x, np.zeros(5), theta), x, atol=1e-15)
    pos = np.array([0, 1, 100, 4097, 32767])
    r = oi.rope_neox(x, pos, theta)
    half = hd // 2
    np.testing.assert_allclose(r[..., :half] ** 2 + r[..., half:] ** 2, x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-10)
    # relative position: <R(q, m), R(k, n)> depends on m - n only
    q, k = rng.standard_normal((2, 1, 1, hd))
    for m, n, s in [(3, 1, 10), (100, 90, 1000), (0, 7, 30000)]:
        a = (oi.rope_neox(q, np.array([m]), theta) * oi.rope_neox(k, np.array([n]), theta)).sum()
        b = (oi.rope_neox(q, np.array([m + s]), theta) * oi.rope_neox(k, np.array([n + s]), theta)).sum()
        assert abs(a - b) < 1e-9
    # composition: R(R(x, a), b) = R(x, a + b)
    a1 = oi.rope_neox(oi.rope_neox(x[:1], np.array([12]), theta), np.array([30]), theta)
    np.testing.assert_allclose(a1, oi.rope_neox(x[:1], np.array([42]), theta), atol=1e-10)


def test_inject_layout_one_hot():
    """Identity weights make Y = H, so each written K/V head is known in
    closed form: a one-hot K head c*e_j normalises to sqrt(hd/(1+eps*hd/c^2))*g_j*e_j
    and then rotates; V is copied; only the request's slots change."""
    L, n_kv, hd = 2, 2, 8
    N = L * 2 * n_kv * hd
    w = np.eye(N)
    B = 2
    row_cu = np.array([0, 2, 3])
    row_pos0 = np.array([5, 0])
    cache_base = np.array([0, 10])
    T_cap = 14
    M = 3
    h = np.zeros((M, N))
    rng = np.random.default_rng(4)
    one_hot = {}
    for m in range(M):
        for l in range(L):
            for g in range(n_kv):
                j = int(rng.integers(0, hd))
                one_hot[(m, l, g)] = j
                h[m, ((l * 2 + 0) * n_kv + g) * hd + j] = 2.0                       # K head
                h[m, ((l * 2 + 1) * n_kv + g) * hd: ((l * 2 + 1) * n_kv + g + 1) * hd] = \
                    np.arange(hd) + 100 * m + 10 * l + g                              # V head
    gains = np.array([[1.0 + 0.5 * k for k in range(hd)], [2.0] * hd])
    kc = np.full((L, T_cap, n_kv, hd), -7.0)
    vc = np.full((L, T_cap, n_kv, hd), -7.0)
    eps = 1e-6
    oi.inject_kv(h, w, gains, row_cu, row_pos0, cache_base, kc, vc, L, n_kv, hd, 1e6, eps)
    written = set()
    for b in range(B):
        for j_row, m in enumerate(range(row_cu[b], row_cu[b + 1])):
            pos = row_pos0[b] + j_row
            slot = cache_base[b] + pos
            written.add(slot)
            for l in range(L):
                for g in range(n_kv):
                    j = one_hot[(m, l, g)]
                    amp = 2.0 / math.sqrt(4.0 / hd + eps) * gains[l, j]
                    i = j % (hd // 2)
                    a = pos * 1e6 ** (-2.0 * i / hd)
                    expect = np.zeros(hd)
                    if j < hd // 2:
                        expect[j], expect[j + hd // 2] = amp * math.cos(a), amp * math.sin(a)
                    else:
                        expect[i], expect[j] = -amp * math.sin(a), amp * math.cos(a)
                    np.testing.assert_allclose(kc[l, slot, g], expect, rtol=2 ** -8, atol=1e-30)
                    np.testing.assert_array_equal(vc[l, slot, g], ob.round_to_bf16(np.arange(hd) + 100 * m + 10 * l + g))
    for s in range(T_cap):
        if s not in written:
            assert (kc[:, s] == -7.0).all() and (vc[:, s] == -7.0).all()


def test_inject_outputs_are_bf16_values():
    rng = np.random.default_rng(5)
    L, n_kv, hd, d_in = 1, 1, 16, 32
    h = ob.round_to_bf16(rng.standard_normal((4, d_in)))
    w = ob.round_to_bf16(rng.standard_normal((L * 2 * n_kv * hd, d_in)) * 0.1)
    kc = np.zeros((L, 4, n_kv, hd))
    vc = np.zeros((L, 4, n_kv, hd))
    oi.inject_kv(h, w, None, np.array([0, 4]), np.array([0]), np.array([0]), kc, vc, L, n_kv, hd, 1e4, 1e-6)
    for arr in (kc, vc):
        np.testing.assert_array_equal(ob.round_to_bf16(arr), arr)
