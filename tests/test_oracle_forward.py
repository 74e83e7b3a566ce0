"""Pins of the drafter-forward oracle (CPU only): one layer against the same
layer built from PyTorch's float64 library routines (rms_norm, linear,
scaled_dot_product_attention, silu), structural special cases (zeroed output
projections make a layer the identity), and closed forms of the pieces."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import forward as of
from oracle.bf16 import round_to_bf16


def make(seed=0, B=2, K=4, d=64, n_q=4, n_kv=2, hd=16, ffn=96, V=50, L=1, ctx=(5, 9)):
    rng = np.random.default_rng(seed)
    ctx = np.array(ctx)
    base = np.concatenate([[0], np.cumsum(ctx + K)[:-1]])
    T = int((ctx + K).sum())
    b16 = lambda *s, std=1.0: round_to_bf16(rng.standard_normal(s) * std)
    layers = [dict(g_attn=b16(d, std=0.2) + 1, w_qkv=b16((n_q + 2 * n_kv) * hd, d, std=d ** -0.5),
                   g_q=b16(hd, std=0.2) + 1, g_k=b16(hd, std=0.2) + 1, w_o=b16(d, n_q * hd, std=(n_q * hd) ** -0.5),
                   g_mlp=b16(d, std=0.2) + 1, w_gu=b16(2 * ffn, d, std=d ** -0.5), w_down=b16(d, ffn, std=ffn ** -0.5))
              for _ in range(L)]
    for w in layers:
        for k in ("g_attn", "g_q", "g_k", "g_mlp"):
            w[k] = round_to_bf16(w[k])
    x = b16(B * K, d)
    kc = b16(L, T, n_kv, hd)
    vc = b16(L, T, n_kv, hd)
    gf = round_to_bf16(1 + rng.standard_normal(d) * 0.2)
    lm = b16(V, d, std=d ** -0.5)
    return dict(x=x, layers=layers, gf=gf, lm=lm, kc=kc, vc=vc, base=base, ctx=ctx, B=B, K=K, n_q=n_q, n_kv=n_kv,
                hd=hd)


def torch_layer(c, theta=1e6, eps=1e-6):
    """The same forward from torch's float64 routines, bf16 rounding at the same points."""
    r = lambda t: t.to(torch.bfloat16).to(torch.float64)
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    B, K, n_q, n_kv, hd = c["B"], c["K"], c["n_q"], c["n_kv"], c["hd"]
    x = T(c["x"])
    pos = T((c["ctx"][:, None] + np.arange(K)[None, :]).reshape(-1))
    half = hd // 2
    inv = torch.pow(torch.tensor(1e6, dtype=torch.float64), -2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = pos[:, None] * inv[None, :]

    def rope(t):  # t [M, heads, hd]
        a, b = t[..., :half], t[..., half:]
        cs, sn = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        return torch.cat([a * cs - b * sn, b * cs + a * sn], dim=-1)

    for l, w in enumerate(c["layers"]):
        W = {k: T(v) for k, v in w.items()}
        xn = r(F.rms_norm(x, (x.shape[1],), W["g_attn"], eps))
        qkv = r(F.linear(xn, W["w_qkv"]))
        q = qkv[:, :n_q * hd].reshape(-1, n_q, hd)
        k = qkv[:, n_q * hd:(n_q + n_kv) * hd].reshape(-1, n_kv, hd)
        v = qkv[:, (n_q + n_kv) * hd:].reshape(-1, n_kv, hd)
        q = r(rope(F.rms_norm(q, (hd,), W["g_q"], eps)))
        k = r(rope(F.rms_norm(k, (hd,), W["g_k"], eps)))
        att = torch.zeros(B * K, n_q, hd, dtype=torch.float64)
        for b in range(B):
            lo, hi = 0, int(c["ctx"][b])
            s0 = int(c["base"][b])
            kc = T(c["kc"][l, s0 + lo:s0 + hi])
            vc = T(c["vc"][l, s0 + lo:s0 + hi])
            keys = torch.cat([kc, k[b * K:(b + 1) * K]], 0)        # [n_keys, n_kv, hd]
            vals = torch.cat([vc, v[b * K:(b + 1) * K]], 0)
            g = n_q // n_kv
            qq = q[b * K:(b + 1) * K].permute(1, 0, 2)               # [n_q, K, hd]
            kk = keys.permute(1, 0, 2).repeat_interleave(g, 0)     # [n_q, n_keys, hd]
            vv = vals.permute(1, 0, 2).repeat_interleave(g, 0)
            o = F.scaled_dot_product_attention(qq[None], kk[None], vv[None])[0]
            att[b * K:(b + 1) * K] = o.permute(1, 0, 2)
        att = r(att)
        x = r(x + F.linear(att.reshape(B * K, -1), W["w_o"]))
        xn = r(F.rms_norm(x, (x.shape[1],), W["g_mlp"], eps))
        gu = r(F.linear(xn, W["w_gu"]))
        Fh = gu.shape[1] // 2
        h = r(F.silu(gu[:, :Fh]) * gu[:, Fh:])
        x = r(x + F.linear(h, W["w_down"]))
    xn = r(F.rms_norm(x, (x.shape[1],), T(c["gf"]), eps))
    return F.linear(xn, T(c["lm"])).numpy()


@pytest.mark.parametrize("L,seed,shape", [
    (1, 0, {}), (2, 1, {}), (3, 7, {}),
    (2, 4, dict(B=3, K=8, d=256, n_q=8, n_kv=2, hd=64, ffn=320, V=300, ctx=(0, 33, 70))),
])
def test_matches_torch_library_routines(L, seed, shape):
    c = make(seed=seed, L=L, **shape)
    o = of.draft_forward(c["x"], c["layers"], c["gf"], c["lm"], c["kc"], c["vc"], c["base"], c["ctx"], c["B"], c["K"],
                         c["n_q"], c["n_kv"], c["hd"])
    t = torch_layer(c)
    # Both sides round the same float64 values to bf16 at the same points, so
    # they differ only by float64 summation order (about 1e-16 relative); that
    # moves a bf16 rounding only for a value within 1e-16 of a rounding
    # boundary (odds near 1e-13 per value), so the logits agree to float64
    # rounding and every row's argmax is the same.
    assert np.abs(o - t).max() <= 1e-12 * np.abs(t).max()
    assert (np.argmax(o, 1) == np.argmax(t, 1)).all()


def test_zero_projections_make_layers_the_identity():
    c = make(seed=2, L=2)
    for w in c["layers"]:
        w["w_o"] = np.zeros_like(w["w_o"])
        w["w_down"] = np.zeros_like(w["w_down"])
    o = of.draft_forward(c["x"], c["layers"], c["gf"], c["lm"], c["kc"], c["vc"], c["base"], c["ctx"], c["B"], c["K"],
                         c["n_q"], c["n_kv"], c["hd"])
    e = of.draft_forward(c["x"], [], c["gf"], c["lm"], c["kc"], c["vc"], c["base"], c["ctx"], c["B"], c["K"], c["n_q"],
                         c["n_kv"], c["hd"])
    np.testing.assert_array_equal(o, e)
    # no layer: the final norm and the head alone
    x = np.asarray(c["x"], np.float64)
    xn = round_to_bf16(x / np.sqrt((x * x).mean(1, keepdims=True) + 1e-6) * c["gf"])
    np.testing.assert_allclose(e, xn @ c["lm"].T, rtol=1e-12)


def test_silu_and_row_norm_closed_forms():
    x = np.array([-3.0, 0.0, 2.0, 40.0])
    np.testing.assert_allclose(of.silu(x), x / (1 + np.exp(-x)))
    assert of.silu(np.array([0.0]))[0] == 0.0 and abs(of.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    rng = np.random.default_rng(3)
    y = of.rms_norm_rows(rng.standard_normal((5, 32)), np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(1)), 1.0, rtol=1e-12)
