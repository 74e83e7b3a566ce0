"""GPU parity of draft_forward (one drafter forward over the block) against
the oracle, through the C ABI: small shapes that span several GEMM tiles and
ragged tails, and the Qwen3-8B drafter's layer and head shapes (hidden 4096,
MLP 12288, vocabulary 151936) with one layer and 160 block rows (two row
tiles, the second ragged).

Bar: logits within 2e-2 of the logit scale, and every row's top-1 token (the
drafter's greedy decision) within 2e-2 of the scale of the oracle's best
logit.  Derivation: both sides round the same intermediates to bf16 (8 bits
of mantissa, half-ulp 2^-9 = 2e-3 relative); the kernels add their products
in fp32 in another order than the fp64 oracle, so an intermediate that lands
near a bf16 rounding boundary can round the other way, one ulp (4e-3 of its
value); such flips are independent and average out over the d-long dot
products downstream, leaving logit errors of a few 1e-3 of the scale, so
2e-2 is a margin of several times over the worst row seen."""
import numpy as np
import pytest
import torch

from oracle import forward as of
from oracle.bf16 import round_f32_to_bf16
from tests.helpers import say

pytestmark = pytest.mark.gpu

TOL = 2e-2


def bits(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda().to(torch.bfloat16).view(
        torch.int16)


def check(g, o, label):
    scale = np.abs(o).max()
    err = np.abs(g - o).max() / scale
    top = np.argmax(g, 1)
    gap = (o.max(1) - o[np.arange(len(o)), top]) / scale
    say(f"  {label}: logits max err / scale {err:.2e}, top-1 agreement {(top == np.argmax(o, 1)).mean():.3f}, "
        f"worst top-1 shortfall {gap.max():.2e}")
    assert err <= TOL
    assert gap.max() <= TOL


def run(c, B, K, n_q, n_kv, ffn, ctx, **kw):
    import block_drafting_amd as bd
    layers = [{k: bits(v) for k, v in w.items()} for w in c["layers"]]
    return bd.draft_forward(bits(c["x"]), layers, bits(c["gf"]), bits(c["lm"]), bits(c["kc"]), bits(c["vc"]),
                            torch.from_numpy(np.asarray(c["base"], np.int64)).cuda(),
                            torch.from_numpy(np.asarray(c["ctx"], np.int32)).cuda(), int(max(ctx)), K, n_q, n_kv,
                            ffn, **kw)


@pytest.mark.parametrize("B,K,d,n_q,n_kv,hd,ffn,V,L,ctx,seed", [
    (2, 4, 256, 4, 2, 64, 512, 1000, 2, (30, 100), 0),
    (3, 16, 512, 8, 2, 128, 768, 3001, 2, (0, 257, 64), 1),
    (1, 8, 128, 2, 1, 128, 256, 500, 1, (40,), 2),
    (9, 16, 256, 4, 2, 64, 640, 2050, 1, (5, 0, 90, 17, 300, 1, 64, 33, 2), 3),  # M = 144: a ragged row tile
])
def test_forward_parity(B, K, d, n_q, n_kv, hd, ffn, V, L, ctx, seed):
    from tests.test_oracle_forward import make
    say(f"draft_forward B={B} K={K} d={d} n_q={n_q} n_kv={n_kv} hd={hd} ffn={ffn} V={V} L={L}")
    c = make(seed=seed, B=B, K=K, d=d, n_q=n_q, n_kv=n_kv, hd=hd, ffn=ffn, V=V, L=L, ctx=ctx)
    o = of.draft_forward(c["x"], c["layers"], c["gf"], c["lm"], c["kc"], c["vc"], c["base"], c["ctx"], B, K, n_q,
                         n_kv, hd)
    g = run(c, B, K, n_q, n_kv, ffn, ctx)
    torch.cuda.synchronize()
    check(g.cpu().numpy().astype(np.float64), o, "small")


def bf16_normal(rng, shape, std):
    """Seeded normal values rounded to bf16, as float32, generated in chunks."""
    out = np.empty(shape, np.float32)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        n = min(step, flat.size - i)
        flat[i:i + n] = round_f32_to_bf16((rng.standard_normal(n, dtype=np.float32) * np.float32(std)))
    return out


def test_forward_parity_8b_drafter_shape():
    B, K, d, n_q, n_kv, hd, ffn, V, L = 10, 16, 4096, 32, 8, 128, 12288, 151936, 1
    ctx = np.array([700, 0, 1500, 33, 4000, 128, 64, 999, 2047, 5])
    say(f"draft_forward 8B drafter shape B={B} K={K} d={d} ffn={ffn} V={V} L={L}")
    rng = np.random.default_rng(8)
    gain = lambda n: round_f32_to_bf16(1 + rng.standard_normal(n, dtype=np.float32) * np.float32(0.2))
    layers = [dict(g_attn=gain(d), w_qkv=bf16_normal(rng, ((n_q + 2 * n_kv) * hd, d), d ** -0.5), g_q=gain(hd),
                   g_k=gain(hd), w_o=bf16_normal(rng, (d, n_q * hd), (n_q * hd) ** -0.5), g_mlp=gain(d),
                   w_gu=bf16_normal(rng, (2 * ffn, d), d ** -0.5), w_down=bf16_normal(rng, (d, ffn), ffn ** -0.5))
              for _ in range(L)]
    T = int((ctx + K).sum())
    base = np.concatenate([[0], np.cumsum(ctx + K)[:-1]])
    c = dict(x=bf16_normal(rng, (B * K, d), 1.0), layers=layers, gf=gain(d), lm=bf16_normal(rng, (V, d), d ** -0.5),
             kc=bf16_normal(rng, (L, T, n_kv, hd), 1.0), vc=bf16_normal(rng, (L, T, n_kv, hd), 1.0), base=base,
             ctx=ctx)
    g = run(c, B, K, n_q, n_kv, ffn, ctx)
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    say("  oracle ...")
    o = of.draft_forward(c["x"], c["layers"], c["gf"], c["lm"], c["kc"], c["vc"], c["base"], c["ctx"], B, K, n_q,
                         n_kv, hd)
    check(g, o, "8B shape")


def test_forward_deterministic():
    """Two calls give bit-identical logits (fixed split order everywhere)."""
    from tests.test_oracle_forward import make
    B, K, d, n_q, n_kv, hd, ffn, V, L, ctx = 4, 16, 512, 8, 2, 128, 1024, 4000, 2, (10, 200, 0, 77)
    say("draft_forward twice")
    c = make(seed=5, B=B, K=K, d=d, n_q=n_q, n_kv=n_kv, hd=hd, ffn=ffn, V=V, L=L, ctx=ctx)
    a = run(c, B, K, n_q, n_kv, ffn, ctx)
    b = run(c, B, K, n_q, n_kv, ffn, ctx)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
