"""GPU parity of draft_forward (one drafter forward over the block, NEXT
row) against the oracle, through the C ABI.  Random weights scaled to keep
activations O(1); bar: logits within 3e-2 of the logit scale and the same
top-1 token on at least 90% of rows (bf16 intermediates, library GEMMs with
their own accumulation order)."""
import numpy as np
import pytest
import torch

from oracle import forward as of
from oracle.bf16 import round_to_bf16
from tests.helpers import bits_to_f64, say

pytestmark = pytest.mark.gpu


def bits(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).cuda()


@pytest.mark.parametrize("B,K,d,n_q,n_kv,hd,ffn,V,L,ctx,seed", [
    (2, 4, 256, 4, 2, 64, 512, 1000, 2, (30, 100), 0),
    (3, 16, 512, 8, 2, 128, 768, 3001, 2, (0, 257, 64), 1),
    (1, 8, 128, 2, 1, 128, 256, 500, 1, (40,), 2),
])
def test_forward_parity(B, K, d, n_q, n_kv, hd, ffn, V, L, ctx, seed):
    import block_drafting_amd as bd
    from tests.test_oracle_forward import make
    say(f"draft_forward B={B} K={K} d={d} n_q={n_q} n_kv={n_kv} hd={hd} ffn={ffn} V={V} L={L}")
    c = make(seed=seed, B=B, K=K, d=d, n_q=n_q, n_kv=n_kv, hd=hd, ffn=ffn, V=V, L=L, ctx=ctx)
    o = of.draft_forward(c["x"], c["layers"], c["gf"], c["lm"], c["kc"], c["vc"], c["base"], c["ctx"], B, K, n_q,
                         n_kv, hd)
    layers = [{k: bits(v) for k, v in w.items()} for w in c["layers"]]
    kc, vc = bits(c["kc"]), bits(c["vc"])
    g = bd.draft_forward(bits(c["x"]), layers, bits(c["gf"]), bits(c["lm"]), kc, vc,
                         torch.from_numpy(np.asarray(c["base"], np.int64)).cuda(),
                         torch.from_numpy(np.asarray(c["ctx"], np.int32)).cuda(), int(max(ctx)), K, n_q, n_kv, ffn)
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    err = np.abs(g - o).max() / np.abs(o).max()
    agree = (np.argmax(g, 1) == np.argmax(o, 1)).mean()
    say(f"  logits max err / scale {err:.2e}, top-1 agreement {agree:.3f}")
    assert err <= 3e-2
    assert agree >= 0.9
