"""verify_block_noalloc (the entry point for callers that cannot allocate)
against verify_block with a caller workspace, through the C ABI: identical
tau, tokens, ratios and margins on two calls in a row, the second with a
smaller input (the static scratch array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from tests.helpers import say
from tests.test_gpu_verify import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import block_drafting_amd as bd
    bd.load()
    return bd


def both(zt, zd, dt, u, T, k=0, p=1.0):
    import block_drafting_amd as bd
    dev = "cuda"
    B, G1, V = zt.shape
    G = G1 - 1
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev) if x is not None else None
    args = (t(zt), t(zd), t(dt.astype(np.int32)), t(u.astype(np.float32)) if u is not None else None, T, k, p)
    res = []
    for fn in (bd.verify_block, bd.verify_block_noalloc):
        ratio = torch.full((B, max(G, 1)), -7.0, dtype=torch.float32, device=dev)
        margin = torch.full((B,), -7.0, dtype=torch.float32, device=dev)
        tau = torch.full((B,), -9, dtype=torch.int32, device=dev)
        out = torch.full((B, G + 1), -9, dtype=torch.int32, device=dev)
        fn(*args, tau=tau, out_tokens=out, accept_ratio=ratio, sample_margin=margin)
        torch.cuda.synchronize()
        res.append({"tau": tau.cpu().numpy(), "out": out.cpu().numpy(), "ratio": ratio.cpu().numpy(),
                    "margin": margin.cpu().numpy()})
    for key in ("tau", "out", "ratio", "margin"):
        np.testing.assert_array_equal(res[1][key], res[0][key], err_msg=key)
    return res[0]


@pytest.mark.parametrize("first,second", [
    # (B, G, V, sigma, T, top_k, top_p, seed): full-vocabulary sampling at the batch-32 shape, then smaller
    ((32, 15, 151936, 1.0, 1.0, 0, 1.0, 90), (4, 3, 5003, 0.5, 0.7, 0, 1.0, 91)),
    # top-k / top-p at the batch-128 shape's filter, then a smaller one
    ((64, 15, 151936, 0.3, 1.0, 20, 0.95, 92), (3, 5, 12345, 0.3, 1.0, 5, 0.8, 93)),
    # greedy, then greedy with fewer drafts
    ((8, 15, 151936, 0.065, 0.0, 0, 1.0, 94), (2, 2, 1000, 0.3, 0.0, 0, 1.0, 95)),
])
def test_noalloc_matches_workspace_call_twice(first, second):
    for B, G, V, sigma, T, k, p, seed in (first, second):
        say(f"noalloc B={B} G={G} V={V} T={T} k={k} p={p}")
        zt, zd, dt, u = synth(B, G, V, sigma, seed, T=max(T, 1.0), top_k=k)
        r = both(zt, zd if T > 0 else None, dt, u if T > 0 else None, T, k, p)
        assert (r["tau"] >= 0).all()


def test_noalloc_rejects_calls_beyond_the_scratch_size():
    import block_drafting_amd as bd
    say("noalloc size limit")
    B, G, V, k = 1024, 15, 151936, 64
    need = bd.verify_block_workspace_size(B, G, V, k)
    assert need > bd.NOALLOC_SCRATCH_BYTES
    dev = "cuda"
    dummy = torch.zeros(64, dtype=torch.float32, device=dev)     # never read: the call fails before any launch
    tau = torch.full((4,), -9, dtype=torch.int32, device=dev)
    st = bd.load().verify_block_noalloc(dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                        B, G, V, 1.0, k, 1.0, tau.data_ptr(), tau.data_ptr(), None, None, None, None,
                                        None)
    assert st == bd.BD_E_WORKSPACE
    assert "static array" in bd.last_error()
    torch.cuda.synchronize()
    assert (tau.cpu().numpy() == -9).all()
