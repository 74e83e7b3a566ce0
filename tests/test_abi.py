"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments on the host with the
documented status codes (no device work is started by any call here)."""
import ctypes
import os
import re

import pytest

import block_drafting_amd as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockdraft.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.lib_path()):
        from block_drafting_amd import build
        build.build()
    return bd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", text, flags=re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("inject_kv", "draft_block_attn", "verify_block", "blockdraft_last_error",
              "inject_kv_workspace_size", "draft_block_attn_workspace_size", "verify_block_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(bd.EXPORTS) <= set(declared_functions())


F = ctypes.c_float


def _verify(lib, **kw):
    a = dict(zt=1 << 20, zd=1 << 20, dt=1 << 20, u=1 << 20, B=2, G=3, V=100, T=1.0, k=0, p=1.0,
             tau=1 << 20, out=1 << 20, ws=1 << 20, wsb=1 << 30)
    a.update(kw)
    return lib.verify_block(a["zt"], a["zd"], a["dt"], a["u"], a["B"], a["G"], a["V"], F(a["T"]), a["k"], F(a["p"]),
                            a["tau"], a["out"], None, None, None, None, a["ws"], a["wsb"], None)


def test_verify_validation_codes(lib):
    assert _verify(lib, zt=None) == bd.BD_E_NULL
    assert _verify(lib, u=None) == bd.BD_E_NULL            # sampling needs uniforms
    assert _verify(lib, zd=None) == bd.BD_E_NULL
    assert _verify(lib, V=0) == bd.BD_E_SHAPE
    assert _verify(lib, G=-1) == bd.BD_E_SHAPE
    assert _verify(lib, T=-1.0) == bd.BD_E_SHAPE
    assert _verify(lib, T=float("nan")) == bd.BD_E_SHAPE
    assert _verify(lib, k=65) == bd.BD_E_UNSUPPORTED
    # top-p without a top-k filter (k = 0 or k >= V) is not supported when sampling
    assert _verify(lib, k=0, p=0.9) == bd.BD_E_UNSUPPORTED
    assert _verify(lib, V=50, k=50, p=0.9) == bd.BD_E_UNSUPPORTED
    assert _verify(lib, V=50, k=60, p=0.9) == bd.BD_E_UNSUPPORTED
    assert "top-p" in bd.last_error()
    assert _verify(lib, B=0, k=20, p=0.9) == bd.BD_OK
    assert _verify(lib, B=0, T=0.0, zd=None, u=None, k=0, p=0.9) == bd.BD_OK   # greedy ignores the filters
    assert _verify(lib, G=65) == bd.BD_E_UNSUPPORTED
    assert _verify(lib, zt=(1 << 20) + 4) == bd.BD_E_UNSUPPORTED   # misaligned logits
    assert _verify(lib, wsb=16) == bd.BD_E_WORKSPACE
    assert _verify(lib, ws=None) == bd.BD_E_WORKSPACE
    assert "workspace" in bd.last_error()
    # greedy needs neither draft logits nor uniforms; B = 0 is a no-op
    assert _verify(lib, B=0) == bd.BD_OK
    assert _verify(lib, B=0, T=0.0, zd=None, u=None) == bd.BD_OK


def _attn(lib, **kw):
    a = dict(q=1 << 20, kb=1 << 20, vb=1 << 20, kc=1 << 20, vc=1 << 20, base=1 << 20, ctx=1 << 20, T_cap=100,
             max_ctx=50, B=2, K=16, n_q=32, n_kv=8, hd=128, W=0, flags=0, out=1 << 20, ws=1 << 20, wsb=1 << 30)
    a.update(kw)
    return lib.draft_block_attn(a["q"], a["kb"], a["vb"], a["kc"], a["vc"], a["base"], a["ctx"], a["T_cap"],
                                a["max_ctx"], a["B"], a["K"], a["n_q"], a["n_kv"], a["hd"], a["W"], a["flags"], F(0.0),
                                a["out"], None, a["ws"], a["wsb"], None)


def test_attention_validation_codes(lib):
    assert _attn(lib, q=None) == bd.BD_E_NULL
    assert _attn(lib, out=None) == bd.BD_E_NULL
    assert _attn(lib, n_q=30) == bd.BD_E_SHAPE
    assert _attn(lib, K=0) == bd.BD_E_SHAPE
    assert _attn(lib, max_ctx=-1) == bd.BD_E_SHAPE
    assert _attn(lib, hd=96) == bd.BD_E_UNSUPPORTED
    assert _attn(lib, flags=4) == bd.BD_E_UNSUPPORTED                 # unknown flag bit
    assert _attn(lib, flags=-1) == bd.BD_E_UNSUPPORTED
    assert _attn(lib, K=65) == bd.BD_E_UNSUPPORTED
    assert _attn(lib, K=64, n_q=24, n_kv=8) == bd.BD_E_UNSUPPORTED    # 3 * 64 rows > 128
    assert _attn(lib, kc=(1 << 20) + 2) == bd.BD_E_UNSUPPORTED
    assert _attn(lib, wsb=0) == bd.BD_E_WORKSPACE
    assert _attn(lib, B=0) == bd.BD_OK


def _inject(lib, **kw):
    a = dict(h=1 << 20, w=1 << 20, g=None, cu=1 << 20, p0=1 << 20, base=1 << 20, kc=1 << 20, vc=1 << 20,
             T_cap=100, B=2, M=32, d_in=256, L=2, n_kv=2, hd=64, theta=1e6, eps=1e-6, ws=1 << 20, wsb=1 << 30)
    a.update(kw)
    return lib.inject_kv(a["h"], a["w"], a["g"], a["cu"], a["p0"], a["base"], a["kc"], a["vc"], a["T_cap"], a["B"],
                         a["M"], a["d_in"], a["L"], a["n_kv"], a["hd"], F(a["theta"]), F(a["eps"]), a["ws"],
                         a["wsb"], None)


def test_inject_validation_codes(lib):
    assert _inject(lib, h=None) == bd.BD_E_NULL
    assert _inject(lib, cu=None) == bd.BD_E_NULL
    assert _inject(lib, M=-1) == bd.BD_E_SHAPE
    assert _inject(lib, theta=0.0) == bd.BD_E_SHAPE
    assert _inject(lib, hd=80) == bd.BD_E_UNSUPPORTED
    assert _inject(lib, d_in=100) == bd.BD_E_UNSUPPORTED
    assert _inject(lib, w=(1 << 20) + 8) == bd.BD_E_UNSUPPORTED
    assert _inject(lib, wsb=1) == bd.BD_E_WORKSPACE
    assert _inject(lib, M=0, ws=None, wsb=0) == bd.BD_OK


def test_workspace_sizes_are_monotone(lib):
    assert bd.verify_block_workspace_size(32, 15, 151936, 0) <= bd.verify_block_workspace_size(64, 15, 151936, 0)
    assert bd.verify_block_workspace_size(8, 15, 151936, 20) > bd.verify_block_workspace_size(8, 15, 151936, 0)
    assert bd.draft_block_attn_workspace_size(0, 16, 32, 8, 128, 4096, 0) == 0
    assert bd.inject_kv_workspace_size(512, 20480, 5, 8, 128) > 0
    # a workspace sized for M rows serves every call with fewer rows
    sizes = [bd.inject_kv_workspace_size(m, 20480, 5, 8, 128) for m in (1, 16, 128, 300, 512, 1024, 3000, 8192)]
    assert sizes == sorted(sizes)
    sizes = [bd.inject_kv_workspace_size(m, 768, 2, 2, 64) for m in (1, 8, 300, 512, 5000)]
    assert sizes == sorted(sizes)


def test_product_path_has_no_fallback(tmp_path):
    with pytest.raises(RuntimeError):
        bd.load(str(tmp_path / "missing.so"))


def _ragged(lib, **kw):
    a = dict(zt=1 << 20, zd=1 << 20, dt=1 << 20, u=1 << 20, cu=1 << 20, B=2, N=7, Gm=4, V=100, T=1.0, k=0, p=1.0,
             tau=1 << 20, out=1 << 20, beta=None, ws=1 << 20, wsb=1 << 30)
    a.update(kw)
    return lib.verify_block_ragged(a["zt"], a["zd"], a["dt"], a["u"], a["cu"], a["B"], a["N"], a["Gm"], a["V"],
                                   F(a["T"]), a["k"], F(a["p"]), a["tau"], a["out"], None, None, None, None,
                                   a["beta"], a["ws"], a["wsb"], None)


def test_ragged_verify_validation_codes(lib):
    assert _ragged(lib, cu=None) == bd.BD_E_NULL
    assert _ragged(lib, zt=None) == bd.BD_E_NULL
    assert _ragged(lib, zd=None) == bd.BD_E_NULL                    # sampling needs draft logits
    assert _ragged(lib, T=0.0, zd=None, beta=1 << 20) == bd.BD_E_NULL  # labels need draft logits
    assert _ragged(lib, N=1) == bd.BD_E_SHAPE                       # fewer target rows than requests
    assert _ragged(lib, N=11) == bd.BD_E_SHAPE                      # more than B * (G_max + 1)
    assert _ragged(lib, Gm=65, N=7) == bd.BD_E_UNSUPPORTED
    assert _ragged(lib, k=65) == bd.BD_E_UNSUPPORTED
    assert _ragged(lib, k=0, p=0.95) == bd.BD_E_UNSUPPORTED          # top-p needs a top-k filter
    assert _ragged(lib, wsb=16) == bd.BD_E_WORKSPACE
    # greedy without drafts at all: only target rows; B = 0 is a no-op
    assert _ragged(lib, B=0, N=0) == bd.BD_OK


def test_ragged_workspace_grows_with_labels(lib):
    a = lib.verify_block_ragged_workspace_size(4, 40, 15, 151936, 0, 0)
    b = lib.verify_block_ragged_workspace_size(4, 40, 15, 151936, 0, 1)
    assert 0 < a < b
    assert lib.verify_block_ragged_workspace_size(4, 3, 15, 100, 0, 0) == 0   # N < B


def test_prefix_schedule_validation_codes(lib):
    c = ctypes.c_void_p
    assert lib.prefix_schedule(None, None, -1, None, None, 1, None, None) == bd.BD_E_SHAPE
    assert lib.prefix_schedule(None, None, 1, None, None, 1, None, None) == bd.BD_E_NULL


def test_commit_round_validation_codes(lib):
    assert lib.commit_round(None, 4, 16, None, None, None, None, None) == bd.BD_E_NULL
    assert lib.commit_round(None, -1, 16, None, None, None, None, None) == bd.BD_E_SHAPE
    assert lib.commit_round(None, 0, 16, None, None, None, None, None) == bd.BD_OK


def test_draft_forward_validation_codes(lib):
    def fwd(**kw):
        a = dict(x=1 << 20, B=2, K=4, d=64, L=0, nq=4, nkv=2, hd=64, ffn=128, V=100, lw=None, gf=1 << 20, lm=1 << 20,
                 kc=1 << 20, vc=1 << 20, base=1 << 20, ctx=1 << 20, T=100, maxc=50, W=0, ws=1 << 20, wsb=1 << 30)
        a.update(kw)
        return lib.draft_forward(a["x"], a["B"], a["K"], a["d"], a["L"], a["nq"], a["nkv"], a["hd"], a["ffn"], a["V"],
                                 a["lw"], a["gf"], a["lm"], a["kc"], a["vc"], a["base"], a["ctx"], a["T"], a["maxc"],
                                 a["W"], F(1e6), F(1e-6), 1 << 20, a["ws"], a["wsb"], None)
    assert fwd(x=None) == bd.BD_E_NULL
    assert fwd(L=1) == bd.BD_E_NULL              # layer weights missing
    assert fwd(nq=3) == bd.BD_E_SHAPE
    assert fwd(hd=96) == bd.BD_E_UNSUPPORTED
    assert fwd(K=65) == bd.BD_E_UNSUPPORTED
    assert fwd(wsb=16) == bd.BD_E_WORKSPACE


def test_select_block_validation_codes(lib):
    P = 1 << 20  # never dereferenced: every case fails before any launch

    def sel(**kw):
        a = dict(z=P, an=P, e=P, f=P, B=2, G=3, V=1000, r=64, tok=P, ws=P, wsb=1 << 30)
        a.update(kw)
        return lib.select_block(a["z"], a["an"], a["e"], a["f"], a["B"], a["G"], a["V"], a["r"], a["tok"], None, None,
                                a["ws"], a["wsb"], None)
    assert sel(B=-1) == bd.BD_E_SHAPE
    assert sel(V=15) == bd.BD_E_UNSUPPORTED       # fewer tokens than candidates
    assert sel(V=600000) == bd.BD_E_UNSUPPORTED
    assert sel(r=12) == bd.BD_E_UNSUPPORTED       # rank not a multiple of 8
    assert sel(r=512) == bd.BD_E_UNSUPPORTED
    assert sel(tok=None) == bd.BD_E_NULL
    assert sel(e=P + 2) == bd.BD_E_UNSUPPORTED    # tables must be 16-byte aligned
    assert sel(wsb=16) == bd.BD_E_WORKSPACE
    assert sel(B=0, z=None, tok=None) == bd.BD_OK  # nothing to do
    assert lib.select_block_workspace_size(2, 3, 1000) > 0
    assert lib.select_block_workspace_size(0, 3, 1000) == 0


def test_noalloc_verify_size_limit_on_the_host(lib):
    # the size check comes before any device call, so it runs without a GPU
    F = ctypes.c_float
    need = lib.verify_block_workspace_size(1024, 15, 151936, 64)
    assert need > bd.NOALLOC_SCRATCH_BYTES
    st = lib.verify_block_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1024, 15, 151936, F(1.0), 64, F(1.0),
                                  1 << 20, 1 << 20, None, None, None, None, None)
    assert st == bd.BD_E_WORKSPACE
    assert "static array" in bd.last_error()
    # the same argument checks as verify_block
    assert lib.verify_block_noalloc(None, 1 << 20, 1 << 20, 1 << 20, 2, 3, 100, F(1.0), 0, F(1.0), 1 << 20, 1 << 20,
                                    None, None, None, None, None) == bd.BD_E_NULL
    assert lib.verify_block_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, 2, 3, 100, F(1.0), 0, F(0.9), 1 << 20,
                                    1 << 20, None, None, None, None, None) == bd.BD_E_UNSUPPORTED
    # B = 0 needs no scratch and launches nothing
    assert lib.verify_block_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, 0, 3, 100, F(1.0), 0, F(1.0), 1 << 20,
                                    1 << 20, None, None, None, None, None) == bd.BD_OK
