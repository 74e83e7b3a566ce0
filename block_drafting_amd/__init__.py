"""Python binding of libblockdraft.so: inject_kv, draft_block_attn, verify_block.

Argument marshalling only.  Every step of the round runs in the HIP kernels
of the library; PyTorch supplies device memory (``tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``).  There is no fallback:
if the library is missing or cannot be loaded, every call raises.

bf16 tensors may be passed as ``torch.bfloat16`` or as ``torch.uint16`` /
``torch.int16`` bit patterns.  Workspaces are allocated with torch when the
caller does not pass one (``workspace=`` takes a ``torch.uint8`` CUDA tensor).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libblockdraft.so")

BD_OK, BD_E_NULL, BD_E_SHAPE, BD_E_UNSUPPORTED, BD_E_WORKSPACE, BD_E_LAUNCH = 0, -1, -2, -3, -4, -5
BD_ATTN_CAUSAL, BD_ATTN_QUERY_WINDOW = 1, 2

EXPORTS = (
    "blockdraft_last_error",
    "inject_kv_workspace_size", "inject_kv",
    "draft_block_attn_workspace_size", "draft_block_attn",
    "verify_block_workspace_size", "verify_block", "verify_block_noalloc",
    "verify_block_ragged_workspace_size", "verify_block_ragged",
    "prefix_schedule", "commit_round",
    "draft_forward_workspace_size", "draft_forward",
    "select_block_workspace_size", "select_block",
)


class BlockDraftError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"[{status}] {text}")
        self.status = status
        self.text = text


_lib = None


def lib_path() -> str:
    return LIB_PATH


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m block_drafting_amd.build`")
    L = ctypes.CDLL(p)
    c_p, c_i32, c_i64, c_f, c_sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.blockdraft_last_error.restype = ctypes.c_char_p
    L.blockdraft_last_error.argtypes = []
    L.inject_kv_workspace_size.restype = c_sz
    L.inject_kv_workspace_size.argtypes = [c_i32] * 5
    L.inject_kv.restype = ctypes.c_int
    L.inject_kv.argtypes = [c_p] * 8 + [c_i64] + [c_i32] * 6 + [c_f, c_f, c_p, c_sz, c_p]
    L.draft_block_attn_workspace_size.restype = c_sz
    L.draft_block_attn_workspace_size.argtypes = [c_i32] * 7
    L.draft_block_attn.restype = ctypes.c_int
    L.draft_block_attn.argtypes = [c_p] * 7 + [c_i64, c_i32] + [c_i32] * 5 + [c_i32, c_i32, c_f, c_p, c_p, c_p, c_sz, c_p]
    L.verify_block_workspace_size.restype = c_sz
    L.verify_block_workspace_size.argtypes = [c_i32] * 4
    L.verify_block.restype = ctypes.c_int
    L.verify_block.argtypes = [c_p] * 4 + [c_i32] * 3 + [c_f, c_i32, c_f] + [c_p] * 6 + [c_p, c_sz, c_p]
    L.verify_block_noalloc.restype = ctypes.c_int
    L.verify_block_noalloc.argtypes = [c_p] * 4 + [c_i32] * 3 + [c_f, c_i32, c_f] + [c_p] * 6 + [c_p]
    L.verify_block_ragged_workspace_size.restype = c_sz
    L.verify_block_ragged_workspace_size.argtypes = [c_i32] * 6
    L.verify_block_ragged.restype = ctypes.c_int
    L.verify_block_ragged.argtypes = [c_p] * 5 + [c_i32] * 4 + [c_f, c_i32, c_f] + [c_p] * 7 + [c_p, c_sz, c_p]
    L.draft_forward_workspace_size.restype = c_sz
    L.draft_forward_workspace_size.argtypes = [c_i32] * 9
    L.draft_forward.restype = ctypes.c_int
    L.draft_forward.argtypes = ([c_p] + [c_i32] * 9 + [c_p] * 7 + [c_i64, c_i32, c_i32, c_f, c_f, c_p, c_p, c_sz,
                                                                   c_p])
    L.commit_round.restype = ctypes.c_int
    L.commit_round.argtypes = [c_p, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p]
    L.select_block_workspace_size.restype = c_sz
    L.select_block_workspace_size.argtypes = [c_i32] * 3
    L.select_block.restype = ctypes.c_int
    L.select_block.argtypes = [c_p] * 4 + [c_i32] * 4 + [c_p] * 3 + [c_p, c_sz, c_p]
    L.prefix_schedule.restype = ctypes.c_int
    L.prefix_schedule.argtypes = [c_p, c_p, c_i32, c_p, c_p, c_i32, c_p, c_p]
    if path is None:
        _lib = L
    return L


def last_error() -> str:
    return load().blockdraft_last_error().decode()


def _check(status: int):
    if status != BD_OK:
        raise BlockDraftError(status, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("blockdraft tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("blockdraft tensors must be contiguous")
    return t.data_ptr()


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError(f"{name} must be bf16 (or its uint16 bits), got {t.dtype}")
    return t


def _typed(t: Optional[torch.Tensor], dtype, name: str):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _workspace(nbytes: int, ws: Optional[torch.Tensor], device) -> tuple:
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------- inject_kv
def inject_kv_workspace_size(M: int, d_in: int, L: int, n_kv: int, hd: int) -> int:
    return int(load().inject_kv_workspace_size(M, d_in, L, n_kv, hd))


def inject_kv(h_target, w_kv, k_norm_w, row_cu, row_pos0, cache_base, k_cache, v_cache,
              rope_theta: float = 1e6, rms_eps: float = 1e-6, workspace=None, stream=None):
    """Project hidden states into every layer's K/V cache (in place).
    k_cache / v_cache: [L, T_cap, n_kv, hd] bf16."""
    L_, T_cap, n_kv, hd = k_cache.shape
    M, d_in = h_target.shape
    B = row_pos0.shape[0]
    _bf16(h_target, "h_target"); _bf16(w_kv, "w_kv"); _bf16(k_cache, "k_cache"); _bf16(v_cache, "v_cache")
    if k_norm_w is not None:
        _bf16(k_norm_w, "k_norm_w")
    _typed(row_cu, torch.int32, "row_cu"); _typed(row_pos0, torch.int32, "row_pos0")
    _typed(cache_base, torch.int64, "cache_base")
    need = inject_kv_workspace_size(M, d_in, L_, n_kv, hd)
    ws, nb = _workspace(need, workspace, h_target.device)
    st = load().inject_kv(_ptr(h_target), _ptr(w_kv), _ptr(k_norm_w), _ptr(row_cu), _ptr(row_pos0),
                          _ptr(cache_base), _ptr(k_cache), _ptr(v_cache), T_cap, B, M, d_in, L_, n_kv, hd,
                          float(rope_theta), float(rms_eps), _ptr(ws), nb, _stream(stream))
    _check(st)
    return ws


# ---------------------------------------------------------------- draft_block_attn
def draft_block_attn_workspace_size(B, K, n_q, n_kv, hd, max_ctx, window) -> int:
    return int(load().draft_block_attn_workspace_size(B, K, n_q, n_kv, hd, max_ctx, window))


def draft_block_attn(q, k_blk, v_blk, k_cache, v_cache, cache_base, ctx_len, max_ctx: int,
                     window: int = 0, flags: int = 0, scale: float = 0.0, out=None, lse=None, workspace=None,
                     stream=None):
    """One layer of block attention. q [B,K,n_q,hd]; k_blk/v_blk [B,K,n_kv,hd];
    k_cache/v_cache [T_cap,n_kv,hd]. flags: BD_ATTN_CAUSAL | BD_ATTN_QUERY_WINDOW.
    Returns (out bf16-bits tensor, lse or None)."""
    B, K, n_q, hd = q.shape
    n_kv = k_blk.shape[2]
    T_cap = k_cache.shape[0]
    for n, t in (("q", q), ("k_blk", k_blk), ("v_blk", v_blk), ("k_cache", k_cache), ("v_cache", v_cache)):
        _bf16(t, n)
    _typed(cache_base, torch.int64, "cache_base"); _typed(ctx_len, torch.int32, "ctx_len")
    if out is None:
        out = torch.empty((B, K, n_q, hd), dtype=q.dtype, device=q.device)
    _typed(lse, torch.float32, "lse")
    need = draft_block_attn_workspace_size(B, K, n_q, n_kv, hd, max_ctx, window)
    ws, nb = _workspace(need, workspace, q.device)
    st = load().draft_block_attn(_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(cache_base), _ptr(ctx_len), T_cap, int(max_ctx), B, K, n_q, n_kv, hd,
                                 int(window), int(flags), float(scale), _ptr(out), _ptr(lse), _ptr(ws), nb, _stream(stream))
    _check(st)
    return out, lse


# ---------------------------------------------------------------- verify_block
def verify_block_workspace_size(B, G, V, top_k) -> int:
    return int(load().verify_block_workspace_size(B, G, V, top_k))


def verify_block(target_logits, draft_logits, draft_tokens, uniforms, temperature: float = 0.0,
                 top_k: int = 0, top_p: float = 1.0, tau=None, out_tokens=None, target_probs=None,
                 draft_probs=None, accept_ratio=None, sample_margin=None, workspace=None, stream=None):
    """Verify G drafted tokens per request. Returns (tau, out_tokens)."""
    B, G1, V = target_logits.shape
    G = G1 - 1
    dev = target_logits.device
    _typed(target_logits, torch.float32, "target_logits")
    _typed(draft_logits, torch.float32, "draft_logits")
    _typed(draft_tokens, torch.int32, "draft_tokens")
    _typed(uniforms, torch.float32, "uniforms")
    if tau is None:
        tau = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    need = verify_block_workspace_size(B, G, V, top_k)
    ws, nb = _workspace(need, workspace, dev)
    st = load().verify_block(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms),
                             B, G, V, float(temperature), int(top_k), float(top_p), _ptr(tau), _ptr(out_tokens),
                             _ptr(target_probs), _ptr(draft_probs), _ptr(accept_ratio), _ptr(sample_margin),
                             _ptr(ws), nb, _stream(stream))
    _check(st)
    return tau, out_tokens


NOALLOC_SCRATCH_BYTES = 32 << 20


def verify_block_noalloc(target_logits, draft_logits, draft_tokens, uniforms, temperature: float = 0.0,
                         top_k: int = 0, top_p: float = 1.0, tau=None, out_tokens=None, target_probs=None,
                         draft_probs=None, accept_ratio=None, sample_margin=None, stream=None):
    """verify_block without a workspace: the library's static per-GPU scratch
    array holds the intermediate records (calls that overlap on one GPU race).
    The outputs must be passed in when the caller cannot allocate. Returns
    (tau, out_tokens)."""
    B, G1, V = target_logits.shape
    G = G1 - 1
    dev = target_logits.device
    _typed(target_logits, torch.float32, "target_logits")
    _typed(draft_logits, torch.float32, "draft_logits")
    _typed(draft_tokens, torch.int32, "draft_tokens")
    _typed(uniforms, torch.float32, "uniforms")
    if tau is None:
        tau = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    st = load().verify_block_noalloc(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms),
                                     B, G, V, float(temperature), int(top_k), float(top_p), _ptr(tau),
                                     _ptr(out_tokens), _ptr(target_probs), _ptr(draft_probs), _ptr(accept_ratio),
                                     _ptr(sample_margin), _stream(stream))
    _check(st)
    return tau, out_tokens


def verify_block_ragged_workspace_size(B, n_target_rows, G_max, V, top_k, want_beta) -> int:
    return int(load().verify_block_ragged_workspace_size(B, n_target_rows, G_max, V, top_k, int(bool(want_beta))))


def verify_block_ragged(target_logits, draft_logits, draft_tokens, uniforms, row_cu, G_max: int,
                        temperature: float = 0.0, top_k: int = 0, top_p: float = 1.0, tau=None, out_tokens=None,
                        target_probs=None, draft_probs=None, accept_ratio=None, sample_margin=None, beta=None,
                        workspace=None, stream=None):
    """Verify requests with their own drafted lengths over packed rows
    (request b: target rows row_cu[b] .. row_cu[b+1] - 1). target_logits
    [N, V]; draft_logits [N - B, V]; row_cu int32 [B + 1] on the device.
    Returns (tau, out_tokens)."""
    N, V = target_logits.shape
    B = row_cu.shape[0] - 1
    dev = target_logits.device
    _typed(target_logits, torch.float32, "target_logits")
    _typed(draft_logits, torch.float32, "draft_logits")
    _typed(draft_tokens, torch.int32, "draft_tokens")
    _typed(uniforms, torch.float32, "uniforms")
    _typed(row_cu, torch.int32, "row_cu")
    _typed(beta, torch.float32, "beta")
    if tau is None:
        tau = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(N, dtype=torch.int32, device=dev)
    need = verify_block_ragged_workspace_size(B, N, G_max, V, top_k, beta is not None)
    ws, nb = _workspace(need, workspace, dev)
    st = load().verify_block_ragged(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms),
                                    _ptr(row_cu), B, N, int(G_max), V, float(temperature), int(top_k), float(top_p),
                                    _ptr(tau), _ptr(out_tokens), _ptr(target_probs), _ptr(draft_probs),
                                    _ptr(accept_ratio), _ptr(sample_margin), _ptr(beta), _ptr(ws), nb,
                                    _stream(stream))
    _check(st)
    return tau, out_tokens


FORWARD_WEIGHTS = ("g_attn", "w_qkv", "g_q", "g_k", "w_o", "g_mlp", "w_gu", "w_down")


def draft_forward_workspace_size(B, K, d_model, n_q, n_kv, hd, ffn, max_ctx, window) -> int:
    return int(load().draft_forward_workspace_size(B, K, d_model, n_q, n_kv, hd, ffn, max_ctx, window))


def draft_forward(x_in, layers, final_norm, lm_head, k_cache, v_cache, cache_base, ctx_len, max_ctx: int, K: int,
                  n_q: int, n_kv: int, ffn: int, window: int = 0, rope_theta: float = 1e6, rms_eps: float = 1e-6,
                  logits=None, workspace=None, stream=None):
    """One drafter forward over the block. x_in [B*K, d] bf16 bits; layers: list of
    dicts of bf16 tensors keyed by FORWARD_WEIGHTS; k_cache / v_cache [L, T_cap,
    n_kv, hd]. Returns fp32 logits [B*K, V]."""
    M, d = x_in.shape
    B = M // K
    L_ = len(layers)
    V = lm_head.shape[0]
    _, T_cap, _, hd = k_cache.shape
    _bf16(x_in, "x_in"); _bf16(lm_head, "lm_head"); _bf16(final_norm, "final_norm")
    _typed(cache_base, torch.int64, "cache_base"); _typed(ctx_len, torch.int32, "ctx_len")
    ptrs = (ctypes.c_void_p * max(1, 8 * L_))()
    for l, w in enumerate(layers):
        for j, name in enumerate(FORWARD_WEIGHTS):
            _bf16(w[name], name)
            ptrs[8 * l + j] = _ptr(w[name])
    if logits is None:
        logits = torch.empty((M, V), dtype=torch.float32, device=x_in.device)
    _typed(logits, torch.float32, "logits")
    need = draft_forward_workspace_size(B, K, d, n_q, n_kv, hd, ffn, max_ctx, window)
    ws, nb = _workspace(need, workspace, x_in.device)
    st = load().draft_forward(_ptr(x_in), B, K, d, L_, n_q, n_kv, hd, ffn, V, ctypes.cast(ptrs, ctypes.c_void_p),
                              _ptr(final_norm), _ptr(lm_head), _ptr(k_cache), _ptr(v_cache), _ptr(cache_base),
                              _ptr(ctx_len), T_cap, int(max_ctx), int(window), float(rope_theta), float(rms_eps),
                              _ptr(logits), _ptr(ws), nb, _stream(stream))
    _check(st)
    return logits


def commit_round(tau, K: int, ctx_len, row_pos0=None, cap=None, done=None, stream=None):
    """Commit a round on the device: row_pos0 = ctx_len before the update
    (where the next round materializes this round's block), then
    ctx_len += tau + 1 in place (tau >= 0); done = tau < 0 or ctx_len + K > cap."""
    for n, t in (("tau", tau), ("ctx_len", ctx_len), ("row_pos0", row_pos0), ("cap", cap), ("done", done)):
        _typed(t, torch.int32, n)
    st = load().commit_round(_ptr(tau), tau.shape[0], int(K), _ptr(ctx_len), _ptr(row_pos0), _ptr(cap), _ptr(done),
                             _stream(stream))
    _check(st)
    return ctx_len


def select_block_workspace_size(B, G, V) -> int:
    return int(load().select_block_workspace_size(B, G, V))


def select_block(logits, anchor, trans_prev, trans_next, tokens=None, scores=None, candidates=None, workspace=None,
                 stream=None):
    """Choose the G drafted tokens of each request through the transition
    cache. logits fp32 [B, G, V]; anchor int32 [B]; trans_prev / trans_next
    bf16 bits [V, r]. Returns tokens int32 [B, G] (scores fp32 [B, G] and
    candidates int32 [B, G, 16] are filled when given)."""
    B, G, V = logits.shape
    r = trans_prev.shape[1]
    dev = logits.device
    _typed(logits, torch.float32, "logits")
    _typed(anchor, torch.int32, "anchor")
    _bf16(trans_prev, "trans_prev")
    _bf16(trans_next, "trans_next")
    _typed(scores, torch.float32, "scores")
    _typed(candidates, torch.int32, "candidates")
    if tokens is None:
        tokens = torch.empty((B, G), dtype=torch.int32, device=dev)
    ws, nb = _workspace(select_block_workspace_size(B, G, V), workspace, dev)
    st = load().select_block(_ptr(logits), _ptr(anchor), _ptr(trans_prev), _ptr(trans_next), B, G, V, r,
                             _ptr(tokens), _ptr(scores), _ptr(candidates), _ptr(ws), nb, _stream(stream))
    _check(st)
    return tokens


def prefix_schedule(survival, sps_b, sps_v):
    """Host prefix scheduler. survival: list of per-request sequences of
    conditional survival probabilities; (sps_b, sps_v) the measured
    batch -> steps-per-second table. Returns (ell list, theta)."""
    import numpy as np
    R = len(survival)
    cu = np.zeros(R + 1, dtype=np.int32)
    for r, c in enumerate(survival):
        cu[r + 1] = cu[r] + len(c)
    flat = np.ascontiguousarray(np.concatenate([np.asarray(c, np.float32) for c in survival]) if R else
                                np.zeros(0, np.float32), dtype=np.float32)
    tb = np.ascontiguousarray(sps_b, dtype=np.float32)
    tv = np.ascontiguousarray(sps_v, dtype=np.float32)
    ell = np.zeros(max(R, 1), dtype=np.int32)
    theta = ctypes.c_double(0.0)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = load().prefix_schedule(P(flat) if flat.size else None, P(cu), R, P(tb), P(tv), len(tb), P(ell),
                                ctypes.byref(theta))
    _check(st)
    return [int(x) for x in ell[:R]], float(theta.value)


__all__ = ["inject_kv", "draft_block_attn", "verify_block", "verify_block_ragged", "prefix_schedule", "commit_round",
           "draft_forward", "draft_forward_workspace_size", "FORWARD_WEIGHTS",
           "inject_kv_workspace_size", "draft_block_attn_workspace_size", "verify_block_workspace_size",
           "verify_block_ragged_workspace_size", "select_block", "select_block_workspace_size", "BlockDraftError", "load", "last_error", "lib_path", "EXPORTS"]
