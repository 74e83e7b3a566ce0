"""Multi-round driver of the drafting path: inject_kv, L x draft_block_attn,
verify_block, then the commit between rounds.

DFlash/Spec V2 blog, A7 (overlap scheduling): host-device synchronisation
between speculative rounds is the first bottleneck once the kernels are fast;
Spec V2 overlaps the host clean-up of round N-1 and the KV allocation of
round N with the device work.  Three ways to chain rounds:

  * ``synced``:  after each round the host reads tau, advances the context
    lengths and uploads them before launching the next round (the device
    waits for the host every round);
  * ``chained``: ``commit_round`` advances the context lengths on the device,
    so the next round is launched without waiting; the committed tokens reach
    the host through an asynchronous copy that the host reads one round late;
  * ``graph``:   the chained round (all kernels and the commit) is captured
    once in a HIP graph and replayed, which also removes the per-kernel launch
    work from the host.

Each round first materializes the K rows the previous round verified at that
block's positions (row_pos0 = the context length before the previous commit),
then attends to the context including the committed ones.  All three produce
the same results (the kernels and their inputs are the same); the runner only
marshals buffers and streams.  Every round verifies
the same logits, so tau repeats, while the contexts grow by tau + 1 per
round: the caches are laid out with room for ``rounds`` more blocks.
"""
from __future__ import annotations

import numpy as np
import torch

import block_drafting_amd as bd


class RoundRunner:
    """Owns the device buffers of a pool of B requests for up to ``rounds``
    rounds.  ``inp`` holds device tensors: h [B*K, d_in] bf16-bits, w, gains,
    q / kb / vb [L, B, K, ...], zt [B, G+1, V], zd [B, G, V] or None, dtok
    [B, G], uni [B, G+1, 2]; ``kc`` / ``vc`` [L, T_cap, n_kv, hd] hold the
    filled context; ``cache_base`` int64 [B]; ``ctx0`` / ``cap`` host int32
    [B] (cap: slots of each request)."""

    def __init__(self, cfg, inp: dict, kc, vc, cache_base, ctx0: np.ndarray, cap: np.ndarray, rounds: int):
        self.cfg = cfg
        self.inp = inp
        self.kc, self.vc = kc, vc
        self.cache_base = cache_base
        dev = kc.device
        self.dev = dev
        B, K, L = cfg.B, cfg.K, cfg.L
        self.ctx0 = np.asarray(ctx0, dtype=np.int32)
        self.cap_h = np.asarray(cap, dtype=np.int32)
        # the attention grid is sized by an upper bound of every round's contexts
        self.max_ctx = int(self.ctx0.max()) + rounds * K
        self.ctx_len = torch.from_numpy(self.ctx0.copy()).to(dev)
        self.row_pos0 = torch.from_numpy(self.ctx0.copy()).to(dev)
        self.cap = torch.from_numpy(self.cap_h.copy()).to(dev)
        self.done = torch.zeros(B, dtype=torch.int32, device=dev)
        self.row_cu = torch.arange(0, (B + 1) * K, K, dtype=torch.int32, device=dev)
        self.tau = torch.zeros(B, dtype=torch.int32, device=dev)
        self.out_tok = torch.zeros((B, cfg.G + 1), dtype=torch.int32, device=dev)
        self.attn_out = torch.zeros((L, B, K, cfg.n_q, cfg.hd), dtype=torch.int16, device=dev)
        u8 = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device=dev)
        self.ws_inj = u8(bd.inject_kv_workspace_size(B * K, cfg.d_in, L, cfg.n_kv, cfg.hd))
        self.ws_att = u8(bd.draft_block_attn_workspace_size(B, K, cfg.n_q, cfg.n_kv, cfg.hd, self.max_ctx,
                                                             cfg.window))
        self.ws_ver = u8(bd.verify_block_workspace_size(B, cfg.G, cfg.V, cfg.top_k))
        # pinned landing buffers for the committed tokens, two rounds deep
        self.h_tau = [torch.empty(B, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.h_out = [torch.empty((B, cfg.G + 1), dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.h_ev = [torch.cuda.Event() for _ in range(2)]
        self.graph = None

    # one round's kernels on the current stream; commit=True adds the device commit
    def _round(self, commit: bool):
        cfg, p = self.cfg, self.inp
        bd.inject_kv(p["h"], p["w"], p["gains"], self.row_cu, self.row_pos0, self.cache_base, self.kc, self.vc,
                     cfg.rope_theta, cfg.rms_eps, workspace=self.ws_inj)
        for l in range(cfg.L):
            bd.draft_block_attn(p["q"][l], p["kb"][l], p["vb"][l], self.kc[l], self.vc[l], self.cache_base,
                                self.ctx_len, self.max_ctx, cfg.window, out=self.attn_out[l], workspace=self.ws_att)
        bd.verify_block(p["zt"], p["zd"], p["dtok"], p["uni"], cfg.temperature, cfg.top_k, cfg.top_p, tau=self.tau,
                        out_tokens=self.out_tok, workspace=self.ws_ver)
        if commit:
            bd.commit_round(self.tau, cfg.K, self.ctx_len, row_pos0=self.row_pos0, cap=self.cap, done=self.done)

    def _land(self, slot: int):
        """Asynchronous copy of this round's tau and tokens to the pinned slot."""
        self.h_tau[slot].copy_(self.tau, non_blocking=True)
        self.h_out[slot].copy_(self.out_tok, non_blocking=True)
        self.h_ev[slot].record()

    def run_synced(self, n: int):
        """The host waits for every round, then advances the contexts itself."""
        log = []
        ctx = self.ctx0.copy()
        for _ in range(n):
            self._round(commit=False)
            tau = self.tau.cpu().numpy()             # waits for the round
            log.append((tau.copy(), self.out_tok.cpu().numpy()))
            self.row_pos0.copy_(torch.from_numpy(ctx.copy()))   # the verified block's positions
            ctx = ctx + np.where(tau >= 0, tau + 1, 0).astype(np.int32)
            self.ctx_len.copy_(torch.from_numpy(ctx))
        torch.cuda.synchronize()
        return log

    def run_chained(self, n: int):
        """Rounds back to back with the commit on the device; round i's tokens
        are read by the host while round i + 1 runs."""
        log = []
        for i in range(n):
            self._round(commit=True)
            self._land(i % 2)
            if i >= 1:
                s = (i - 1) % 2
                self.h_ev[s].synchronize()               # round i - 1 only
                log.append((self.h_tau[s].numpy().copy(), self.h_out[s].numpy().copy()))
        if n:
            s = (n - 1) % 2
            self.h_ev[s].synchronize()
            log.append((self.h_tau[s].numpy().copy(), self.h_out[s].numpy().copy()))
        return log

    def capture(self):
        """Capture one chained round (after the caller ran one eagerly, so
        every lazily initialised value is in place)."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self._round(commit=True)
        torch.cuda.synchronize()
        self.graph = g

    def run_graph(self, n: int):
        log = []
        for i in range(n):
            self.graph.replay()
            self._land(i % 2)
            if i >= 1:
                s = (i - 1) % 2
                self.h_ev[s].synchronize()
                log.append((self.h_tau[s].numpy().copy(), self.h_out[s].numpy().copy()))
        if n:
            s = (n - 1) % 2
            self.h_ev[s].synchronize()
            log.append((self.h_tau[s].numpy().copy(), self.h_out[s].numpy().copy()))
        return log

    def reset(self, ctx_h: np.ndarray = None):
        """Back to the starting contexts (the caches keep what was written:
        restore them too for a bit-identical rerun)."""
        c = torch.from_numpy((self.ctx0 if ctx_h is None else ctx_h).astype(np.int32).copy())
        self.ctx_len.copy_(c)
        self.row_pos0.copy_(c)
        self.done.zero_()
        torch.cuda.synchronize()


def layout_with_room(ctx_len: np.ndarray, K: int, rounds: int):
    """Cache slots with room for ``rounds`` more blocks per request: request b
    owns ctx_len[b] + (rounds + 1) * K slots from cache_base[b].  Returns
    (cache_base int64 [B], cap int32 [B], T_cap)."""
    span = ctx_len.astype(np.int64) + (rounds + 1) * K
    base = np.zeros(len(ctx_len), dtype=np.int64)
    base[1:] = np.cumsum(span)[:-1]
    return base, span.astype(np.int32), int(span.sum())
