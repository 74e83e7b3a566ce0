"""Chained rounds (NEXT row: overlap of the host bookkeeping with the device):
the device commit against the oracle, and the three ways of chaining rounds
(host-synchronised, device-chained, HIP-graph replay) against each other,
bit for bit, over several rounds with growing contexts.  The graph is
replayed several times with eager work and synchronisation in between."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import commit as oc
from tests.helpers import say

pytestmark = pytest.mark.gpu

ROUNDS = 4
CFG = wl.Config("rounds", B=4, K=16, L=2, n_q=32, n_kv=8, hd=128, d_in=1024, V=20000, ctx_kind="uniform",
                ctx_a=100, ctx_b=700, temperature=1.0, sigma=0.5)


def test_commit_kernel_matches_oracle():
    import block_drafting_amd as bd
    say("commit kernel")
    rng = np.random.default_rng(1)
    B, K = 1000, 16
    tau = rng.integers(-1, 16, B).astype(np.int32)
    ctx = rng.integers(0, 5000, B).astype(np.int32)
    cap = (ctx + rng.integers(0, 40, B)).astype(np.int32)
    t = lambda x: torch.from_numpy(x.copy()).cuda()
    c, p, d = t(ctx), torch.full((B,), -5, dtype=torch.int32, device="cuda"), torch.full((B,), -5, dtype=torch.int32,
                                                                                        device="cuda")
    bd.commit_round(t(tau), K, c, row_pos0=p, cap=t(cap), done=d)
    torch.cuda.synchronize()
    oc_ctx, oc_pos, oc_done = oc.commit_round(tau, ctx, K, cap)
    np.testing.assert_array_equal(c.cpu().numpy(), oc_ctx)
    np.testing.assert_array_equal(p.cpu().numpy(), oc_pos)
    np.testing.assert_array_equal(d.cpu().numpy(), oc_done)


def build_runner(rounds):
    import block_drafting_amd as bd
    from block_drafting_amd.runner import RoundRunner, layout_with_room
    cfg = CFG
    r = wl.make_round(cfg, seed=3)
    base, cap, T_cap = layout_with_room(r.ctx_len, cfg.K, rounds)
    dev = torch.device("cuda")
    i16 = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    kc = torch.zeros((cfg.L, T_cap, cfg.n_kv, cfg.hd), dtype=torch.int16, device=dev)
    vc = torch.zeros_like(kc)
    cb = torch.from_numpy(base).to(dev)
    w, gains = i16(r.w_bits), i16(r.k_norm_bits)
    bits, cu, first = wl.context_hidden(cfg, r.ctx_len, seed=3)
    bd.inject_kv(i16(bits), w, gains, torch.from_numpy(cu).to(dev), torch.from_numpy(first).to(dev), cb, kc, vc,
                 cfg.rope_theta, cfg.rms_eps)
    inp = dict(h=i16(r.h_round_bits), w=w, gains=gains, q=i16(r.q_bits), kb=i16(r.k_blk_bits), vb=i16(r.v_blk_bits),
               zt=torch.from_numpy(r.z_target).to(dev), zd=torch.from_numpy(r.z_draft).to(dev),
               dtok=torch.from_numpy(r.draft_tokens).to(dev), uni=torch.from_numpy(r.uniforms).to(dev))
    torch.cuda.synchronize()
    return RoundRunner(cfg, inp, kc, vc, cb, r.ctx_len, cap, rounds)


def snapshot(run):
    torch.cuda.synchronize()
    return dict(ctx=run.ctx_len.cpu().numpy().copy(), kc=run.kc.cpu().numpy().copy(), vc=run.vc.cpu().numpy().copy(),
                attn=run.attn_out.cpu().numpy().copy())


def same_log(a, b):
    assert len(a) == len(b)
    for (ta, oa), (tb, ob) in zip(a, b):
        np.testing.assert_array_equal(ta, tb)
        np.testing.assert_array_equal(oa, ob)


def same_state(a, b):
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_synced_chained_and_graph_rounds_agree():
    say(f"rounds: B={CFG.B} K={CFG.K} L={CFG.L} x {ROUNDS}")
    run = build_runner(ROUNDS)
    kc0, vc0 = run.kc.clone(), run.vc.clone()

    def restart():
        run.kc.copy_(kc0)
        run.vc.copy_(vc0)
        run.reset()

    log_s = run.run_synced(ROUNDS)
    st_s = snapshot(run)
    # contexts grew by tau + 1 per round
    tau = log_s[0][0]
    assert (st_s["ctx"] == run.ctx0 + ROUNDS * (tau + 1)).all()
    restart()
    log_c = run.run_chained(ROUNDS)
    st_c = snapshot(run)
    same_log(log_s, log_c)
    same_state(st_s, st_c)
    # graph: captured after one eager round (then restarted), replayed with
    # eager rounds and synchronisation in between
    restart()
    run.run_chained(1)
    run.capture()
    for rep in range(3):
        say(f"  graph replay pass {rep}")
        restart()
        log_g = run.run_graph(ROUNDS)
        st_g = snapshot(run)
        same_log(log_s, log_g)
        same_state(st_s, st_g)
        restart()
        run.run_chained(2)            # eager work between the replays
        torch.cuda.synchronize()
