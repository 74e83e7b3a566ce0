"""GPU parity of inject_kv against the oracle (called through the C ABI).

Bar: for every written slot, per layer, max |gpu - oracle| / max |oracle|
<= 2e-2 for K and for V (bf16 inputs, fp32 accumulation, bf16 outputs); every
slot the call must not write keeps its old bits.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import inject as oi
from tests.helpers import bits_to_f64, cuda_bits, host_bits, rel_err, say

pytestmark = pytest.mark.gpu

TOL = 2e-2
SENTINEL = 0x3F80  # bf16 1.0


def run_case(L, n_kv, hd, d_in, rows_per_req, pos0, seed, gains=True, theta=1e6, eps=1e-6, extra=7,
             w_std=0.02):
    rng = np.random.default_rng(seed)
    B = len(rows_per_req)
    row_cu = np.zeros(B + 1, np.int32)
    row_cu[1:] = np.cumsum(rows_per_req)
    M = int(row_cu[-1])
    pos0 = np.asarray(pos0, np.int32)
    span = pos0.astype(np.int64) + np.asarray(rows_per_req) + extra
    base = np.zeros(B, np.int64)
    base[1:] = np.cumsum(span)[:-1]
    T_cap = int(span.sum())
    h, _ = wl.bf16_normal(rng, (M, d_in))
    w, _ = wl.bf16_normal(rng, (L * 2 * n_kv * hd, d_in), std=w_std)
    g = wl.to_bf16_bits((1.0 + 0.3 * rng.standard_normal((L, hd))).astype(np.float32)) if gains else None
    import block_drafting_amd as bd
    kc = torch.full((L, T_cap, n_kv, hd), SENTINEL, dtype=torch.int16, device="cuda")
    vc = torch.full((L, T_cap, n_kv, hd), SENTINEL, dtype=torch.int16, device="cuda")
    say(f"inject L={L} n_kv={n_kv} hd={hd} d_in={d_in} M={M} rows={list(rows_per_req)[:6]}")
    bd.inject_kv(cuda_bits(h), cuda_bits(w), cuda_bits(g) if gains else None,
                 torch.from_numpy(row_cu).cuda(), torch.from_numpy(pos0).cuda(), torch.from_numpy(base).cuda(),
                 kc, vc, theta, eps)
    torch.cuda.synchronize()
    gk, gv = host_bits(kc), host_bits(vc)
    ok = np.full((L, T_cap, n_kv, hd), 1.0)
    ov_ = np.full((L, T_cap, n_kv, hd), 1.0)
    oi.inject_kv(bits_to_f64(h), bits_to_f64(w), bits_to_f64(g) if gains else None, row_cu, pos0, base,
                 ok, ov_, L, n_kv, hd, theta, eps)
    written = np.zeros(T_cap, bool)
    for b in range(B):
        s0 = base[b] + pos0[b]
        written[s0: s0 + rows_per_req[b]] = True
    worst = 0.0
    for l in range(L):
        if written.any():
            worst = max(worst, rel_err(bits_to_f64(gk[l, written]), ok[l, written]),
                        rel_err(bits_to_f64(gv[l, written]), ov_[l, written]))
    assert (gk[:, ~written] == SENTINEL).all() and (gv[:, ~written] == SENTINEL).all()
    say(f"  worst relative error {worst:.2e}")
    assert worst <= TOL
    return worst


def test_tiny_config_round_and_prefill():
    cfg = wl.CONFIGS["tiny"]
    run_case(cfg.L, cfg.n_kv, cfg.hd, cfg.d_in, [cfg.K], [512], 0)        # one round: 8 rows at 512..519
    run_case(cfg.L, cfg.n_kv, cfg.hd, cfg.d_in, [512], [0], 1)            # prefill of the context


def test_ragged_requests_large_positions():
    run_case(3, 4, 128, 1024, [5, 0, 70, 1], [0, 3, 32000, 32767 - 1], 2)


def test_m_above_256_without_whole_head_tiles_uses_big_tiles():
    """M = 300 with 3 KV heads of 128 (n_kv * hd = 384: the 256-column tiles
    would straddle heads, so not the fused wide kernel): 256-row split tiles
    and the finish pass."""
    run_case(2, 3, 128, 512, [150, 150], [100, 0], 3)


def test_m_up_to_256_streams_the_weights():
    """M = 200 and M = 256 (the largest): the weight-streaming GEMM with its
    d_in split and the finish pass."""
    run_case(2, 8, 128, 1024, [120, 80], [100, 0], 12)
    run_case(1, 4, 64, 640, [16] * 16, list(range(0, 1600, 100)), 13)


def test_finish_rows_wider_than_one_workgroup():
    """n_kv * hd above 1024 (more K and V items per row than the finish pass's
    256 threads): 24 heads of 128 at M = 32 (weight-streaming GEMM, long d_in
    split) and 12 heads of 128 at M = 300 (256-column tiles, split)."""
    run_case(1, 24, 128, 8192, [16, 16], [5, 900], 14)
    run_case(1, 12, 128, 1024, [200, 100], [0, 3000], 15)


def test_wide_tiles_two_m_tiles_one_step_splits():
    """M = 700: three 256-row tiles of the wide kernel, the last ragged; d_in =
    128 gives two 64-wide steps, split one per workgroup, then the finish pass."""
    run_case(1, 2, 128, 128, [400, 300], [5, 20000], 7)


def test_wide_tiles_hd64_long_k():
    """M = 513 (one row into the third tile), hd = 64, d_in = 2048 (32 steps in
    16 splits)."""
    run_case(2, 4, 64, 2048, [500, 13], [0, 77], 8)


def test_wide_unsplit_fused_epilogue_hd128():
    """M = 516 > 256 with d_in = 64 (one step, so no split): the 256 x 256 tiles
    run RMSNorm, RoPE and the scatter in the projection's own epilogue; ragged
    requests, positions up to 32 700, a last tile four rows deep."""
    run_case(2, 2, 128, 64, [300, 5, 211], [0, 32700, 1000], 9)


def test_wide_unsplit_fused_epilogue_hd64():
    """The unsplit fused epilogue at hd = 64 (two heads per wave), with and
    without gains."""
    run_case(1, 4, 64, 64, [257, 3], [11, 20000], 10)
    run_case(2, 4, 64, 64, [40, 400], [3, 0], 11, gains=False)


def test_wide_persistent_many_tiles_hd128():
    """M = 4300 rows x 4096 outputs at d_in = 128: 17 x 16 = 272 unsplit tiles,
    more than the CUs, so the persistent projection walks its XCD super-tiles
    (full 8-column super-tiles, a last row tile 204 rows deep)."""
    run_case(2, 8, 128, 128, [2000, 2300], [0, 30000], 12)


def test_wide_persistent_narrow_hd64():
    """The persistent projection with two column tiles (super-tiles mostly
    empty) and 129 row tiles, hd = 64, one step of d_in, three ragged requests."""
    run_case(1, 4, 64, 64, [20000, 12900, 77], [5, 0, 40000], 13)


def test_no_gains_hd64():
    run_case(2, 3, 64, 640, [40, 9], [7, 1000], 4, gains=False)


@pytest.mark.parametrize("n_kv,M,d_in,used", [(2, 20, 256, 12), (4, 300, 64, 261), (4, 600, 128, 333)])
def test_rows_past_row_cu_end_are_not_written(n_kv, M, d_in, used):
    """row_cu[B] < M: trailing rows of H are ignored (small tiles; the wide
    tiles unsplit with the fused epilogue; the wide tiles split)."""
    import block_drafting_amd as bd
    say(f"rows past row_cu: n_kv={n_kv} M={M} d_in={d_in} used={used}")
    rng = np.random.default_rng(5)
    L, hd = 1, 64
    T = M + 20
    h, _ = wl.bf16_normal(rng, (M, d_in))
    w, _ = wl.bf16_normal(rng, (L * 2 * n_kv * hd, d_in), std=0.02)
    kc = torch.full((L, T, n_kv, hd), SENTINEL, dtype=torch.int16, device="cuda")
    vc = torch.full((L, T, n_kv, hd), SENTINEL, dtype=torch.int16, device="cuda")
    bd.inject_kv(cuda_bits(h), cuda_bits(w), None, torch.tensor([0, used], dtype=torch.int32, device="cuda"),
                 torch.tensor([0], dtype=torch.int32, device="cuda"),
                 torch.tensor([0], dtype=torch.int64, device="cuda"), kc, vc)
    torch.cuda.synchronize()
    for c in (host_bits(kc), host_bits(vc)):
        assert (c[:, used:] == SENTINEL).all() and (c[:, :used] != SENTINEL).any()


def test_deterministic_run_to_run():
    a = run_case(2, 8, 128, 2048, [64, 64], [10, 4000], 6)
    b = run_case(2, 8, 128, 2048, [64, 64], [10, 4000], 6)
    assert a == b


def _full_size_sampled_rows(name, rows):
    """One round's projection at the configuration's full size on the GPU
    (every row of every request); the oracle checks the sampled rows."""
    import block_drafting_amd as bd
    cfg = wl.CONFIGS[name]
    r = wl.make_round(cfg, parts=("inject",), random_gains=True)
    say(f"full-size {name} inject M={cfg.B * cfg.K} d_in={cfg.d_in}")
    T_cap = r.T_cap
    kc = torch.full((cfg.L, T_cap, cfg.n_kv, cfg.hd), SENTINEL, dtype=torch.int16, device="cuda")
    vc = torch.full((cfg.L, T_cap, cfg.n_kv, cfg.hd), SENTINEL, dtype=torch.int16, device="cuda")
    bd.inject_kv(cuda_bits(r.h_round_bits), cuda_bits(r.w_bits), cuda_bits(r.k_norm_bits),
                 torch.from_numpy(r.row_cu).cuda(), torch.from_numpy(r.row_pos0).cuda(),
                 torch.from_numpy(r.cache_base).cuda(), kc, vc, cfg.rope_theta, cfg.rms_eps)
    torch.cuda.synchronize()
    rows = np.asarray(rows)
    b_of = rows // cfg.K
    j_of = rows % cfg.K
    pos0 = (r.row_pos0[b_of] + j_of).astype(np.int32)
    slots = torch.from_numpy(r.cache_base[b_of] + pos0).cuda()
    gk, gv = host_bits(kc[:, slots]), host_bits(vc[:, slots])
    w = bits_to_f64(r.w_bits)
    h = bits_to_f64(r.h_round_bits[rows])
    g = bits_to_f64(r.k_norm_bits)
    row_cu = np.arange(len(rows) + 1, dtype=np.int32)
    ok = np.zeros((cfg.L, len(rows), cfg.n_kv, cfg.hd))
    ov_ = np.zeros((cfg.L, len(rows), cfg.n_kv, cfg.hd))
    oi.inject_kv(h, w, g, row_cu, pos0, np.arange(len(rows)) - pos0, ok, ov_, cfg.L, cfg.n_kv, cfg.hd,
                 cfg.rope_theta, cfg.rms_eps)
    for l in range(cfg.L):
        ek = rel_err(bits_to_f64(gk[l]), ok[l])
        ev = rel_err(bits_to_f64(gv[l]), ov_[l])
        say(f"  layer {l}: K rel err {ek:.2e}  V rel err {ev:.2e}")
        assert ek <= TOL and ev <= TOL


def test_full_size_8b_round_sampled_rows():
    """M = 512 rows (B = 32, K = 16), d_in = 20480, 5 layers x 8 heads x 128:
    the wide 256 x 256 tiles split over d_in; the oracle checks 8 rows."""
    _full_size_sampled_rows("qwen3-8b", [0, 15, 16, 100, 257, 300, 498, 511])


def test_full_size_4b_round_all_rows():
    """Batch 1 (M = 16, d_in = 12800): the small-M, weight-bound tiles; the
    oracle checks every row."""
    _full_size_sampled_rows("qwen3-4b", list(range(16)))


def test_full_size_27b_round_sampled_rows():
    """Batch 8 (M = 128, d_in = 25600, 524 MB of weights)."""
    _full_size_sampled_rows("27b-long", [0, 1, 31, 64, 77, 127])


def test_full_size_sweep_round_sampled_rows():
    """Batch 128 (M = 2048: eight 256-row tiles of the wide kernel)."""
    _full_size_sampled_rows("sweep-b128", [0, 511, 512, 1000, 1535, 1536, 2047])


def device_bf16_normal(M, d, seed):
    """[M, d] standard normal bf16 (as int16 bits) drawn on the device in row
    slices, so no full-size float32 copy is ever held."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    h = torch.empty((M, d), dtype=torch.int16, device="cuda")
    step = max(1, (1 << 28) // d)
    for i in range(0, M, step):
        n = min(step, M - i)
        h[i:i + n] = torch.randn((n, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    return h


@pytest.mark.parametrize("name", ["qwen3-8b", "27b-long", "sweep-b128"])
def test_prefill_scale_materialization_sampled_rows(name):
    """Immediate materialization of a whole context batch (NEXT row): every
    request's context at once, M = the sum of the workload's context lengths
    in one call (about 74k rows for the 8B round's batch, 262k for the 27B
    batch at d_in 25600, 411k for the batch of 128 lognormal contexts); the
    oracle checks 12 sampled rows."""
    import block_drafting_amd as bd
    cfg = wl.CONFIGS[name]
    r = wl.make_round(cfg, parts=("inject",), random_gains=True)
    ctx = r.ctx_len.astype(np.int64)
    M = int(ctx.sum())
    row_cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    pos0 = np.zeros(cfg.B, np.int32)
    say(f"prefill-scale inject {name} M={M} d_in={cfg.d_in}")
    h = device_bf16_normal(M, cfg.d_in, 11)
    kc = torch.full((cfg.L, r.T_cap, cfg.n_kv, cfg.hd), SENTINEL, dtype=torch.int16, device="cuda")
    vc = torch.full_like(kc, SENTINEL)
    bd.inject_kv(h, cuda_bits(r.w_bits), cuda_bits(r.k_norm_bits), torch.from_numpy(row_cu).cuda(),
                 torch.from_numpy(pos0).cuda(), torch.from_numpy(r.cache_base).cuda(), kc, vc, cfg.rope_theta,
                 cfg.rms_eps)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.sort(np.concatenate([[0, M - 1, int(row_cu[1]), int(row_cu[1]) - 1], rng.integers(0, M, 8)]))
    b_of = np.searchsorted(row_cu, rows, side="right") - 1
    p_of = (rows - row_cu[b_of]).astype(np.int32)
    slots = r.cache_base[b_of] + p_of
    hr = host_bits(h[torch.from_numpy(rows).cuda()])
    gk, gv = host_bits(kc[:, torch.from_numpy(slots).cuda()]), host_bits(vc[:, torch.from_numpy(slots).cuda()])
    ok = np.zeros((cfg.L, len(rows), cfg.n_kv, cfg.hd))
    ov_ = np.zeros((cfg.L, len(rows), cfg.n_kv, cfg.hd))
    oi.inject_kv(bits_to_f64(hr), bits_to_f64(r.w_bits), bits_to_f64(r.k_norm_bits),
                 np.arange(len(rows) + 1, dtype=np.int32), p_of, np.arange(len(rows)) - p_of, ok, ov_, cfg.L,
                 cfg.n_kv, cfg.hd, cfg.rope_theta, cfg.rms_eps)
    for l in range(cfg.L):
        ek = rel_err(bits_to_f64(gk[l]), ok[l])
        ev = rel_err(bits_to_f64(gv[l]), ov_[l])
        say(f"  layer {l}: K rel err {ek:.2e}  V rel err {ev:.2e}")
        assert ek <= TOL and ev <= TOL
    del h, kc, vc
    torch.cuda.empty_cache()
