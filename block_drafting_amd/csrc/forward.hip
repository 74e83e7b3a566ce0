// One drafter forward over a block (random-init weights welcome): the pass a
// DFlash drafter makes once per round, to measure a whole draft step against
// the block size.
//
// DFlash/Spec V2 blog, A2: the drafter is a few transformer layers whose
// attention reads the target's injected context K/V plus the block's own
// K/V, and one forward yields all K positions (so its cost should stay close
// to flat in K).  The layers follow the Qwen3 layout the pages' drafters are
// built on: pre-norm RMSNorm; fused Q/K/V projection; per-head RMSNorm of Q
// and K; RoPE at the absolute position ctx + i; block attention over the
// context window plus the block (draft_block_attn); output projection with
// the residual; RMSNorm; SiLU-gated MLP with the residual; final RMSNorm and
// the LM head (fp32 logits).
//
// The GEMMs are this library's weight-streaming kernel (fg_gemm below): every
// weight byte is read once per call, the block's rows are re-read from L2,
// fp32 partial sums over d_in splits go to the workspace, and the kernel that
// consumes a projection adds its splits in a fixed order (the Q/K norm + RoPE
// kernel, the residual add + RMSNorm kernel, the SiLU-gate kernel), so a split
// costs no extra launch.  Attention is this library's kernel.
#include "bd_common.hpp"
#include "bd_launch.hpp"

#include <algorithm>
#include <cmath>

namespace bd {

// ---------------------------------------------------------------- weight-streaming GEMM
// P[s][m][n] = sum over the d_in steps of split s of X[m][k] W[n][k]: X the
// block's rows [M, Kd] (bf16), W a weight [N, Kd] (bf16), P fp32.  At the
// drafter's M = B K (a few hundred rows at most) the product is bound by
// reading W, so the tiling is chosen for streaming it once: a workgroup holds
// all rows of a 128-row M tile against 32 FN weight rows, and walks its d_in
// range in 64-wide steps.  Both operands go straight from global memory to
// LDS (global_load_lds, 16 bytes per lane; W non-temporal, X through the
// caches, since every workgroup re-reads it) through a ring of NS stages; the
// refill of a stage is issued between the MFMAs of the current one.  Four
// waves, wave w owning rows 32 w .. 32 w + 31 of the M tile; each computes the
// transposed tile D = W . X^T on 32x32x16 bf16 MFMAs, so a lane ends up with
// one row and 16 columns (four runs of four), stored as 16-byte pieces.
// The (N tile, M tile, split) triples are numbered with the M tiles and
// splits of an N tile adjacent, and spread over the eight XCDs in contiguous
// ranges (launch index b runs triple (b mod 8) * per_xcd + b / 8), so the M
// tiles sharing a weight tile sit on one XCD and read it through its L2.
constexpr int FG_BM = 128, FG_BK = 64, FG_T = 256;

struct FgArgs {
  const uint16_t* X;  // [M, Kd]
  const uint16_t* W;  // [N, Kd]
  float* P;           // [S][M][N]
  int M, N, Kd, S, steps_per_split, MT, total, per_xcd;
};

// byte offset of 16-byte piece c (of 8) of row `row` in a stage: two rows per
// 256-byte line, pieces XOR-permuted by the line so that the fragment reads
// (16 lanes: 16 consecutive rows at one piece) hit distinct banks
__device__ __forceinline__ int fg_piece(int row, int c) {
  const int line = row >> 1;
  return (line * 16 + ((((row & 1) << 3) | c) ^ (line & 7))) * 16;
}

template <int FN, int NS>
__global__ __launch_bounds__(FG_T) void fg_gemm(FgArgs g) {
  constexpr int BN = 32 * FN;
  constexpr int XB = FG_BM * FG_BK * 2, WB = BN * FG_BK * 2, SB = XB + WB;
  constexpr int XPW = XB / 1024 / 4, WPW = WB / 1024 / 4;  // loads per wave per stage
  constexpr int LPW = XPW + WPW;
  static_assert(NS >= 2 && NS * SB <= 160 * 1024, "LDS ring");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * SB];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 31, h = lane >> 5;
  const int b = blockIdx.x;
  const int u = (b & 7) * g.per_xcd + (b >> 3);
  if (u >= g.total) return;
  const int s = u % g.S, rest = u / g.S;
  const int mt = rest % g.MT, tn = rest / g.MT;
  const int m0 = mt * FG_BM, n0 = tn * BN;
  const int step0 = s * g.steps_per_split;
  const int ns = min(g.steps_per_split, g.Kd / FG_BK - step0);

  // per-lane byte offsets of this wave's loads: load q fills the stage's piece
  // slots 64 (w + 4 q) + lane; the (row, piece) placed there by fg_piece
  uint32_t offX[XPW], offW[WPW];
#pragma unroll
  for (int q = 0; q < XPW; ++q) {
    const int ps = (w + 4 * q) * 64 + lane;
    const int line = ps >> 4, lc = (ps & 15) ^ (line & 7);
    const int row = 2 * line + (lc >> 3), c = lc & 7;
    const int m = min(m0 + row, g.M - 1) - m0;  // rows past M re-read row M - 1; never stored
    offX[q] = uint32_t(m * g.Kd * 2 + c * 16);
  }
#pragma unroll
  for (int q = 0; q < WPW; ++q) {
    const int ps = (w + 4 * q) * 64 + lane;
    const int line = ps >> 4, lc = (ps & 15) ^ (line & 7);
    const int row = 2 * line + (lc >> 3), c = lc & 7;
    const int n = min(n0 + row, g.N - 1) - n0;  // rows past N re-read row N - 1; never stored
    offW[q] = uint32_t(n * g.Kd * 2 + c * 16);
  }
  const uint16_t* Xb = g.X + size_t(m0) * g.Kd + size_t(step0) * FG_BK;
  const uint16_t* Wb = g.W + size_t(n0) * g.Kd + size_t(step0) * FG_BK;
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring)));
  // load d of this wave for step st: its W loads first, then its X loads
  auto issue = [&](int st, int d) {
    const uint32_t sb = l0 + (st % NS) * SB;
    if (d < WPW) dma16<true>(Wb + size_t(st) * FG_BK, offW[d], sb + XB + (w + 4 * d) * 1024);
    else dma16<false>(Xb + size_t(st) * FG_BK, offX[d - WPW], sb + (w + 4 * (d - WPW)) * 1024);
  };

  floatx16 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) acc[j] = floatx16{};

  for (int st = 0; st < NS - 1 && st < ns; ++st)
#pragma unroll
    for (int d = 0; d < LPW; ++d) issue(st, d);

  constexpr int NMF = (FG_BK / 16) * FN;  // MFMAs per step
  constexpr int EVERY = NMF / LPW >= 2 ? 2 : 1;
  for (int k = 0; k < ns; ++k) {
    // step k has landed once no more than the loads of the later steps
    // already issued (k + 1 .. min(k + NS - 2, ns - 1)) are outstanding
    vm_wait_le<(NS - 2) * LPW>(min(NS - 2, ns - 1 - k) * LPW);
    __syncthreads();
    const int kn = k + NS - 1;  // refills the slot read in iteration k - 1
    const uint8_t* Xs = ring + (k % NS) * SB;
    const uint8_t* Ws = Xs + XB;
#pragma unroll
    for (int kk = 0; kk < FG_BK / 16; ++kk) {
      const bf16x8 xf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Xs + fg_piece(32 * w + lr, 2 * kk + h)));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const bf16x8 wf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Ws + fg_piece(32 * j + lr, 2 * kk + h)));
        acc[j] = mfma32x32x16(wf, xf, acc[j]);  // D = W . X^T
        const int mi = kk * FN + j;
        if (kn < ns && mi % EVERY == 0 && mi / EVERY < LPW) issue(kn, mi / EVERY);
      }
    }
#pragma unroll
    for (int d = (NMF + EVERY - 1) / EVERY; d < LPW; ++d)
      if (kn < ns) issue(kn, d);
  }

  // lane (lr, h) of wave w: row m0 + 32 w + lr, columns n0 + 32 j + 8 q + 4 h + e
  const int m = m0 + 32 * w + lr;
  if (m >= g.M) return;
  float* P = g.P + (size_t(s) * g.M + m) * g.N;
  const bool vec = (g.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * j + 8 * q + 4 * h;
      if (vec && n + 3 < g.N) {
        *reinterpret_cast<floatx4*>(P + n) =
            floatx4{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) P[n + e] = acc[j][4 * q + e];
      }
    }
}

namespace {

struct FgPlan {
  int FN, S, steps_per_split, MT, total;
};

int fg_cus() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

// Tile width and d_in split of one projection.  Per candidate (tile width
// 32 FN, split S) the time is estimated as the rounds of workgroups over the
// CUs times one workgroup's time, that being its weight bytes over its share
// of HBM bandwidth or its operand bytes (weights plus rows) over one CU's
// load rate, whichever is longer, plus a fixed cost per d_in step; splits add
// their partial sums' write and read-back.
FgPlan fg_plan(int M, int N, int Kd, bool split = true) {
  const int cus = fg_cus();
  const double hbm = 6.0e12, cu_load = 60e9, step_cost = 40e-9, part_bw = 8.0e12;
  const int MT = (M + FG_BM - 1) / FG_BM;
  const int steps = Kd / FG_BK;
  FgPlan best{8, 1, steps, MT, 0};
  double best_t = 1e30;
  for (int FN : {2, 4, 8}) {
    const int tiles = (N + 32 * FN - 1) / (32 * FN) * MT;
    for (int S = 1; S <= (split ? std::min(steps, 32) : 1); ++S) {
      const int sps = (steps + S - 1) / S;
      const int Sr = (steps + sps - 1) / sps;
      if (Sr != S) continue;
      const long nwg = long(tiles) * S;
      const long active = std::min<long>(nwg, cus);
      const long rounds = (nwg + cus - 1) / cus;
      const double wb = 64.0 * FN * sps * FG_BK, xb = 2.0 * FG_BM * sps * FG_BK;
      const double per_wg = std::max(wb / MT / (hbm / active), (wb + xb) / cu_load) + sps * step_cost;
      const double t = rounds * per_wg + (S > 1 ? double(S) * M * N * 8.0 / part_bw : 0.0);
      if (t < best_t * 0.98) {
        best_t = t;
        best = FgPlan{FN, S, sps, MT, int(nwg)};
      }
    }
  }
  return best;
}

template <int FN>
hipError_t fg_launch_fn(const FgArgs& a, int grid, hipStream_t stream) {
  constexpr int NS = (FG_BM + 32 * FN) * FG_BK * 2 * 4 <= 160 * 1024 ? 4 : 3;
  hipLaunchKernelGGL((fg_gemm<FN, NS>), dim3(grid), dim3(FG_T), 0, stream, a);
  return hipGetLastError();
}

// P = the split partials of X . W^T (or, with S = 1 forced, the product itself)
hipError_t fg_run(const FgPlan& p, const uint16_t* X, const uint16_t* W, float* P, int M, int N, int Kd,
                  hipStream_t stream) {
  FgArgs a{};
  a.X = X; a.W = W; a.P = P;
  a.M = M; a.N = N; a.Kd = Kd; a.S = p.S; a.steps_per_split = p.steps_per_split; a.MT = p.MT;
  a.total = p.total;
  a.per_xcd = (p.total + 7) / 8;
  const int grid = 8 * a.per_xcd;
  switch (p.FN) {
    case 2: return fg_launch_fn<2>(a, grid, stream);
    case 4: return fg_launch_fn<4>(a, grid, stream);
    default: return fg_launch_fn<8>(a, grid, stream);
  }
}

}  // namespace

// ---------------------------------------------------------------- the consumers
// sum of the S split partials of element i (stride: one split), in split order
__device__ __forceinline__ float split_sum(const float* P, size_t stride, int S, size_t i) {
  float v = P[i];
  for (int s = 1; s < S; ++s) v += P[size_t(s) * stride + i];
  return v;
}

// RMSNorm of each row of x [M, d] (bf16) with gain g [d]: out = x / rms * g
__global__ __launch_bounds__(256) void fw_rmsnorm(const uint16_t* x, const uint16_t* g, int d, float eps,
                                                  uint16_t* out) {
  __shared__ float s_w[4];
  const int m = blockIdx.x, t = threadIdx.x;
  const uint16_t* xr = x + size_t(m) * d;
  float ss = 0.f;
  for (int i = t; i < d; i += 256) {
    const float v = bf16_to_f32(xr[i]);
    ss += v * v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((t & 63) == 0) s_w[t >> 6] = ss;
  __syncthreads();
  const float tot = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  const float inv = 1.0f / sqrtf(tot / float(d) + eps);
  uint16_t* orow = out + size_t(m) * d;
  for (int i = t; i < d; i += 256) orow[i] = f32_to_bf16(bf16_to_f32(xr[i]) * inv * bf16_to_f32(g[i]));
}

// Residual add then RMSNorm, per row m: x_out = bf16(x_res + sum of the S
// partials of the projection), xn = bf16(x_out / rms(x_out) * g).  x_out may
// be x_res (each element is read and written by the same thread).
__global__ __launch_bounds__(256) void fw_add_rmsnorm(const uint16_t* x_res, const float* P, int S, int M, int d,
                                                      const uint16_t* g, float eps, uint16_t* x_out,
                                                      uint16_t* xn) {
  __shared__ float s_w[4];
  const int m = blockIdx.x, t = threadIdx.x;
  const size_t stride = size_t(M) * d;
  float ss = 0.f;
  for (int i = t; i < d; i += 256) {
    const size_t e = size_t(m) * d + i;
    const uint16_t v = f32_to_bf16(bf16_to_f32(x_res[e]) + split_sum(P, stride, S, e));
    x_out[e] = v;
    const float f = bf16_to_f32(v);
    ss += f * f;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((t & 63) == 0) s_w[t >> 6] = ss;
  __syncthreads();
  const float tot = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  const float inv = 1.0f / sqrtf(tot / float(d) + eps);
  for (int i = t; i < d; i += 256) {
    const size_t e = size_t(m) * d + i;
    xn[e] = f32_to_bf16(bf16_to_f32(x_out[e]) * inv * bf16_to_f32(g[i]));
  }
}

struct QkArgs {
  const float* P;       // [S][M][(n_q + 2 n_kv) hd] partials of the Q/K/V projection
  const uint16_t* gq;   // [hd]
  const uint16_t* gk;   // [hd]
  const int32_t* ctx_len;
  uint16_t* q;          // [M, n_q hd]
  uint16_t* kb;         // [M, n_kv hd]
  uint16_t* vb;         // [M, n_kv hd]
  int M, S, K, n_q, n_kv, hd;
  float eps;
  double inv_freq[64];
};

// Per row m = b K + i: the projection (its splits summed, rounded to bf16),
// then RMSNorm of every Q and K head with its gain and RoPE (pairs d, d + hd/2)
// at position ctx_len[b] + i; V rounded and copied.  One thread per (head, dim
// pair).
__global__ __launch_bounds__(256) void fw_qk_norm_rope(QkArgs a) {
  const int m = blockIdx.x, t = threadIdx.x;
  const int b = m / a.K, i = m - b * a.K;
  const int pos = a.ctx_len[b] + i;
  const int hd = a.hd, half = hd >> 1;
  const int nh = a.n_q + a.n_kv;  // heads that get norm + RoPE
  const int ld = (a.n_q + 2 * a.n_kv) * hd;
  const size_t stride = size_t(a.M) * ld, row = size_t(m) * ld;
  auto val = [&](int c) { return bf16_to_f32(f32_to_bf16(split_sum(a.P, stride, a.S, row + c))); };
  // half / 64 threads per head when hd = 128 (a wave covers one head)
  for (int it = t; it < nh * half; it += 256) {
    const int head = it / half, d = it - head * half;
    const float xa = val(head * hd + d), xb = val(head * hd + half + d);
    float ss = xa * xa + xb * xb;
    // the head's half threads are consecutive lanes of one wave (half <= 64)
    for (int o = half >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / float(hd) + a.eps);
    const uint16_t* g = head < a.n_q ? a.gq : a.gk;
    const float va = xa * inv * bf16_to_f32(g[d]), vb = xb * inv * bf16_to_f32(g[half + d]);
    // angle pos * theta^(-2d/hd) in fp64, reduced in fp64, fp32 sin / cos
    float sn, cs;
    sincos_angle(double(pos) * a.inv_freq[d], &sn, &cs);
    uint16_t* dst = head < a.n_q ? a.q + (size_t(m) * a.n_q + head) * hd
                                 : a.kb + (size_t(m) * a.n_kv + (head - a.n_q)) * hd;
    dst[d] = f32_to_bf16(va * cs - vb * sn);
    dst[half + d] = f32_to_bf16(vb * cs + va * sn);
  }
  for (int c = t; c < a.n_kv * hd; c += 256)
    a.vb[size_t(m) * a.n_kv * hd + c] = f32_to_bf16(split_sum(a.P, stride, a.S, row + size_t(nh) * hd + c));
}

// h = bf16(silu(gate) * up) with gate and up the rounded sums of the gate/up
// projection's splits (a row of it: gate (F), then up (F))
__global__ __launch_bounds__(256) void fw_silu_mul(const float* P, int S, int M, int F, uint16_t* h) {
  const int m = blockIdx.x;
  const size_t stride = size_t(M) * 2 * F, row = size_t(m) * 2 * F;
  for (int c = threadIdx.x; c < F; c += 256) {
    const float g = bf16_to_f32(f32_to_bf16(split_sum(P, stride, S, row + c)));
    const float u = bf16_to_f32(f32_to_bf16(split_sum(P, stride, S, row + F + c)));
    h[size_t(m) * F + c] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
  }
}

namespace {

inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

struct FwLayout {
  size_t x, xn, q, kb, vb, att, h, part, attn_ws, total;
};

// the largest partial-sum buffer of the layer projections (the LM head writes
// the logits directly)
size_t fw_part_bytes(int M, int d, int n_q, int n_kv, int hd, int ffn) {
  size_t mx = 0;
  const int shapes[4][2] = {{(n_q + 2 * n_kv) * hd, d}, {d, n_q * hd}, {2 * ffn, d}, {d, ffn}};
  for (const auto& sh : shapes) {
    const FgPlan p = fg_plan(M, sh[0], sh[1]);
    mx = std::max(mx, size_t(p.S) * M * sh[0] * 4);
  }
  return mx;
}

FwLayout fw_layout(int B, int K, int d, int n_q, int n_kv, int hd, int ffn, int max_ctx, int window) {
  const size_t M = size_t(B) * K;
  FwLayout L{};
  size_t o = 0;
  L.x = o; o += al(M * d * 2);
  L.xn = o; o += al(M * d * 2);
  L.q = o; o += al(M * size_t(n_q) * hd * 2);
  L.kb = o; o += al(M * size_t(n_kv) * hd * 2);
  L.vb = o; o += al(M * size_t(n_kv) * hd * 2);
  L.att = o; o += al(M * size_t(n_q) * hd * 2);
  L.h = o; o += al(M * size_t(ffn) * 2);
  L.part = o; o += al(M > 0 ? fw_part_bytes(int(M), d, n_q, n_kv, hd, ffn) : 0);
  L.attn_ws = o; o += al(attn_ws_bytes(B, K, n_q, n_kv, hd, max_ctx, window));
  L.total = o;
  return L;
}

}  // namespace

size_t forward_ws_bytes(int B, int K, int d, int n_q, int n_kv, int hd, int ffn, int max_ctx, int window) {
  return fw_layout(B, K, d, n_q, n_kv, hd, ffn, max_ctx, window).total;
}

hipError_t launch_forward(const uint16_t* x_in, int B, int K, int d, int L, int n_q, int n_kv, int hd, int ffn,
                          int V, const uint16_t* const* lw, const uint16_t* g_final, const uint16_t* w_lm,
                          const uint16_t* kc, const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                          int64_t T_cap, int max_ctx, int window, float rope_theta, float eps, float* logits,
                          void* ws, hipStream_t stream) {
  const int M = B * K;
  const FwLayout Lo = fw_layout(B, K, d, n_q, n_kv, hd, ffn, max_ctx, window);
  char* w = static_cast<char*>(ws);
  auto Pb = [&](size_t off) { return reinterpret_cast<uint16_t*>(w + off); };
  uint16_t *x = Pb(Lo.x), *xn = Pb(Lo.xn), *q = Pb(Lo.q), *kb = Pb(Lo.kb), *vb = Pb(Lo.vb), *att = Pb(Lo.att),
           *h = Pb(Lo.h);
  float* part = reinterpret_cast<float*>(w + Lo.part);
  QkArgs qa{};
  qa.P = part; qa.ctx_len = ctx_len; qa.q = q; qa.kb = kb; qa.vb = vb;
  qa.M = M; qa.K = K; qa.n_q = n_q; qa.n_kv = n_kv; qa.hd = hd; qa.eps = eps;
  for (int i = 0; i < hd / 2; ++i) qa.inv_freq[i] = pow(double(rope_theta), -2.0 * i / double(hd));
  const int n_qkv = (n_q + 2 * n_kv) * hd;
  const size_t layer_cache = size_t(T_cap) * n_kv * hd;
  const FgPlan p_qkv = fg_plan(M, n_qkv, d), p_o = fg_plan(M, d, n_q * hd), p_gu = fg_plan(M, 2 * ffn, d),
               p_dn = fg_plan(M, d, ffn);
  const FgPlan p_lm = fg_plan(M, V, d, false);  // the logits are written directly: no split
  hipError_t e = hipSuccess;
#define FW_TRY(x)                        \
  do {                                   \
    if ((e = (x)) != hipSuccess) return e; \
  } while (0)
  if (L == 0) {
    hipLaunchKernelGGL(fw_rmsnorm, dim3(M), dim3(256), 0, stream, x_in, g_final, d, eps, xn);
  } else {
    hipLaunchKernelGGL(fw_rmsnorm, dim3(M), dim3(256), 0, stream, x_in, lw[0], d, eps, xn);
  }
  for (int l = 0; l < L; ++l) {
    const uint16_t* w_qkv = lw[8 * l + 1];
    const uint16_t* g_q = lw[8 * l + 2];
    const uint16_t* g_k = lw[8 * l + 3];
    const uint16_t* w_o = lw[8 * l + 4];
    const uint16_t* g_mlp = lw[8 * l + 5];
    const uint16_t* w_gu = lw[8 * l + 6];
    const uint16_t* w_dn = lw[8 * l + 7];
    const uint16_t* g_next = l + 1 < L ? lw[8 * (l + 1)] : g_final;  // the norm after this layer
    const uint16_t* xr = l == 0 ? x_in : x;  // the residual stream
    FW_TRY(fg_run(p_qkv, xn, w_qkv, part, M, n_qkv, d, stream));
    qa.gq = g_q; qa.gk = g_k; qa.S = p_qkv.S;
    hipLaunchKernelGGL(fw_qk_norm_rope, dim3(M), dim3(256), 0, stream, qa);
    FW_TRY(launch_attn(q, kb, vb, kc + l * layer_cache, vc + l * layer_cache, cache_base, ctx_len, T_cap, max_ctx,
                       B, K, n_q, n_kv, hd, window, 0, 0.f, att, nullptr, w + Lo.attn_ws, stream));
    FW_TRY(fg_run(p_o, att, w_o, part, M, d, n_q * hd, stream));
    hipLaunchKernelGGL(fw_add_rmsnorm, dim3(M), dim3(256), 0, stream, xr, part, p_o.S, M, d, g_mlp, eps, x, xn);
    FW_TRY(fg_run(p_gu, xn, w_gu, part, M, 2 * ffn, d, stream));
    hipLaunchKernelGGL(fw_silu_mul, dim3(M), dim3(256), 0, stream, part, p_gu.S, M, ffn, h);
    FW_TRY(fg_run(p_dn, h, w_dn, part, M, d, ffn, stream));
    hipLaunchKernelGGL(fw_add_rmsnorm, dim3(M), dim3(256), 0, stream, x, part, p_dn.S, M, d, g_next, eps, x, xn);
  }
#undef FW_TRY
  return fg_run(p_lm, xn, w_lm, logits, M, V, d, stream);
}

}  // namespace bd
