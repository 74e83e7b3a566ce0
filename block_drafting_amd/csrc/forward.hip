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
#include <map>
#include <mutex>
#include <tuple>

namespace bd {

// ---------------------------------------------------------------- weight-streaming GEMM
// P[s][m][n] = sum over the d_in steps of split s of X[m][k] W[n][k]: X the
// block's rows [M, Kd] (bf16), W a weight [N, Kd] (bf16), P fp32.  At the
// drafter's M = B K (a few hundred rows at most) the product is bound by
// reading W, so the kernel is built to stream it once, evenly over the CUs:
//   * work: the 32-row blocks of W (32 output columns each), per (M tile of
//     BM rows, d_in split) "plane"; each plane's blocks are cut into G nearly
//     equal contiguous ranges, one per workgroup, and a workgroup walks its
//     range in chunks of at most FN blocks, every chunk over the split's d_in
//     steps (64 wide), storing the chunk's fp32 tile when its last step is
//     done.  The plans give each workgroup one chunk and launch a whole
//     number of rounds of workgroups over the CUs (one resident per CU), so
//     the rounds finish together and a workgroup's stores come after its
//     loads: stores issued while a CU streams slow its loads down.
//   * waves: four loader waves only issue the operand loads and wait for them;
//     eight compute waves only read LDS, run the MFMAs and store the results.
//     Stores and loads share one completion counter, so a wave that did both
//     would stall its next load wait on its own stores; split this way the
//     loads keep NS - 1 steps in flight across chunk boundaries and the stores
//     drain in the background.  One barrier per step: the loaders reach it
//     once the step has landed, the compute waves once the previous step's
//     fragments are read, so after it the step is readable and the slot of the
//     previous step can be refilled.
//   * loads: both operands go straight from global memory to LDS
//     (global_load_lds, 16 bytes per lane; W non-temporal, X through the
//     caches, since every workgroup re-reads it) through a ring of NS stages;
//     loads of W rows past the chunk and of X rows past M are not issued.
//   * math: the compute waves form WMW (along M) x 8 / WMW (along N) groups;
//     wave (wm, wn) computes rows 32 wm .. 32 wm + 31 of the M tile against
//     FNW = FN WMW / 8 blocks, as the transposed product D = W . X^T on
//     32x32x16 bf16 MFMAs, so a lane ends up with one row and 16 columns per
//     block (four runs of four), stored as 16-byte pieces.
//   * placement: with several M tiles, workgroup u = ((s G + g) MT + mt)
//     (split, range, M tile) runs at launch index b with u = (b mod 8) per_xcd
//     + b / 8, so the M tiles reading one weight range share it through their
//     XCD's L2; with one M tile, u = b.
constexpr int FG_BK = 64, FG_NC = 8, FG_NL = 4, FG_T = 64 * (FG_NC + FG_NL);

struct FgArgs {
  const uint16_t* X;  // [M, Kd]
  const uint16_t* W;  // [N, Kd]
  float* P;           // [S][M][N]
  int M, N, Kd, S, steps_per_split, MT, G, nwg, per_xcd;
};

// byte offset of 16-byte piece c (of 8) of row `row` in a stage: two rows per
// 256-byte line, pieces XOR-permuted by the line so that the fragment reads
// (16 lanes: 16 consecutive rows at one piece) hit distinct banks
__device__ __forceinline__ int fg_piece(int row, int c) {
  const int line = row >> 1;
  return (line * 16 + ((((row & 1) << 3) | c) ^ (line & 7))) * 16;
}

template <int FN, int WMW>
struct FgShape {
  static constexpr int BM = 32 * WMW, BN = 32 * FN;
  static constexpr int XB = BM * FG_BK * 2, WB = BN * FG_BK * 2, SB = XB + WB;
  static constexpr int NS = 160 * 1024 / SB > 4 ? 4 : 160 * 1024 / SB;
  static constexpr int XPW = XB / 1024 / FG_NL, WPW = WB / 1024 / FG_NL;  // loads per loader wave per step
  static constexpr int FNW = FN * WMW / FG_NC;                              // blocks per compute wave
  static_assert(NS >= 2 && XPW >= 1 && WPW >= 1 && FNW >= 1, "shape");
};

template <int FN, int WMW>
__global__ __launch_bounds__(FG_T) void fg_gemm(FgArgs g) {
  using Sh = FgShape<FN, WMW>;
  constexpr int BM = Sh::BM, XB = Sh::XB, SB = Sh::SB, NS = Sh::NS, XPW = Sh::XPW, WPW = Sh::WPW;
  constexpr int FNW = Sh::FNW, LMAX = XPW + WPW;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * SB];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int b = blockIdx.x;
  const int u = g.MT > 1 ? (b & 7) * g.per_xcd + (b >> 3) : b;
  if (u >= g.nwg) return;
  const int mt = u % g.MT, rest = u / g.MT;
  const int gi = rest % g.G, s = rest / g.G;
  const int NB = (g.N + 31) >> 5;
  const int blk0 = int(int64_t(gi) * NB / g.G), blk1 = int(int64_t(gi + 1) * NB / g.G);
  const int nch = (blk1 - blk0 + FN - 1) / FN;
  if (nch == 0) return;
  const int m0 = mt * BM, mrows = min(BM, g.M - m0);
  const int step0 = s * g.steps_per_split;
  const int ns = min(g.steps_per_split, g.Kd / FG_BK - step0);
  const int T = nch * ns;  // linear steps: chunk ci, step k at ci * ns + k
  auto rows_of = [&](int ci) {  // rows of W in chunk ci
    const int cb = blk0 + ci * FN;
    return min(32 * min(FN, blk1 - cb), g.N - 32 * cb);
  };

  if (w >= FG_NC) {
    // ------------------------------------------------ loader waves
    const int lw = w - FG_NC;
    // load q of loader lw fills the stage's piece slots 64 (lw + 4 q) + lane:
    // rows 8 (lw + 4 q) + rsub, piece c (the inverse of fg_piece)
    const int lc = (lane & 15) ^ ((4 * lw + (lane >> 4)) & 7);
    const int rsub = 2 * (lane >> 4) + (lc >> 3), c16 = (lc & 7) * 16;
    const int r8x = (mrows + 7) >> 3;
    const int nX = r8x > lw ? min(XPW, (r8x - lw + 3) >> 2) : 0;
    auto nw_of = [&](int ci) {
      const int r8 = (rows_of(ci) + 7) >> 3;
      return r8 > lw ? min(WPW, (r8 - lw + 3) >> 2) : 0;
    };
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring)));
    const int Kd2 = g.Kd * 2;
    // all loads of linear step li (chunk ci, step k): W first, then X
    auto issue_step = [&](int li, int ci, int k) {
      const int cb = blk0 + ci * FN;
      const int rv = rows_of(ci), nw = nw_of(ci);
      const uint16_t* wb = g.W + size_t(32 * cb) * g.Kd + size_t(step0 + k) * FG_BK;
      const uint16_t* xb = g.X + size_t(m0) * g.Kd + size_t(step0 + k) * FG_BK;
      const uint32_t sb = l0 + (li % NS) * SB;
#pragma unroll
      for (int q = 0; q < WPW; ++q)
        if (q < nw) {
          const int row = min(8 * (lw + 4 * q) + rsub, rv - 1);
          dma16<true>(wb, uint32_t(row * Kd2 + c16), sb + XB + (lw + 4 * q) * 1024);
        }
#pragma unroll
      for (int q = 0; q < XPW; ++q)
        if (q < nX) {
          const int row = min(8 * (lw + 4 * q) + rsub, mrows - 1);
          dma16<false>(xb, uint32_t(row * Kd2 + c16), sb + (lw + 4 * q) * 1024);
        }
    };
    int ic = 0, ik = 0;  // chunk and step of the next step to issue
    int li = 0;
    for (; li < NS - 1 && li < T; ++li) {
      issue_step(li, ic, ik);
      if (++ik == ns) {
        ik = 0;
        ++ic;
      }
    }
    int cc = 0, ck = 0;  // chunk and step of the step being waited for
    for (int ls = 0; ls < T; ++ls) {
      // step ls has landed once no more than this wave's loads of the later
      // steps already issued (ls + 1 .. li - 1) are outstanding (loads
      // complete in order)
      int pend = 0;
      {
        int c = cc, k = ck;
        for (int j = ls + 1; j < li; ++j) {
          if (++k == ns) {
            k = 0;
            ++c;
          }
          pend += nX + nw_of(c);
        }
      }
      vm_wait_le<(NS - 2) * LMAX>(pend);
      __builtin_amdgcn_s_barrier();
      // the slot of step ls - 1 is free: refill it with step ls + NS - 1
      if (li < T) {
        issue_step(li, ic, ik);
        ++li;
        if (++ik == ns) {
          ik = 0;
          ++ic;
        }
      }
      if (++ck == ns) {
        ck = 0;
        ++cc;
      }
    }
    return;
  }

  // -------------------------------------------------- compute waves
  const int wm = w % WMW, wn = w / WMW;
  const int lr = lane & 31, h = lane >> 5;
  const bool live = 32 * wm < mrows;
  int ls = 0;
  for (int ci = 0; ci < nch; ++ci) {
    const int cb = blk0 + ci * FN;
    floatx16 acc[FNW];
#pragma unroll
    for (int j = 0; j < FNW; ++j) acc[j] = floatx16{};
    for (int k = 0; k < ns; ++k, ++ls) {
      __builtin_amdgcn_s_barrier();
      const uint8_t* Xs = ring + (ls % NS) * SB;
      const uint8_t* Ws = Xs + XB;
      // fragments of round kk + 1 are read while round kk's MFMAs run; every
      // block is computed, also past the chunk or past M (not stored)
      bf16x8 xf[2], wf[2][FNW];
      auto read_round = [&](int kk, int buf) {
        xf[buf] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Xs + fg_piece(32 * wm + lr, 2 * kk + h)));
#pragma unroll
        for (int j = 0; j < FNW; ++j)
          wf[buf][j] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(Ws + fg_piece(32 * (wn * FNW + j) + lr, 2 * kk + h)));
      };
      read_round(0, 0);
#pragma unroll
      for (int kk = 0; kk < FG_BK / 16; ++kk) {
        if (kk + 1 < FG_BK / 16) read_round(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int j = 0; j < FNW; ++j) acc[j] = mfma32x32x16(wf[kk & 1][j], xf[kk & 1], acc[j]);  // D = W . X^T
      }
      // the fragments are in registers (the MFMAs consumed them): the slot may
      // be refilled after the next barrier
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }

    // the chunk is done: lane (lr, h) of wave (wm, wn) holds row m0 + 32 wm +
    // lr, columns 32 (cb + wn FNW + j) + 8 q + 4 h + e.  (Stores slow down the
    // CU's streaming loads while any are in flight, so plans give a workgroup
    // one chunk where they can: its stores then come after its last load.)
    const int nb = min(FN, blk1 - cb);
    const int m = m0 + 32 * wm + lr;
    if (live && m < g.M) {
      float* P = g.P + (size_t(s) * g.M + m) * g.N;
      const bool vec = (g.N & 3) == 0;
#pragma unroll
      for (int j = 0; j < FNW; ++j) {
        if (wn * FNW + j >= nb) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = 32 * (cb + wn * FNW + j) + 8 * q + 4 * h;
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
    }
  }
}

namespace {

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

}  // namespace

// M tile (32 WMW rows), chunk width (at most FN blocks of 32 columns), d_in
// split S and ranges per plane G of one projection.  Candidates: one chunk per
// workgroup with a whole number of rounds of workgroups over the CUs (G =
// rounds x CUs / planes), or one round whose workgroups walk several chunks
// (G = CUs / planes).  The estimate per candidate is rounds x (the largest of
// a workgroup's share of the weight bytes over its share of HBM bandwidth, its
// operand bytes over one CU's load rate, and its steps over the steps in
// flight times the load latency; plus the ring's first fill), plus the split
// partials' write and read-back.  Its constants were fitted to timings of
// every candidate at the drafter's shapes (hidden 4096, MLP 12288, vocabulary
// 151936, M = 16 .. 512), where its pick is within a few per cent of the best.
static FgPlan fg_plan_search(int M, int N, int Kd, bool split) {
  const int cus = fg_cus();
  const double hbm = 5.5e12, cu_load = 40e9, latency = 3e-6, ramp = 1e-6;
  const int WMW = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  const int BM = 32 * WMW;
  const int MT = (M + BM - 1) / BM;
  const int steps = Kd / FG_BK;
  const int NB = (N + 31) / 32;
  const int mrows = std::min(M, BM);
  FgPlan best{8, WMW, 1, steps, MT, std::max(1, std::min(NB, cus / MT)), 0};
  best.nwg = MT * best.G;
  double best_t = 1e30;
  for (int FN : {4, 8}) {
    if (FN == 4 && WMW != 4) continue;
    const int sb = (BM + 32 * FN) * FG_BK * 2;
    const int ns_ring = std::min(4, 160 * 1024 / sb);  // the kernel's ring depth
    for (int S = 1; S <= (split ? std::min(steps, 32) : 1); ++S) {
      const int sps = (steps + S - 1) / S;
      if ((steps + sps - 1) / sps != S) continue;
      const int planes = MT * S;
      if (planes > cus) break;
      for (int rounds = 0; rounds <= 64; ++rounds) {
        // rounds == 0: one round, several chunks per workgroup
        const int G = std::min(NB, std::max(1, (rounds ? rounds : 1) * cus / planes));
        const int bpw = (NB + G - 1) / G;  // blocks of the widest range
        if (rounds > 0 && bpw > FN) continue;
        const int chunks = (bpw + FN - 1) / FN;
        const int nwg = planes * G;
        const int r = (nwg + cus - 1) / cus;
        const double kb = double(sps) * FG_BK * 2;  // bytes of one row over a split
        const double wb = 32.0 * bpw * kb, xb = double(mrows) * kb * chunks;
        const double per_wg = std::max(std::max(wb / MT / (hbm / cus), (wb + xb) / cu_load),
                                       double(chunks) * sps * latency / (ns_ring - 1));
        const double t = r * (per_wg + ramp) + (S > 1 ? 8.0 * S * M * N / hbm : 0.0);
        if (t < best_t * 0.999) {
          best_t = t;
          best = FgPlan{FN, WMW, S, sps, MT, G, nwg};
        }
        if (rounds > 0 && G == NB) break;
      }
    }
  }
  return best;
}

// The search above takes tens of microseconds; calls repeat a few shapes, so
// the plans are kept per (M, N, Kd, split).
FgPlan fg_plan(int M, int N, int Kd, bool split) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, bool>, FgPlan> memo;
  const auto key = std::make_tuple(M, N, Kd, split);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  const FgPlan p = fg_plan_search(M, N, Kd, split);
  std::lock_guard<std::mutex> lock(mu);
  memo.emplace(key, p);
  return p;
}

namespace {

template <int FN, int WMW>
hipError_t fg_launch_shape(const FgArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fg_gemm<FN, WMW>), dim3(grid), dim3(FG_T), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// P = the split partials of X . W^T (with S = 1, the product itself)
hipError_t fg_run(const FgPlan& p, const uint16_t* X, const uint16_t* W, float* P, int M, int N, int Kd,
                  hipStream_t stream) {
  FgArgs a{};
  a.X = X; a.W = W; a.P = P;
  a.M = M; a.N = N; a.Kd = Kd; a.S = p.S; a.steps_per_split = p.steps_per_split; a.MT = p.MT; a.G = p.G;
  a.nwg = p.nwg;
  a.per_xcd = (p.nwg + 7) / 8;
  const int grid = p.MT > 1 ? 8 * a.per_xcd : p.nwg;  // (the remap needs a multiple of 8)
  if (p.WMW == 1) return fg_launch_shape<8, 1>(a, grid, stream);
  if (p.WMW == 2) return fg_launch_shape<8, 2>(a, grid, stream);
  if (p.FN == 4) return fg_launch_shape<4, 4>(a, grid, stream);
  return fg_launch_shape<8, 4>(a, grid, stream);
}


// ---------------------------------------------------------------- the consumers
// Every consumer adds the S split partials of each element in split order, 16
// bytes (four columns) per load, and spreads its rows over the whole chip.

__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
// sum over s < S of load(s), added in order of s; the loads are issued four at
// a time so that a wave waits for one round trip per four splits
template <typename T, typename Load, typename Add>
__device__ __forceinline__ T split_sum(int S, Load load, Add add) {
  T v = load(0);
  int s = 1;
  for (; s + 3 < S; s += 4) {
    const T a = load(s), b = load(s + 1), c = load(s + 2), d = load(s + 3);
    v = add(add(add(add(v, a), b), c), d);
  }
  for (; s < S; ++s) v = add(v, load(s));
  return v;
}
__device__ __forceinline__ float4 split_sum4(const float* P, size_t stride, int S, size_t e) {
  return split_sum<float4>(
      S, [&](int s) { return *reinterpret_cast<const float4*>(P + size_t(s) * stride + e); }, add4);
}
__device__ __forceinline__ float4 bf16x4_to_f32(uint2 b) {
  return make_float4(bf16_to_f32(uint16_t(b.x & 0xffff)), bf16_to_f32(uint16_t(b.x >> 16)),
                     bf16_to_f32(uint16_t(b.y & 0xffff)), bf16_to_f32(uint16_t(b.y >> 16)));
}
__device__ __forceinline__ uint2 f32x4_to_bf16(float4 v) {
  return make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}
__device__ __forceinline__ float4 round_bf16x4(float4 v) { return bf16x4_to_f32(f32x4_to_bf16(v)); }

constexpr int FW_NT = 1024;  // threads of a row-norm workgroup

// (Residual add then) RMSNorm, one workgroup per row m, four columns per
// thread: with partials P, x_out = bf16(x_res + their sum) (x_out may be x_res:
// each element is read and written by the same thread); without, the row is
// x_res itself and x_out is not written.  xn = bf16(row / rms(row) * g).
// Requires d % 4 == 0.
__global__ __launch_bounds__(FW_NT) void fw_add_rmsnorm(const uint16_t* x_res, const float* P, int S, int M, int d,
                                                        const uint16_t* g, float eps, uint16_t* x_out, uint16_t* xn) {
  __shared__ float s_w[FW_NT / 64];
  const int m = blockIdx.x, t = threadIdx.x;
  const size_t stride = size_t(M) * d, row = size_t(m) * d;
  float ss = 0.f;
  for (int c = 4 * t; c < d; c += 4 * FW_NT) {
    float4 v = bf16x4_to_f32(*reinterpret_cast<const uint2*>(x_res + row + c));
    if (P) {
      const float4 p = split_sum4(P, stride, S, row + c);
      v = round_bf16x4(make_float4(v.x + p.x, v.y + p.y, v.z + p.z, v.w + p.w));
      *reinterpret_cast<uint2*>(x_out + row + c) = f32x4_to_bf16(v);
    }
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((t & 63) == 0) s_w[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < FW_NT / 64; ++i) tot += s_w[i];
  const float inv = 1.0f / sqrtf(tot / float(d) + eps);
  const uint16_t* src = P ? x_out : x_res;
  for (int c = 4 * t; c < d; c += 4 * FW_NT) {
    const float4 v = bf16x4_to_f32(*reinterpret_cast<const uint2*>(src + row + c));
    const float4 gg = bf16x4_to_f32(*reinterpret_cast<const uint2*>(g + c));
    *reinterpret_cast<uint2*>(xn + row + c) =
        f32x4_to_bf16(make_float4(v.x * inv * gg.x, v.y * inv * gg.y, v.z * inv * gg.z, v.w * inv * gg.w));
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

// One wave per (row m = b K + i, head): the projection's splits summed and
// rounded to bf16; a Q or K head then gets RMSNorm with its gain and RoPE
// (pairs d, d + hd/2, lane d) at position ctx_len[b] + i; a V head is copied.
// Grid: (M, ceil((n_q + 2 n_kv) / 4)), four waves per workgroup.
__global__ __launch_bounds__(256) void fw_qk_norm_rope(QkArgs a) {
  const int m = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int hd = a.hd, half = hd >> 1;
  const int head = blockIdx.y * 4 + (t >> 6);
  const int nh = a.n_q + 2 * a.n_kv;
  if (head >= nh) return;
  const int b = m / a.K, i = m - b * a.K;
  const int pos = a.ctx_len[b] + i;
  const int ld = nh * hd;
  const size_t stride = size_t(a.M) * ld, base = size_t(m) * ld + size_t(head) * hd;
  // the pair (c, c + half) of this lane, its splits summed, rounded to bf16
  const int c = lane < half ? lane : 0;
  const float2 pr = split_sum<float2>(
      a.S, [&](int s) {
        const float* p = a.P + size_t(s) * stride + base + c;
        return make_float2(p[0], p[half]);
      },
      [](float2 x, float2 y) { return make_float2(x.x + y.x, x.y + y.y); });
  const float xa0 = bf16_to_f32(f32_to_bf16(pr.x)), xb0 = bf16_to_f32(f32_to_bf16(pr.y));
  if (head >= a.n_q + a.n_kv) {  // V head
    if (lane < half) {
      uint16_t* dst = a.vb + (size_t(m) * a.n_kv + (head - a.n_q - a.n_kv)) * hd;
      dst[lane] = f32_to_bf16(xa0);
      dst[half + lane] = f32_to_bf16(xb0);
    }
    return;
  }
  const bool on = lane < half;
  const float xa = on ? xa0 : 0.f, xb = on ? xb0 : 0.f;
  float ss = xa * xa + xb * xb;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (!on) return;
  const float inv = 1.0f / sqrtf(ss / float(hd) + a.eps);
  const uint16_t* g = head < a.n_q ? a.gq : a.gk;
  const float va = xa * inv * bf16_to_f32(g[lane]), vb = xb * inv * bf16_to_f32(g[half + lane]);
  // angle pos * theta^(-2d/hd) in fp64, reduced in fp64, fp32 sin / cos
  float sn, cs;
  sincos_angle(double(pos) * kernarg_elem<double>(offsetof(QkArgs, inv_freq), lane), &sn, &cs);
  uint16_t* dst = head < a.n_q ? a.q + (size_t(m) * a.n_q + head) * hd
                               : a.kb + (size_t(m) * a.n_kv + (head - a.n_q)) * hd;
  dst[lane] = f32_to_bf16(va * cs - vb * sn);
  dst[half + lane] = f32_to_bf16(vb * cs + va * sn);
}

// h = bf16(silu(gate) * up) with gate and up the rounded sums of the gate/up
// projection's splits (a row of it: gate (F), then up (F)); four columns per
// thread over the whole [M, F] output.  Requires F % 4 == 0.
__global__ __launch_bounds__(256) void fw_silu_mul(const float* P, int S, int M, int F, uint16_t* h) {
  const size_t stride = size_t(M) * 2 * F;
  const size_t n4 = size_t(M) * (F / 4);
  for (size_t u = blockIdx.x * size_t(256) + threadIdx.x; u < n4; u += size_t(gridDim.x) * 256) {
    const size_t m = u / (F / 4), c = (u - m * (F / 4)) * 4;
    const float4 gt = round_bf16x4(split_sum4(P, stride, S, m * 2 * F + c));
    const float4 up = round_bf16x4(split_sum4(P, stride, S, m * 2 * F + F + c));
    const float4 r = make_float4(gt.x / (1.0f + expf(-gt.x)) * up.x, gt.y / (1.0f + expf(-gt.y)) * up.y,
                                 gt.z / (1.0f + expf(-gt.z)) * up.z, gt.w / (1.0f + expf(-gt.w)) * up.w);
    *reinterpret_cast<uint2*>(h + m * F + c) = f32x4_to_bf16(r);
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
  const dim3 qk_grid(M, (n_q + 2 * n_kv + 3) / 4);
  const int silu_blocks = int(std::min<size_t>((size_t(M) * (ffn / 4) + 255) / 256, 4096));
  hipLaunchKernelGGL(fw_add_rmsnorm, dim3(M), dim3(FW_NT), 0, stream, x_in, nullptr, 0, M, d, L == 0 ? g_final : lw[0],
                     eps, nullptr, xn);
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
    hipLaunchKernelGGL(fw_qk_norm_rope, qk_grid, dim3(256), 0, stream, qa);
    FW_TRY(launch_attn(q, kb, vb, kc + l * layer_cache, vc + l * layer_cache, cache_base, ctx_len, T_cap, max_ctx,
                       B, K, n_q, n_kv, hd, window, 0, 0.f, att, nullptr, w + Lo.attn_ws, stream));
    FW_TRY(fg_run(p_o, att, w_o, part, M, d, n_q * hd, stream));
    hipLaunchKernelGGL(fw_add_rmsnorm, dim3(M), dim3(FW_NT), 0, stream, xr, part, p_o.S, M, d, g_mlp, eps, x, xn);
    FW_TRY(fg_run(p_gu, xn, w_gu, part, M, 2 * ffn, d, stream));
    hipLaunchKernelGGL(fw_silu_mul, dim3(silu_blocks), dim3(256), 0, stream, part, p_gu.S, M, ffn, h);
    FW_TRY(fg_run(p_dn, h, w_dn, part, M, d, ffn, stream));
    hipLaunchKernelGGL(fw_add_rmsnorm, dim3(M), dim3(FW_NT), 0, stream, x, part, p_dn.S, M, d, g_next, eps, x, xn);
  }
#undef FW_TRY
  return fg_run(p_lm, xn, w_lm, logits, M, V, d, stream);
}

}  // namespace bd
