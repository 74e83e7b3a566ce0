// inject_kv kernels: the layer-batched projection of target hidden states
// into every draft layer's K/V, with RMSNorm + RoPE + bf16 + cache scatter.
//
// DFlash/Spec V2 blog, summary and A2: KV_draft^(l) = Projection^(l)(H_target)
// for every draft layer l.  A7: all layers' projections run as one batched
// linear map, followed by a fused Norm + RoPE post-processing step, and the
// result goes straight into the draft KV cache before the draft forward
// (immediate materialization; the target latents are not kept).
//
// The projection Y = H . W^T runs on the gfx950 32x32x16 bf16 MFMA with fp32
// accumulation: 256 x 256 tiles (ik_proj; ik_proj_persist when there are more
// unsplit tiles than CUs) for more than 256 rows, the weight-streaming GEMM of
// the drafter forward (fg_run) up to 256 rows, and ik_gemm's smaller tiles when
// the K/V blocks do not divide into 256 columns.  The epilogue normalises each
// K head (RMS over hd, times the gain), rotates the half-split pairs
// (i, i + hd/2) by pos * theta^(-2i/hd), rounds K and V to bf16 and writes them
// to the request's cache slot: inside ik_proj when its tile needs no split over
// d_in, otherwise in ik_finish (one workgroup per (row, layer)), which first
// adds the splits' fp32 partials in a fixed order.
#include "bd_common.hpp"
#include "bd_gemm.hpp"
#include "bd_launch.hpp"

#include <math.h>

namespace bd {

// ---------------------------------------------------------------- wide-M projection
// For M > 256: one workgroup computes a 256 x 256 output tile (two heads of one
// layer's K or V block at hd 128) over its d_in range; the two row tiles of a
// column block and the d_in splits of a tile sit at launch indices congruent
// modulo 8, so they share an XCD and its L2.  Eight waves as 4 (M) x 2 (N), each
// a 64 x 128 tile of 32x32x16 MFMAs: a wave holds whole heads, so the RMSNorm
// sum of a row is a reduction over 32 lanes and the rotary pairs (d, d + hd/2)
// sit in the same lane.  Both operands reach LDS straight from global memory
// (global_load_lds, 16 bytes per lane) through rings of SA (H) and SW (W)
// stages of BK-wide d_in steps; in iteration k a loading wave issues its W loads
// of step k + SW - 1, then its H loads of step k + SA - 1 (SW >= SA, so the W
// loads of a step are always older than its H loads).  A row is BK / 8 pieces of
// 16 bytes; the pieces of each 256-byte line are XOR-permuted so the operand
// reads (16 lanes: 16 rows, one piece each) are conflict-free.
//
// With a split over d_in, each split stores its fp32 partial tile to the
// workspace and ik_finish adds the partials in split order and runs the
// epilogue.  With no split the epilogue runs in this kernel: per-head RMSNorm
// and gain, rotary embedding at the row's position, bf16, and the scatter into
// the cache slots (the row map comes from ik_prep).
constexpr int WBM = 256, WBN = 256;
constexpr int WNW = 8, WNT = 64 * WNW;
constexpr int WMW = 4, WNWN = 2;          // waves along M and along N
constexpr int WFM = WBM / WMW / 32;       // 32-row blocks per wave (2)
constexpr int WFN = WBN / WNWN / 32;      // 32-column blocks per wave (4)
static_assert(WFN == 4, "a wave spans 128 columns");
#ifndef BD_GEMM_WIDE_BK
#define BD_GEMM_WIDE_BK 64
#endif
#ifndef BD_GEMM_WIDE_SA
#define BD_GEMM_WIDE_SA 2
#endif
#ifndef BD_GEMM_WIDE_SW
#define BD_GEMM_WIDE_SW 2
#endif
// Split workgroups grouped by d_in range per XCD (1) or launched as (tile, split) (0)
#ifndef BD_GEMM_XCD_MAP
#define BD_GEMM_XCD_MAP 1
#endif
constexpr int WBK = BD_GEMM_WIDE_BK, WSA = BD_GEMM_WIDE_SA, WSW = BD_GEMM_WIDE_SW;
static_assert(WSW >= WSA && WSA >= 2, "ring depths");
constexpr int WA_BYTES = WBM * WBK * 2;
constexpr int WW_BYTES = WBN * WBK * 2;
// Waves that issue the operand loads: one per SIMD, so each SIMD's other
// wave never stalls on a load issue and keeps the matrix pipe busy while its
// partner waits (measured: about 1.5% faster than every wave issuing its
// share, and two loading waves slower).
#ifndef BD_GEMM_WIDE_LOAD_WAVES
#define BD_GEMM_WIDE_LOAD_WAVES 4
#endif
constexpr int WLW = BD_GEMM_WIDE_LOAD_WAVES;
static_assert(WLW <= WNW && (WBN * WBK * 2 / 1024) % WLW == 0, "loading waves");
constexpr int WA_PW = WA_BYTES / 1024 / WLW;  // H loads per loading wave per step
constexpr int WW_PW = WW_BYTES / 1024 / WLW;  // W loads per loading wave per step
static_assert(WSA * WA_BYTES + WSW * WW_BYTES <= 160 * 1024, "LDS");

// byte offset of piece c (16 bytes) of row `row` in a stage
__device__ __forceinline__ int wpiece(int row, int c) {
  constexpr int P = WBK / 8, RPL = 16 / P;  // pieces per row, rows per line
  const int line = row / RPL;
  return (line * 16 + (((row % RPL) * P + c) ^ (line & (P - 1)))) * 16;
}

// ops a wave issues after its H loads of step k (loads complete in order, so
// once no more than these remain, step k's H and W loads have landed)
__device__ __forceinline__ int wide_younger(int k, int ns) {
  int n = 0;
  // rest of the iteration that issued H step k (k - SA + 1): nothing after H
  for (int j = k - WSA + 2; j <= k - 1; ++j) {
    if (j + WSW - 1 < ns) n += WW_PW;
    if (j + WSA - 1 < ns) n += WA_PW;
  }
  return n;
}

struct ProjArgs {
  const uint16_t* A;        // [M, Kd]
  const uint16_t* Bw;       // [N, Kd]
  float* part;              // [S][M][N] partial sums (S > 1)
  const int64_t* rslot;     // [M] cache slot of each row, -1 if the row is not written
  const int32_t* rpos;      // [M] absolute position of each row
  const uint16_t* gain;     // [L][hd] or NULL
  const int32_t* row_cu;
  const int32_t* row_pos0;
  const int64_t* cache_base;
  uint16_t* kc;
  uint16_t* vc;
  int64_t T_cap;
  int M, N, Kd, S, steps_per_split, tiles_n;
  int B, n_kv;
  float eps;
  double inv_freq[64];
};

// Epilogue of one tile from the summed accumulators.  The tile is computed
// transposed (D = W . H^T), so in block (i, j) lane (lr, h) holds row
// 64 wm + 32 i + lr of the tile at the 16 columns 128 wn + 32 j + 8 q + 4 h + e
// (r = 4 q + e).  K heads get RMSNorm x gain and the rotary embedding, V heads
// are copied; both are rounded to bf16 and written to the row's cache slot,
// four consecutive dims per 8-byte store.  lds_g / lds_f: this tile's gains
// (fp32) and inverse frequencies (fp64) staged in LDS.
template <int HD>
__device__ __forceinline__ void proj_epilogue(const ProjArgs& a, floatx16 (&acc)[WFM][WFN], int n0, int wn,
                                              int lane, const int64_t (&slot)[WFM], const int (&pos)[WFM],
                                              const float* lds_g, const double* lds_f) {
  constexpr int BPH = HD / 32;                // 32-column blocks per head
  const int h = lane >> 5;
  const int c0 = n0 + 128 * wn;               // first column of this wave
  const int kvw = a.n_kv * HD;                // columns of one layer's K (or V) block
  const int blk = c0 / kvw;
  const int l = blk >> 1;
  const bool is_k = (blk & 1) == 0;
  const int g0 = (c0 - blk * kvw) / HD;       // first head of this wave
  uint16_t* cache = is_k ? a.kc : a.vc;
#pragma clang loop unroll(full)
  for (int i = 0; i < WFM; ++i) {
    if (is_k) {
      // RMS over each head: this lane's 16 values per block, then the other half
      float s0 = 0.f, s1 = 0.f;
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j)
#pragma clang loop unroll(full)
        for (int r = 0; r < 16; ++r) {
          const float v = acc[i][j][r];
          if (HD == 128 || j < 2) s0 += v * v; else s1 += v * v;
        }
      s0 += xor_lane<32>(s0);
      if constexpr (HD == 64) s1 += xor_lane<32>(s1);
      const float inv0 = 1.0f / sqrtf(s0 / float(HD) + a.eps);
      const float inv1 = HD == 128 ? inv0 : 1.0f / sqrtf(s1 / float(HD) + a.eps);
      // fully unrolled: the accumulators are indexed by r (a loop left rolled
      // would put them in private memory)
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int dd = 8 * (r >> 2) + 4 * h + (r & 3);  // dim within a 32-column block
        // angle pos * theta^(-2d/hd) in fp64, reduced in fp64; HD 128: dims dd
        // and 32 + dd; HD 64: dim dd (both heads)
        float sn[2], cs[2];
#pragma clang loop unroll(full)
        for (int pp = 0; pp < (HD == 128 ? 2 : 1); ++pp)
          sincos_angle(double(pos[i]) * lds_f[32 * pp + dd], &sn[pp], &cs[pp]);
        if constexpr (HD == 64) {
          sn[1] = sn[0];
          cs[1] = cs[0];
        }
        // pairs (d, d + hd/2): HD 128 blocks (0, 2) and (1, 3); HD 64 (0, 1) and (2, 3)
#pragma clang loop unroll(full)
        for (int pp = 0; pp < 2; ++pp) {
          const int ja = HD == 128 ? pp : 2 * pp, jb = HD == 128 ? pp + 2 : 2 * pp + 1;
          const int d = (HD == 128 ? 32 * pp : 0) + dd;
          const float inv = (HD == 128 || pp == 0) ? inv0 : inv1;
          const float xa = acc[i][ja][r] * inv * lds_g[d];
          const float xb = acc[i][jb][r] * inv * lds_g[d + HD / 2];
          acc[i][ja][r] = xa * cs[pp] - xb * sn[pp];
          acc[i][jb][r] = xb * cs[pp] + xa * sn[pp];
        }
      }
    }
    if (slot[i] >= 0) {
      uint16_t* dst = cache + ((size_t(l) * a.T_cap + slot[i]) * a.n_kv + g0) * HD;
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j)
#pragma clang loop unroll(full)
        for (int q = 0; q < 4; ++q) {
          const int col = (j / BPH) * HD + 32 * (j % BPH) + 8 * q + 4 * h;
          const uint2 v = make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                     pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
          *reinterpret_cast<uint2*>(dst + col) = v;
        }
    }
  }
}

// One 256 x 256 output tile over one d_in range (split), from the workgroup's
// LDS rings; the caller's rings are free on entry and free again on return
// once the workgroup has passed a barrier.
template <int HD>
__device__ __forceinline__ void proj_tile(const ProjArgs& g, int tile, int split, uint8_t* ringA, uint8_t* ringW) {
  constexpr int P = WBK / 8;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WNWN, wn = w % WNWN;
  const int lr = lane & 31, h = lane >> 5;
  const int tm = tile / g.tiles_n, tn = tile - tm * g.tiles_n;
  const int m0 = tm * WBM, n0 = tn * WBN;
  const int step0 = split * g.steps_per_split;
  const int ns = min(g.steps_per_split, g.Kd / WBK - step0);
  const uint32_t lA = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ringA)));
  const uint32_t lW = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ringW)));

  // per-lane byte offsets of this wave's loads from the tile's first row at the
  // step's first column: load q of a loading wave fills piece slots
  // 64 (w + WLW q) + lane of a stage
  uint32_t offA[WA_PW], offW[WW_PW];
#pragma unroll
  for (int q = 0; q < WA_PW; ++q) {
    const int ps = (w + WLW * q) * 64 + lane;
    // the (row, piece) that wpiece places at slot ps
    constexpr int RPL = 16 / P;
    const int line = ps >> 4, lc = (ps & 15) ^ (line & (P - 1));
    const int row = line * RPL + lc / P, c = lc % P;
    const int m = min(m0 + row, g.M - 1) - m0;  // rows past M re-read row M - 1; never stored
    offA[q] = uint32_t(m * g.Kd * 2 + c * 16);
  }
#pragma unroll
  for (int q = 0; q < WW_PW; ++q) {
    const int ps = (w + WLW * q) * 64 + lane;
    constexpr int RPL = 16 / P;
    const int line = ps >> 4, lc = (ps & 15) ^ (line & (P - 1));
    const int row = line * RPL + lc / P, c = lc % P;
    offW[q] = uint32_t(row * g.Kd * 2 + c * 16);
  }
  const uint16_t* Abase = g.A + size_t(m0) * g.Kd + size_t(step0) * WBK;
  const uint16_t* Wbase = g.Bw + size_t(n0) * g.Kd + size_t(step0) * WBK;

  floatx16 acc[WFM][WFN];
#pragma unroll
  for (int i = 0; i < WFM; ++i)
#pragma unroll
    for (int j = 0; j < WFN; ++j) acc[i][j] = floatx16{};

  // prologue: the iterations before the loop, W steps 0 .. SW - SA - 1 alone,
  // then (W step j + SW - 1, H step j + SA - 1) for j = -(SA - 1) .. -1
  for (int k = 0; k < WSW - WSA && k < ns && w < WLW; ++k)
#pragma unroll
    for (int q = 0; q < WW_PW; ++q)
      dma16<true>(Wbase + size_t(k) * WBK, offW[q], lW + (k % WSW) * WW_BYTES + (w + WLW * q) * 1024);
  for (int j = -(WSA - 1); j < 0 && w < WLW; ++j) {
    const int kw = j + WSW - 1, ka = j + WSA;
    if (kw < ns)
#pragma unroll
      for (int q = 0; q < WW_PW; ++q)
        dma16<true>(Wbase + size_t(kw) * WBK, offW[q], lW + (kw % WSW) * WW_BYTES + (w + WLW * q) * 1024);
    if (ka - 1 < ns && ka - 1 >= 0)
#pragma unroll
      for (int q = 0; q < WA_PW; ++q)
        dma16<false>(Abase + size_t(ka - 1) * WBK, offA[q], lA + ((ka - 1) % WSA) * WA_BYTES + (w + WLW * q) * 1024);
  }
  for (int k = 0; k < ns; ++k) {
    vm_wait_le<(WSA - 2) * (WA_PW + WW_PW)>(wide_younger(k, ns));
    __syncthreads();
    // refill the stages consumed in iteration k - 1: this wave's W loads, then
    // its H loads (in that order), one after every few MFMAs so that their
    // issue overlaps the MFMAs instead of stalling the SIMD after the barrier
    const int kw = k + WSW - 1, ka = k + WSA - 1;
    auto refill = [&](int d) {
      if (w >= WLW) return;
      if (d < WW_PW) {
        if (kw < ns) dma16<true>(Wbase + size_t(kw) * WBK, offW[d], lW + (kw % WSW) * WW_BYTES + (w + WLW * d) * 1024);
      } else {
        const int q = d - WW_PW;
        if (ka < ns) dma16<false>(Abase + size_t(ka) * WBK, offA[q], lA + (ka % WSA) * WA_BYTES + (w + WLW * q) * 1024);
      }
    };
    constexpr int NDMA = WW_PW + WA_PW;
    constexpr int NMF = (WBK / 16) * WFM * WFN;
#ifdef BD_GEMM_DMA_EVERY
    constexpr int EVERY = BD_GEMM_DMA_EVERY;
#else
    constexpr int EVERY = NMF / NDMA > 2 ? 2 : (NMF / NDMA > 0 ? NMF / NDMA : 1);
#endif
    const uint8_t* As = ringA + (k % WSA) * WA_BYTES;
    const uint8_t* Ws = ringW + (k % WSW) * WW_BYTES;
#pragma unroll
    for (int kk = 0; kk < WBK / 16; ++kk) {
      bf16x8 af[WFM], bfr[WFN];
#pragma unroll
      for (int i = 0; i < WFM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + wpiece(32 * (WFM * wm + i) + lr, 2 * kk + h)));
#pragma unroll
      for (int j = 0; j < WFN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Ws + wpiece(32 * (WFN * wn + j) + lr, 2 * kk + h)));
#pragma unroll
      for (int i = 0; i < WFM; ++i)
#pragma unroll
        for (int j = 0; j < WFN; ++j) {
          acc[i][j] = mfma32x32x16(bfr[j], af[i], acc[i][j]);  // D = W . H^T
          const int m = (kk * WFM + i) * WFN + j;
          if (m % EVERY == 0 && m / EVERY < NDMA) refill(m / EVERY);
        }
    }
    // loads not yet issued (when there are more loads than MFMA slots)
#pragma unroll
    for (int d = (NMF + EVERY - 1) / EVERY; d < NDMA; ++d) refill(d);
  }

  // ------------------------------------------------ split over d_in: partials
  // With a split, the fp32 partial goes to P[split][m][n] for the finish pass
  // (four consecutive columns per 16-byte store).  A reduction inside this
  // kernel (the last split of a tile adding the others' partials) was measured
  // slower: the one reducing CU per tile must read the other splits' 512 KB at
  // its own load rate, which costs as much as the finish pass over all CUs.
  if (g.S > 1) {
    float* P = g.part + size_t(split) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < WFM; ++i) {
      const int m = m0 + 64 * wm + 32 * i + lr;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < WFN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + 128 * wn + 32 * j + 8 * q + 4 * h;
          *reinterpret_cast<floatx4*>(P + size_t(m) * g.N + n) =
              floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
    }
    return;
  }

  // ------------------------------------------------ epilogue
  // this lane's two output rows (64 wm + 32 i + lr): cache slot and position
  int64_t rslot[WFM];
  int rpos[WFM];
#pragma unroll
  for (int i = 0; i < WFM; ++i) {
    const int m = m0 + 64 * wm + 32 * i + lr;
    rslot[i] = m < g.M ? g.rslot[m] : -1;
    rpos[i] = m < g.M ? g.rpos[m] : 0;
  }
  __syncthreads();  // the rings are free: this tile's gains and frequencies go there
  const int kvw = g.n_kv * HD;
  const int l = n0 / (2 * kvw);
  float* lds_g = reinterpret_cast<float*>(ringW);
  double* lds_f = reinterpret_cast<double*>(ringW + HD * 4);
  for (int d = t; d < HD; d += WNT) lds_g[d] = g.gain ? bf16_to_f32(g.gain[l * HD + d]) : 1.f;
  if (t < HD / 2) lds_f[t] = kernarg_elem<double>(offsetof(ProjArgs, inv_freq), t);
  __syncthreads();
  proj_epilogue<HD>(g, acc, n0, wn, lane, rslot, rpos, lds_g, lds_f);
}

template <int HD>
__global__ __launch_bounds__(WNT) void ik_proj(ProjArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ringA[WSA * WA_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ringW[WSW * WW_BYTES];
#if BD_GEMM_XCD_MAP
  // launch index L sits on XCD L mod 8; the workgroups run in the order
  // (split, column tile) major, row tile minor, and XCD x takes the x-th
  // eighth of that order, so its workgroups share few H blocks (one d_in
  // range) and each W block between the row tiles
  const int tiles_m = (g.M + WBM - 1) / WBM;
  const int total = tiles_m * g.tiles_n * g.S;
  const int per_x = (total + 7) / 8;
  const int q = (blockIdx.x & 7) * per_x + (blockIdx.x >> 3);
  if (q >= total) return;
  const int sc = q / tiles_m;
  proj_tile<HD>(g, (q % tiles_m) * g.tiles_n + sc % g.tiles_n, sc / g.tiles_n, ringA, ringW);
#else
  proj_tile<HD>(g, blockIdx.x, blockIdx.y, ringA, ringW);
#endif
}

// Persistent form of the unsplit projection (many tiles per CU, e.g. a whole
// prefill's rows): one workgroup per CU walks its tiles.  The grid is a
// multiple of 8, and launch index w is taken to sit on XCD w mod 8 (the
// dispatcher's round-robin; any other placement gives the same results, only
// less L2 reuse).  The tiles form super-tiles of SM row tiles x SN column
// tiles, one tile per workgroup of an XCD; XCD x takes super-tiles x, x + 8,
// x + 16, ... in row-major order, so the workgroups of one XCD work on one
// super-tile at a time and share its SM H row blocks and SN W column blocks in
// their L2.
#ifndef BD_PERSIST_SN
#define BD_PERSIST_SN 8
#endif
struct PersistPlan {
  int SM, SN, n_sm, n_sn;
};

__device__ __forceinline__ PersistPlan persist_plan(const ProjArgs& g) {
  PersistPlan p;
  const int n_loc = gridDim.x >> 3;
  p.SN = (n_loc % BD_PERSIST_SN == 0) ? BD_PERSIST_SN : n_loc;
  p.SM = n_loc / p.SN;
  const int tiles_m = (g.M + WBM - 1) / WBM;
  p.n_sm = (tiles_m + p.SM - 1) / p.SM;
  p.n_sn = (g.tiles_n + p.SN - 1) / p.SN;
  return p;
}

template <int HD>
__global__ __launch_bounds__(WNT) void ik_proj_persist(ProjArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t ringA[WSA * WA_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ringW[WSW * WW_BYTES];
  const PersistPlan p = persist_plan(g);
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int tiles_m = (g.M + WBM - 1) / WBM;
  for (int s = x; s < p.n_sm * p.n_sn; s += 8) {
    const int tm = (s / p.n_sn) * p.SM + j / p.SN;
    const int tn = (s % p.n_sn) * p.SN + j % p.SN;
    if (tm < tiles_m && tn < g.tiles_n) {
      proj_tile<HD>(g, tm * g.tiles_n + tn, 0, ringA, ringW);
      __syncthreads();  // the epilogue's use of the rings ends before the next tile's loads
    }
  }
}

// Before an unsplit projection: the cache slot (-1: not written) and absolute
// position of every row.
__global__ void ik_prep(ProjArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.M) return;
  int64_t slot = -1;
  int pos = 0;
  if (a.B > 0 && i < a.row_cu[a.B]) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.row_cu[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int jrow = i - a.row_cu[lo];
    pos = a.row_pos0[lo] + jrow;
    const int64_t s = a.cache_base[lo] + pos;
    if (jrow >= 0 && s >= 0 && s < a.T_cap) slot = s;
  }
  const_cast<int64_t*>(a.rslot)[i] = slot;
  const_cast<int32_t*>(a.rpos)[i] = pos;
}
struct FinishArgs {
  const float* P;  // [S][M][N]
  const uint16_t* gain;  // [L][hd] or NULL
  const int32_t* row_cu;
  const int32_t* row_pos0;
  const int64_t* cache_base;
  uint16_t* kc;
  uint16_t* vc;
  int64_t T_cap;
  int B, M, N, S, L, n_kv, hd;
  float eps;
  double inv_freq[64];
};

// A thread item is eight values of one (row, layer): a K item holds dims d0..d0+3
// and hd/2+d0..hd/2+d0+3 of one head (the rotary pairs), a V item eight
// consecutive columns; either is two float4 per split.  The K and V items of the
// row run side by side, every split's loads of an item are issued before the
// first is added (in split order), and the row's request is looked up while
// they are in flight.
constexpr int FIN_SG = 4;  // splits whose loads are in flight together

struct FinRow {
  bool valid;
  int pos;
  int64_t slot;
};

// request, position and cache slot of row m (uniform); row_cu is non-decreasing
__device__ __forceinline__ FinRow fin_lookup(const FinishArgs& f, int m) {
  FinRow r{false, 0, 0};
  if (f.B <= 0 || m >= f.row_cu[f.B]) return r;
  int lo = 0, hi = f.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (f.row_cu[mid] <= m) lo = mid; else hi = mid - 1;
  }
  const int j = m - f.row_cu[lo];
  r.pos = f.row_pos0[lo] + j;
  r.slot = f.cache_base[lo] + r.pos;
  r.valid = j >= 0 && r.slot >= 0 && r.slot < f.T_cap;
  return r;
}

// One item (thread it of the row's 2 n_kv hd / 8): loads every split, then adds
// them in split order and writes the eight outputs.  FIRST: the row lookup runs
// between the first splits' loads and their use (it precedes every store of the
// kernel, so its reads are scalar and do not wait for the vector loads).
template <bool FIRST>
__device__ __forceinline__ void fin_item(const FinishArgs& f, int m, int l, int it, FinRow& row) {
  const int hd = f.hd, half = hd >> 1;
  const int tph = hd / 8;                 // K items per head
  const int n_items_k = f.n_kv * tph;     // as many V items (n_kv * hd / 8)
  const size_t MN = size_t(f.M) * f.N;
  const float* prow = f.P + size_t(m) * f.N + size_t(l) * 2 * f.n_kv * hd;  // the layer's K columns, then V
  const bool act = it < 2 * n_items_k;
  const bool isk = it < n_items_k;
  int head = 0, d0 = 0, off0 = 0, off1 = 0;
  if (isk) {
    head = it / tph;
    d0 = 4 * (it - head * tph);
    off0 = head * hd + d0;
    off1 = off0 + half;
  } else {
    off0 = f.n_kv * hd + (it - n_items_k) * 8;
    off1 = off0 + 4;
  }
  float xa[4] = {0.f, 0.f, 0.f, 0.f}, xb[4] = {0.f, 0.f, 0.f, 0.f};
  double fr[4] = {0.0, 0.0, 0.0, 0.0};
  uint16_t ga[4] = {0, 0, 0, 0}, gb[4] = {0, 0, 0, 0};
  for (int s0 = 0; s0 < f.S; s0 += FIN_SG) {
    float4 va[FIN_SG], vb[FIN_SG];
#pragma unroll
    for (int u = 0; u < FIN_SG; ++u) {
      va[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      vb[u] = va[u];
    }
#pragma unroll
    for (int u = 0; u < FIN_SG; ++u)
      if (s0 + u < f.S && act) {
        va[u] = *reinterpret_cast<const float4*>(prow + (s0 + u) * MN + off0);
        vb[u] = *reinterpret_cast<const float4*>(prow + (s0 + u) * MN + off1);
      }
    if (s0 == 0 && isk) {
      // the item's rotary frequencies and gains, in flight with the partials
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        fr[c] = kernarg_elem<double>(offsetof(FinishArgs, inv_freq), d0 + c);
        if (f.gain) {
          ga[c] = f.gain[l * hd + d0 + c];
          gb[c] = f.gain[l * hd + half + d0 + c];
        }
      }
    }
    if (FIRST && s0 == 0) row = fin_lookup(f, m);
#pragma unroll
    for (int u = 0; u < FIN_SG; ++u)
      if (s0 + u < f.S) {
        xa[0] += va[u].x; xa[1] += va[u].y; xa[2] += va[u].z; xa[3] += va[u].w;
        xb[0] += vb[u].x; xb[1] += vb[u].y; xb[2] += vb[u].z; xb[3] += vb[u].w;
      }
  }
  if (!row.valid || !act) return;
  if (isk) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) ss += xa[c] * xa[c] + xb[c] * xb[c];
    for (int o = tph >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / float(hd) + f.eps);
    uint16_t oa[4], ob[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gxa = f.gain ? bf16_to_f32(ga[c]) : 1.f, gxb = f.gain ? bf16_to_f32(gb[c]) : 1.f;
      const float a = xa[c] * inv * gxa, bb = xb[c] * inv * gxb;
      // angle pos * theta^(-2i/hd), i = d0 + c, in fp64, reduced in fp64
      float sn, cs;
      sincos_angle(double(row.pos) * fr[c], &sn, &cs);
      oa[c] = f32_to_bf16(a * cs - bb * sn);
      ob[c] = f32_to_bf16(bb * cs + a * sn);
    }
    uint16_t* kd = f.kc + ((size_t(l) * f.T_cap + row.slot) * f.n_kv + head) * hd;
    *reinterpret_cast<uint2*>(kd + d0) = make_uint2(oa[0] | (uint32_t(oa[1]) << 16), oa[2] | (uint32_t(oa[3]) << 16));
    *reinterpret_cast<uint2*>(kd + half + d0) = make_uint2(ob[0] | (uint32_t(ob[1]) << 16), ob[2] | (uint32_t(ob[3]) << 16));
  } else {
    uint16_t* vd = f.vc + (size_t(l) * f.T_cap + row.slot) * f.n_kv * hd + (off0 - f.n_kv * hd);
    *reinterpret_cast<uint4*>(vd) = make_uint4(pack_bf16x2(xa[0], xa[1]), pack_bf16x2(xa[2], xa[3]),
                                               pack_bf16x2(xb[0], xb[1]), pack_bf16x2(xb[2], xb[3]));
  }
}

__global__ __launch_bounds__(256) void ik_finish(FinishArgs f) {
  const int m = blockIdx.x, l = blockIdx.y, t = threadIdx.x;
  FinRow row;
  fin_item<true>(f, m, l, t, row);
  if (!row.valid) return;
  const int n_items = 2 * f.n_kv * (f.hd / 8);
  for (int base = 256; base < n_items; base += 256) fin_item<false>(f, m, l, base + t, row);
}

// ---------------------------------------------------------------- host side
static inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

#ifndef BD_GEMM_BN
#define BD_GEMM_BN 128
#endif
#ifndef BD_GEMM_BK
#define BD_GEMM_BK 64
#endif
#ifndef BD_GEMM_WGS
#define BD_GEMM_WGS 512
#endif


struct GemmPlan {
  int bm, bn, bk, S, steps_per_split, tiles;
  bool wide;
  bool stream;  // the weight-streaming GEMM (fg_run) with plan f
  FgPlan f;
};

// The persistent form of the unsplit projection (1) or one workgroup per tile (0)
#ifndef BD_INJECT_PERSIST
#define BD_INJECT_PERSIST 1
#endif

// Rows up to which the projection runs as the weight-streaming GEMM
#ifndef BD_INJECT_STREAM_M
#define BD_INJECT_STREAM_M 256
#endif

// The fused 256 x 256 projection covers M > 256 when every 256-column tile
// lies inside one layer's K or V block (n_kv * hd a multiple of 256); its d_in
// split comes from a cost model of waves and partial traffic.  Up to
// BD_INJECT_STREAM_M rows the projection is bound by streaming the weights
// and runs as the library's weight-streaming GEMM (warp-specialised loader
// waves, a planned d_in split).  Otherwise 256 x BD_GEMM_BN tiles split until
// about BD_GEMM_WGS run.  Every split is followed by the finish pass.
static bool wide_fits(int M, int n_kv, int hd) {
  return M > 256 && (hd == 64 || hd == 128) && (size_t(n_kv) * hd) % WBN == 0;
}

// Compute units of the current device (queried once; 256 if the query fails).
static int inject_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    return cus;
  }();
  return n;
}

static GemmPlan gemm_plan(int M, int N, int Kd, bool wide) {
  GemmPlan p{};
  p.wide = wide;
  if (p.wide) {
    p.bm = WBM; p.bn = WBN; p.bk = WBK;
    p.tiles = ((M + WBM - 1) / WBM) * (N / WBN);
    const int steps = Kd / WBK;
    // the split over d_in with the least modelled time: one workgroup per CU
    // (the LDS rings allow no more), so the busiest CU runs ceil(tiles S /
    // CUs) workgroups of ceil(steps / S) steps (about 1.7 us per step at full
    // load); a split adds its fp32 partials, written once and read once by
    // the finish pass at about 6 TB/s
    const int cus = inject_cus();
    int best_S = 1;
    double best = 1e30;
    for (int S = 1; S <= 8 && S <= steps; ++S) {
      const double waves = double((long long)p.tiles * S + cus - 1) / cus;
      const double t = double(int(waves)) * double((steps + S - 1) / S) * 1.7e-6 +
                       (S > 1 ? 2.0 * S * double(M) * N * 4 / 6e12 : 0.0);
      if (t < best * 0.999) { best = t; best_S = S; }
    }
    p.steps_per_split = (steps + best_S - 1) / best_S;
    p.S = (steps + p.steps_per_split - 1) / p.steps_per_split;
    return p;
  }
  if (M <= BD_INJECT_STREAM_M) {
    p.stream = true;
    p.f = fg_plan(M, N, Kd);
    p.S = p.f.S;
    p.steps_per_split = p.f.steps_per_split;
    p.bm = p.bn = p.bk = p.tiles = 0;
    return p;
  }
  const bool big = M > 128 && N % BD_GEMM_BN == 0;
  p.bm = big ? 256 : 64;
  p.bn = big ? BD_GEMM_BN : 128;
  p.bk = big ? BD_GEMM_BK : 64;
  const int target = big ? BD_GEMM_WGS : 512;
  const int tm = (M + p.bm - 1) / p.bm;
  p.tiles = tm * (N / p.bn);
  const int steps = Kd / p.bk;
  int S = (target + p.tiles / 2) / p.tiles;
  if (S > steps) S = steps;
  if (S < 1) S = 1;
  p.steps_per_split = (steps + S - 1) / S;
  p.S = (steps + p.steps_per_split - 1) / p.steps_per_split;
  return p;
}

// workspace: projection without a split: row slots [M] (int64) and positions
// [M] (int32); with a split (either kernel): the partials [S][M][N] fp32 of the
// finish pass
struct WideLayout {
  size_t rslot, rpos, total;
};
static WideLayout wide_layout(int M) {
  WideLayout w{};
  size_t o = 0;
  w.rslot = o; o += al(size_t(M) * 8);
  w.rpos = o; o += al(size_t(M) * 4);
  w.total = o;
  return w;
}

// workspace a call with exactly M rows uses
static size_t ws_bytes_exact(int M, int d_in, int N, int n_kv, int hd) {
  const bool wide = wide_fits(M, n_kv, hd);
  GemmPlan p = gemm_plan(M, N, d_in, wide);
  if (wide && p.S == 1) return wide_layout(M).total;
  return al(size_t(p.S) * M * N * 4);
}

size_t inject_ws_bytes_call(int M, int d_in, int L, int n_kv, int hd) {
  if (M <= 0) return 0;
  return ws_bytes_exact(M, d_in, L * 2 * n_kv * hd, n_kv, hd);
}

// The size reported covers every call with up to M rows (the unsplit wide
// projection needs less than a smaller, split one): the largest exact need
// over M' <= M.  Within one tile count the need grows with M', so the row
// counts that end a tile (and M itself) are the only candidates.
size_t inject_ws_bytes(int M, int d_in, int L, int n_kv, int hd) {
  if (M <= 0) return 0;
  const int N = L * 2 * n_kv * hd;
  size_t need = ws_bytes_exact(M, d_in, N, n_kv, hd);
  for (int m = 1; m < M && m <= 256; ++m) {
    const size_t x = ws_bytes_exact(m, d_in, N, n_kv, hd);
    if (x > need) need = x;
  }
  for (long long m = 256; m < M; m += 256) {
    const size_t x = ws_bytes_exact(int(m), d_in, N, n_kv, hd);
    if (x > need) need = x;
  }
  return need;
}

hipError_t launch_inject(const uint16_t* h, const uint16_t* w, const uint16_t* gain, const int32_t* row_cu,
                         const int32_t* row_pos0, const int64_t* cache_base, uint16_t* kc, uint16_t* vc,
                         int64_t T_cap, int B, int M, int d_in, int L, int n_kv, int hd, float theta,
                         float eps, void* ws, hipStream_t stream) {
  if (M == 0 || B == 0) return hipSuccess;
  const int N = L * 2 * n_kv * hd;
  const bool wide = wide_fits(M, n_kv, hd);
  GemmPlan p = gemm_plan(M, N, d_in, wide);
  dim3 grid(p.tiles, p.S);
  if (wide) {
    ProjArgs a{};
    a.A = h; a.Bw = w; a.gain = gain; a.row_cu = row_cu; a.row_pos0 = row_pos0; a.cache_base = cache_base;
    a.kc = kc; a.vc = vc; a.T_cap = T_cap;
    a.M = M; a.N = N; a.Kd = d_in; a.S = p.S; a.steps_per_split = p.steps_per_split; a.tiles_n = N / WBN;
    a.B = B; a.n_kv = n_kv; a.eps = eps;
    for (int i = 0; i < hd / 2; ++i) a.inv_freq[i] = pow(double(theta), -2.0 * i / double(hd));
    if (p.S == 1) {
      // fused epilogue: the row map first
      const WideLayout wl = wide_layout(M);
      a.rslot = reinterpret_cast<const int64_t*>(static_cast<char*>(ws) + wl.rslot);
      a.rpos = reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + wl.rpos);
      hipLaunchKernelGGL(ik_prep, dim3((M + 255) / 256), dim3(256), 0, stream, a);
    } else {
      a.part = static_cast<float*>(ws);
    }
    // more unsplit tiles than CUs: the persistent form, one workgroup per CU
    // (the grid a multiple of 8 for its XCD placement)
    const int pgrid = inject_cus() / 8 * 8;
    if (BD_INJECT_PERSIST && p.S == 1 && pgrid >= 8 && p.tiles > inject_cus()) {
      if (hd == 128) hipLaunchKernelGGL(ik_proj_persist<128>, dim3(pgrid), dim3(WNT), 0, stream, a);
      else hipLaunchKernelGGL(ik_proj_persist<64>, dim3(pgrid), dim3(WNT), 0, stream, a);
    } else {
      const dim3 g1 = BD_GEMM_XCD_MAP ? dim3((p.tiles * p.S + 7) / 8 * 8) : grid;
      if (hd == 128) hipLaunchKernelGGL(ik_proj<128>, g1, dim3(WNT), 0, stream, a);
      else hipLaunchKernelGGL(ik_proj<64>, g1, dim3(WNT), 0, stream, a);
    }
    if (p.S == 1) return hipGetLastError();
  }
  if (!wide && p.stream) {
    const hipError_t e = fg_run(p.f, h, w, static_cast<float*>(ws), M, N, d_in, stream);
    if (e != hipSuccess) return e;
  } else if (!wide) {
    GemmArgs g;
    g.A = h; g.Bw = w; g.P = static_cast<float*>(ws);
    g.M = M; g.N = N; g.Kd = d_in; g.S = p.S; g.steps_per_split = p.steps_per_split;
    g.tiles_n = N / p.bn;
    if (p.bm == 256) hipLaunchKernelGGL((ik_gemm<256, BD_GEMM_BN, BD_GEMM_BK>), grid, dim3(GT), 0, stream, g);
    else hipLaunchKernelGGL((ik_gemm<64, 128, 64>), grid, dim3(GT), 0, stream, g);
  }

  FinishArgs f{};
  f.P = static_cast<float*>(ws); f.gain = gain; f.row_cu = row_cu; f.row_pos0 = row_pos0; f.cache_base = cache_base;
  f.kc = kc; f.vc = vc; f.T_cap = T_cap;
  f.B = B; f.M = M; f.N = N; f.S = p.S; f.L = L; f.n_kv = n_kv; f.hd = hd; f.eps = eps;
  for (int i = 0; i < hd / 2; ++i) f.inv_freq[i] = pow(double(theta), -2.0 * i / double(hd));
  hipLaunchKernelGGL(ik_finish, dim3(M, L), dim3(256), 0, stream, f);
  return hipGetLastError();
}

}  // namespace bd
