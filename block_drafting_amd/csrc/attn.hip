// draft_block_attn kernels: split-KV block attention with an exact
// log-sum-exp merge.
//
// DFlash/Spec V2 blog, A2: each draft layer attends to the context K/V that
// was injected from the target, and one forward covers the whole block.
// DSpine article, "principle": DFlash's block positions see each other in
// both directions; "what these weights are": an 8192-token sliding window.
// Didi EAGLE-3 article, 5.3: attention computed over disjoint key sets merges
// exactly through each part's running maximum and normaliser (streaming
// softmax), which is what lets the context be cut into chunks that run on
// different compute units.
//
// Item = (request b, KV head g): its visible context in 64-key tiles plus one
// tile holding the K in-block keys.  The item's query rows are the group's
// (n_q / n_kv) heads at all K block positions (row r = i * group + hh).  The
// partial kernel is persistent and balanced: all tiles of all items form one
// sequence and each workgroup takes an equal run of it (the schedule is
// rebuilt on the device from ctx_len, so ragged batches need no host copy of
// the lengths); it writes one partial (O, max, normaliser) per item it
// touches, and the merge kernel combines an item's partials exactly.  Each
// wave owns 16-row blocks; the key tile is staged once in LDS and shared by
// the four waves.
//
// Per 64-key tile and 16-row block, with the gfx950 16x16x32 bf16 MFMA:
//   S^T[key][row] = K[key][:] . Q[row][:]          (A = K from LDS, B = Q regs)
//   online softmax per row in the exp2 domain
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]  (A = V from LDS, B = P regs)
// Keeping keys on the M side of S^T puts one row per lane column, so P leaves
// the accumulators already in the B-operand layout (with a fixed permutation
// of the 32 keys of a k-step that V's fragment reproduces).
#include "bd_common.hpp"
#include "bd_launch.hpp"

#include <math.h>

namespace bd {

constexpr int AT = 256;  // threads per workgroup (4 waves)

// Register budget of the persistent partial kernel (waves per SIMD it must
// allow); its grid is the number of workgroups that are resident at once
// (CUs x workgroups per CU from the occupancy query), at most BD_ATTN_GRID.
#ifndef BD_ATTN_GRID
#define BD_ATTN_GRID 1024
#endif
#ifndef BD_ATTN_WPE
#define BD_ATTN_WPE 2
#endif
#define BD_ATTN_OCC __attribute__((amdgpu_waves_per_eu(BD_ATTN_WPE)))
constexpr int TK = 64;   // keys per tile

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kb;
  const uint16_t* vb;
  const uint16_t* kc;
  const uint16_t* vc;
  const int64_t* cache_base;
  const int32_t* ctx_len;
  int64_t T_cap;
  int B, K, n_q, n_kv, group, R;  // R = K * group query rows per item
  int window, max_ctx;
  int grid;                       // workgroups of the partial kernel
  int tmin;                       // fewest tiles a workgroup takes
  float sl2;                      // scale * log2(e)
  uint16_t* out;
  float* lse;
  float* wo;   // [items + grid][R][HD] partial outputs
  float* wml;  // [items + grid][R][2]  running max (exp2 domain), normaliser
};

// visible context of request b, or ok = false when its metadata is invalid
__device__ __forceinline__ bool visible(const AttnArgs& a, int b, int64_t& base, int& lo, int& hi) {
  base = a.cache_base[b];
  int ctx = a.ctx_len[b];
  if (ctx < 0 || ctx > a.max_ctx || base < 0 || base + ctx > a.T_cap) return false;
  lo = (a.window > 0 && ctx > a.window) ? ctx - a.window : 0;
  hi = ctx;
  return true;
}

// Tiles of request b: its visible context in 64-key tiles, then one tile for
// the block keys.  Invalid requests get the block tile only.
__device__ __forceinline__ int req_tiles(const AttnArgs& a, int b) {
  int64_t base;
  int lo, hi;
  if (!visible(a, b, base, lo, hi)) return 1;
  return (hi - lo + TK - 1) / TK + 1;
}

constexpr int TMIN = 4;     // fewest tiles a workgroup takes
constexpr int MAXSEG = 64;  // partial records one merge may combine

// Shared schedule: every workgroup (and the merge) derives the same tile
// prefix over requests from ctx_len: item i = b * n_kv + g owns global tiles
// [s_i, s_i + nt_b) with s_i = n_kv * P_b + g * nt_b, P_b = sum_{b' < b} nt_b'.
// Workgroup w takes global tiles [w * tpw, (w + 1) * tpw).
struct Sched {
  int total;  // all tiles
  int tpw;    // tiles per workgroup
};

__device__ Sched build_sched(const AttnArgs& a, int* s_pref /* [B + 1] */) {
  const int t = threadIdx.x;
  // per-request tile counts, prefix by one thread per 256 requests (B <= 4096)
  for (int b = t; b < a.B; b += AT) s_pref[b + 1] = req_tiles(a, b);
  __syncthreads();
  if (t == 0) {
    s_pref[0] = 0;
    for (int b = 0; b < a.B; ++b) s_pref[b + 1] += s_pref[b];
  }
  __syncthreads();
  Sched s;
  s.total = a.n_kv * s_pref[a.B];
  int tpw = (s.total + a.grid - 1) / a.grid;
  s.tpw = tpw < a.tmin ? a.tmin : tpw;
  return s;
}

// request holding global tile x (binary search over the prefix)
__device__ __forceinline__ int find_req(const AttnArgs& a, const int* s_pref, int x) {
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a.n_kv * s_pref[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Loads of one tile into registers: K as 16-byte pieces t + p * AT (key =
// piece / (HD/8)); V as keys 4 kg .. 4 kg + 3 of column piece vd for threads
// t < (HD/8) * 16 (kg = t % 16, vd = t / 16).  Loads are unconditional (keys
// past the tile's end re-read key 0) so they stay in flight until used; the
// caller masks keys >= the returned count.
template <int HD>
__device__ __forceinline__ int fetch_tile(const AttnArgs& a, int ti, int nt, int b, int g, int64_t cbase, int lo,
                                          int nctx, int t, u32x4 (&pk)[TK * HD / 8 / AT], u32x4 (&pv)[4]) {
  constexpr int PPT = TK * HD / 8 / AT;
  constexpr int NDC = HD / 8;
  constexpr int VTH = NDC * (TK / 4);
  const size_t kstride = size_t(a.n_kv) * HD;
  const int kg = t & 15, vd = t >> 4;
  const uint16_t* kp;
  const uint16_t* vp;
  int nkeys;
  if (ti == nt - 1) {
    kp = a.kb + (size_t(b) * a.K * a.n_kv + g) * HD;
    vp = a.vb + (size_t(b) * a.K * a.n_kv + g) * HD;
    nkeys = a.K;
  } else {
    const int k0 = ti * TK;
    kp = a.kc + (size_t(cbase + lo + k0) * a.n_kv + g) * HD;
    vp = a.vc + (size_t(cbase + lo + k0) * a.n_kv + g) * HD;
    nkeys = min(TK, nctx - k0);
  }
#pragma unroll
  for (int p = 0; p < PPT; ++p) {
    const int piece = t + p * AT;
    const int key = piece / NDC, dc = piece - key * NDC;
    pk[p] = ld_stream_v(kp + size_t(key < nkeys ? key : 0) * kstride + dc * 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 4 * kg + i;
    const bool in = t < VTH && key < nkeys;
    pv[i] = ld_stream_v(vp + (in ? size_t(key) * kstride + vd * 8 : 0));
  }
  return nkeys;
}

// One key tile (in LDS) against the wave's 16-row blocks: scores, online
// softmax in the exp2 domain, and the P.V accumulation.
template <int HD, int RB>
__device__ __forceinline__ void tile_math(const AttnArgs& a, const uint16_t* Ks, const uint16_t* Vt, int nvalid,
                                          int w, int lr, int q4, const bf16x8 (&qf)[RB][HD / 32],
                                          floatx4 (&acc)[RB][HD / 16], float (&m_run)[RB], float (&l_run)[RB]) {
  constexpr int LS = HD + 8;
  constexpr int LV = TK + 8;
  constexpr int NKS = HD / 32;
  constexpr int NDB = HD / 16;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    if ((w + 4 * j) * 16 >= a.R) continue;
    floatx4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&Ks[(kb * 16 + lr) * LS + ks * 32 + q4 * 8]);
        s[kb] = mfma16x16x32(as_bf16x8(kv), qf[j][ks], s[kb]);
      }
    }
    // lane holds keys kb*16 + 4*q4 + r for row lr
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * 16 + q4 * 4 + r;
        float v = s[kb][r] * a.sl2;
        v = key < nvalid ? v : -INFINITY;
        s[kb][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run[j], tmax);
    const float alpha = exp2f(m_run[j] - m_new);
    m_run[j] = m_new;
    float psum = 0.f;
    uint32_t pw[8];  // P^T fragments: two k-steps of 32 keys, 4 dwords each
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float pe[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pe[r] = exp2f(s[2 * ks2][r] - m_new);
        pe[4 + r] = exp2f(s[2 * ks2 + 1][r] - m_new);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) psum += pe[r];
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[ks2 * 4 + r] = pack_bf16x2(pe[2 * r], pe[2 * r + 1]);
    }
    l_run[j] = l_run[j] * alpha + psum;
#pragma unroll
    for (int d = 0; d < NDB; ++d) acc[j][d] *= alpha;
    // O^T += V^T P^T; the V fragment of lane (dim = 16d + lr) holds the
    // same 8 keys of the k-step, in the same order, as its P fragment
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pw[ks2 * 4], pw[ks2 * 4 + 1], pw[ks2 * 4 + 2], pw[ks2 * 4 + 3]));
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const uint4 vf = *reinterpret_cast<const uint4*>(&Vt[(d * 16 + lr) * LV + ks2 * 32 + q4 * 8]);
        acc[j][d] = mfma16x16x32(as_bf16x8(vf), pb, acc[j][d]);
      }
    }
  }
}

template <int HD, int RB>
__global__ __launch_bounds__(AT) BD_ATTN_OCC void attn_partial(AttnArgs a) {
  constexpr int LS = HD + 8;          // K tile row stride (elements)
  constexpr int LV = TK + 8;          // V^T tile row stride (elements)
  constexpr int PIECES = TK * HD / 8;  // 16-byte pieces per tile
  constexpr int PPT = PIECES / AT;     // K pieces per thread
  constexpr int NDC = HD / 8;          // 16-byte pieces per key row
  constexpr int VTH = NDC * (TK / 4);  // threads staging V (4 keys x 16 bytes each)
  constexpr int NKS = HD / 32;         // k-steps of the score MFMA
  constexpr int NDB = HD / 16;         // dim blocks of the output MFMA
  // K tile row-major [key][dim]; V tile transposed [dim][column] with key k at
  // column vcol(k): within each 32 keys, keys 4q..4q+3 and 16+4q..16+4q+3 sit
  // side by side at columns 8q..8q+7, which is the order in which a lane's P
  // fragment holds them, so a V fragment is one 16-byte LDS read.
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TK * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HD * LV];
  extern __shared__ int s_pref[];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lr = lane & 15, q4 = lane >> 4;
  const Sched sc = build_sched(a, s_pref);
  const int wg = blockIdx.x;
  int x = wg * sc.tpw;
  const int x_end = min(x + sc.tpw, sc.total);
  const size_t kstride = size_t(a.n_kv) * HD;

  while (x < x_end) {
    // the segment of this workgroup inside one item
    const int b = find_req(a, s_pref, x);
    const int nt = s_pref[b + 1] - s_pref[b];
    const int g = (x - a.n_kv * s_pref[b]) / nt;
    const int item_s = a.n_kv * s_pref[b] + g * nt;
    const int t0 = x - item_s;                      // first tile of the item we take
    const int t1 = min(nt, x_end - item_s);         // one past the last
    const int item = b * a.n_kv + g;
    int64_t cbase;
    int lo, hi;
    const bool ok = visible(a, b, cbase, lo, hi);
    const int nctx = ok ? hi - lo : 0;              // context keys of the item

    // query fragments: B operand of S^T, lane holds Q[row][32ks + 8q4 .. +8]
    bf16x8 qf[RB][NKS];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int row = (w + 4 * j) * 16 + lr;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < a.R) {
          const int i = row / a.group, hh = row - i * a.group;
          const uint16_t* qp = a.q + ((size_t(b) * a.K + i) * a.n_q + g * a.group + hh) * HD + ks * 32 + q4 * 8;
          v = *reinterpret_cast<const uint4*>(qp);
        }
        qf[j][ks] = as_bf16x8(v);
      }
    }
    floatx4 acc[RB][NDB];
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      m_run[j] = -INFINITY;
      l_run[j] = 0.f;
#pragma unroll
      for (int d = 0; d < NDB; ++d) acc[j][d] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // tile ti < nt - 1: context keys [lo + 64 ti, ...); tile nt - 1: block keys
    // K: thread loads pieces t + p * AT (key = piece / NDC, 16-byte column
    // piece % NDC); V: thread t < VTH loads keys 4 kg .. 4 kg + 3 of 16-byte
    // column vd, kg = t % 16, vd = t / 16.
    const int kg = t & 15, vd = t >> 4;
    u32x4 pk[PPT], pv[4];
    int nvalid_next = fetch_tile<HD>(a, t0, nt, b, g, cbase, lo, nctx, t, pk, pv);
    // all tiles but the last: the look-ahead fetch is unconditional
    for (int ti = t0; ti < t1; ++ti) {
      const int nvalid = nvalid_next;
      __syncthreads();
      // the loads were unconditional: keys past the tile's valid count are
      // zeroed here, where the data is consumed
      const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < PPT; ++p) {
        const int piece = t + p * AT;
        const int key = piece / NDC, dc = piece - key * NDC;
        *reinterpret_cast<u32x4*>(&Ks[key * LS + dc * 8]) = key < nvalid ? pk[p] : z4;
      }
      if (t < VTH) {
        // transpose 4 keys x 8 dims into 8 dims x 4 keys (bf16 pairs)
        const int col = 32 * (kg >> 3) + 8 * (kg & 3) + 4 * ((kg >> 2) & 1);
        const u32x4 a0 = 4 * kg + 0 < nvalid ? pv[0] : z4;
        const u32x4 a1 = 4 * kg + 1 < nvalid ? pv[1] : z4;
        const u32x4 a2 = 4 * kg + 2 < nvalid ? pv[2] : z4;
        const u32x4 a3 = 4 * kg + 3 < nvalid ? pv[3] : z4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint2 even = make_uint2((a0[m] & 0xffffu) | (a1[m] << 16), (a2[m] & 0xffffu) | (a3[m] << 16));
          const uint2 odd = make_uint2((a0[m] >> 16) | (a1[m] & 0xffff0000u), (a2[m] >> 16) | (a3[m] & 0xffff0000u));
          *reinterpret_cast<uint2*>(&Vt[(vd * 8 + 2 * m) * LV + col]) = even;
          *reinterpret_cast<uint2*>(&Vt[(vd * 8 + 2 * m + 1) * LV + col]) = odd;
        }
      }
      __syncthreads();
      if (ti + 1 == t1) {
        tile_math<HD, RB>(a, Ks, Vt, nvalid, w, lr, q4, qf, acc, m_run, l_run);
        break;
      }
      nvalid_next = fetch_tile<HD>(a, ti + 1, nt, b, g, cbase, lo, nctx, t, pk, pv);
      tile_math<HD, RB>(a, Ks, Vt, nvalid, w, lr, q4, qf, acc, m_run, l_run);
    }

    // partial result of (item, workgroup): slot item + wg is unique because a
    // later item only starts in a workgroup at or after this one's last
    const size_t slot = size_t(item) + wg;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int row = (w + 4 * j) * 16 + lr;
      float l = l_run[j];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      if (row < a.R) {
        float* o = a.wo + (slot * a.R + row) * HD;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
          *reinterpret_cast<floatx4*>(o + d * 16 + q4 * 4) = acc[j][d];
        if (q4 == 0) {
          a.wml[(slot * a.R + row) * 2] = m_run[j];
          a.wml[(slot * a.R + row) * 2 + 1] = l;
        }
      }
    }
    x = item_s + t1;
  }
}

template <int HD>
__global__ __launch_bounds__(AT) void attn_merge(AttnArgs a) {
  extern __shared__ int s_pref[];
  __shared__ float s_f[MAXSEG * 128];  // per record and row: 2^(m - M) / L
  __shared__ int s_ns;
  const int item = blockIdx.x, t = threadIdx.x;
  const int b = item / a.n_kv, g = item - b * a.n_kv;
  const Sched sc = build_sched(a, s_pref);
  const int nt = s_pref[b + 1] - s_pref[b];
  const int item_s = a.n_kv * s_pref[b] + g * nt;
  const int w0 = item_s / sc.tpw, w1 = (item_s + nt - 1) / sc.tpw;
  const int ns = w1 - w0 + 1;
  int64_t cbase;
  int lo, hi;
  const bool ok = visible(a, b, cbase, lo, hi) && ns <= MAXSEG;
  const size_t slot0 = size_t(item) + w0;
  if (t < a.R) {
    const int row = t;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.wml[((slot0 + s) * a.R + row) * 2]);
    float L = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = a.wml[((slot0 + s) * a.R + row) * 2];
      L += a.wml[((slot0 + s) * a.R + row) * 2 + 1] * exp2f(ms - M);
    }
    const float inv = 1.f / L;
    if (ok)
      for (int s = 0; s < ns; ++s) s_f[s * 128 + row] = exp2f(a.wml[((slot0 + s) * a.R + row) * 2] - M) * inv;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = (size_t(b) * a.K + i) * a.n_q + g * a.group + hh;
    if (a.lse) a.lse[oidx] = ok ? (M + log2f(L)) * 0.6931471805599453f : NAN;
  }
  __syncthreads();
  // outputs four dims at a time; the records of one float4 load independently
  for (int e4 = t; e4 < a.R * HD / 4; e4 += AT) {
    const int row = e4 / (HD / 4), d4 = (e4 - row * (HD / 4)) * 4;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = (size_t(b) * a.K + i) * a.n_q + g * a.group + hh;
    uint2 packed;
    if (!ok) {
      packed = make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    } else {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < ns; ++s) {
        const float f = s_f[s * 128 + row];
        const float4 v = *reinterpret_cast<const float4*>(a.wo + ((slot0 + s) * a.R + row) * HD + d4);
        o.x += v.x * f; o.y += v.y * f; o.z += v.z * f; o.w += v.w * f;
      }
      packed = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
    }
    *reinterpret_cast<uint2*>(a.out + oidx * HD + d4) = packed;
  }
}

// ---------------------------------------------------------------- host side
static inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int PARTIAL_GRID = BD_ATTN_GRID;

// At least TMIN tiles per workgroup, and enough that one item (at most
// vis/64 + 1 tiles) spans no more than MAXSEG workgroups.
static int attn_tmin(int max_ctx, int window) {
  const int vis = (window > 0 && max_ctx > window) ? window : max_ctx;
  const int nt_max = (vis + TK - 1) / TK + 1;
  const int t = (nt_max + MAXSEG - 3) / (MAXSEG - 2);
  return t > TMIN ? t : TMIN;
}

// upper bound of the grid (sizes the workspace)
static int attn_grid(int B, int n_kv, int max_ctx, int window) {
  const int vis = (window > 0 && max_ctx > window) ? window : max_ctx;
  const long long tiles = (long long)B * n_kv * ((vis + TK - 1) / TK + 1);  // upper bound
  const int tmin = attn_tmin(max_ctx, window);
  long long g = (tiles + tmin - 1) / tmin;
  if (g > PARTIAL_GRID) g = PARTIAL_GRID;
  if (g < 1) g = 1;
  return int(g);
}

// Workgroups of attn_partial<HD, RB> that fit on the device at once (queried
// once per variant; falls back to two per CU on 256 CUs).
template <int HD, int RB>
static int resident_partial() {
  static const int n = [] {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, attn_partial<HD, RB>, AT, 4096) != hipSuccess || per < 1)
      per = 2;
    return cus * per;
  }();
  return n;
}

size_t attn_ws_bytes(int B, int K, int n_q, int n_kv, int hd, int max_ctx, int window) {
  if (B <= 0) return 0;
  const size_t R = size_t(K) * (n_q / n_kv);
  const size_t slots = size_t(B) * n_kv + attn_grid(B, n_kv, max_ctx, window);
  return al(slots * R * hd * 4) + al(slots * R * 2 * 4);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kb, const uint16_t* vb, const uint16_t* kc,
                       const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                       int64_t T_cap, int max_ctx, int B, int K, int n_q, int n_kv, int hd, int window,
                       float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  AttnArgs a{};
  a.q = q; a.kb = kb; a.vb = vb; a.kc = kc; a.vc = vc;
  a.cache_base = cache_base; a.ctx_len = ctx_len; a.T_cap = T_cap;
  a.B = B; a.K = K; a.n_q = n_q; a.n_kv = n_kv; a.group = n_q / n_kv; a.R = K * a.group;
  a.window = window; a.max_ctx = max_ctx;
  a.tmin = attn_tmin(max_ctx, window);
  const bool two = a.R > 64;
  const int resident = hd == 128 ? (two ? resident_partial<128, 2>() : resident_partial<128, 1>())
                                 : (two ? resident_partial<64, 2>() : resident_partial<64, 1>());
  a.grid = attn_grid(B, n_kv, max_ctx, window);
  if (a.grid > resident) a.grid = resident;
  const float sc = scale > 0.f ? scale : float(1.0 / sqrt(double(hd)));
  a.sl2 = float(double(sc) * 1.4426950408889634);
  a.out = out; a.lse = lse;
  const size_t R = size_t(a.R);
  const size_t slots = size_t(B) * n_kv + a.grid;
  a.wo = static_cast<float*>(ws);
  a.wml = reinterpret_cast<float*>(static_cast<char*>(ws) + al(slots * R * hd * 4));
  const size_t pref_bytes = size_t(B + 1) * sizeof(int);
  if (hd == 128) {
    if (two) hipLaunchKernelGGL((attn_partial<128, 2>), dim3(a.grid), dim3(AT), pref_bytes, stream, a);
    else hipLaunchKernelGGL((attn_partial<128, 1>), dim3(a.grid), dim3(AT), pref_bytes, stream, a);
    hipLaunchKernelGGL(attn_merge<128>, dim3(B * n_kv), dim3(AT), pref_bytes, stream, a);
  } else {
    if (two) hipLaunchKernelGGL((attn_partial<64, 2>), dim3(a.grid), dim3(AT), pref_bytes, stream, a);
    else hipLaunchKernelGGL((attn_partial<64, 1>), dim3(a.grid), dim3(AT), pref_bytes, stream, a);
    hipLaunchKernelGGL(attn_merge<64>, dim3(B * n_kv), dim3(AT), pref_bytes, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bd
