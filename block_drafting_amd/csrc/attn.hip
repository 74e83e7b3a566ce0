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
// Item = (request b, KV head g): its visible context in 32-key tiles plus
// ceil(K/32) tiles holding the K in-block keys.  The item's query rows are the
// group's (n_q / n_kv) heads at all K block positions (row r = i * group + hh);
// each wave owns 32 of them.  The partial kernel is persistent and balanced:
// all tiles of all items form one sequence and each workgroup takes an equal
// run of it (the schedule is rebuilt on the device from ctx_len, so ragged
// batches need no host copy of the lengths); it writes one partial (O, max,
// normaliser) per item it touches, and the merge kernel combines an item's
// partials exactly.  A key tile is staged once in LDS and shared by the waves.
//
// Per 32-key tile and 32-row wave, with the gfx950 32x32x16 bf16 MFMA:
//   S^T[key][row] = K[key][:] . Q[row][:]          (A = K from LDS, B = Q regs)
//   online softmax per row in the exp2 domain
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]  (A = V from LDS, B = P regs)
// Keys on the M side of S^T put one query row per lane column, so the score
// accumulators already hold the B operand of the P.V product: within each 16
// keys a lane holds keys 4h..4h+3 and 8+4h..8+4h+3 (h = lane / 32), and V^T is
// staged with exactly that key order so its fragment is one 16-byte LDS read.
#include "bd_common.hpp"
#include "bd_launch.hpp"

#include <math.h>

namespace bd {

constexpr int TK = 32;   // keys per tile
constexpr int MT = 256;  // threads of a merge workgroup

// Register budget of the persistent partial kernel (waves per SIMD it must
// allow); its grid is the number of workgroups resident at once (CUs x
// workgroups per CU from the occupancy query), at most BD_ATTN_GRID.
#ifndef BD_ATTN_GRID
#define BD_ATTN_GRID 2048
#endif
#ifndef BD_ATTN_WPE
#define BD_ATTN_WPE 2
#endif
#define BD_ATTN_OCC(NW) __attribute__((amdgpu_waves_per_eu(NW == 1 ? 1 : BD_ATTN_WPE)))

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
  int nbt;                        // tiles of block keys per item, ceil(K / 32)
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

// Tiles of request b: its visible context in 32-key tiles, then the block
// keys.  Invalid requests get the block tiles only.
__device__ __forceinline__ int req_tiles(const AttnArgs& a, int b) {
  int64_t base;
  int lo, hi;
  if (!visible(a, b, base, lo, hi)) return a.nbt;
  return (hi - lo + TK - 1) / TK + a.nbt;
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
  // per-request tile counts, prefix by thread 0
  for (int b = t; b < a.B; b += blockDim.x) s_pref[b + 1] = req_tiles(a, b);
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

// Staging of one 32-key tile by NT threads: K as 16-byte pieces
// t + p * NT (key = piece / (HD/8)); V as units u = t + i * NT < 8 * (HD/8),
// each four keys 4 kg .. 4 kg + 3 (kg = u % 8) of one 16-byte dim piece
// vd = u / 8.  Loads are unconditional (keys past the tile end re-read a
// valid line) so they stay in flight until used; the stager masks keys >=
// the returned count.
template <int HD, int NT>
struct TileRegs {
  static constexpr int KPIECES = TK * HD / 8;
  static constexpr int KP = (KPIECES + NT - 1) / NT;
  static constexpr int VUNITS = (TK / 4) * (HD / 8);
  static constexpr int VU = (VUNITS + NT - 1) / NT;
  u32x4 k[KP];
  u32x4 v[VU][4];
};

template <int HD, int NT>
__device__ __forceinline__ int fetch_tile(const AttnArgs& a, int ti, int nct, int nt, int b, int g,
                                          int64_t cbase, int lo, int nctx, int t, TileRegs<HD, NT>& r) {
  using TR = TileRegs<HD, NT>;
  const size_t kstride = size_t(a.n_kv) * HD;
  const uint16_t* kp;
  const uint16_t* vp;
  int nkeys;
  if (ti >= nt) {
    // past the segment: the same number of loads from one valid line, so the
    // count of loads in flight does not depend on the path
    kp = a.kb + (size_t(b) * a.K * a.n_kv + g) * HD;
    vp = kp;
    nkeys = 0;
  } else if (ti >= nct) {
    const int k0 = (ti - nct) * TK;
    kp = a.kb + ((size_t(b) * a.K + k0) * a.n_kv + g) * HD;
    vp = a.vb + ((size_t(b) * a.K + k0) * a.n_kv + g) * HD;
    nkeys = min(TK, a.K - k0);
  } else {
    const int k0 = ti * TK;
    kp = a.kc + (size_t(cbase + lo + k0) * a.n_kv + g) * HD;
    vp = a.vc + (size_t(cbase + lo + k0) * a.n_kv + g) * HD;
    nkeys = min(TK, nctx - k0);
  }
#pragma unroll
  for (int p = 0; p < TR::KP; ++p) {
    const int piece = t + p * NT;
    const int key = piece / (HD / 8), dc = piece - key * (HD / 8);
    const bool in = piece < TR::KPIECES && key < nkeys;
    r.k[p] = ld_stream_v(kp + (in ? size_t(key) * kstride + dc * 8 : 0));
  }
#pragma unroll
  for (int i = 0; i < TR::VU; ++i) {
    const int u = t + i * NT;
    const int kg = u & 7, vd = u >> 3;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int key = 4 * kg + c;
      const bool in = u < TR::VUNITS && key < nkeys;
      r.v[i][c] = ld_stream_v(vp + (in ? size_t(key) * kstride + vd * 8 : 0));
    }
  }
  return nkeys;
}

// LDS column of key 4 kg within a tile's V^T rows (see the header comment)
__device__ __forceinline__ int vcol(int kg) { return 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1); }

template <int HD, int NT>
__device__ __forceinline__ void stage_tile(const TileRegs<HD, NT>& r, int nvalid, int t, uint16_t* Ks, uint16_t* Vt) {
  using TR = TileRegs<HD, NT>;
  constexpr int LS = HD + 8;
  constexpr int LV = TK + 8;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < TR::KP; ++p) {
    const int piece = t + p * NT;
    const int key = piece / (HD / 8), dc = piece - key * (HD / 8);
    if (piece < TR::KPIECES) *reinterpret_cast<u32x4*>(&Ks[key * LS + dc * 8]) = key < nvalid ? r.k[p] : z4;
  }
#pragma unroll
  for (int i = 0; i < TR::VU; ++i) {
    const int u = t + i * NT;
    if (u < TR::VUNITS) {
      const int kg = u & 7, vd = u >> 3;
      const int col = vcol(kg);
      const u32x4 a0 = 4 * kg + 0 < nvalid ? r.v[i][0] : z4;
      const u32x4 a1 = 4 * kg + 1 < nvalid ? r.v[i][1] : z4;
      const u32x4 a2 = 4 * kg + 2 < nvalid ? r.v[i][2] : z4;
      const u32x4 a3 = 4 * kg + 3 < nvalid ? r.v[i][3] : z4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // dims 2m and 2m + 1 of the piece, keys 4 kg .. 4 kg + 3
        const uint2 even = make_uint2((a0[m] & 0xffffu) | (a1[m] << 16), (a2[m] & 0xffffu) | (a3[m] << 16));
        const uint2 odd = make_uint2((a0[m] >> 16) | (a1[m] & 0xffff0000u), (a2[m] >> 16) | (a3[m] & 0xffff0000u));
        *reinterpret_cast<uint2*>(&Vt[(vd * 8 + 2 * m) * LV + col]) = even;
        *reinterpret_cast<uint2*>(&Vt[(vd * 8 + 2 * m + 1) * LV + col]) = odd;
      }
    }
  }
}

// One key tile (in LDS) against the wave's 32 query rows: scores, online
// softmax in the exp2 domain, and the P.V accumulation.
template <int HD>
__device__ __forceinline__ void tile_math(const AttnArgs& a, const uint16_t* Ks, const uint16_t* Vt, int nvalid,
                                          int lane, const bf16x8 (&qf)[HD / 16], floatx16 (&acc)[HD / 32],
                                          float& m_run, float& l_run) {
  constexpr int LS = HD + 8;
  constexpr int LV = TK + 8;
  const int lr = lane & 31, h = lane >> 5;
  floatx16 s = {};
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) {
    const u32x4 kf = *reinterpret_cast<const u32x4*>(&Ks[lr * LS + ks * 16 + h * 8]);
    s = mfma32x32x16(__builtin_bit_cast(bf16x8, kf), qf[ks], s);
  }
  // lane holds keys 8 (r / 4) + 4 h + r % 4 of row lr
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + 4 * h + (r & 3);
    const float v = key < nvalid ? s[r] * a.sl2 : -INFINITY;
    s[r] = v;
    tmax = fmaxf(tmax, v);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(m_run, tmax);
  const float alpha = exp2_hw(m_run - m_new);
  m_run = m_new;
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = exp2_hw(s[r] - m_new);
    psum += s[r];
  }
  l_run = l_run * alpha + psum;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int d = 0; d < HD / 32; ++d) acc[d] *= alpha;
  }
  // P^T fragments of the two 16-key steps: registers 8 s2 .. 8 s2 + 7
  bf16x8 pb[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    pb[s2] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(s[8 * s2 + 0], s[8 * s2 + 1]),
                                                   pack_bf16x2(s[8 * s2 + 2], s[8 * s2 + 3]),
                                                   pack_bf16x2(s[8 * s2 + 4], s[8 * s2 + 5]),
                                                   pack_bf16x2(s[8 * s2 + 6], s[8 * s2 + 7])));
#pragma unroll
  for (int d = 0; d < HD / 32; ++d)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const u32x4 vf = *reinterpret_cast<const u32x4*>(&Vt[(d * 32 + lr) * LV + s2 * 16 + h * 8]);
      acc[d] = mfma32x32x16(__builtin_bit_cast(bf16x8, vf), pb[s2], acc[d]);
    }
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) BD_ATTN_OCC(NW) void attn_partial(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int LS = HD + 8;
  constexpr int LV = TK + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TK * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HD * LV];
  extern __shared__ int s_pref[];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const Sched sc = build_sched(a, s_pref);
  const int wg = blockIdx.x;
  int x = wg * sc.tpw;
  const int x_end = min(x + sc.tpw, sc.total);
  const int row = w * 32 + lr;  // this lane's query row

  while (x < x_end) {
    // the segment of this workgroup inside one item
    const int b = find_req(a, s_pref, x);
    const int nt = s_pref[b + 1] - s_pref[b];
    const int g = (x - a.n_kv * s_pref[b]) / nt;
    const int item_s = a.n_kv * s_pref[b] + g * nt;
    const int t0 = x - item_s;                      // first tile of the item we take
    const int t1 = min(nt, x_end - item_s);         // one past the last
    const int item = b * a.n_kv + g;
    const int nct = nt - a.nbt;                     // context tiles of the item
    int64_t cbase = 0;
    int lo = 0, hi = 0;
    const bool ok = visible(a, b, cbase, lo, hi);
    const int nctx = ok ? hi - lo : 0;

    // query fragments: B operand of S^T, lane holds Q[row][16 ks + 8 h .. +8]
    bf16x8 qf[HD / 16];
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < a.R) {
        const int i = row / a.group, hh = row - i * a.group;
        v = *reinterpret_cast<const uint4*>(a.q + ((size_t(b) * a.K + i) * a.n_q + g * a.group + hh) * HD + ks * 16 + h * 8);
      }
      qf[ks] = as_bf16x8(v);
    }
    floatx16 acc[HD / 32];
#pragma unroll
    for (int d = 0; d < HD / 32; ++d) acc[d] = floatx16{};
    float m_run = -INFINITY, l_run = 0.f;

    TileRegs<HD, NT> regs;
    int nvalid_next = fetch_tile<HD, NT>(a, t0, nct, nt, b, g, cbase, lo, nctx, t, regs);
    for (int ti = t0; ti < t1; ++ti) {
      const int nvalid = nvalid_next;
      __syncthreads();
      stage_tile<HD, NT>(regs, nvalid, t, Ks, Vt);
      __syncthreads();
      // look-ahead for the next tile (past the segment end: a dummy fetch of
      // one line), in flight during this tile's MFMAs
      nvalid_next = fetch_tile<HD, NT>(a, ti + 1 < t1 ? ti + 1 : nt, nct, nt, b, g, cbase, lo, nctx, t, regs);
      tile_math<HD>(a, Ks, Vt, nvalid, lane, qf, acc, m_run, l_run);
    }

    // partial result of (item, workgroup): slot item + wg is unique because a
    // later item only starts in a workgroup at or after this one's last
    const size_t slot = size_t(item) + wg;
    const float l = l_run + __shfl_xor(l_run, 32);
    if (row < a.R) {
      float* o = a.wo + (slot * a.R + row) * HD;
#pragma unroll
      for (int d = 0; d < HD / 32; ++d)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<float4*>(o + d * 32 + 8 * r4 + 4 * h) =
              make_float4(acc[d][4 * r4], acc[d][4 * r4 + 1], acc[d][4 * r4 + 2], acc[d][4 * r4 + 3]);
      if (h == 0) {
        a.wml[(slot * a.R + row) * 2] = m_run;
        a.wml[(slot * a.R + row) * 2 + 1] = l;
      }
    }
    x = item_s + t1;
  }
}

constexpr int MRS = 16;  // query rows per merge workgroup

template <int HD>
__global__ __launch_bounds__(MT) void attn_merge(AttnArgs a) {
  extern __shared__ int s_pref[];
  __shared__ float s_f[MAXSEG * MRS];  // per record and row: 2^(m - M) / L
  const int item = blockIdx.x, r0 = blockIdx.y * MRS, t = threadIdx.x;
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
  const int nr = min(MRS, a.R - r0);
  if (nr <= 0) return;
  if (t < nr) {
    const int row = r0 + t;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.wml[((slot0 + s) * a.R + row) * 2]);
    float L = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = a.wml[((slot0 + s) * a.R + row) * 2];
      L += a.wml[((slot0 + s) * a.R + row) * 2 + 1] * exp2f(ms - M);
    }
    const float inv = 1.f / L;
    if (ok)
      for (int s = 0; s < ns; ++s) s_f[s * MRS + t] = exp2f(a.wml[((slot0 + s) * a.R + row) * 2] - M) * inv;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = (size_t(b) * a.K + i) * a.n_q + g * a.group + hh;
    if (a.lse) a.lse[oidx] = ok ? (M + log2f(L)) * 0.6931471805599453f : NAN;
  }
  __syncthreads();
  // outputs four dims at a time; the records of one float4 load independently
  for (int e4 = t; e4 < nr * HD / 4; e4 += MT) {
    const int rr = e4 / (HD / 4), d4 = (e4 - rr * (HD / 4)) * 4;
    const int row = r0 + rr;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = (size_t(b) * a.K + i) * a.n_q + g * a.group + hh;
    uint2 packed;
    if (!ok) {
      packed = make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    } else {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < ns; ++s) {
        const float f = s_f[s * MRS + rr];
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
// ceil(vis/32) + 2 tiles) spans no more than MAXSEG workgroups.
static int attn_tmin(int max_ctx, int window) {
  const int vis = (window > 0 && max_ctx > window) ? window : max_ctx;
  const int nt_max = (vis + TK - 1) / TK + 2;
  const int t = (nt_max + MAXSEG - 3) / (MAXSEG - 2);
  return t > TMIN ? t : TMIN;
}

// upper bound of the grid (sizes the workspace)
static int attn_grid(int B, int n_kv, int max_ctx, int window) {
  const int vis = (window > 0 && max_ctx > window) ? window : max_ctx;
  const long long tiles = (long long)B * n_kv * ((vis + TK - 1) / TK + 2);  // upper bound
  const int tmin = attn_tmin(max_ctx, window);
  long long g = (tiles + tmin - 1) / tmin;
  if (g > PARTIAL_GRID) g = PARTIAL_GRID;
  if (g < 1) g = 1;
  return int(g);
}

// Workgroups of attn_partial<HD, NW> that fit on the device at once (queried
// once per variant; falls back to two per CU on 256 CUs).
template <int HD, int NW>
static int resident_partial() {
  static const int n = [] {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, attn_partial<HD, NW>, 64 * NW, 4096) != hipSuccess ||
        per < 1)
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

// one partial-kernel variant: NW = ceil(R / 32) waves of 32 query rows
template <int HD, int NW>
static void run_partial(AttnArgs& a, size_t pref_bytes, hipStream_t stream) {
  const int resident = resident_partial<HD, NW>();
  if (a.grid > resident) a.grid = resident;
  hipLaunchKernelGGL((attn_partial<HD, NW>), dim3(a.grid), dim3(64 * NW), pref_bytes, stream, a);
}

template <int HD>
static void run_attn(AttnArgs& a, size_t pref_bytes, hipStream_t stream) {
  switch ((a.R + 31) / 32) {
    case 1: run_partial<HD, 1>(a, pref_bytes, stream); break;
    case 2: run_partial<HD, 2>(a, pref_bytes, stream); break;
    case 3: run_partial<HD, 3>(a, pref_bytes, stream); break;
    default: run_partial<HD, 4>(a, pref_bytes, stream); break;
  }
  hipLaunchKernelGGL(attn_merge<HD>, dim3(a.B * a.n_kv, (a.R + MRS - 1) / MRS), dim3(MT), pref_bytes, stream, a);
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
  a.nbt = (K + TK - 1) / TK;
  a.tmin = attn_tmin(max_ctx, window);
  // the workspace holds items + attn_grid() partial slots; the launch may use fewer
  a.grid = attn_grid(B, n_kv, max_ctx, window);
  const float sc = scale > 0.f ? scale : float(1.0 / sqrt(double(hd)));
  a.sl2 = float(double(sc) * 1.4426950408889634);
  a.out = out; a.lse = lse;
  const size_t R = size_t(a.R);
  const size_t slots = size_t(B) * n_kv + a.grid;
  a.wo = static_cast<float*>(ws);
  a.wml = reinterpret_cast<float*>(static_cast<char*>(ws) + al(slots * R * hd * 4));
  const size_t pref_bytes = size_t(B + 1) * sizeof(int);
  if (hd == 128) run_attn<128>(a, pref_bytes, stream);
  else run_attn<64>(a, pref_bytes, stream);
  return hipGetLastError();
}

}  // namespace bd
