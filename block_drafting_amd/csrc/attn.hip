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
// allow); its grid is at most the number of workgroups resident at once (CUs x
// workgroups per CU from the occupancy query) and at most BD_ATTN_GRID: three
// workgroups per CU of 256 (measured at the 8B round: 68.0 us per call against
// 71.8 us with all four that fit, 76 us with two).
#ifndef BD_ATTN_GRID
#define BD_ATTN_GRID 768
#endif
#ifndef BD_ATTN_WPE
#define BD_ATTN_WPE 2
#endif
// stages of the partial kernel's LDS tile ring (S - 1 tiles in flight)
#ifndef BD_ATTN_STAGES
#define BD_ATTN_STAGES 2
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
  int Rp;                         // R rounded up to whole 32-row wave blocks
  int window, max_ctx;
  int flags;                      // 1: causal in-block keys, 2: per-query window
  int nbt;                        // tiles of block keys per item, ceil(K / 32)
  int grid;                       // workgroups of the partial kernel
  int tmin;                       // fewest tiles a workgroup takes
  float sl2;                      // scale * log2(e)
  uint16_t* out;
  float* lse;
  uint16_t* wo;  // [items + grid][Rp / 32][HD / 32][2][64 lanes][8] partial O / l (bf16)
  float* wml;  // [items + grid][Rp][2]  running max (exp2 domain), normaliser
  int2* ihdr;  // [items] first record slot and record count of each item
};

// visible context of request b, or ok = false when its metadata is invalid
// (cache_base and ctx_len are read through the constant address space: they do
// not change during a call, so uniform reads become scalar loads)
typedef const __attribute__((address_space(4))) int64_t c_int64;
typedef const __attribute__((address_space(4))) int32_t c_int32;
__device__ __forceinline__ bool visible(const AttnArgs& a, int b, int64_t& base, int& lo, int& hi) {
  base = ((c_int64*)a.cache_base)[b];
  int ctx = ((c_int32*)a.ctx_len)[b];
  if (ctx < 0 || ctx > a.max_ctx || base < 0 || base + ctx > a.T_cap) return false;
  // the keys of block position 0 under a per-query window, else of every
  // position: the union over the block either way
  const int w_lo = (a.flags & 2) ? ctx + 1 - a.window : ctx - a.window;
  lo = (a.window > 0 && w_lo > 0) ? w_lo : 0;
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

constexpr int TMIN = 2;     // fewest tiles a workgroup takes (small problems: more, shorter runs)
constexpr int MAXSEG = 64;  // partial records one merge may combine
constexpr int MGRP = 8;     // records whose loads the merge keeps in flight together

// Shared schedule: every workgroup (and the merge) derives the same tile
// prefix over requests from ctx_len: item i = b * n_kv + g owns global tiles
// [s_i, s_i + nt_b) with s_i = n_kv * P_b + g * nt_b, P_b = sum_{b' < b} nt_b'.
// Workgroup w < ge takes global tiles [floor(w T / ge), floor((w + 1) T / ge))
// (T tiles in all): every workgroup of the grid gets floor or ceil of T / ge.
// Measured: weighting the shares (e.g. more work for the workgroups placed
// first on a CU, whose older waves win the issue arbitration) does not help,
// since a CU's workgroups share its bandwidth.
//
// Head-synchronous form (BD_ATTN_HEADSYNC): every KV head's items form their
// own sequence of T1 = sum_b nt_b tiles (requests in order), cut the same way
// for all heads: workgroup w serves head w mod n_kv in group w / n_kv, and
// group j takes tiles [floor(j T1 / ge1), floor((j + 1) T1 / ge1)) of its
// head's sequence (ge1 groups).  The n_kv workgroups of a group read the same
// cache rows' heads at about the same time.  Records: head g, request b, group
// j at slot g (B + ge1) + b + j.
#ifndef BD_ATTN_HEADSYNC
#define BD_ATTN_HEADSYNC 1
#endif
struct Sched {
  int total;  // all tiles (head-synchronous: tiles of one head's sequence)
  int ge;     // workgroups with work
  int ge1;    // head-synchronous: groups of n_kv workgroups
};

// first tile of workgroup w (head-synchronous: of group w, in its head's sequence)
__device__ __forceinline__ int sched_start(const Sched& s, int w) {
  return int((long long)s.total * w / (BD_ATTN_HEADSYNC ? s.ge1 : s.ge));
}

// workgroup (head-synchronous: group) holding tile x: the last w with start(w) <= x
__device__ __forceinline__ int sched_owner(const Sched& s, int x) {
  return int((((long long)x + 1) * (BD_ATTN_HEADSYNC ? s.ge1 : s.ge) - 1) / s.total);
}

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
  // values read from LDS are the same in every lane: keep them in scalar registers
#if BD_ATTN_HEADSYNC
  s.total = __builtin_amdgcn_readfirstlane(s_pref[a.B]);
  // every share at least tmin tiles (fewer groups for small problems); the
  // host makes the grid at least n_kv
  const int gmax = a.grid / a.n_kv;
  s.ge1 = (long long)s.total >= (long long)gmax * a.tmin ? gmax : (s.total / a.tmin > 1 ? s.total / a.tmin : 1);
  s.ge = s.ge1 * a.n_kv;
#else
  s.total = __builtin_amdgcn_readfirstlane(a.n_kv * s_pref[a.B]);
  // every share at least tmin tiles (fewer workgroups for small problems)
  s.ge = (long long)s.total >= (long long)a.grid * a.tmin ? a.grid : (s.total / a.tmin > 1 ? s.total / a.tmin : 1);
  s.ge1 = 0;
#endif
  return s;
}

// request holding global tile x (head-synchronous: tile x of a head's
// sequence), by a binary search over the prefix
__device__ __forceinline__ int find_req(const AttnArgs& a, const int* s_pref, int x) {
  const int f = BD_ATTN_HEADSYNC ? 1 : a.n_kv;
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (f * s_pref[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- tile ring
// A stage of the LDS ring holds one 32-key tile: K, then V, each [32 keys][HD]
// bf16 as 16-byte pieces, 16 pieces to a 256-byte line (HD = 128: one key per
// line, HD = 64: two).  Tiles arrive straight from HBM (global_load_lds, 16
// bytes per lane, a wave filling 1 KB of consecutive pieces), so the pieces of
// a line are XOR-permuted by swz(line) instead of padded.  swz makes both MFMA
// operand reads conflict-free: the K reads (16 lanes, 16 keys, one piece each)
// need a bijection over 16 consecutive keys, the V transpose reads (32 lanes,
// 4 aligned keys x 4 consecutive pieces) need those 4 keys to differ in piece
// bits 2..3 (HD = 128), or two consecutive lines in bit 2 (HD = 64).
template <int HD>
__device__ __forceinline__ int swz(int line) {
  if constexpr (HD == 128) return ((line & 3) << 2) | ((line >> 2) & 3);
  else return ((line & 1) << 2) | ((line >> 1) & 3);
}

// byte offset, inside a K or V tile, of dims [8c, 8c + 8) of key `key`
template <int HD>
__device__ __forceinline__ int piece_off(int key, int c) {
  constexpr int P = HD / 8;
  const int flat = key * P + c, line = flat >> 4;
  return (line * 16 + ((flat & 15) ^ swz<HD>(line))) * 16;
}

// Tiles are consumed in order and loads complete in order, so tile x is in LDS
// once no more than the loads of the `ahead` tiles issued after it remain.
template <int L, int A>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if constexpr (A == 0) {
    vm_wait<0>();
  } else {
    if (ahead >= A) vm_wait<A * L>();
    else wait_tiles<L, A - 1>(ahead);
  }
}

// Position of a workgroup in its run of tiles: request b, KV head g, tile ti
// of that item (context tiles first, then block tiles).
struct Cur {
  int b, g, ti, nt, nct, lo, nctx;
  int64_t cbase;
};

__device__ __forceinline__ void cur_item(const AttnArgs& a, const int* s_pref, Cur& c) {
  c.b = __builtin_amdgcn_readfirstlane(c.b);
  c.nt = __builtin_amdgcn_readfirstlane(s_pref[c.b + 1] - s_pref[c.b]);
  c.nct = c.nt - a.nbt;
  int64_t base = 0;
  int lo = 0, hi = 0;
  const bool ok = visible(a, c.b, base, lo, hi);
  c.cbase = ok ? base : 0;
  c.lo = ok ? lo : 0;
  c.nctx = ok ? hi - lo : 0;
}

// cursor at tile x (head-synchronous: tile x of head g's sequence)
__device__ __forceinline__ void cur_init(const AttnArgs& a, const int* s_pref, Cur& c, int x, int g) {
  c.b = __builtin_amdgcn_readfirstlane(find_req(a, s_pref, x));
#if BD_ATTN_HEADSYNC
  c.g = g;
  c.ti = x - __builtin_amdgcn_readfirstlane(s_pref[c.b]);
#else
  (void)g;
  const int nt = __builtin_amdgcn_readfirstlane(s_pref[c.b + 1] - s_pref[c.b]);
  const int r = x - a.n_kv * __builtin_amdgcn_readfirstlane(s_pref[c.b]);
  c.g = r / nt;
  c.ti = r - c.g * nt;
#endif
  cur_item(a, s_pref, c);
}

__device__ __forceinline__ void cur_next(const AttnArgs& a, const int* s_pref, Cur& c) {
  if (++c.ti < c.nt) return;
  c.ti = 0;
  if (BD_ATTN_HEADSYNC || ++c.g == a.n_kv) {
    if (!BD_ATTN_HEADSYNC) c.g = 0;
    if (++c.b >= a.B) return;  // past the last tile: never read
  }
  cur_item(a, s_pref, c);
}

// record slot of the cursor's item in workgroup wg
__device__ __forceinline__ size_t rec_slot(const AttnArgs& a, const Sched& sc, int b, int g, int wg) {
#if BD_ATTN_HEADSYNC
  return size_t(g) * (a.B + sc.ge1) + b + wg / a.n_kv;
#else
  (void)sc;
  return size_t(b) * a.n_kv + g + wg;
#endif
}

// first record slot and record count of item (b, g)
__device__ __forceinline__ void item_records(const AttnArgs& a, const Sched& sc, const int* s_pref, int b, int g,
                                             size_t& slot0, int& nrec) {
  const int nt = s_pref[b + 1] - s_pref[b];
#if BD_ATTN_HEADSYNC
  const int s0 = s_pref[b];
  const int w0 = sched_owner(sc, s0), w1 = sched_owner(sc, s0 + nt - 1);
  slot0 = size_t(g) * (a.B + sc.ge1) + b + w0;
#else
  const int s0 = a.n_kv * s_pref[b] + g * nt;
  const int w0 = sched_owner(sc, s0), w1 = sched_owner(sc, s0 + nt - 1);
  slot0 = size_t(b) * a.n_kv + g + w0;
#endif
  nrec = w1 - w0 + 1;
}

// first K and V rows of the cursor's tile; returns its number of keys (>= 1)
template <int HD>
__device__ __forceinline__ int tile_src(const AttnArgs& a, const Cur& c, const uint16_t*& kp, const uint16_t*& vp) {
  if (c.ti >= c.nct) {
    const int k0 = (c.ti - c.nct) * TK;
    const size_t o = ((size_t(c.b) * a.K + k0) * a.n_kv + c.g) * HD;
    kp = a.kb + o;
    vp = a.vb + o;
    return min(TK, a.K - k0);
  }
  const int k0 = c.ti * TK;
  const size_t o = (size_t(c.cbase + c.lo + k0) * a.n_kv + c.g) * HD;
  kp = a.kc + o;
  vp = a.vc + o;
  return min(TK, c.nctx - k0);
}

// Loads of one tile into a ring stage: 2 * NH one-KB wave loads spread over
// the waves (wave w issues loads w, w + NW, ...; its t-th is load w + t NW).
// Lane l of load j fills piece slot 64 (j % NH) + l of the K (j < NH) or V
// half.  lane_piece() gives that slot's key and 16-byte column; for a full
// tile the byte offsets from the tile's first row are fixed per lane and
// computed once (voff); a short tile re-reads its last key in place of the
// missing ones (their scores are masked).
template <int HD>
__device__ __forceinline__ void lane_piece(int jj, int lane, int& key, int& cc) {
  constexpr int P = HD / 8;
  const int ps = jj * 64 + lane, line = ps >> 4;
  const int flat = line * 16 + ((ps & 15) ^ swz<HD>(line));
  key = flat / P;
  cc = flat % P;
}

template <int HD, int NW>
struct IssuePlan {
  static constexpr int TB = TK * HD * 2, NH = TB / 1024;
  static constexpr int LMAX = (2 * NH + NW - 1) / NW;
  uint32_t voff[LMAX];  // byte offsets of a full tile
};

template <int HD, int NW>
__device__ __forceinline__ void plan_init(IssuePlan<HD, NW>& pl, int kstride_bytes, int w, int lane) {
  using PL = IssuePlan<HD, NW>;
#pragma unroll
  for (int t = 0; t < PL::LMAX; ++t) {
    const int j = w + t * NW;
    const int jj = j >= PL::NH ? j - PL::NH : j;
    int key, cc;
    lane_piece<HD>(jj, lane, key, cc);
    pl.voff[t] = uint32_t(key * kstride_bytes + cc * 16);
  }
}

template <int HD, int NW>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Cur& c, const IssuePlan<HD, NW>& pl,
                                           uint32_t stage, int w, int lane) {
  using PL = IssuePlan<HD, NW>;
  const uint16_t* kp;
  const uint16_t* vp;
  const int nkeys = tile_src<HD>(a, c, kp, vp);
  const int kstride_bytes = a.n_kv * HD * 2;
#pragma unroll
  for (int t = 0; t < PL::LMAX; ++t) {
    const int j = w + t * NW;
    if (j < 2 * PL::NH) {
      const bool isv = j >= PL::NH;
      const int jj = isv ? j - PL::NH : j;
      uint32_t off = pl.voff[t];
      if (nkeys < TK) {
        int key, cc;
        lane_piece<HD>(jj, lane, key, cc);
        off = uint32_t(min(key, nkeys - 1) * kstride_bytes + cc * 16);
      }
      dma16(isv ? vp : kp, off, stage + (isv ? PL::TB : 0) + jj * 1024);
    }
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two probabilities to packed bf16 (round to nearest even)
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Query fragments of item (b, g) for this lane's row (rows past R re-read row
// R - 1; their results are never used): the B operand of S^T, lane holds
// Q[row][16 ks + 8 h .. + 8].
template <int HD>
__device__ __forceinline__ void load_q(const AttnArgs& a, int b, int g, int row, int h, bf16x8 (&qf)[HD / 16]) {
  const int r = min(row, a.R - 1);
  const int i = r / a.group, hh = r - i * a.group;
  const uint16_t* p = a.q + ((size_t(b) * a.K + i) * a.n_q + g * a.group + hh) * HD + h * 8;
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(p + ks * 16));
}

// One key tile (K at byte kt, V at byte vt of LDS) against the wave's 32 query
// rows: scores, online softmax in the exp2 domain, and the P.V accumulation.
// All K fragment reads are issued before the score MFMAs and all V^T fragment
// reads before the softmax, so the LDS latency is paid about once per phase
// rather than once per MFMA.
template <int HD>
__device__ __forceinline__ void tile_math(const AttnArgs& a, const uint8_t* lds, uint32_t kt, uint32_t vt,
                                          bool mask, int klo, int khi, int lane, const bf16x8 (&qf)[HD / 16],
                                          floatx16 (&acc)[HD / 32], float& m_run, float& l_run) {
  const int lr = lane & 31, h = lane >> 5;
  u32x4 kf[HD / 16];
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks)
    kf[ks] = *reinterpret_cast<const u32x4*>(lds + kt + piece_off<HD>(lr, 2 * ks + h));
  floatx16 s = {};
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) s = mfma32x32x16(__builtin_bit_cast(bf16x8, kf[ks]), qf[ks], s);
  // V^T fragments by transpose reads: in each group of 16 lanes, lane 4e + q
  // points at key k0 + e, dims 4q .. 4q + 3 of the group's 16 dims, and lane i
  // receives dim i of keys k0 .. k0 + 3.  Two reads give the lane's 8 keys
  // (4h .. 4h + 3 and 8 + 4h .. 8 + 4h + 3 of the 16-key step).
  const int gi = lane & 15, e = gi >> 2, q = gi & 3, gh = (lane >> 4) & 1;
  bf16x8 vf[HD / 32][2];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d) {
    const int c = 4 * d + 2 * gh + (q >> 1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int k0 = 16 * s2 + 4 * h + e;
      const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(lds + vt + piece_off<HD>(k0, c) + 8 * (q & 1)));
      const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(lds + vt + piece_off<HD>(k0 + 8, c) + 8 * (q & 1)));
      vf[d][s2] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  // lane holds keys 8 (r / 4) + 4 h + r % 4 of row lr; keys outside the
  // lane's [klo, khi) get -inf (short tiles, and the causal / per-query
  // window bounds): key - klo < khi - klo as unsigned
  float tmax = -INFINITY;
  if (mask) {
    const int kb = 4 * h - klo;
    const unsigned span = khi > klo ? unsigned(khi - klo) : 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = unsigned(kb + 8 * (r >> 2) + (r & 3)) < span ? s[r] : -INFINITY;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  // running maximum in the exp2 domain (scores times scale * log2(e) > 0); a
  // row that has seen no key yet keeps m = -inf, l = 0
  const float m_new = fmaxf(m_run, tmax * a.sl2);
  const bool none = m_new == -INFINITY;
  const float alpha = none ? 1.f : exp2_hw(m_run - m_new);
  const float mu = none ? 0.f : m_new;
  m_run = m_new;
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = exp2_hw(fmaf(s[r], a.sl2, -mu));
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
    pb[s2] = __builtin_bit_cast(bf16x8, make_uint4(pk_bf16(s[8 * s2 + 0], s[8 * s2 + 1]),
                                                   pk_bf16(s[8 * s2 + 2], s[8 * s2 + 3]),
                                                   pk_bf16(s[8 * s2 + 4], s[8 * s2 + 5]),
                                                   pk_bf16(s[8 * s2 + 6], s[8 * s2 + 7])));
#pragma unroll
  for (int d = 0; d < HD / 32; ++d)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) acc[d] = mfma32x32x16(vf[d][s2], pb[s2], acc[d]);
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) BD_ATTN_OCC(NW) void attn_partial(AttnArgs a) {
  constexpr int S = BD_ATTN_STAGES;
  constexpr int TB = TK * HD * 2;
  constexpr int NI = 2 * TB / 1024;          // one-KB loads per tile
  constexpr int LMAX = (NI + NW - 1) / NW;   // loads per tile of wave 0
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * 2 * TB];
  extern __shared__ int s_pref[];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 31, h = lane >> 5;
  const Sched sc = build_sched(a, s_pref);
  const int wg = blockIdx.x;
  if (wg >= sc.ge) return;
  const int sw = BD_ATTN_HEADSYNC ? wg / a.n_kv : wg;  // share index (head-synchronous: group)
  const int x0 = sched_start(sc, sw);
  const int x_end = sched_start(sc, sw + 1);
  if (x0 >= x_end) return;
  const bool full_wave = (NI % NW == 0) || w < NI % NW;  // issues LMAX loads per tile
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring)));
  const int row = w * 32 + lr;  // this lane's query row

  IssuePlan<HD, NW> plan;
  plan_init<HD, NW>(plan, a.n_kv * HD * 2, w, lane);
  Cur ic, cc;
  cur_init(a, s_pref, ic, x0, wg % a.n_kv);
  cc = ic;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    if (x0 + s < x_end) {
      issue_tile<HD, NW>(a, ic, plan, ring0 + s * 2 * TB, w, lane);
      cur_next(a, s_pref, ic);
    }
  }

  bf16x8 qf[HD / 16];
  floatx16 acc[HD / 32];
  float m_run = -INFINITY, l_run = 0.f;
  bool first_seg = false;  // the current segment starts at the item's first tile
  int stage = 0;
  int ready = x0 - 1;  // tiles up to here are known to be in LDS
  for (int x = x0; x < x_end; ++x) {
    if (x > ready) {
      const int ahead = min(S - 2, x_end - 1 - x);
      if (full_wave) wait_tiles<LMAX, S - 2>(ahead);
      else wait_tiles<(LMAX > 1 ? LMAX - 1 : 1), S - 2>(ahead);
    }
    __syncthreads();
    if (x == x0) {
      load_q<HD>(a, cc.b, cc.g, row, h, qf);
      vm_wait<0>();
      ready = x + S - 2;
    }
    if (x == x0 || cc.ti == 0) {
#pragma unroll
      for (int d = 0; d < HD / 32; ++d) acc[d] = floatx16{};
      m_run = -INFINITY;
      l_run = 0.f;
      first_seg = cc.ti == 0;
    }
    // refill the stage that every wave finished with before the barrier
    if (x + S - 1 < x_end) {
      const int st = stage == 0 ? S - 1 : stage - 1;
      issue_tile<HD, NW>(a, ic, plan, ring0 + st * 2 * TB, w, lane);
      cur_next(a, s_pref, ic);
    }
    const uint16_t* kp;
    const uint16_t* vp;
    const int nvalid = tile_src<HD>(a, cc, kp, vp);
    // valid keys of this lane's row in the tile: [klo, khi)
    int klo = 0, khi = nvalid;
    if (a.flags) {
      const int i = min(row, a.R - 1) / a.group;  // block position of the row
      if (cc.ti >= cc.nct) {
        const int j0 = (cc.ti - cc.nct) * TK;      // first block key of the tile
        if (a.flags & 1) khi = min(khi, i - j0 + 1);
        if ((a.flags & 2) && a.window > 0) klo = max(klo, i - a.window + 1 - j0);
      } else if ((a.flags & 2) && a.window > 0) {
        // context position p = lo + key: query i needs p >= ctx + i + 1 - W
        const int ctx = cc.lo + cc.nctx;
        klo = max(klo, max(0, ctx + i + 1 - a.window) - cc.lo - cc.ti * TK);
      }
    }
    tile_math<HD>(a, ring, stage * 2 * TB, stage * 2 * TB + TB, nvalid < TK || a.flags != 0, klo, khi, lane, qf,
                  acc, m_run, l_run);

    if (x == x_end - 1 || cc.ti == cc.nt - 1) {
      if (x < x_end - 1) {
        // the next item's query rows, waited for before this segment's stores
        // are issued: a store is never waited for inside the loop (stores may
        // complete out of order with loads; the tile waits above rely only on
        // loads completing in order)
        Cur nx = cc;
        cur_next(a, s_pref, nx);
        load_q<HD>(a, nx.b, nx.g, row, h, qf);
        vm_wait<0>();
        ready = x + S - 1;
      }
      // partial result of (item, workgroup): slot item + wg is unique because a
      // later item only starts in a workgroup at or after this one's last.
      // O / l is stored in bf16 (the normaliser l and the running max stay
      // fp32) in accumulator order, so each store is one contiguous KB: the
      // 16 bytes (d, rp, lane) hold dims 32 d + 16 rp + 4 h .. + 3 and
      // 32 d + 16 rp + 8 + 4 h .. + 3 of row lr
      const size_t slot = rec_slot(a, sc, cc.b, cc.g, wg);
      const float l = l_run + __shfl_xor(l_run, 32);
      const float il = l > 0.f ? 1.f / l : 0.f;  // l = 0: no key of this segment was visible
      uint16_t* o = a.wo + (slot * (a.Rp / 32) + w) * (32 * HD);
#pragma unroll
      for (int d = 0; d < HD / 32; ++d)
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
          const floatx16& c = acc[d];
          const int r0 = 8 * rp;
          *reinterpret_cast<uint4*>(o + ((d * 2 + rp) * 64 + lane) * 8) =
              make_uint4(pk_bf16(c[r0] * il, c[r0 + 1] * il), pk_bf16(c[r0 + 2] * il, c[r0 + 3] * il),
                         pk_bf16(c[r0 + 4] * il, c[r0 + 5] * il), pk_bf16(c[r0 + 6] * il, c[r0 + 7] * il));
        }
      if (h == 0) *reinterpret_cast<float2*>(a.wml + (slot * a.Rp + row) * 2) = make_float2(m_run, l);
      if (first_seg && t == 0) {
        // the item's first record is this one: its slot and record count for the merge
        size_t s0;
        int nrec;
        item_records(a, sc, s_pref, cc.b, cc.g, s0, nrec);
        a.ihdr[size_t(cc.b) * a.n_kv + cc.g] = make_int2(int(s0), nrec);
      }
    }
    cur_next(a, s_pref, cc);
    stage = stage == S - 1 ? 0 : stage + 1;
  }
}

// One workgroup per (item, 32-row wave block): the records' (max, normaliser)
// pairs are read in parallel into LDS, each row's weights 2^(m_s - M) / L
// follow (the rows' records shared out over the threads), then the weighted
// sum of the records in their stored (accumulator) order, with the loads of
// eight records in flight together (a small batch spreads an item over many
// workgroups: 32 records at batch 1), transposed through LDS so the bf16 rows
// leave whole.
template <int HD>
__global__ __launch_bounds__(MT) void attn_merge(AttnArgs a) {
  constexpr int TPR = MT / 32;       // threads per row in the weight pass
  constexpr int NP = 32 * HD / 8;    // 16-byte pieces of a record's row block
  constexpr int PPT = NP / MT;
  extern __shared__ int s_pref[];
  __shared__ float2 s_ml[MAXSEG * 32];                                  // [record][row]
  __shared__ float s_f[MAXSEG * 32];                                    // [record][row]
  __shared__ __attribute__((aligned(16))) uint16_t s_o[32 * (HD + 8)];  // bf16 rows
  const int item = blockIdx.x, wb = blockIdx.y, t = threadIdx.x;
  const int b = item / a.n_kv, g = item - b * a.n_kv;
  const int2 ih = a.ihdr[item];  // written by the partial kernel
  const size_t slot0 = size_t(ih.x);
  const int nrec = ih.y;
  const int ns = min(nrec, MAXSEG);
  int64_t cbase;
  int lo, hi;
  const bool ok = visible(a, b, cbase, lo, hi) && nrec <= MAXSEG;
  const int nr = min(32, a.R - 32 * wb);  // valid rows of this block
  // 16 bytes p of a record: (d, rp, lane) -> row lane % 32, dims
  // 32 d + 16 rp + 4 (lane / 32) .. + 3 and the same + 8
  const uint16_t* base = a.wo + (slot0 * (a.Rp / 32) + wb) * (32 * HD);
  const size_t rstride = size_t(a.Rp) * HD;  // elements between consecutive records
  // the (max, normaliser) pairs and the first MGRP records' pieces, all in flight together
  uint4 v[MGRP][PPT];
  {
    const int s = t >> 5, r = t & 31;
    const float2 ml0 = *reinterpret_cast<const float2*>(a.wml + ((slot0 + min(s, ns - 1)) * a.Rp + 32 * wb + r) * 2);
#pragma unroll
    for (int u = 0; u < MGRP; ++u) {
      const int su = min(u, ns - 1);  // a repeated record gets weight 0
#pragma unroll
      for (int k = 0; k < PPT; ++k)
        v[u][k] = *reinterpret_cast<const uint4*>(base + su * rstride + size_t(t + k * MT) * 8);
    }
    if (t < ns * 32) s_ml[t] = ml0;
  }
  for (int e = t + MT; e < ns * 32; e += MT) {
    const int s = e >> 5, r = e & 31;
    s_ml[e] = *reinterpret_cast<const float2*>(a.wml + ((slot0 + s) * a.Rp + 32 * wb + r) * 2);
  }
  __syncthreads();
  {
    // TPR threads per row (consecutive lanes), each taking every TPR-th
    // record; the partial maxima and sums are combined across them
    const int r = t / TPR, q = t % TPR;
    float M = -INFINITY;
    for (int s = q; s < ns; s += TPR) M = fmaxf(M, s_ml[s * 32 + r].x);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    for (int s = q; s < ns; s += TPR) L += s_ml[s * 32 + r].y * exp2f(s_ml[s * 32 + r].x - M);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) L += __shfl_xor(L, o);
    const float inv = 1.f / L;
    // records hold O_s / l_s: weight l_s 2^(m_s - M) / L
    for (int s = q; s < ns; s += TPR) s_f[s * 32 + r] = s_ml[s * 32 + r].y * exp2f(s_ml[s * 32 + r].x - M) * inv;
    if (q == 0 && r < nr && a.lse) {
      const int row = 32 * wb + r;
      const int i = row / a.group, hh = row - i * a.group;
      a.lse[(size_t(b) * a.K + i) * a.n_q + g * a.group + hh] = ok ? (M + log2f(L)) * 0.6931471805599453f : NAN;
    }
  }
  __syncthreads();
  float o[PPT][8];
#pragma unroll
  for (int k = 0; k < PPT; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[k][e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += MGRP) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < MGRP; ++u) {
        const int s = min(s0 + u, ns - 1);  // a repeated record gets weight 0
#pragma unroll
        for (int k = 0; k < PPT; ++k)
          v[u][k] = *reinterpret_cast<const uint4*>(base + s * rstride + size_t(t + k * MT) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < MGRP; ++u) {
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int rr = (t + k * MT) & 31;
        const float f = s0 + u < ns ? s_f[(s0 + u) * 32 + rr] : 0.f;
        const uint32_t wd[4] = {v[u][k].x, v[u][k].y, v[u][k].z, v[u][k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[k][2 * e] += bf16_to_f32(uint16_t(wd[e] & 0xffffu)) * f;
          o[k][2 * e + 1] += bf16_to_f32(uint16_t(wd[e] >> 16)) * f;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int p = t + k * MT;
    const int lane = p & 63, dr = p >> 6, d = dr >> 1, rp = dr & 1;
    const int rr = lane & 31, dim = 32 * d + 16 * rp + 4 * (lane >> 5);
    const uint2 lo4 = ok ? make_uint2(pack_bf16x2(o[k][0], o[k][1]), pack_bf16x2(o[k][2], o[k][3]))
                         : make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    const uint2 hi4 = ok ? make_uint2(pack_bf16x2(o[k][4], o[k][5]), pack_bf16x2(o[k][6], o[k][7]))
                         : make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    *reinterpret_cast<uint2*>(&s_o[rr * (HD + 8) + dim]) = lo4;
    *reinterpret_cast<uint2*>(&s_o[rr * (HD + 8) + dim + 8]) = hi4;
  }
  __syncthreads();
  // whole rows out: 16 bytes per thread
  for (int e = t; e < nr * (HD / 8); e += MT) {
    const int rr = e / (HD / 8), c8 = (e - rr * (HD / 8)) * 8;
    const int row = 32 * wb + rr;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = (size_t(b) * a.K + i) * a.n_q + g * a.group + hh;
    *reinterpret_cast<uint4*>(a.out + oidx * HD + c8) = *reinterpret_cast<const uint4*>(&s_o[rr * (HD + 8) + c8]);
  }
}

// The same merge split over the head dimension, for few (item, row block)
// pairs (a small batch, whose items each span many workgroups: 32 records at
// batch 1): one workgroup per (item, 32-row block, 32-dimension group), whose
// threads take one 16-byte piece of the group each, in RS record phases
// (phase r adds records r, r + RS, ...; the phases are added in order through
// LDS at the end).  Each workgroup then reads a quarter of the records' bytes
// (at hd 128) with as many loads in flight, so four times the CUs share them.
template <int HD>
__global__ __launch_bounds__(MT) void attn_merge_split(AttnArgs a) {
  constexpr int TPR = MT / 32;       // threads per row in the weight pass
  constexpr int NPD = 32 * 32 / 8;   // pieces of a 32-dimension group of a row block: 128
  constexpr int RS = MT / NPD;       // record phases
  static_assert(RS >= 1 && MT % NPD == 0, "merge shape");
  extern __shared__ int s_pref[];
  __shared__ float2 s_ml[MAXSEG * 32];                                  // [record][row]
  __shared__ float s_f[MAXSEG * 32];                                    // [record][row]
  __shared__ float s_red[(RS - 1) * NPD * 8 + 1];                      // later phases' sums
  __shared__ __attribute__((aligned(16))) uint16_t s_o[32 * (32 + 8)];  // bf16 row slices
  const int item = blockIdx.x, wb = blockIdx.y, dg = blockIdx.z, t = threadIdx.x;
  const int b = item / a.n_kv, g = item - b * a.n_kv;
  const int2 ih = a.ihdr[item];  // written by the partial kernel
  const size_t slot0 = size_t(ih.x);
  const int nrec = ih.y;
  const int ns = min(nrec, MAXSEG);
  int64_t cbase;
  int lo, hi;
  const bool ok = visible(a, b, cbase, lo, hi) && nrec <= MAXSEG;
  const int nr = min(32, a.R - 32 * wb);
  for (int e = t; e < ns * 32; e += MT) {
    const int s = e >> 5, r = e & 31;
    s_ml[e] = *reinterpret_cast<const float2*>(a.wml + ((slot0 + s) * a.Rp + 32 * wb + r) * 2);
  }
  __syncthreads();
  {
    const int r = t / TPR, q = t % TPR;
    float M = -INFINITY;
    for (int s = q; s < ns; s += TPR) M = fmaxf(M, s_ml[s * 32 + r].x);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    for (int s = q; s < ns; s += TPR) L += s_ml[s * 32 + r].y * exp2f(s_ml[s * 32 + r].x - M);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) L += __shfl_xor(L, o);
    const float inv = 1.f / L;
    for (int s = q; s < ns; s += TPR) s_f[s * 32 + r] = s_ml[s * 32 + r].y * exp2f(s_ml[s * 32 + r].x - M) * inv;
    if (dg == 0 && q == 0 && r < nr && a.lse) {
      const int row = 32 * wb + r;
      const int i = row / a.group, hh = row - i * a.group;
      a.lse[(size_t(b) * a.K + i) * a.n_q + g * a.group + hh] = ok ? (M + log2f(L)) * 0.6931471805599453f : NAN;
    }
  }
  __syncthreads();
  // piece pp of the group (pieces (d, rp, lane) with d = dg: 2 x 64)
  const int pp = t % NPD, ph = t / NPD;
  const int rr = pp & 31;
  const uint16_t* base = a.wo + (slot0 * (a.Rp / 32) + wb) * (32 * HD) + size_t(dg * NPD + pp) * 8;
  const size_t rstride = size_t(a.Rp) * HD;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int s0 = ph; s0 < ns; s0 += RS * MGRP) {
    uint4 v[MGRP];
#pragma unroll
    for (int u = 0; u < MGRP; ++u) v[u] = *reinterpret_cast<const uint4*>(base + min(s0 + u * RS, ns - 1) * rstride);
#pragma unroll
    for (int u = 0; u < MGRP; ++u) {
      const int s = s0 + u * RS;
      const float f = s < ns ? s_f[s * 32 + rr] : 0.f;
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] += bf16_to_f32(uint16_t(wd[e] & 0xffffu)) * f;
        o[2 * e + 1] += bf16_to_f32(uint16_t(wd[e] >> 16)) * f;
      }
    }
  }
  if (ph > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_red[((ph - 1) * NPD + pp) * 8 + e] = o[e];
  }
  __syncthreads();
  if (ph == 0) {
    for (int q = 1; q < RS; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += s_red[((q - 1) * NPD + pp) * 8 + e];
    const int lane = pp & 63, rp = pp >> 6;
    const int dim = 16 * rp + 4 * (lane >> 5);  // within the group
    const uint2 lo4 = ok ? make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]))
                         : make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    const uint2 hi4 = ok ? make_uint2(pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]))
                         : make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    *reinterpret_cast<uint2*>(&s_o[rr * 40 + dim]) = lo4;
    *reinterpret_cast<uint2*>(&s_o[rr * 40 + dim + 8]) = hi4;
  }
  __syncthreads();
  // the group's 32 dimensions of each row: 64 bytes, 16 per thread
  for (int e = t; e < nr * 4; e += MT) {
    const int r2 = e >> 2, c8 = (e & 3) * 8;
    const int row = 32 * wb + r2;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = (size_t(b) * a.K + i) * a.n_q + g * a.group + hh;
    *reinterpret_cast<uint4*>(a.out + oidx * HD + 32 * dg + c8) = *reinterpret_cast<const uint4*>(&s_o[r2 * 40 + c8]);
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
  if (g < n_kv) g = n_kv;  // head-synchronous schedule: one group at least
  if (g < 1) g = 1;
  return int(g);
}

// Compute units of the current device (queried once; 256 if the query fails).
static int device_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    return cus;
  }();
  return n;
}

// Workgroups of attn_partial<HD, NW> that fit on the device at once (queried
// once per variant; falls back to two per CU).
template <int HD, int NW>
static int resident_partial() {
  static const int n = [] {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, attn_partial<HD, NW>, 64 * NW, 4096) != hipSuccess ||
        per < 1)
      per = 2;
    return device_cus() * per;
  }();
  return n;
}

size_t attn_ws_bytes(int B, int K, int n_q, int n_kv, int hd, int max_ctx, int window) {
  if (B <= 0) return 0;
  const size_t Rp = (size_t(K) * (n_q / n_kv) + 31) / 32 * 32;
  const size_t slots = size_t(B) * n_kv + attn_grid(B, n_kv, max_ctx, window);
  return al(slots * Rp * hd * 2) + al(slots * Rp * 2 * 4) + al(size_t(B) * n_kv * 8);
}

// one partial-kernel variant: NW = ceil(R / 32) waves of 32 query rows
template <int HD, int NW>
static void run_partial(AttnArgs& a, size_t pref_bytes, hipStream_t stream) {
  const int resident = resident_partial<HD, NW>();
  // at most the resident workgroups, but never fewer than one group of n_kv
  // (the head-synchronous schedule needs a workgroup per head; nothing waits on
  // another workgroup, so workgroups beyond the resident ones simply run later)
  if (a.grid > resident) a.grid = resident > a.n_kv ? resident : a.n_kv;
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
  // few (item, row block) pairs: split each over its 32-dimension groups
  if (a.B * a.n_kv * (a.Rp / 32) < device_cus())
    hipLaunchKernelGGL(attn_merge_split<HD>, dim3(a.B * a.n_kv, a.Rp / 32, HD / 32), dim3(MT), pref_bytes, stream,
                       a);
  else
    hipLaunchKernelGGL(attn_merge<HD>, dim3(a.B * a.n_kv, a.Rp / 32), dim3(MT), pref_bytes, stream, a);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kb, const uint16_t* vb, const uint16_t* kc,
                       const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                       int64_t T_cap, int max_ctx, int B, int K, int n_q, int n_kv, int hd, int window,
                       int flags, float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  AttnArgs a{};
  a.q = q; a.kb = kb; a.vb = vb; a.kc = kc; a.vc = vc;
  a.cache_base = cache_base; a.ctx_len = ctx_len; a.T_cap = T_cap;
  a.B = B; a.K = K; a.n_q = n_q; a.n_kv = n_kv; a.group = n_q / n_kv; a.R = K * a.group;
  a.Rp = (a.R + 31) / 32 * 32;
  a.window = window; a.max_ctx = max_ctx; a.flags = flags;
  a.nbt = (K + TK - 1) / TK;
  a.tmin = attn_tmin(max_ctx, window);
  // the workspace holds items + attn_grid() partial slots; the launch may use fewer
  a.grid = attn_grid(B, n_kv, max_ctx, window);
  const float sc = scale > 0.f ? scale : float(1.0 / sqrt(double(hd)));
  a.sl2 = float(double(sc) * 1.4426950408889634);
  a.out = out; a.lse = lse;
  const size_t Rp = size_t(a.Rp);
  const size_t slots = size_t(B) * n_kv + a.grid;
  a.wo = static_cast<uint16_t*>(ws);
  a.wml = reinterpret_cast<float*>(static_cast<char*>(ws) + al(slots * Rp * hd * 2));
  a.ihdr = reinterpret_cast<int2*>(static_cast<char*>(ws) + al(slots * Rp * hd * 2) + al(slots * Rp * 2 * 4));
  const size_t pref_bytes = size_t(B + 1) * sizeof(int);
  if (hd == 128) run_attn<128>(a, pref_bytes, stream);
  else run_attn<64>(a, pref_bytes, stream);
  return hipGetLastError();
}

}  // namespace bd
