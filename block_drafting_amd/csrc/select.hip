// select_block kernels: choosing the drafted tokens of a block through a
// transition cache.
//
// DSpine article, "principle": every block position keeps its 16 best
// candidates, the scores of all pairings of adjacent positions' candidates are
// computed at once into 16 x 16 tables (the transition cache), and the tokens
// are then chosen from left to right by looking up the row of the token just
// chosen.  DSpark tutorial, "semi-autoregressive generation": the dependence on
// the previous token is an offset to the position's logits from a low-rank
// (rank 256) transition matrix.  Here the score of token b at drafted position
// t after token a is z_t(b) + E[a] . F[b] (E, F [V, r] bf16); position 0's
// predecessor is the anchor token; ties go to the better base logit.
//
// Three launches:
//   sel_chunk_top  (chunk, row): the chunk's 16 best logits (value desc, index
//                  asc).  Per wave the 16th best lane maximum bounds the
//                  wave's 16 best from below, so only elements at or above it
//                  are ranked; a wave with more than WCAP of them (ties) sends
//                  the chunk to an exact 16-round selection.
//   sel_table      (position, request): merges the chunk lists of its position
//                  and of the one before, stages the predecessors' E rows and
//                  the candidates' F rows in LDS and computes the position's
//                  16 x 16 table (one entry per thread).
//   sel_walk       (request): the tables, 32 positions at a time, in LDS; one
//                  lane walks them.
#include "bd_common.hpp"
#include "bd_launch.hpp"

#include <math.h>

namespace bd {

constexpr int ST = 256;        // threads of a workgroup
constexpr int SCH = 8192;      // logits per chunk
constexpr int SPT = SCH / ST;  // 32 per thread
constexpr int NC = 16;         // candidates per position
constexpr int WCAP = 64;       // threshold candidates a wave may keep

struct SelArgs {
  const float* z;         // [B * G][V] base logits of the drafted positions
  const int32_t* anchor;  // [B]
  const uint16_t* E;      // [V][r] predecessor representation (bf16)
  const uint16_t* F;      // [V][r] successor representation (bf16)
  int B, G, V, r, nch;
  float* ctv;             // [rows][nch][NC] chunk candidates: values
  int* cti;               //                                   indices
  float* tab;             // [rows][NC][NC] tables (position 0: row 0 only)
  int* cand;              // [rows][NC] merged candidates
  int32_t* tokens;        // [B][G]
  float* scores;          // [B][G] or NULL
  int32_t* cand_out;      // [B][G][NC] or NULL
};

// the total order: larger value first, then lower index
__device__ __forceinline__ bool sel_better(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// element of slot s (0..31) of thread t in a chunk starting at `start`
template <bool VEC>
__device__ __forceinline__ int sel_slot(int start, int s, int t) {
  return VEC ? start + 4 * ((s >> 2) * ST + t) + (s & 3) : start + s * ST + t;
}

// ------------------------------------------------------------- chunk top-16
template <bool VEC>
__global__ __launch_bounds__(ST) void sel_chunk_top(SelArgs a) {
  __shared__ float s_v[4 * WCAP];
  __shared__ int s_i[4 * WCAP];
  __shared__ int s_n[4];
  __shared__ int s_over;
  __shared__ float s_rv[4];
  __shared__ int s_ri[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = blockIdx.x, row = blockIdx.y;
  const int start = c * SCH;
  const float* zr = a.z + size_t(row) * a.V;
  float x[SPT];
  if (VEC) {
#pragma unroll
    for (int j = 0; j < SPT / 4; ++j) {
      const int e = start + 4 * (j * ST + t);
      float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (e < a.V) f = *reinterpret_cast<const float4*>(zr + e);  // V % 4 == 0: all four in the row
      x[4 * j] = f.x; x[4 * j + 1] = f.y; x[4 * j + 2] = f.z; x[4 * j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int e = start + s * ST + t;
      x[s] = e < a.V ? zr[e] : -INFINITY;
    }
  }
  // this lane's best valid element
  float bv = -INFINITY;
  int bi = INT32_MAX;
#pragma unroll
  for (int s = 0; s < SPT; ++s) {
    const int e = sel_slot<VEC>(start, s, t);
    if (e < a.V && sel_better(x[s], e, bv, bi)) { bv = x[s]; bi = e; }
  }
  // the wave's lane maxima sorted best first (bitonic network over the lanes)
  float sv = bv;
  int si = bi;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float ov = __shfl_xor(sv, j);
      const int oi = __shfl_xor(si, j);
      const bool lower = (lane & j) == 0, desc = (lane & k) == 0;
      // in a descending run the lower lane keeps the better of the pair
      const bool take = (lower == desc) ? sel_better(ov, oi, sv, si) : sel_better(sv, si, ov, oi);
      if (take) { sv = ov; si = oi; }
    }
  const float tv = __shfl(sv, NC - 1);
  const int ti = __shfl(si, NC - 1);
  // candidates: valid elements not worse than the threshold
  int cnt = 0;
#pragma unroll
  for (int s = 0; s < SPT; ++s) {
    const int e = sel_slot<VEC>(start, s, t);
    cnt += (e < a.V && !sel_better(tv, ti, x[s], e)) ? 1 : 0;
  }
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  const int total = __shfl(inc, 63);
  if (t == 0) s_over = 0;
  __syncthreads();
  if (lane == 0) s_n[w] = total;
  if (total > WCAP) {
    if (lane == 0) s_over = 1;
  } else {
    int pos = w * WCAP + inc - cnt;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int e = sel_slot<VEC>(start, s, t);
      if (e < a.V && !sel_better(tv, ti, x[s], e)) { s_v[pos] = x[s]; s_i[pos] = e; ++pos; }
    }
  }
  __syncthreads();
  float* ov = a.ctv + (size_t(row) * a.nch + c) * NC;
  int* oi = a.cti + (size_t(row) * a.nch + c) * NC;
  if (!s_over) {
    // exact ranks among the kept candidates (keys are distinct: ranks are)
    const int wt = t / WCAP, k = t % WCAP;
    if (k < s_n[wt]) {
      const float v = s_v[t];
      const int i = s_i[t];
      int rank = 0;
      for (int w2 = 0; w2 < 4; ++w2)
        for (int k2 = 0; k2 < s_n[w2]; ++k2) rank += sel_better(s_v[w2 * WCAP + k2], s_i[w2 * WCAP + k2], v, i) ? 1 : 0;
      if (rank < NC) { ov[rank] = v; oi[rank] = i; }
    }
    // fewer than NC valid elements in the chunk: the rest of the list is empty
    const int n = s_n[0] + s_n[1] + s_n[2] + s_n[3];
    if (t >= n && t < NC) { ov[t] = -INFINITY; oi[t] = INT32_MAX; }
    return;
  }
  // exact selection, one element per round (ties beyond WCAP per wave)
  unsigned taken = 0u;
  for (int r = 0; r < NC; ++r) {
    float v = -INFINITY;
    int i = INT32_MAX;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int e = sel_slot<VEC>(start, s, t);
      if (e < a.V && !(taken >> s & 1u) && sel_better(x[s], e, v, i)) { v = x[s]; i = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(v, o);
      const int i2 = __shfl_xor(i, o);
      if (sel_better(v2, i2, v, i)) { v = v2; i = i2; }
    }
    if (lane == 0) { s_rv[w] = v; s_ri[w] = i; }
    __syncthreads();
    v = s_rv[0];
    i = s_ri[0];
    for (int w2 = 1; w2 < 4; ++w2)
      if (sel_better(s_rv[w2], s_ri[w2], v, i)) { v = s_rv[w2]; i = s_ri[w2]; }
    __syncthreads();
    if (t == 0) { ov[r] = i == INT32_MAX ? -INFINITY : v; oi[r] = i; }
#pragma unroll
    for (int s = 0; s < SPT; ++s)
      if (sel_slot<VEC>(start, s, t) == i) taken |= 1u << s;
  }
}

// ------------------------------------------------------------- tables
// the NC best of a row's chunk lists (rank counting over nch * NC entries)
__device__ __forceinline__ void merge_row(const SelArgs& a, int row, float* s_mv, int* s_mi, int* out_i,
                                          float* out_v) {
  const int n = a.nch * NC;
  const float* gv = a.ctv + size_t(row) * n;
  const int* gi = a.cti + size_t(row) * n;
  for (int e = threadIdx.x; e < n; e += ST) { s_mv[e] = gv[e]; s_mi[e] = gi[e]; }
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += ST) {
    const float v = s_mv[e];
    const int i = s_mi[e];
    if (i == INT32_MAX) continue;  // empty list entry
    int rank = 0;
    for (int k = 0; k < n; ++k) rank += sel_better(s_mv[k], s_mi[k], v, i) ? 1 : 0;
    if (rank < NC) {
      out_i[rank] = i;
      if (out_v) out_v[rank] = v;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(ST) void sel_table(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sel_lds[];
  // [nch * NC] merge values and indices, then E rows [NC][r] and F rows [NC][r]
  float* s_mv = reinterpret_cast<float*>(sel_lds);
  int* s_mi = reinterpret_cast<int*>(s_mv + a.nch * NC);
  uint16_t* s_E = reinterpret_cast<uint16_t*>(s_mi + a.nch * NC);
  uint16_t* s_F = s_E + NC * a.r;
  __shared__ int s_prev[NC], s_cur[NC];
  __shared__ float s_z[NC];
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int row = b * a.G + t;
  merge_row(a, row, s_mv, s_mi, s_cur, s_z);
  int n_prev = NC;
  if (t > 0) {
    merge_row(a, row - 1, s_mv, s_mi, s_prev, nullptr);
  } else {
    n_prev = 1;
    if (tid == 0) s_prev[0] = a.anchor[b];
  }
  if (tid < NC) {
    a.cand[size_t(row) * NC + tid] = s_cur[tid];
    if (a.cand_out) a.cand_out[size_t(row) * NC + tid] = s_cur[tid];
  }
  __syncthreads();
  // rows of E for the predecessors and of F for the candidates (an anchor
  // outside the vocabulary reads as a zero row; its request is flagged by
  // sel_walk)
  const int pr = a.r / 8;  // 16-byte pieces per row
  for (int e = tid; e < 2 * NC * pr; e += ST) {
    const int which = e / (NC * pr), rr = (e / pr) % NC, p = e % pr;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (which == 0) {
      const int tok = s_prev[rr < n_prev ? rr : 0];
      if (tok >= 0 && tok < a.V) v = *reinterpret_cast<const uint4*>(a.E + size_t(tok) * a.r + p * 8);
      *reinterpret_cast<uint4*>(s_E + rr * a.r + p * 8) = v;
    } else {
      v = *reinterpret_cast<const uint4*>(a.F + size_t(s_cur[rr]) * a.r + p * 8);
      *reinterpret_cast<uint4*>(s_F + rr * a.r + p * 8) = v;
    }
  }
  __syncthreads();
  // entry (i, j) = z(c_j) + E[p_i] . F[c_j], the products added in order k
  const int i = tid / NC, j = tid % NC;
  if (i < n_prev) {
    const uint16_t* er = s_E + i * a.r;
    const uint16_t* fr = s_F + j * a.r;
    float dot = 0.f;
    for (int k = 0; k < a.r; k += 8) {
      const uint4 ev = *reinterpret_cast<const uint4*>(er + k);
      const uint4 fv = *reinterpret_cast<const uint4*>(fr + k);
      const uint32_t ew[4] = {ev.x, ev.y, ev.z, ev.w}, fw[4] = {fv.x, fv.y, fv.z, fv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dot = fmaf(bf16_to_f32(uint16_t(ew[q] & 0xffffu)), bf16_to_f32(uint16_t(fw[q] & 0xffffu)), dot);
        dot = fmaf(bf16_to_f32(uint16_t(ew[q] >> 16)), bf16_to_f32(uint16_t(fw[q] >> 16)), dot);
      }
    }
    a.tab[(size_t(row) * NC + i) * NC + j] = s_z[j] + dot;
  }
}

// ------------------------------------------------------------- walk
constexpr int WALK_GROUP = 32;  // positions whose tables are in LDS at once

__global__ __launch_bounds__(64) void sel_walk(SelArgs a) {
  __shared__ float s_t[WALK_GROUP * NC * NC];
  __shared__ int s_c[WALK_GROUP * NC];
  __shared__ int s_j;
  const int b = blockIdx.x, lane = threadIdx.x;
  const size_t r0 = size_t(b) * a.G;
  const int anc = a.anchor[b];
  const bool ok = anc >= 0 && anc < a.V;
  if (lane == 0) s_j = 0;
  for (int t0 = 0; t0 < a.G; t0 += WALK_GROUP) {
    const int ng = min(WALK_GROUP, a.G - t0);
    __syncthreads();
    for (int e = lane; e < ng * NC * NC; e += 64) {
      const int tt = t0 + e / (NC * NC), ij = e % (NC * NC);
      // position 0 has row 0 only
      s_t[e] = (tt == 0 && ij >= NC) ? 0.f : a.tab[(r0 + t0) * NC * NC + e];
    }
    for (int e = lane; e < ng * NC; e += 64) s_c[e] = a.cand[(r0 + t0) * NC + e];
    __syncthreads();
    if (lane == 0) {
      int jp = s_j;
      for (int u = 0; u < ng; ++u) {
        const int t = t0 + u;
        const float* rowp = s_t + (u * NC + (t == 0 ? 0 : jp)) * NC;
        int j = 0;
        float best = rowp[0];
        for (int k = 1; k < NC; ++k)
          if (rowp[k] > best) { best = rowp[k]; j = k; }  // first maximum
        a.tokens[r0 + t] = ok ? s_c[u * NC + j] : -1;
        if (a.scores) a.scores[r0 + t] = ok ? best : NAN;
        jp = j;
      }
      s_j = jp;
    }
  }
}

// ------------------------------------------------------------- host side
static inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

size_t select_ws_bytes(int B, int G, int V) {
  if (B <= 0 || G <= 0) return 0;
  const size_t rows = size_t(B) * G, nch = (size_t(V) + SCH - 1) / SCH;
  return al(rows * nch * NC * 4) * 2 + al(rows * NC * NC * 4) + al(rows * NC * 4);
}

hipError_t launch_select(const float* z, const int32_t* anchor, const uint16_t* E, const uint16_t* F, int B, int G,
                         int V, int r, int32_t* tokens, float* scores, int32_t* cand, void* ws, hipStream_t stream) {
  if (B == 0 || G == 0) return hipSuccess;
  SelArgs a{};
  a.z = z; a.anchor = anchor; a.E = E; a.F = F;
  a.B = B; a.G = G; a.V = V; a.r = r;
  a.nch = (V + SCH - 1) / SCH;
  const size_t rows = size_t(B) * G;
  char* w = static_cast<char*>(ws);
  a.ctv = reinterpret_cast<float*>(w);
  w += al(rows * a.nch * NC * 4);
  a.cti = reinterpret_cast<int*>(w);
  w += al(rows * a.nch * NC * 4);
  a.tab = reinterpret_cast<float*>(w);
  w += al(rows * NC * NC * 4);
  a.cand = reinterpret_cast<int*>(w);
  a.tokens = tokens; a.scores = scores; a.cand_out = cand;
  const dim3 g1(a.nch, unsigned(rows));
  if ((V & 3) == 0) hipLaunchKernelGGL(sel_chunk_top<true>, g1, dim3(ST), 0, stream, a);
  else hipLaunchKernelGGL(sel_chunk_top<false>, g1, dim3(ST), 0, stream, a);
  const size_t lds2 = size_t(a.nch) * NC * 8 + size_t(2) * NC * r * 2;
  hipLaunchKernelGGL(sel_table, dim3(G, B), dim3(ST), lds2, stream, a);
  hipLaunchKernelGGL(sel_walk, dim3(B), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bd
