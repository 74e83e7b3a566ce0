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
//                  asc).  The chunk's 16th best lane maximum bounds its 16
//                  best from below (found by a bitwise search over
//                  order-preserving keys, per wave and then over the waves'
//                  survivors), so only elements at or above it are ranked, in
//                  one wave-wide sort; more than WCAP of them in a wave, or
//                  more than 64 in all (ties), sends the chunk to an exact
//                  16-round selection.
//   sel_table      (position, request): merges the chunk lists of its position
//                  and of the one before, stages the predecessors' E rows and
//                  the candidates' F rows in LDS and computes the position's
//                  16 x 16 table on the matrix cores.
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
constexpr int WCAP = 64;
constexpr int SEL_ROW_PAD = 8;  // bf16 elements of padding per staged E / F row       // threshold candidates a wave may keep

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

// the total order: larger value first, then lower index (no short circuit:
// the compiler keeps it a select rather than a branch)
// keep the better of this lane's (v, i) and lane l ^ J's
template <int J>
__device__ __forceinline__ void keep_better(float& v, int& i) {
  const float v2 = xor_lane<J>(v);
  const int i2 = xor_lane<J>(i);
  const bool t = sel_better(v2, i2, v, i);
  v = t ? v2 : v;
  i = t ? i2 : i;
}

// element of slot s (0..SPT-1) of thread t in a chunk starting at `start`
template <bool VEC>
__device__ __forceinline__ int sel_slot(int start, int s, int t) {
  return VEC ? start + 4 * ((s >> 2) * ST + t) + (s & 3) : start + s * ST + t;
}

// one (value, index) per lane, sorted best first across the wave (bitonic
// network over the lanes)
// ------------------------------------------------------------- chunk top-16
template <bool VEC>
__global__ __launch_bounds__(ST) void sel_chunk_top(SelArgs a) {
  __shared__ float s_v[4 * WCAP];
  __shared__ int s_i[4 * WCAP];
  __shared__ int s_n[4];
  __shared__ int s_over;
  __shared__ float s_rv[4];
  __shared__ int s_ri[4];
  __shared__ uint32_t s_k[4 * NC];
  __shared__ uint32_t s_tk;
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
  // Elements past V read as -inf at their own index (>= V), so they rank
  // after every real element: no bounds checks below.  This lane's best: its
  // slots increase with the index, so the first strict maximum is the lowest
  // index among equals.
  float bv = x[0];
  int bs = 0;
#pragma unroll
  for (int s = 1; s < SPT; ++s) {
    const bool gt = x[s] > bv;
    bv = gt ? x[s] : bv;
    bs = gt ? s : bs;
  }
  int bi = VEC ? start + 4 * ((bs >> 2) * ST + t) + (bs & 3) : start + bs * ST + t;
  // The chunk's 16th largest lane maximum bounds its 16 best from below (16
  // elements are at least that large).  Each wave finds its own 16th largest
  // lane maximum and hands its 16 lane maxima at or above it to wave 0, which
  // takes the 16th largest of those 64: every one of the chunk's 16 largest
  // lane maxima is among its wave's 16 largest.
  {
    const uint32_t kb = order_key(bv);
    const uint32_t tw = wave_nth_key(kb, NC);
    const bool p = kb >= tw;  // at least NC lanes
    const unsigned long long m = __ballot(p);
    const int pos = __builtin_amdgcn_mbcnt_hi(unsigned(m >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(m), 0u));
    if (p && pos < NC) s_k[w * NC + pos] = kb;
  }
  if (t == 0) s_over = 0;
  __syncthreads();
  if (w == 0) {
    const uint32_t tc = wave_nth_key(s_k[lane], NC);
    if (lane == 0) s_tk = tc;
  }
  __syncthreads();
  const float tv = key_value(s_tk);
  // candidates: elements at or above the bound (equal values past its index
  // come along too, which only adds candidates), appended slot by slot (one
  // compare and a ballot per slot; most slots hold none)
  int total = 0;
#pragma unroll
  for (int s = 0; s < SPT; ++s) {
    const int e = sel_slot<VEC>(start, s, t);
    const bool p = x[s] >= tv;
    const unsigned long long m = __ballot(p);
    if (m) {
      const int below = __builtin_amdgcn_mbcnt_hi(unsigned(m >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(m), 0u));
      const int pos = total + below;
      if (p && pos < WCAP) { s_v[w * WCAP + pos] = x[s]; s_i[w * WCAP + pos] = e; }
      total += __popcll(m);
    }
  }
  if (lane == 0) s_n[w] = total;
  if (total > WCAP && lane == 0) s_over = 1;
  __syncthreads();
  float* ov = a.ctv + (size_t(row) * a.nch + c) * NC;
  int* oi = a.cti + (size_t(row) * a.nch + c) * NC;
  const int n0 = s_n[0], n01 = n0 + s_n[1], n012 = n01 + s_n[2], nall = n012 + s_n[3];
  if (!s_over && nall <= 64) {
    // wave 0 sorts all candidates (one per lane, the four lists one after
    // the other, empty lanes last) and keeps the first 16
    if (w == 0) {
      float v = -INFINITY;
      int i = INT32_MAX;
      if (lane < nall) {
        const int ww = (lane >= n0) + (lane >= n01) + (lane >= n012);
        const int off = lane - (ww == 0 ? 0 : ww == 1 ? n0 : ww == 2 ? n01 : n012);
        v = s_v[ww * WCAP + off];
        i = s_i[ww * WCAP + off];
      }
      wave_sort_best_first(v, i);
      // fewer than NC elements in the chunk: the list ends in empty entries
      if (lane < NC) {
        const bool real = i < a.V;
        ov[lane] = real ? v : -INFINITY;
        oi[lane] = real ? i : INT32_MAX;
      }
    }
    return;
  }
  // exact selection, one element per round (ties beyond WCAP per wave)
  unsigned long long taken = 0ull;
  for (int r = 0; r < NC; ++r) {
    float v = -INFINITY;
    int i = INT32_MAX;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int e = sel_slot<VEC>(start, s, t);
      if (!(taken >> s & 1ull) && sel_better(x[s], e, v, i)) { v = x[s]; i = e; }
    }
    keep_better<32>(v, i);
    keep_better<16>(v, i);
    keep_better<8>(v, i);
    keep_better<4>(v, i);
    keep_better<2>(v, i);
    keep_better<1>(v, i);
    if (lane == 0) { s_rv[w] = v; s_ri[w] = i; }
    __syncthreads();
    v = s_rv[0];
    i = s_ri[0];
    for (int w2 = 1; w2 < 4; ++w2)
      if (sel_better(s_rv[w2], s_ri[w2], v, i)) { v = s_rv[w2]; i = s_ri[w2]; }
    __syncthreads();
    if (t == 0) {
      const bool real = i < a.V;
      ov[r] = real ? v : -INFINITY;
      oi[r] = real ? i : INT32_MAX;
    }
#pragma unroll
    for (int s = 0; s < SPT; ++s)
      if (sel_slot<VEC>(start, s, t) == i) taken |= 1ull << s;
  }
}

// ------------------------------------------------------------- tables
// The NC best of a row's chunk lists (each sorted best first, already in
// LDS), merged by one wave: lane l holds the head of list l; each round the
// best head is taken and its lane moves to its next entry.
__device__ __forceinline__ void merge_lists(int nch, const float* s_mv, const int* s_mi, int* out_i, float* out_v) {
  const int lane = threadIdx.x & 63;
  int h = 0;  // this lane's position in its list
  float hv = -INFINITY;
  int hi = INT32_MAX;
  if (lane < nch) { hv = s_mv[lane * NC]; hi = s_mi[lane * NC]; }
  for (int r = 0; r < NC; ++r) {
    float v = hv;
    int i = hi;
    keep_better<32>(v, i);
    keep_better<16>(v, i);
    keep_better<8>(v, i);
    keep_better<4>(v, i);
    keep_better<2>(v, i);
    keep_better<1>(v, i);
    if (lane == 0) {
      out_i[r] = i;
      if (out_v) out_v[r] = v;
    }
    if (hi == i && i != INT32_MAX) {  // indices are unique across the lists
      ++h;
      hv = h < NC ? s_mv[lane * NC + h] : -INFINITY;
      hi = h < NC ? s_mi[lane * NC + h] : INT32_MAX;
    }
  }
}

__global__ __launch_bounds__(ST) void sel_table(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sel_lds[];
  // [2][nch * NC] list values and indices, then E rows [NC][r + pad] and F rows [NC][r + pad]
  float* s_mv = reinterpret_cast<float*>(sel_lds);
  int* s_mi = reinterpret_cast<int*>(s_mv + 2 * a.nch * NC);
  uint16_t* s_E = reinterpret_cast<uint16_t*>(s_mi + 2 * a.nch * NC);
  // rows padded by 16 bytes: the 16 candidate rows one read phase touches
  // then start 4 banks apart and cover all 64 banks
  const int rs = (a.r + 31) / 32 * 32 + SEL_ROW_PAD;
  uint16_t* s_F = s_E + NC * rs;
  __shared__ int s_prev[NC], s_cur[NC];
  __shared__ float s_z[NC];
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int row = b * a.G + t;
  // the chunk lists of this position (first half of the buffers) and of the
  // one before (second half) in one round of loads; wave 0 merges this
  // position's, wave 1 the previous one's
  const int n = a.nch * NC;
  const int nrows = t > 0 ? 2 : 1;
  int anc = 0;  // position 0's predecessor, loaded with the lists
  if (t == 0 && tid == 0) anc = a.anchor[b];
  {
    constexpr int PER = 2 * 64 * NC / ST;  // at most 64 chunks per row
    float bv[PER];
    int bi[PER];
    // unconditional loads (past the end: the last entry again), so that all
    // are in flight together; only the LDS stores are conditional
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = min(tid + u * ST, nrows * n - 1);
      const size_t src = size_t(row - e / n) * n + e % n;
      bv[u] = a.ctv[src];
      bi[u] = a.cti[src];
    }
    // the values are needed here, so no load is moved into the conditional
    // stores below (which would wait for each in turn)
#pragma unroll
    for (int u = 0; u < PER; ++u) asm volatile("" : "+v"(bv[u]), "+v"(bi[u]));
    asm volatile("" : "+v"(anc));
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * ST;
      if (e < nrows * n) { s_mv[e] = bv[u]; s_mi[e] = bi[u]; }
    }
  }
  if (t == 0 && tid == 0) s_prev[0] = anc;
  __syncthreads();
  const int n_prev = t > 0 ? NC : 1;
  if (tid < 64) merge_lists(a.nch, s_mv, s_mi, s_cur, s_z);
  else if (tid < 128 && t > 0) merge_lists(a.nch, s_mv + n, s_mi + n, s_prev, nullptr);
  __syncthreads();
  if (tid < NC) {
    a.cand[size_t(row) * NC + tid] = s_cur[tid];
    if (a.cand_out) a.cand_out[size_t(row) * NC + tid] = s_cur[tid];
  }
  __syncthreads();
  // rows of E for the predecessors and of F for the candidates (an anchor
  // outside the vocabulary reads as a zero row; its request is flagged by
  // sel_walk)
  // Rows are staged with r rounded up to 32 (zeros past r), the MFMA's k
  // step, plus the bank padding.
  const int pr = a.r / 8;                 // 16-byte pieces per row
  const int pr32 = (a.r + 31) / 32 * 4;   // the same, zero-padded to 32 elements
  {
    constexpr int PER = 2 * NC * 32 / ST;  // r <= 256: at most 32 pieces per row
    uint4 buf[PER];
    // one unconditional load per piece from a valid row (clamped index, an
    // invalid anchor's row replaced by zeros afterwards), all in flight together
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = min(tid + u * ST, 2 * NC * pr32 - 1);
      const int which = e / (NC * pr32), rr = (e / pr32) % NC, p = e % pr32;
      const int tok = which == 0 ? s_prev[rr < n_prev ? rr : 0] : s_cur[rr];
      const bool valid = tok >= 0 && tok < a.V;
      const uint16_t* base = which == 0 ? a.E : a.F;
      const uint4 v = *reinterpret_cast<const uint4*>(base + size_t(valid ? tok : 0) * a.r + min(p, pr - 1) * 8);
      buf[u] = valid && p < pr ? v : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) asm volatile("" : "+v"(buf[u].x), "+v"(buf[u].y), "+v"(buf[u].z), "+v"(buf[u].w));
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * ST;
      if (e < 2 * NC * pr32) {
        const int which = e / (NC * pr32), rr = (e / pr32) % NC, p = e % pr32;
        *reinterpret_cast<uint4*>((which == 0 ? s_E : s_F) + rr * rs + p * 8) = buf[u];
      }
    }
  }
  __syncthreads();
  // entry (i, j) = z(c_j) + E[p_i] . F[c_j]: one 16 x 16 product over k on
  // the matrix cores (16x16x32 bf16, fp32 accumulation).  Lane l supplies row
  // l % 16 of E and of F, k octet l / 16 of each 32-step, and receives
  // entries (4 (l / 16) + q, l % 16), q = 0..3.
  if (tid < 64) {
    const int lr = tid & 15, kq = tid >> 4;
    floatx4 d = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < pr32 * 8; k0 += 32) {
      const bf16x8 ea = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(s_E + lr * rs + k0 + 8 * kq));
      const bf16x8 fb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(s_F + lr * rs + k0 + 8 * kq));
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea, fb, d, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * kq + q;
      if (i < n_prev) a.tab[(size_t(row) * NC + i) * NC + lr] = s_z[lr] + d[q];
    }
  }
}

// ------------------------------------------------------------- walk
constexpr int WALK_GROUP = 32;  // positions whose tables are in LDS at once

__global__ __launch_bounds__(64) void sel_walk(SelArgs a) {
  __shared__ __attribute__((aligned(16))) float s_t[WALK_GROUP * NC * NC];
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
    // every load of the group in flight before the first LDS store (position
    // 0's rows past the first are never read)
    const float4* src = reinterpret_cast<const float4*>(a.tab + (r0 + t0) * NC * NC);
    const int n4 = ng * NC * NC / 4;  // at most 64 per lane
    constexpr int PER = WALK_GROUP * NC * NC / 4 / 64;
    float4 buf[PER];
    int cbuf[WALK_GROUP * NC / 64];
    // unconditional loads (past the group: its last entry again) so that all
    // are in flight together
#pragma unroll
    for (int u = 0; u < PER; ++u) buf[u] = src[min(lane + u * 64, n4 - 1)];
#pragma unroll
    for (int u = 0; u < WALK_GROUP * NC / 64; ++u) cbuf[u] = a.cand[(r0 + t0) * NC + min(lane + u * 64, ng * NC - 1)];
    // (the LDS arrays hold a whole group: entries past this one's end are
    // written too and never read)
#pragma unroll
    for (int u = 0; u < PER; ++u) reinterpret_cast<float4*>(s_t)[lane + u * 64] = buf[u];
#pragma unroll
    for (int u = 0; u < WALK_GROUP * NC / 64; ++u) s_c[lane + u * 64] = cbuf[u];
    __syncthreads();
    // 16 lanes read the visited row at once; the best (lowest j on ties) wins
    int jp = s_j;
    for (int u = 0; u < ng; ++u) {
      const int t = t0 + u;
      const int j = lane & (NC - 1);
      float v = s_t[(u * NC + (t == 0 ? 0 : jp)) * NC + j];
      int jj = j;
      keep_better<8>(v, jj);
      keep_better<4>(v, jj);
      keep_better<2>(v, jj);
      keep_better<1>(v, jj);
      if (lane == 0) {
        a.tokens[r0 + t] = ok ? s_c[u * NC + jj] : -1;
        if (a.scores) a.scores[r0 + t] = ok ? v : NAN;
      }
      jp = jj;
    }
    if (lane == 0) s_j = jp;
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
  const size_t lds2 = size_t(2) * a.nch * NC * 8 + size_t(2) * NC * ((r + 31) / 32 * 32 + SEL_ROW_PAD) * 2;
  hipLaunchKernelGGL(sel_table, dim3(G, B), dim3(ST), lds2, stream, a);
  hipLaunchKernelGGL(sel_walk, dim3(B), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bd
