// verify_block kernels: vocabulary-row statistics, the per-request decision
// chain, and the residual / extra-token draw.
//
// DSpark tutorial, "speculative decoding basics": prefix acceptance, one
// replacement at the first disagreement, one extra token per round, and the
// losslessness of the rejection rule (accept with min(1, P/Q), else draw from
// the normalised max(0, P - Q)).  DSpine article, "principle": greedy
// matching; "speed-up": temperature / top-k / top-p; "tuning and memory":
// batched verification can flip near-tied tokens, hence the fixed reduction
// orders here and the ratio / margin diagnostics.
//
// Pass 1 streams every logits row once, in chunks of 8192, with persistent
// workgroups that each take an equal run of (row, chunk) pairs and write one
// record per row they touch: vb_stats_stream the maximum and its lowest
// index and the sum of exp((z - max) / T) (fp32 lanes, fp64 across lanes),
// vb_topk_stream under top-k the k best (value desc, index asc).  Greedy and
// top-k: pass 2 (vb_decide, one workgroup per request, after vb_merge_rows
// under top-k) merges the records of its rows, applies the filters, runs the
// accept chain and draws over the filtered support.  Full-vocabulary
// sampling needs the chosen row pair once more: there pass 2
// (vb_decide_sums, one workgroup per (chunk, request)) merges the request's
// rows and runs the accept chain in every workgroup, then sums the draw
// weights of its chunk, and vb_draw_pick scans the one chunk that holds the
// crossing.
#include "bd_common.hpp"
#include "bd_launch.hpp"

#include <math.h>

namespace bd {

constexpr int VT = 256;        // threads of a stats / draw workgroup
constexpr int VCH = 8192;      // logits per chunk (32 per thread)
constexpr int VPT = VCH / VT;  // 32
constexpr int TOPK_MAX = 64;
// Vector rows: a chunk's draw-weight sum is also kept per run of SUBLEN
// consecutive logits (run k = 4 j + w: the slot group j of wave w), so the
// draw can find the run holding the crossing without re-reading the chunk.
constexpr int NSUB = VPT / 4 * (VT / 64);  // 32
constexpr int SUBLEN = VCH / NSUB;         // 256
constexpr int PICK_FAST_NCH = 64;          // chunks whose run sums the draw keeps in LDS
// Target workgroups of the streaming statistics pass and its register budget
// (waves per SIMD) so that they are all resident at once.
#ifndef BD_STATS_GRID
#define BD_STATS_GRID 1024
#endif
#ifndef BD_STATS_WPE
#define BD_STATS_WPE 4
#endif
#define BD_STATS_OCC __attribute__((amdgpu_waves_per_eu(BD_STATS_WPE)))
constexpr int STATS_GRID = BD_STATS_GRID;

enum { JOB_NONE = 0, JOB_RESID = 1, JOB_BONUS = 2 };

// The full-vocabulary draw of one request: the position, the kind, the
// uniform, and the row maxima and 1 / sums of the row pair (one load).
struct alignas(32) DrawJob {
  int pos, kind;
  float u2, mt, st, md, sd, pad;
};

// -------------------------------------------------------------------------
// element access: thread t holds, for j = 0..7 and c = 0..3 (vector rows) the
// logit at chunk offset 4 * (j * 256 + t) + c, or for j = 0..31 (scalar rows)
// the logit at chunk offset j * 256 + t.  Both orders increase with the slot.
// -------------------------------------------------------------------------
template <bool VEC>
__device__ __forceinline__ int slot_offset(int s, int t) {
  if (VEC) return 4 * ((s >> 2) * VT + t) + (s & 3);
  return s * VT + t;
}

template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int start, int V, int t,
                                           float (&x)[VPT]) {
  // Every lane loads unconditionally (slots past the row end re-read the row
  // start) and the values are used raw: callers mask slots with index >= V at
  // the point of use.  Keeping selects off the loaded registers lets the
  // loads stay in flight until the data is consumed.
  if (VEC) {
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j) {
      const int e = start + 4 * (j * VT + t);
      const float4 f = *reinterpret_cast<const float4*>(row + (e < V ? e : 0));
      x[4 * j] = f.x; x[4 * j + 1] = f.y; x[4 * j + 2] = f.z; x[4 * j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = start + j * VT + t;
      x[j] = row[e < V ? e : 0];
    }
  }
}

// Block-wide (value, index) argmax; lds needs 2 * (VT / 64) words.
__device__ __forceinline__ void block_argmax(float& v, int& i, float* lv, int* li) {
  wave_argmax(v, i);
  int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) { lv[w] = v; li[w] = i; }
  __syncthreads();
  v = lv[0]; i = li[0];
#pragma unroll
  for (int k = 1; k < VT / 64; ++k)
    if (better(lv[k], li[k], v, i)) { v = lv[k]; i = li[k]; }
}

__device__ __forceinline__ double block_sum_f64(double s, double* ld) {
  s = wave_sum(s);
  int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) ld[w] = s;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int k = 0; k < VT / 64; ++k) r += ld[k];
  return r;
}

// Descending bitonic sort of one float per lane across the wave.
__device__ __forceinline__ float wave_sort_desc(float v) {
  int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      float o = __shfl_xor(v, stride);
      bool desc = (lane & size) == 0 || size == 64;
      bool lower = (lane & stride) == 0;
      v = (lower == desc) ? fmaxf(v, o) : fminf(v, o);
    }
  }
  return v;
}

// Statistics records: workgroup w of pass 1 takes the global chunks
// [w * cpw, (w + 1) * cpw) of the row-major (row, chunk) sequence and writes
// one record per row it touches, at slot row + w (unique: a later row starts
// in a workgroup at or after the last one of an earlier row).
struct VerifyWs {
  float* cmax;   // [slots]
  int* carg;     // [slots]
  double* csum;  // [slots]
  float* ctv;    // [slots][k]
  int* cti;      // [slots][k]
  float* rmax;   // [rows]
  int* rarg;     // [rows]
  double* rsum;  // [rows]
  int* rkn;      // [rows]           kept count after filters
  int* rki;      // [rows][TOPK_MAX] kept indices (value desc, index asc)
  double* rkp;   // [rows][TOPK_MAX] kept probabilities
  DrawJob* job;  // [B]             the draw each request needs
  double* jsum;  // [B][nch]
  double* jsub;  // [B][nch][NSUB]  vector rows: sums over runs of SUBLEN logits
  double* jbeta; // [n_draft][nch]  per-chunk sums of min(P, Q) (labels, full vocabulary)
};

struct VerifyArgs {
  const float* zt;
  const float* zd;
  const int* dtok;
  const float* uni;
  int B, G, V, nch;      // G: drafted tokens per request (the largest one with row_cu)
  int cpw;               // consecutive (row, chunk) pairs per statistics workgroup
  int n_trows, n_rows;   // target rows; all rows with the draft rows
  const int* row_cu;     // [B + 1] first target row of each request, or NULL: B * (G + 1)
  float T;               // temperature used for probabilities (1 when greedy)
  float c2;              // log2(e) / T
  int greedy, topk, need_sum;
  float top_p;
  int* tau;
  int* out;
  float* tprob;
  float* dprob;
  float* ratio;
  float* margin;
  float* beta;           // [n_draft] confidence label of each drafted position, or NULL
  VerifyWs ws;
};

// Rows of request b: target rows t0 .. t0 + G, draft rows d0 .. d0 + G - 1
// (packed: d0 = t0 - b).  With a row map the request is valid when its rows
// lie inside the packed arrays with room for one row per other request and
// 0 <= G <= the largest G; an invalid request gets tau = -1 and nothing else.
struct ReqRows {
  int t0, d0, G;
  bool ok;
};

__device__ __forceinline__ ReqRows req_rows(const VerifyArgs& a, int b) {
  ReqRows r;
  if (!a.row_cu) {
    r.t0 = b * (a.G + 1);
    r.d0 = b * a.G;
    r.G = a.G;
    r.ok = true;
    return r;
  }
  const int c0 = a.row_cu[b], c1 = a.row_cu[b + 1];
  r.G = c1 - c0 - 1;
  r.t0 = c0;
  r.d0 = c0 - b;
  r.ok = c0 >= b && r.G >= 0 && r.G <= a.G && c1 <= a.n_trows - (a.B - 1 - b);
  if (!r.ok) { r.t0 = 0; r.d0 = 0; r.G = 0; }
  return r;
}

__device__ __forceinline__ const float* row_ptr(const VerifyArgs& a, int r) {
  return r < a.n_trows ? a.zt + size_t(r) * a.V : a.zd + size_t(r - a.n_trows) * a.V;
}

// -------------------------------------------------------------------------
// Pass 1, streaming form (no top-k): a persistent workgroup walks its run of
// (row, chunk) pairs, keeping the next chunk's non-temporal loads in flight
// while it reduces the current one.  Every thread keeps its own running
// maximum (lowest index on ties) and sum of exp((z - max) / T) in fp64,
// rescaled when its maximum grows; at the end of each row (or of the run) the
// workgroup combines its threads into one record.
// -------------------------------------------------------------------------
template <bool VEC>
__device__ __forceinline__ void load_stream_chunk(const float* __restrict__ row, int start, int V, int t,
                                                  float (&x)[VPT]) {
  if (VEC) {
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j) {
      const int e = start + 4 * (j * VT + t);
      const float4 f = ld_stream(row + (e < V ? e : 0));
      x[4 * j] = f.x; x[4 * j + 1] = f.y; x[4 * j + 2] = f.z; x[4 * j + 3] = f.w;
    }
  } else {
    load_chunk<false>(row, start, V, t, x);
  }
}

// ARG: keep the index of the maximum (greedy decisions need it; sampling
// needs only the maximum and the sum, and the plain maximum is a third of the
// per-logit selects: 2.3 us of the 8B round's 95.5 us pass).  Without ARG,
// `it` only marks that the thread has seen a logit (any value but INT32_MAX).
template <bool VEC, bool ARG = true>
__device__ __forceinline__ void consume_chunk(const VerifyArgs& a, const float (&x)[VPT], int start, int t,
                                              float& mt, int& it, double& st) {
  float cm = -INFINITY;
  int ci = INT32_MAX;
  if (start + VCH <= a.V) {
    // full chunk (every chunk of a row but its last): no bounds checks; the
    // slots increase with the index, so the first strict maximum in slot
    // order is the lowest index; the sum folds the scale into one FMA
    cm = x[0];
    if constexpr (ARG) {
      int cs = 0;
#pragma unroll
      for (int s = 1; s < VPT; ++s)
        if (x[s] > cm) { cm = x[s]; cs = s; }
      ci = start + (VEC ? 4 * ((cs >> 2) * VT + t) + (cs & 3) : cs * VT + t);
    } else {
#pragma unroll
      for (int s = 1; s < VPT; ++s) cm = x[s] > cm ? x[s] : cm;
      ci = 0;
    }
    const bool first = it == INT32_MAX;
    const float mn = first ? cm : fmaxf(mt, cm);
    if (a.need_sum && mn != -INFINITY) {
      if (!first && mn > mt && st != 0.0) st *= exp2(double(mt - mn) * double(a.c2));
      const float nb = -mn * a.c2;
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < VPT; ++s) part += exp2_hw(fmaf(x[s], a.c2, nb));
      st += double(part);
    }
    if (first || cm > mt) { mt = cm; it = ci; }
    return;
  }
#pragma unroll
  for (int s = 0; s < VPT; ++s) {
    const int e = start + slot_offset<VEC>(s, t);
    if (e < a.V && (x[s] > cm || ci == INT32_MAX)) { cm = x[s]; ci = e; }
  }
  if (ci == INT32_MAX) return;
  const bool first = it == INT32_MAX;
  const float mn = first ? cm : fmaxf(mt, cm);
  if (a.need_sum && mn != -INFINITY) {
    if (!first && mn > mt && st != 0.0) st *= exp2(double(mt - mn) * double(a.c2));
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const float p = exp2_hw((x[s] - mn) * a.c2);
      part += (start + slot_offset<VEC>(s, t) < a.V) ? p : 0.f;
    }
    st += double(part);
  }
  if (first || cm > mt) { mt = cm; it = ci; }
}

// one record of (row, workgroup) from the threads' running statistics
__device__ __forceinline__ void flush_row(const VerifyArgs& a, size_t slot, float& mt, int& it, double& st,
                                          float* s_v, int* s_i, double* s_d) {
  float bv = mt;
  int bi = it;
  block_argmax(bv, bi, s_v, s_i);  // (without ARG the indices are placeholders)
  if (threadIdx.x == 0) { a.ws.cmax[slot] = bv; a.ws.carg[slot] = bi; }
  if (a.need_sum) {
    double contrib = 0.0;
    if (it != INT32_MAX && st != 0.0) contrib = st * exp2(double(mt - bv) * double(a.c2));
    const double S = block_sum_f64(contrib, s_d);
    if (threadIdx.x == 0) a.ws.csum[slot] = S;
  }
  mt = -INFINITY;
  it = INT32_MAX;
  st = 0.0;
}

template <bool VEC, bool ARG>
__global__ __launch_bounds__(VT) BD_STATS_OCC void vb_stats_stream(VerifyArgs a) {
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  __shared__ double s_d[4];
  const int t = threadIdx.x, w = blockIdx.x;
  const long long total = (long long)a.n_rows * a.nch;
  const long long x0 = (long long)w * a.cpw;
  const long long x1 = min(total, x0 + a.cpw);
  if (x0 >= x1) return;
  float mt = -INFINITY;
  int it = INT32_MAX;
  double st = 0.0;
  float xa[VPT], xb[VPT];
  auto rowp = [&](long long x) { return row_ptr(a, int(x / a.nch)); };
  auto cstart = [&](long long x) { return int(x % a.nch) * VCH; };
  auto row_ends = [&](long long x) { return x + 1 == x1 || (x + 1) % a.nch == 0; };
  load_stream_chunk<VEC>(rowp(x0), cstart(x0), a.V, t, xa);
  long long x = x0;
  // steady state: both look-ahead loads are unconditional, so the compiler
  // can wait for exactly the chunk it consumes
  while (x + 2 < x1) {
    load_stream_chunk<VEC>(rowp(x + 1), cstart(x + 1), a.V, t, xb);
    consume_chunk<VEC, ARG>(a, xa, cstart(x), t, mt, it, st);
    if (row_ends(x)) flush_row(a, size_t(x / a.nch) + w, mt, it, st, s_v, s_i, s_d);
    load_stream_chunk<VEC>(rowp(x + 2), cstart(x + 2), a.V, t, xa);
    consume_chunk<VEC, ARG>(a, xb, cstart(x + 1), t, mt, it, st);
    if (row_ends(x + 1)) flush_row(a, size_t((x + 1) / a.nch) + w, mt, it, st, s_v, s_i, s_d);
    x += 2;
  }
  // the last one or two chunks
  if (x + 1 < x1) {
    load_stream_chunk<VEC>(rowp(x + 1), cstart(x + 1), a.V, t, xb);
    consume_chunk<VEC, ARG>(a, xa, cstart(x), t, mt, it, st);
    if (row_ends(x)) flush_row(a, size_t(x / a.nch) + w, mt, it, st, s_v, s_i, s_d);
    consume_chunk<VEC, ARG>(a, xb, cstart(x + 1), t, mt, it, st);
    flush_row(a, size_t((x + 1) / a.nch) + w, mt, it, st, s_v, s_i, s_d);
  } else {
    consume_chunk<VEC, ARG>(a, xa, cstart(x), t, mt, it, st);
    flush_row(a, size_t(x / a.nch) + w, mt, it, st, s_v, s_i, s_d);
  }
}

// -------------------------------------------------------------------------
// Pass 1, streaming top-k form: a persistent workgroup walks its run of (row,
// chunk) pairs as the streaming form does, in half chunks (16 logits per
// thread, the next half's loads in flight).  Each wave keeps, for the row it
// is in, a bound and an LDS list of its logits that beat it, with no barrier
// inside the row: at the row's first half chunk of the run the bound is the
// k-th largest of the wave's 64 lane maxima (k of its logits are at least that
// large, so each of the wave's own k best, value desc and index asc, is too).
// Every half chunk appends the wave's logits that beat the bound.  When the
// list would overflow (or holds 2k entries still under that first bound) the
// list's k best replace it and the k-th of them becomes the bound (strict from
// then on: later logits have larger indices, so an equal value comes after
// it); a half chunk that still does not fit falls back to k rounds of a wave
// argmax over the wave's own logits of it.  The row's k best are among the
// union of the waves' own k best: at the row's last half chunk of the run wave
// 0 selects them from the four lists for the record, whose first entry is
// also the record's maximum and lowest-index argmax.
// -------------------------------------------------------------------------
constexpr int TKW_CAP = 256;       // list entries per wave (values and indices: 8 KB per workgroup)
constexpr int TKW_Q = TKW_CAP / 64;
constexpr int HPT = VPT / 2;       // logits per thread of a half chunk
constexpr int HCH = VCH / 2;       // logits of a half chunk

// the logits of the half chunk at `start` (thread t: slot s < HPT at
// start + slot_offset(s, t)); slots past the row re-read its first logit
template <bool VEC>
__device__ __forceinline__ void load_half(const float* __restrict__ row, int start, int V, int t, float (&x)[HPT]) {
  if (VEC) {
#pragma unroll
    for (int j = 0; j < HPT / 4; ++j) {
      const int e = start + 4 * (j * VT + t);
      const float4 f = ld_stream(row + (e < V ? e : 0));
      x[4 * j] = f.x; x[4 * j + 1] = f.y; x[4 * j + 2] = f.z; x[4 * j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
      const int e = start + j * VT + t;
      x[j] = row[e < V ? e : 0];
    }
  }
}

// The k best (value desc, index asc) of up to 64 Q entries held in the
// wave's registers (empty entries: index INT32_MAX), by the whole wave: the
// k-th largest value key T by a bitwise search (one ballot count per bit and
// register), then the entries with key >= T (ties at T included) staged in
// LDS and sorted by a wave bitonic sort.  More than 64 of those (heavy ties)
// fall back to k rounds of a wave argmax over the registers.  Lane r < k gets
// pick r (value -inf, index INT32_MAX when there are fewer than k entries).
// The staging area (64 entries) may be where the entries were loaded from:
// every lane holds its entries before it is written.
template <int Q>
__device__ __forceinline__ void wave_top_k(const float (&v)[Q], const int (&id)[Q], int k, float* stage_v,
                                           int* stage_i, float& mv, int& mi) {
  const int lane = threadIdx.x & 63;
  uint32_t key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) key[q] = id[q] == INT32_MAX ? 0u : order_key(v[q]);  // real keys are >= 1
  uint32_t T = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int n = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) n += __popcll(__ballot(key[q] >= c));
    if (n >= k) T = c;
  }
  if (T == 0) T = 1;  // fewer than k entries: all of them
  int m = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) m += __popcll(__ballot(key[q] >= T));
  mv = -INFINITY;
  mi = INT32_MAX;
  if (m <= 64) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int off = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const bool p = key[q] >= T;
      const unsigned long long msk = __ballot(p);
      const int pos = off + __builtin_amdgcn_mbcnt_hi(unsigned(msk >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(msk), 0u));
      if (p) { stage_v[pos] = v[q]; stage_i[pos] = id[q]; }
      off += __popcll(msk);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float sv = lane < m ? stage_v[lane] : -INFINITY;
    int si = lane < m ? stage_i[lane] : INT32_MAX;
    wave_sort_best_first(sv, si);
    if (lane < k) { mv = sv; mi = si; }
    return;
  }
  float pv = INFINITY;
  int pi = -1;
  for (int r = 0; r < k; ++r) {
    float cv = -INFINITY;
    int ci = INT32_MAX;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if ((pi < 0 || better(pv, pi, v[q], id[q])) && better(v[q], id[q], cv, ci)) { cv = v[q]; ci = id[q]; }
    wave_argmax(cv, ci);
    if (ci == INT32_MAX) break;
    if (lane == r) { mv = cv; mi = ci; }
    pv = cv;
    pi = ci;
  }
}

struct TopkState {
  int cnt;     // entries of the wave's list
  float tv;    // bound: a logit is a candidate when v > tv (strict) or v >= tv
  int strict;
};

// the wave's list replaced by its k best, best first; the k-th becomes the
// (strict) bound when there were at least k entries
__device__ __forceinline__ void topk_trim(TopkState& st, float* lv, int* li, int k) {
  const int lane = threadIdx.x & 63;
  float v[TKW_Q];
  int id[TKW_Q];
#pragma unroll
  for (int q = 0; q < TKW_Q; ++q) {
    const int j = lane + 64 * q;
    v[q] = j < st.cnt ? lv[j] : -INFINITY;
    id[q] = j < st.cnt ? li[j] : INT32_MAX;
  }
  float mv;
  int mi;
  wave_top_k<TKW_Q>(v, id, k, lv, li, mv, mi);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int kept = st.cnt < k ? st.cnt : k;
  if (lane < kept) { lv[lane] = mv; li[lane] = mi; }
  if (st.cnt >= k) {
    st.tv = lane_value(mv, k - 1);
    st.strict = 1;
  }
  st.cnt = kept;
}

// Appends the wave's logits of the half chunk that beat the bound to its
// list (one ballot per slot; a slot no lane hits costs one compare).  Entries
// past the capacity are not written; returns false when some did not fit.
template <bool VEC, bool STRICT, bool FULL>
__device__ __forceinline__ bool topk_append(const VerifyArgs& a, TopkState& st, const float (&x)[HPT], int start,
                                            float* lv, int* li) {
  const int t = threadIdx.x;
  int base = st.cnt;
#pragma unroll
  for (int s = 0; s < HPT; ++s) {
    const int e = start + slot_offset<VEC>(s, t);
    const bool hit = (STRICT ? x[s] > st.tv : x[s] >= st.tv) && (FULL || e < a.V);
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int pos = base + __builtin_amdgcn_mbcnt_hi(unsigned(m >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(m), 0u));
      if (hit && pos < TKW_CAP) { lv[pos] = x[s]; li[pos] = e; }
      base += __popcll(m);
    }
  }
  st.cnt = base < TKW_CAP ? base : TKW_CAP;
  return base <= TKW_CAP;
}

template <bool VEC>
__device__ __forceinline__ bool topk_append(const VerifyArgs& a, TopkState& st, const float (&x)[HPT], int start,
                                            float* lv, int* li) {
  if (start + HCH <= a.V)
    return st.strict ? topk_append<VEC, true, true>(a, st, x, start, lv, li)
                     : topk_append<VEC, false, true>(a, st, x, start, lv, li);
  return st.strict ? topk_append<VEC, true, false>(a, st, x, start, lv, li)
                   : topk_append<VEC, false, false>(a, st, x, start, lv, li);
}

template <bool VEC>
__device__ __forceinline__ void topk_half(const VerifyArgs& a, TopkState& st, const float (&x)[HPT], int start,
                                          bool first, bool last, size_t slot, float* s_bv, int* s_bi, int* s_cnt) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int k = a.topk;
  float* lv = s_bv + w * TKW_CAP;
  int* li = s_bi + w * TKW_CAP;
  if (first) {
    float lm = -INFINITY;
#pragma unroll
    for (int s = 0; s < HPT; ++s) lm = (start + slot_offset<VEC>(s, t) < a.V) ? fmaxf(lm, x[s]) : lm;
    st.cnt = 0;
    st.tv = key_value(wave_nth_key(order_key(lm), k));
    st.strict = 0;
  }
  const int cnt0 = st.cnt;
  if (!topk_append<VEC>(a, st, x, start, lv, li)) {
    // the half chunk did not fit: its entries are dropped, the list trimmed
    // to its k best (a stricter bound), and the half chunk appended again
    st.cnt = cnt0;
    topk_trim(st, lv, li, k);
    const int cnt1 = st.cnt;
    if (!topk_append<VEC>(a, st, x, start, lv, li)) {
      // still too many: the wave's own k best of the half chunk, k rounds
      // of a wave argmax
      st.cnt = cnt1;
      float pv = INFINITY;
      int pi = -1;
      for (int r = 0; r < k; ++r) {
        float cv = -INFINITY;
        int ci = INT32_MAX;
#pragma unroll
        for (int s = 0; s < HPT; ++s) {
          const int e = start + slot_offset<VEC>(s, t);
          if (e < a.V && (pi < 0 || better(pv, pi, x[s], e)) && better(x[s], e, cv, ci)) { cv = x[s]; ci = e; }
        }
        wave_argmax(cv, ci);
        if (ci == INT32_MAX) break;
        if (lane == 0) { lv[st.cnt] = cv; li[st.cnt] = ci; }
        ++st.cnt;
        pv = cv;
        pi = ci;
      }
    }
  } else if (!st.strict && st.cnt > 2 * k) {
    // the first bound is loose: once the list holds 2k the k-th best becomes
    // the bound
    topk_trim(st, lv, li, k);
  }
  if (last) {
    // the record: each wave's k best, then the k best of those four lists
    topk_trim(st, lv, li, k);
    if (lane == 0) s_cnt[w] = st.cnt;
    __syncthreads();
    if (w == 0) {
      float v[VT / 64];
      int id[VT / 64];
#pragma unroll
      for (int q = 0; q < VT / 64; ++q) {
        const bool ok = lane < s_cnt[q];
        v[q] = ok ? s_bv[q * TKW_CAP + lane] : -INFINITY;
        id[q] = ok ? s_bi[q * TKW_CAP + lane] : INT32_MAX;
      }
      float mv;
      int mi;
      wave_top_k<VT / 64>(v, id, k, s_bv, s_bi, mv, mi);
      if (lane < k) { a.ws.ctv[slot * k + lane] = mv; a.ws.cti[slot * k + lane] = mi; }
      if (lane == 0) { a.ws.cmax[slot] = mv; a.ws.carg[slot] = mi; }
    }
    __syncthreads();
  }
}

template <bool VEC>
__global__ __launch_bounds__(VT) BD_STATS_OCC void vb_topk_stream(VerifyArgs a) {
  __shared__ float s_bv[(VT / 64) * TKW_CAP];
  __shared__ int s_bi[(VT / 64) * TKW_CAP];
  __shared__ int s_cnt[VT / 64];
  const int t = threadIdx.x, w = blockIdx.x;
  const long long total = (long long)a.n_rows * a.nch;
  const long long x0 = (long long)w * a.cpw;
  const long long x1 = min(total, x0 + a.cpw);
  if (x0 >= x1) return;
  // half chunks h = 2 x + half of the chunks x in [x0, x1)
  const long long h0 = 2 * x0, h1 = 2 * x1;
  TopkState st{0, -INFINITY, 0};
  float xa[HPT], xb[HPT];
  auto rowp = [&](long long h) { return row_ptr(a, int((h >> 1) / a.nch)); };
  auto hstart = [&](long long h) { return int((h >> 1) % a.nch) * VCH + int(h & 1) * HCH; };
  auto is_first = [&](long long h) { return (h & 1) == 0 && (h == h0 || (h >> 1) % a.nch == 0); };
  auto is_last = [&](long long h) { return (h & 1) == 1 && (h + 1 == h1 || ((h >> 1) + 1) % a.nch == 0); };
  auto slot = [&](long long h) { return size_t((h >> 1) / a.nch) + size_t(w); };
  // two half chunks per iteration (h0 and h1 are even): register double buffer
  load_half<VEC>(rowp(h0), hstart(h0), a.V, t, xa);
  for (long long h = h0; h < h1; h += 2) {
    load_half<VEC>(rowp(h + 1), hstart(h + 1), a.V, t, xb);
    topk_half<VEC>(a, st, xa, hstart(h), is_first(h), false, slot(h), s_bv, s_bi, s_cnt);
    // the look-ahead past the run re-reads its last half chunk (in bounds, never consumed)
    const long long hn = h + 2 < h1 ? h + 2 : h + 1;
    load_half<VEC>(rowp(hn), hstart(hn), a.V, t, xa);
    topk_half<VEC>(a, st, xb, hstart(h + 1), false, is_last(h + 1), slot(h + 1), s_bv, s_bi, s_cnt);
  }
}

// -------------------------------------------------------------------------
// Draw weights of the full-vocabulary draw: the residual max(0, p - q) or p.
// p(x) = exp((z - max) / T) / S evaluated in fp32.
// -------------------------------------------------------------------------
struct DrawRow {
  const float* zt;
  const float* zd;  // NULL for the extra-token draw
  float mt, md, st, sd;  // row maxima and 1 / sums
};

__device__ __forceinline__ float draw_weight(const DrawRow& r, float c2, float zt, float zd, bool resid) {
  float p = exp2_hw((zt - r.mt) * c2) * r.st;
  if (!resid) return p;
  float q = exp2_hw((zd - r.md) * c2) * r.sd;
  return fmaxf(0.f, p - q);
}

// -------------------------------------------------------------------------
// Pass 2: one workgroup per request.
// -------------------------------------------------------------------------
// The row's merged maximum, lowest-index argmax and (when asked) sum of
// exp((z - max) / T) from its records: slots row + w for the workgroups w of
// the statistics pass that covered it.  The records of the first 64 are kept
// in registers between the two reductions.
__device__ __forceinline__ int row_records(const VerifyArgs& a, int row, size_t& slot0) {
  const long long w0 = (long long)row * a.nch / a.cpw;
  const long long w1 = ((long long)row * a.nch + a.nch - 1) / a.cpw;
  slot0 = size_t(row) + size_t(w0);
  return int(w1 - w0 + 1);
}

__device__ __forceinline__ void merge_stats(const VerifyArgs& a, int row, int lane, float& v, int& i, double& S) {
  size_t slot0;
  const int nrec = row_records(a, row, slot0);
  v = -INFINITY;
  i = INT32_MAX;
  float cm0 = -INFINITY;
  double cs0 = 0.0;
  if (lane < nrec) {
    cm0 = a.ws.cmax[slot0 + lane];
    i = a.ws.carg[slot0 + lane];
    if (a.need_sum) cs0 = a.ws.csum[slot0 + lane];
    v = cm0;
  }
  for (int c = lane + 64; c < nrec; c += 64) {
    const size_t rc = slot0 + c;
    const float cv = a.ws.cmax[rc];
    const int ci = a.ws.carg[rc];
    if (better(cv, ci, v, i)) { v = cv; i = ci; }
  }
  wave_argmax(v, i);
  S = 0.0;
  if (a.need_sum && v != -INFINITY) {
    if (cm0 != -INFINITY) S = cs0 * exp2(double(cm0 - v) * double(a.c2));
    for (int c = lane + 64; c < nrec; c += 64) {
      const size_t rc = slot0 + c;
      const float cm = a.ws.cmax[rc];
      if (cm != -INFINITY) S += a.ws.csum[rc] * exp2(double(cm - v) * double(a.c2));
    }
    S = wave_sum(S);
  }
}

// s_v / s_i: LDS room for the row's nrec * k chunk-list entries (used with a
// top-k filter only, by a one-wave workgroup)
__device__ void merge_row(const VerifyArgs& a, int row, int lane, float* s_v = nullptr, int* s_i = nullptr) {
  float v;
  int i;
  double S;
  merge_stats(a, row, lane, v, i, S);
  if (lane == 0) {
    a.ws.rmax[row] = v;
    a.ws.rarg[row] = i;
    a.ws.rsum[row] = S;
  }
  if (a.topk > 0) {
    // k best of the chunk lists, then softmax over them and the top-p cut
    size_t slot0;
    const int nrec = row_records(a, row, slot0);
    const int k = a.topk;
    const int ncand = nrec * k;
    const float* cv = a.ws.ctv + slot0 * k;
    const int* ci = a.ws.cti + slot0 * k;
    float pv = INFINITY;
    int pi = -1;
    int* ki = a.ws.rki + size_t(row) * TOPK_MAX;
    double* kp = a.ws.rkp + size_t(row) * TOPK_MAX;
    float kv_lane = -INFINITY;  // lane r keeps the r-th kept value
    int kept = 0;
    if (ncand <= 64) {
      // every candidate in one lane: the k best are the first k lanes after a
      // wave-wide bitonic sort (value desc, index asc; empty entries, index
      // INT32_MAX, sort last)
      float sv = -INFINITY;
      int si = INT32_MAX;
      if (lane < ncand) { sv = cv[lane]; si = ci[lane]; }
      wave_sort_best_first(sv, si);
      kept = __popcll(__ballot(lane < k && si != INT32_MAX));
      if (lane < kept) { kv_lane = sv; ki[lane] = si; }
    } else if (s_v && nrec <= 64) {
      // the chunk lists are sorted best first: a k-way merge, lane l holding
      // list l's head and the round's winner advancing (the lists staged in
      // LDS, loaded eight per lane at a time)
      for (int j0 = 0; j0 < ncand; j0 += 8 * 64) {
        float vb8[8];
        int ib8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int jc = min(j0 + lane + 64 * c, ncand - 1);
          vb8[c] = cv[jc];
          ib8[c] = ci[jc];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(vb8[c]), "+v"(ib8[c]));
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (j0 + lane + 64 * c < ncand) { s_v[j0 + lane + 64 * c] = vb8[c]; s_i[j0 + lane + 64 * c] = ib8[c]; }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      int h = 0;
      float hv = lane < nrec ? s_v[lane * k] : -INFINITY;
      int hi = lane < nrec ? s_i[lane * k] : INT32_MAX;
      for (int r = 0; r < k; ++r) {
        float bv = hv;
        int bi = hi;
        wave_argmax(bv, bi);
        if (bi == INT32_MAX) break;
        if (hi == bi) {  // indices are distinct: exactly one lane wins
          ++h;
          hv = h < k ? s_v[lane * k + h] : -INFINITY;
          hi = h < k ? s_i[lane * k + h] : INT32_MAX;
        }
        if (lane == r) { kv_lane = bv; ki[r] = bi; }
        ++kept;
      }
    } else {
      // each round the best candidate strictly after the previous pick
      for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int bi = INT32_MAX;
        for (int j = lane; j < ncand; j += 64) {
          float x = cv[j];
          int id = ci[j];
          if (id == INT32_MAX) continue;
          if ((pi < 0 || better(pv, pi, x, id)) && better(x, id, bv, bi)) { bv = x; bi = id; }
        }
        wave_argmax(bv, bi);
        if (bi == INT32_MAX) break;
        if (lane == r) { kv_lane = bv; ki[r] = bi; }
        pv = bv; pi = bi;
        ++kept;
      }
    }
    // softmax over the kept set in fp64: x_j = z_j / T, e_j = exp(x_j - x_0)
    double x0 = double(lane_value(kv_lane, 0)) / double(a.T);
    double e = 0.0;
    if (lane < kept) e = exp(double(kv_lane) / double(a.T) - x0);
    // sum in kept order (lane 0 first), the same sequential order everywhere
    double tot = 0.0;
    for (int r = 0; r < kept; ++r) tot += lane_value(e, r);
    double p = (lane < kept) ? e / tot : 0.0;
    int n = kept;
    if (a.top_p < 1.0f) {
      double run = 0.0;
      n = kept;
      for (int r = 0; r < kept; ++r) {
        run += lane_value(p, r);
        if (run >= double(a.top_p)) { n = r + 1; break; }
      }
      if (n < 1) n = 1;
      double tot2 = 0.0;
      for (int r = 0; r < n; ++r) tot2 += lane_value(p, r);
      p = (lane < n) ? p / tot2 : 0.0;
    }
    if (lane < n) kp[lane] = p;
    if (lane == 0) a.ws.rkn[row] = n;
  }
}

// Kept probability, in the row whose kept list lane s holds as (kid, kpd)
// for s < nd, of the token `tok` this lane asks for (0 when not kept).
__device__ __forceinline__ double kept_lookup(int tok, int kid, double kpd, int nd) {
  double q = 0.0;
  for (int s = 0; s < nd; ++s) {
    const int ts = lane_value(kid, s);
    const double ps = lane_value(kpd, s);
    if (ts == tok) q = ps;
  }
  return q;
}

__device__ __forceinline__ double kept_prob(const VerifyArgs& a, int row, int tok) {
  int n = a.ws.rkn[row];
  const int* ki = a.ws.rki + size_t(row) * TOPK_MAX;
  const double* kp = a.ws.rkp + size_t(row) * TOPK_MAX;
  for (int j = 0; j < n; ++j)
    if (ki[j] == tok) return kp[j];
  return 0.0;
}

constexpr int DT = 1024;  // threads of the decision workgroup (16 waves)

// One wave per (request, row): the row's statistics records merged, and with
// a top-k filter its kept list (k rounds of a wave-wide argmax).  Spread over
// the whole chip rather than one workgroup per request.
__global__ __launch_bounds__(64) void vb_merge_rows(VerifyArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char mr_lds[];  // [nrec * k] values, then indices
  const int b = blockIdx.x, lane = threadIdx.x, j = blockIdx.y;
  const ReqRows rr = req_rows(a, b);
  if (!rr.ok) return;
  const int G = rr.G;
  const bool drafts = a.n_rows > a.n_trows;
  const int n_my = (G + 1) + (drafts ? G : 0);
  if (j >= n_my) return;
  const int row = j <= G ? rr.t0 + j : a.n_trows + rr.d0 + (j - G - 1);
  size_t slot0;
  const int nrec = row_records(a, row, slot0);
  float* s_v = reinterpret_cast<float*>(mr_lds);
  merge_row(a, row, lane, s_v, reinterpret_cast<int*>(s_v + nrec * a.topk));
}

__global__ __launch_bounds__(DT) void vb_decide(VerifyArgs a) {
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const ReqRows rr = req_rows(a, b);
  if (!rr.ok) {
    if (t == 0) a.tau[b] = -1;
    return;
  }
  const int G = rr.G;
  const bool drafts = a.n_rows > a.n_trows;
  // rows of this request: G+1 target rows, then G draft rows when present
  if (a.topk == 0) {
    // no kept lists: the rows' merges are short, done here
    const int n_my = (G + 1) + (drafts ? G : 0);
    for (int j = w; j < n_my; j += DT / 64) {
      const int row = j <= G ? rr.t0 + j : a.n_trows + rr.d0 + (j - G - 1);
      merge_row(a, row, lane);
    }
    __threadfence_block();
    __syncthreads();
  }
  // with a top-k filter the rows were merged by vb_merge_rows; with sampling, P(d) and Q(d) of
  // each drafted token from its rows' kept lists, one wave per position
  __shared__ double s_pq[2 * 64];  // [position] P(d), then [G + position] Q(d)
  if (!a.greedy) {
    for (int i = w; i < G; i += DT / 64) {
      const int d = a.dtok[rr.d0 + i];
      const int trow = rr.t0 + i, drow = a.n_trows + rr.d0 + i;
      const int nt = a.ws.rkn[trow], nd = a.ws.rkn[drow];
      const int kit = lane < nt ? a.ws.rki[size_t(trow) * TOPK_MAX + lane] : -1;
      const double kpt = lane < nt ? a.ws.rkp[size_t(trow) * TOPK_MAX + lane] : 0.0;
      const int kid = lane < nd ? a.ws.rki[size_t(drow) * TOPK_MAX + lane] : -2;
      const double kpd = lane < nd ? a.ws.rkp[size_t(drow) * TOPK_MAX + lane] : 0.0;
      const unsigned long long ft = __ballot(lane < nt && kit == d);
      const unsigned long long fd = __ballot(lane < nd && kid == d);
      if (lane == 0) {
        s_pq[i] = ft ? lane_value(kpt, __ffsll((long long)ft) - 1) : 0.0;
        s_pq[G + i] = fd ? lane_value(kpd, __ffsll((long long)fd) - 1) : 0.0;
      }
    }
  }
  __syncthreads();
  if (!a.greedy && a.beta) {
    // label of position i: sum over P's kept support of min(P, Q), in the
    // order of P's kept list; one wave per position
    for (int i = w; i < G; i += DT / 64) {
      const int trow = rr.t0 + i, drow = a.n_trows + rr.d0 + i;
      const int nt = a.ws.rkn[trow], nd = a.ws.rkn[drow];
      const int kit = lane < nt ? a.ws.rki[size_t(trow) * TOPK_MAX + lane] : -1;
      const double kpt = lane < nt ? a.ws.rkp[size_t(trow) * TOPK_MAX + lane] : 0.0;
      const int kid = lane < nd ? a.ws.rki[size_t(drow) * TOPK_MAX + lane] : -2;
      const double kpd = lane < nd ? a.ws.rkp[size_t(drow) * TOPK_MAX + lane] : 0.0;
      const double q = kept_lookup(kit, kid, kpd, nd);
      const double m = fmin(kpt, q);
      double sm = 0.0;
      for (int s2 = 0; s2 < nt; ++s2) sm += lane_value(m, s2);
      if (lane == 0) a.beta[rr.d0 + i] = float(sm);
    }
  }
  if (w != 0) return;

  // decisions, one lane per drafted position (G <= 64)
  bool acc = false;
  float ratio = 0.f;
  int d = -1;
  if (lane < G) {
    d = a.dtok[rr.d0 + lane];
    const int trow = rr.t0 + lane;
    const int drow = a.n_trows + rr.d0 + lane;
    if (a.greedy) {
      acc = (d == a.ws.rarg[trow]);
      ratio = acc ? 1.f : 0.f;
      if (a.beta) a.beta[rr.d0 + lane] = a.ws.rarg[trow] == a.ws.rarg[drow] ? 1.f : 0.f;
    } else {
      double p = 0.0, q = 0.0;
      if (d >= 0 && d < a.V) {
        p = s_pq[lane];      // target row of position lane
        q = s_pq[G + lane];  // draft row of position lane
      }
      float p32 = float(p), q32 = float(q);
      ratio = p32 / q32;
      float u = a.uni[(size_t(rr.t0) + lane) * 2];
      acc = u < ratio;
    }
    if (a.ratio) a.ratio[rr.d0 + lane] = ratio;
  }
  unsigned long long rej = __ballot(lane < G && !acc);
  int tau = rej ? __ffsll((long long)rej) - 1 : G;
  if (lane == 0) a.tau[b] = tau;
  for (int i = lane; i <= G; i += 64) {
    if (i < tau) a.out[rr.t0 + i] = a.dtok[rr.d0 + i];
    else if (i > tau) a.out[rr.t0 + i] = -1;
  }
  const int trow = rr.t0 + tau;
  if (a.greedy) {
    if (lane == 0) {
      a.out[rr.t0 + tau] = a.ws.rarg[trow];
      if (a.margin) a.margin[b] = INFINITY;
    }
    return;
  }
  // top-k: draw over the kept support (full-vocabulary sampling runs
  // vb_decide_sums instead of this kernel)
  const float u2 = a.uni[(size_t(rr.t0) + tau) * 2 + 1];
  // draw over P's kept support in vocabulary order, the whole wave: lane s
  // holds kept entry s; its rank by index orders the sequential sums
  const int n = a.ws.rkn[trow];
  const int idx = lane < n ? a.ws.rki[size_t(trow) * TOPK_MAX + lane] : INT32_MAX;
  const double pw = lane < n ? a.ws.rkp[size_t(trow) * TOPK_MAX + lane] : 0.0;
  int rank = 0;
  for (int s2 = 0; s2 < n; ++s2) rank += lane_value(idx, s2) < idx;
  double wt = pw;
  if (tau < G) {
    const int drow = a.n_trows + rr.d0 + tau;
    const int nd = a.ws.rkn[drow];
    const int kid = lane < nd ? a.ws.rki[size_t(drow) * TOPK_MAX + lane] : -2;
    const double kpd = lane < nd ? a.ws.rkp[size_t(drow) * TOPK_MAX + lane] : 0.0;
    const double r = pw - kept_lookup(idx, kid, kpd, nd);
    wt = r > 0.0 ? r : 0.0;
  }
  // the lane holding rank k
  auto at_rank = [&](int k2) { return __ffsll((long long)__ballot(lane < n && rank == k2)) - 1; };
  double Z = 0.0;
  for (int k2 = 0; k2 < n; ++k2) Z += lane_value(wt, at_rank(k2));
  if (tau < G && Z == 0.0) {
    wt = pw;  // the residual vanished: draw from P itself
    for (int k2 = 0; k2 < n; ++k2) Z += lane_value(wt, at_rank(k2));
  }
  const double tgt = double(u2) * Z;
  int pick = -1;
  double run = 0.0, mg = 0.0;
  for (int k2 = 0; k2 < n; ++k2) {
    const double prev = run;
    run += lane_value(wt, at_rank(k2));
    if (run > tgt) { pick = k2; mg = fmin(tgt - prev, run - tgt); break; }
  }
  if (pick < 0) {
    for (int k2 = n - 1; k2 >= 0; --k2)
      if (lane_value(wt, at_rank(k2)) > 0.0) { pick = k2; break; }
    if (pick < 0) pick = n - 1;
    mg = 0.0;
  }
  const int tok = lane_value(idx, at_rank(pick));
  if (lane == 0) {
    a.out[rr.t0 + tau] = tok;
    if (a.margin) a.margin[b] = float(mg);
  }
}

__device__ __forceinline__ DrawRow job_row(const VerifyArgs& a, int b, const DrawJob& j) {
  DrawRow r;
  const ReqRows rr = req_rows(a, b);
  r.zt = a.zt + size_t(rr.t0 + j.pos) * a.V;
  r.zd = j.kind == JOB_RESID ? a.zd + size_t(rr.d0 + j.pos) * a.V : nullptr;
  r.mt = j.mt;
  r.st = j.st;
  r.md = j.md;
  r.sd = j.sd;
  return r;
}

// Eight sums over the wave at once: lane 8 j + i (i < 8) ends with the sum of
// v[j] over all 64 lanes.  Three halving exchanges (each lane keeps the half
// of its values its half of the wave owns) and three plain butterfly steps:
// 14 exchanges of doubles instead of 48 for eight separate reductions.
__device__ __forceinline__ double wave_sum8(const double (&v)[8]) {
  const int lane = threadIdx.x & 63;
  const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
  double k4[4], k2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) k4[i] = (h5 ? v[i + 4] : v[i]) + __shfl_xor(h5 ? v[i] : v[i + 4], 32);
#pragma unroll
  for (int i = 0; i < 2; ++i) k2[i] = (h4 ? k4[i + 2] : k4[i]) + __shfl_xor(h4 ? k4[i] : k4[i + 2], 16);
  double k1 = (h3 ? k2[1] : k2[0]) + __shfl_xor(h3 ? k2[0] : k2[1], 8);
  k1 += __shfl_xor(k1, 4);
  k1 += __shfl_xor(k1, 2);
  k1 += __shfl_xor(k1, 1);
  return k1;
}

// Full-vocabulary sampling, pass 2: workgroup (c, b) merges request b's
// 2G + 1 rows, runs the accept chain (every workgroup of the request reaches
// the same decision from the same records), and sums the draw weights of
// chunk c of the row pair at the first rejection (or of the extra target
// row).  Workgroup (0, b) also writes tau, the accepted tokens, the ratios,
// the row statistics and the draw job.  The draft logits at the drafted
// tokens are loaded before the merge, which they do not depend on.
template <bool VEC>
__global__ __launch_bounds__(VT) void vb_decide_sums(VerifyArgs a) {
  __shared__ float s_m[2 * 64 + 1];
  __shared__ int s_i[2 * 64 + 1];
  __shared__ double s_s[2 * 64 + 1];
  __shared__ double s_d[4];
  __shared__ int s_tau;
  const int b = blockIdx.y, c = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const ReqRows rr = req_rows(a, b);
  if (!rr.ok) {
    if (c == 0 && t == 0) {
      a.tau[b] = -1;
      DrawJob jb = {};
      jb.kind = JOB_NONE;
      a.ws.job[b] = jb;
    }
    return;
  }
  const int G = rr.G;
  int d = -1;
  float zt_d = 0.f, zd_d = 0.f, u = 0.f;
  if (w == 0 && lane < G) {
    d = a.dtok[rr.d0 + lane];
    u = a.uni[(size_t(rr.t0) + lane) * 2];
    if (d >= 0 && d < a.V) {
      zt_d = a.zt[size_t(rr.t0 + lane) * a.V + d];
      zd_d = a.zd[size_t(rr.d0 + lane) * a.V + d];
    }
  }
  // rows j = 0..G: target rows, j = G + 1..2G: draft rows; thread j merges
  // row j's few records in record order, so all rows' loads are in flight
  // together
  const int n_my = 2 * G + 1;
  if (t < n_my) {
    const int row = t <= G ? rr.t0 + t : a.n_trows + rr.d0 + (t - G - 1);
    size_t slot0;
    const int nrec = row_records(a, row, slot0);
    float v = -INFINITY;
    int i = INT32_MAX;
    for (int r = 0; r < nrec; ++r) {
      const float cv = a.ws.cmax[slot0 + r];
      const int ci = a.ws.carg[slot0 + r];
      if (better(cv, ci, v, i)) { v = cv; i = ci; }
    }
    double S = 0.0;
    if (v != -INFINITY)
      for (int r = 0; r < nrec; ++r) {
        const float cm = a.ws.cmax[slot0 + r];
        if (cm != -INFINITY) S += a.ws.csum[slot0 + r] * exp2(double(cm - v) * double(a.c2));
      }
    s_m[t] = v;
    s_i[t] = i;
    s_s[t] = S;
  }
  __syncthreads();
  if (w == 0) {
    bool acc = false;
    float ratio = 0.f;
    if (lane < G) {
      double p = 0.0, q = 0.0;
      if (d >= 0 && d < a.V) {
        const double Tt = double(a.T);
        p = exp(double(zt_d) / Tt - double(s_m[lane]) / Tt) / s_s[lane];
        q = exp(double(zd_d) / Tt - double(s_m[G + 1 + lane]) / Tt) / s_s[G + 1 + lane];
      }
      const float p32 = float(p), q32 = float(q);
      ratio = p32 / q32;
      acc = u < ratio;
    }
    const unsigned long long rej = __ballot(lane < G && !acc);
    const int tau = rej ? __ffsll((long long)rej) - 1 : G;
    if (lane == 0) s_tau = tau;
    if (c == 0) {
      if (lane < G && a.ratio) a.ratio[rr.d0 + lane] = ratio;
      if (lane == 0) a.tau[b] = tau;
      for (int i = lane; i <= G; i += 64) {
        if (i < tau) a.out[rr.t0 + i] = a.dtok[rr.d0 + i];
        else if (i > tau) a.out[rr.t0 + i] = -1;
      }
      for (int j = lane; j < n_my; j += 64) {
        const int row = j <= G ? rr.t0 + j : a.n_trows + rr.d0 + (j - G - 1);
        a.ws.rmax[row] = s_m[j];
        a.ws.rarg[row] = s_i[j];
        a.ws.rsum[row] = s_s[j];
      }
      if (lane == 0) {
        DrawJob jb;
        jb.pos = tau;
        jb.kind = tau < G ? JOB_RESID : JOB_BONUS;
        jb.u2 = a.uni[(size_t(rr.t0) + tau) * 2 + 1];
        jb.mt = s_m[tau];
        jb.st = float(1.0 / s_s[tau]);
        jb.md = tau < G ? s_m[G + 1 + tau] : 0.f;
        jb.sd = tau < G ? float(1.0 / s_s[G + 1 + tau]) : 0.f;
        jb.pad = 0.f;
        a.ws.job[b] = jb;
      }
    }
  }
  __syncthreads();
  const int tau = s_tau;
  const bool resid = tau < G;
  DrawRow r;
  r.zt = a.zt + size_t(rr.t0 + tau) * a.V;
  r.zd = resid ? a.zd + size_t(rr.d0 + tau) * a.V : nullptr;
  r.mt = s_m[tau];
  r.st = float(1.0 / s_s[tau]);
  r.md = resid ? s_m[G + 1 + tau] : 0.f;
  r.sd = resid ? float(1.0 / s_s[G + 1 + tau]) : 0.f;
  const int start = c * VCH;
  float xt[VPT], xd[VPT];
  load_chunk<VEC>(r.zt, start, a.V, t, xt);
  if (resid) load_chunk<VEC>(r.zd, start, a.V, t, xd);
  if constexpr (VEC) {
    // run sums (wave w, slot group j: logits 1024 j + 256 w .. + 255 of the
    // chunk), then the chunk sum as their sum in run order
    __shared__ double s_sub[NSUB];
    double ls[VPT / 4];
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j) {
      ls[j] = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = start + slot_offset<true>(4 * j + q, t);
        if (e < a.V) ls[j] += double(draw_weight(r, a.c2, xt[4 * j + q], resid ? xd[4 * j + q] : 0.f, resid));
      }
    }
    const double sj = wave_sum8(ls);  // lane 8 j: the wave's sum of slot group j
    if ((lane & 7) == 0) s_sub[4 * (lane >> 3) + w] = sj;
    __syncthreads();
    if (t < NSUB) a.ws.jsub[(size_t(b) * a.nch + c) * NSUB + t] = s_sub[t];
    if (t == 0) {
      double sum = 0.0;
      for (int k = 0; k < NSUB; ++k) sum += s_sub[k];
      a.ws.jsum[size_t(b) * a.nch + c] = sum;
    }
  } else {
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = start + slot_offset<VEC>(j, t);
      if (e < a.V) sum += double(draw_weight(r, a.c2, xt[j], resid ? xd[j] : 0.f, resid));
    }
    sum = block_sum_f64(sum, s_d);
    if (t == 0) a.ws.jsum[size_t(b) * a.nch + c] = sum;
  }
  if (a.beta) {
    // confidence labels: this chunk's sum of min(P_i, Q_i) for every drafted
    // position i of the request (vb_draw_pick adds the chunks up)
    for (int i = 0; i < G; ++i) {
      DrawRow rb;
      rb.zt = a.zt + size_t(rr.t0 + i) * a.V;
      rb.zd = a.zd + size_t(rr.d0 + i) * a.V;
      rb.mt = s_m[i];
      rb.st = float(1.0 / s_s[i]);
      rb.md = s_m[G + 1 + i];
      rb.sd = float(1.0 / s_s[G + 1 + i]);
      load_chunk<VEC>(rb.zt, start, a.V, t, xt);
      load_chunk<VEC>(rb.zd, start, a.V, t, xd);
      double sm = 0.0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int e = start + slot_offset<VEC>(j, t);
        if (e < a.V) {
          const float pp = exp2_hw((xt[j] - rb.mt) * a.c2) * rb.st;
          const float qq = exp2_hw((xd[j] - rb.md) * a.c2) * rb.sd;
          sm += double(fminf(pp, qq));
        }
      }
      sm = block_sum_f64(sm, s_d);
      if (t == 0) a.ws.jbeta[size_t(rr.d0 + i) * a.nch + c] = sm;
    }
  }
}

// The thread's 32 consecutive logits of a row, starting at element e0.
__device__ __forceinline__ void load_run(const float* __restrict__ row, int e0, int V, bool vec, float (&x)[VPT]) {
  if (vec && e0 + VPT <= V) {
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(row + e0 + 4 * j);
      x[4 * j] = f.x; x[4 * j + 1] = f.y; x[4 * j + 2] = f.z; x[4 * j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPT; ++j) x[j] = (e0 + j < V) ? row[e0 + j] : -INFINITY;
  }
}

// Exclusive prefix sum over the workgroup's threads (thread order), fp64.
__device__ __forceinline__ double block_exclusive_scan(double v, double* s_w /* [4] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  double base = 0.0;
  for (int k = 0; k < w; ++k) base += s_w[k];
  return base + inc - v;
}

// Scan one chunk for the first running sum above tgt.  Returns the vocabulary
// index (or INT32_MAX) and the margin through the shared outputs.
template <bool VEC, bool USE_P>
__device__ __forceinline__ void scan_chunk(const VerifyArgs& a, const DrawRow& r, bool resid, int c, double base,
                                           double tgt, int* s_pick, double* s_mg, double* s_w) {
  constexpr bool use_p = USE_P;
  const int t = threadIdx.x;
  const int start = c * VCH + t * VPT;
  const bool vec = VEC;
  float xt[VPT], xd[VPT];
  load_run(r.zt, start, a.V, vec, xt);
  if (resid && !use_p) load_run(r.zd, start, a.V, vec, xd);
  float wv[VPT];
  double mine = 0.0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    float wgt = 0.f;
    if (start + j < a.V) wgt = use_p ? draw_weight(r, a.c2, xt[j], 0.f, false)
                                     : draw_weight(r, a.c2, xt[j], resid ? xd[j] : 0.f, resid);
    wv[j] = wgt;
    mine += double(wgt);
  }
  double run = base + block_exclusive_scan(mine, s_w);
  int pick = INT32_MAX;
  double mg = 0.0;
  for (int j = 0; j < VPT; ++j) {
    const double prev = run;
    run += double(wv[j]);
    if (run > tgt) { pick = start + j; mg = fmin(tgt - prev, run - tgt); break; }
  }
  // lowest pick wins
  int best = pick;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o));
  __syncthreads();
  if (t == 0) *s_pick = INT32_MAX;
  __syncthreads();
  if ((t & 63) == 0) atomicMin(s_pick, best);
  __syncthreads();
  if (pick != INT32_MAX && pick == *s_pick) *s_mg = mg;
  __syncthreads();
}

// last x in chunk c with a positive weight (INT32_MAX if none)
__device__ int last_positive(const VerifyArgs& a, const DrawRow& r, bool resid, bool use_p, int c,
                             int* s_pick) {
  const int t = threadIdx.x;
  int best = -1;
  for (int j = 0; j < VPT; ++j) {
    int e = c * VCH + t * VPT + j;
    if (e < a.V) {
      float wgt = use_p ? draw_weight(r, a.c2, r.zt[e], 0.f, false)
                        : draw_weight(r, a.c2, r.zt[e], resid ? r.zd[e] : 0.f, resid);
      if (wgt > 0.f) best = e;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o));
  __syncthreads();
  if (t == 0) *s_pick = -1;
  __syncthreads();
  if ((t & 63) == 0) atomicMax(s_pick, best);
  __syncthreads();
  return *s_pick;
}

// Shared state of the draw: the scan's per-wave totals, the pick and its
// margin, the crossing chunk.
struct PickLds {
  double ex[4];
  double d[4];
  double mg;
  int pick;
  int chunk;
};

// Every case the common path of vb_draw_pick does not finish: vocabularies
// of more than VT chunks (the sums are walked in order), a residual whose
// weights all rounded to zero (the draw then uses P), and no crossing found
// (the last positive weight wins).  Out of line so that the common path stays
// short in the instruction cache.  For nch <= VT, Z, chunk and base_c come
// from the common path's scan.
template <bool VEC>
__device__ __forceinline__ void draw_pick_rest(const VerifyArgs& a, const DrawRow& r, bool resid, int b, int pos,
                                            float u2, double Z, int chunk, double base_c, PickLds* sh) {
  const int t = threadIdx.x;
  const double* cs = a.ws.jsum + size_t(b) * a.nch;
  bool use_p = false;
  if (a.nch > VT) {
    Z = 0.0;
    for (int c = 0; c < a.nch; ++c) Z += cs[c];
  }
  if (resid && Z == 0.0) {
    // every residual weight rounded to zero: draw from P instead
    use_p = true;
    chunk = -1;
    double tot_p = 0.0;
    for (int c = 0; c < a.nch; ++c) {
      double s = 0.0;
      for (int j = 0; j < VPT; ++j) {
        int e = c * VCH + t * VPT + j;
        if (e < a.V) s += double(draw_weight(r, a.c2, r.zt[e], 0.f, false));
      }
      tot_p += block_sum_f64(s, sh->d);
    }
    Z = tot_p;
  }
  const double tgt = double(u2) * Z;
  if (a.nch > VT && !use_p) {
    // chunk holding the crossing, walking the sums in order
    __syncthreads();
    if (t == 0) {
      double run = 0.0;
      int ch = -1;
      for (int c = 0; c < a.nch; ++c) {
        run += cs[c];
        if (run > tgt) { ch = c; break; }
      }
      sh->chunk = ch;
    }
    __syncthreads();
    chunk = sh->chunk;
    base_c = 0.0;
    if (chunk >= 0)
      for (int c = 0; c < chunk; ++c) base_c += cs[c];
  }
  int pick = INT32_MAX;
  double mg = 0.0;
  if (!use_p && chunk >= 0) {
    scan_chunk<VEC, false>(a, r, resid, chunk, base_c, tgt, &sh->pick, &sh->mg, sh->ex);
    pick = sh->pick;
    mg = sh->mg;
    if (pick == INT32_MAX) {
      pick = last_positive(a, r, resid, false, chunk, &sh->pick);
      mg = 0.0;
    }
  } else if (use_p) {
    // P-weights: walk chunk by chunk
    double run = 0.0;
    for (int c = 0; c < a.nch && pick == INT32_MAX; ++c) {
      scan_chunk<VEC, true>(a, r, resid, c, run, tgt, &sh->pick, &sh->mg, sh->ex);
      if (sh->pick != INT32_MAX) { pick = sh->pick; mg = sh->mg; break; }
      double s = 0.0;
      for (int j = 0; j < VPT; ++j) {
        int e = c * VCH + t * VPT + j;
        if (e < a.V) s += double(draw_weight(r, a.c2, r.zt[e], 0.f, false));
      }
      run += block_sum_f64(s, sh->d);
    }
  }
  if (pick == INT32_MAX || pick < 0) {
    // no crossing anywhere: the last x with a positive weight
    int last = -1;
    for (int c = a.nch - 1; c >= 0 && last < 0; --c) last = last_positive(a, r, resid, use_p, c, &sh->pick);
    pick = last >= 0 ? last : a.V - 1;
    mg = 0.0;
  }
  if (t == 0) {
    a.out[req_rows(a, b).t0 + pos] = pick;
    if (a.margin) a.margin[b] = float(mg);
  }
}

// The run of SUBLEN logits that holds the crossing, scanned by one wave:
// lane l takes logits 4 l .. 4 l + 3 of the run, an inclusive scan over the
// lanes gives each lane's running start.  Returns the pick (INT32_MAX when
// rounding put the crossing outside the run) and its margin.
__device__ __forceinline__ int scan_run(const VerifyArgs& a, const DrawRow& r, bool resid, int e0, double base,
                                        double tgt, double& mg) {
  const int lane = threadIdx.x & 63;
  const int e = e0 + 4 * lane;
  float wv[4] = {0.f, 0.f, 0.f, 0.f};
  if (e < a.V) {  // V % 4 == 0: the whole group of four is in the row
    const float4 ft = *reinterpret_cast<const float4*>(r.zt + e);
    float4 fd = make_float4(0.f, 0.f, 0.f, 0.f);
    if (resid) fd = *reinterpret_cast<const float4*>(r.zd + e);
    wv[0] = draw_weight(r, a.c2, ft.x, fd.x, resid);
    wv[1] = draw_weight(r, a.c2, ft.y, fd.y, resid);
    wv[2] = draw_weight(r, a.c2, ft.z, fd.z, resid);
    wv[3] = draw_weight(r, a.c2, ft.w, fd.w, resid);
  }
  double mine = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) mine += double(wv[q]);
  double inc = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  double run = base + (inc - mine);
  int pick = INT32_MAX;
  double m = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double prev = run;
    run += double(wv[q]);
    if (pick == INT32_MAX && run > tgt) { pick = e + q; m = fmin(tgt - prev, run - tgt); }
  }
  const unsigned long long hit = __ballot(pick != INT32_MAX);
  if (!hit) return INT32_MAX;
  const int src = __ffsll((long long)hit) - 1;
  mg = __shfl(m, src);
  return __shfl(pick, src);
}

// One workgroup per request: the chunk sums of the draw weights give Z and,
// through an exclusive scan in chunk order, the chunk whose running end first
// exceeds u' Z.  Vector rows then walk that chunk's run sums in order and scan
// the one run holding the crossing; other rows scan the whole chunk.  What
// this does not settle (rounding at a boundary, residual weights that all
// rounded to zero, very large vocabularies) goes to draw_pick_rest.
template <bool VEC>
__global__ __launch_bounds__(VT) void vb_draw_pick(VerifyArgs a) {
  __shared__ PickLds sh;
  __shared__ double s_sub[VEC ? PICK_FAST_NCH * NSUB : 1];
  __shared__ int s_done;
  const int b = blockIdx.x, t = threadIdx.x;
  const ReqRows rr = req_rows(a, b);
  if (!rr.ok) return;
  if (a.beta && t < rr.G) {
    // confidence label of drafted position t: its chunk sums in chunk order
    const double* pb = a.ws.jbeta + size_t(rr.d0 + t) * a.nch;
    double sm = 0.0;
    for (int c = 0; c < a.nch; ++c) sm += pb[c];
    a.beta[rr.d0 + t] = float(sm);
  }
  // the job, this thread's chunk sum and the run sums are loaded together
  const DrawJob jb = a.ws.job[b];
  const double* cs = a.ws.jsum + size_t(b) * a.nch;
  const double cs_t = t < a.nch ? cs[t] : 0.0;
  const bool fast_runs = VEC && a.nch <= PICK_FAST_NCH;
  if (fast_runs) {
    const double* sub = a.ws.jsub + size_t(b) * a.nch * NSUB;
    for (int i = t; i < a.nch * NSUB; i += VT) s_sub[i] = sub[i];
  }
  const int pos = jb.pos;
  const bool resid = jb.kind == JOB_RESID;
  const DrawRow r = job_row(a, b, jb);
  const float u2 = jb.u2;
  double Z = 0.0, base_c = 0.0;
  int chunk = -1;
  if (a.nch <= VT) {
    const double excl = block_exclusive_scan(cs_t, sh.ex);
    if (t == a.nch - 1) sh.mg = excl + cs_t;  // total, in the scan's order
    if (t == 0) { sh.chunk = INT32_MAX; s_done = 0; }
    __syncthreads();
    Z = sh.mg;
    if (!(resid && Z == 0.0)) {
      const double tgt0 = double(u2) * Z;
      if (t < a.nch && excl + cs_t > tgt0) atomicMin(&sh.chunk, t);
    }
    __syncthreads();
    if (sh.chunk != INT32_MAX && sh.chunk == t) sh.mg = excl;
    __syncthreads();
    chunk = sh.chunk == INT32_MAX ? -1 : sh.chunk;
    base_c = chunk >= 0 ? sh.mg : 0.0;
    __syncthreads();
    const double tgt = double(u2) * Z;
    if (chunk >= 0 && fast_runs) {
      if (t < 64) {
        // the chunk's runs in order: the first whose running end exceeds tgt
        int k = -1;
        double bsub = 0.0;
        if (t == 0) {
          double run = base_c;
          for (int i = 0; i < NSUB; ++i) {
            const double prev = run;
            run += s_sub[chunk * NSUB + i];
            if (run > tgt) { k = i; bsub = prev; break; }
          }
        }
        k = __shfl(k, 0);
        bsub = __shfl(bsub, 0);
        if (k >= 0) {
          const int e0 = chunk * VCH + (k >> 2) * (4 * VT) + (k & 3) * SUBLEN;
          double mg = 0.0;
          const int pick = scan_run(a, r, resid, e0, bsub, tgt, mg);
          if (pick != INT32_MAX && t == 0) {
            a.out[rr.t0 + pos] = pick;
            if (a.margin) a.margin[b] = float(mg);
            s_done = 1;
          }
        }
      }
      __syncthreads();
      if (s_done) return;
    } else if (chunk >= 0) {
      scan_chunk<VEC, false>(a, r, resid, chunk, base_c, tgt, &sh.pick, &sh.mg, sh.ex);
      const int pick = sh.pick;
      if (pick != INT32_MAX) {
        if (t == 0) {
          a.out[rr.t0 + pos] = pick;
          if (a.margin) a.margin[b] = float(sh.mg);
        }
        return;
      }
    }
  }
  draw_pick_rest<VEC>(a, r, resid, b, pos, u2, Z, chunk, base_c, &sh);
}

// probabilities for the test path: full rows of the (filtered) P and Q
__global__ __launch_bounds__(VT) void vb_write_probs(VerifyArgs a) {
  const int row = blockIdx.x / a.nch;
  const int c = blockIdx.x - row * a.nch;
  const int t = threadIdx.x;
  float* dst;
  if (row < a.n_trows) {
    if (!a.tprob) return;
    dst = a.tprob + size_t(row) * a.V;
  } else {
    if (!a.dprob) return;
    dst = a.dprob + size_t(row - a.n_trows) * a.V;
  }
  const float* z = row_ptr(a, row);
  const float m = a.ws.rmax[row];
  const bool filt = a.topk > 0 && !a.greedy;
  const float inv = float(1.0 / a.ws.rsum[row]);
  for (int j = 0; j < VPT; ++j) {
    int e = c * VCH + j * VT + t;
    if (e >= a.V) break;
    float p;
    if (filt) p = float(kept_prob(a, row, e));
    else p = exp2_hw((z[e] - m) * a.c2) * inv;
    dst[e] = p;
  }
}

// -------------------------------------------------------------------------
// host side
// -------------------------------------------------------------------------
static inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

struct VerifyLayout {
  size_t cmax, carg, csum, ctv, cti, rmax, rarg, rsum, rkn, rki, rkp, job, jsum, jsub, jbeta, total;
};

// n_trows target rows (B * (G + 1) without a row map), as many minus B draft rows
static VerifyLayout verify_layout(int B, int n_trows, int V, int top_k, bool beta) {
  VerifyLayout L{};
  const size_t nch = (size_t(V) + VCH - 1) / VCH;
  const size_t rows = 2 * size_t(n_trows) - size_t(B);
  const size_t n_draft = size_t(n_trows) - size_t(B);
  // record slots: row + workgroup, with at most min(rows * nch, STATS_GRID)
  // workgroups in pass 1
  const size_t rc = rows + (rows * nch < size_t(STATS_GRID) ? rows * nch : size_t(STATS_GRID));
  const size_t k = top_k > 0 ? size_t(top_k) : 0;
  size_t o = 0;
  L.cmax = o; o += al(rc * 4);
  L.carg = o; o += al(rc * 4);
  L.csum = o; o += al(rc * 8);
  L.ctv = o; o += al(rc * k * 4);
  L.cti = o; o += al(rc * k * 4);
  L.rmax = o; o += al(rows * 4);
  L.rarg = o; o += al(rows * 4);
  L.rsum = o; o += al(rows * 8);
  L.rkn = o; o += al(rows * 4);
  L.rki = o; o += al(k ? rows * TOPK_MAX * 4 : 0);
  L.rkp = o; o += al(k ? rows * TOPK_MAX * 8 : 0);
  L.job = o; o += al(size_t(B) * sizeof(DrawJob));
  L.jsum = o; o += al(size_t(B) * nch * 8);
  L.jsub = o; o += al(size_t(B) * nch * NSUB * 8);
  L.jbeta = o; o += al(beta && top_k == 0 ? n_draft * nch * 8 : 0);
  L.total = o;
  return L;
}

size_t verify_ws_bytes(int B, int n_trows, int V, int top_k, bool beta) {
  if (B <= 0) return 0;
  return verify_layout(B, n_trows, V, top_k, beta).total;
}

hipError_t launch_verify(const float* zt, const float* zd, const int* dtok, const float* uni,
                         const int* row_cu, int B, int n_trows, int G, int V, float temperature, int top_k,
                         float top_p, int* tau, int* out, float* tprob, float* dprob, float* ratio, float* margin,
                         float* beta, void* ws, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const bool greedy = temperature == 0.0f;
  const int k = (!greedy && top_k > 0 && top_k < V) ? top_k : 0;
  VerifyLayout L = verify_layout(B, n_trows, V, k, beta != nullptr);
  char* w = static_cast<char*>(ws);
  VerifyArgs a{};
  a.zt = zt; a.zd = zd; a.dtok = dtok; a.uni = uni;
  a.B = B; a.G = G; a.V = V;
  a.nch = (V + VCH - 1) / VCH;
  a.n_trows = n_trows;
  a.row_cu = row_cu;
  const bool draft_rows = !greedy || dprob != nullptr || beta != nullptr;
  a.n_rows = a.n_trows + (draft_rows && zd ? n_trows - B : 0);
  a.T = greedy ? 1.0f : temperature;
  a.c2 = float(1.4426950408889634 / double(a.T));
  a.greedy = greedy;
  a.topk = k;
  a.top_p = greedy ? 1.0f : top_p;
  a.need_sum = (!greedy && k == 0) || (greedy && (tprob || dprob));
  a.tau = tau; a.out = out; a.tprob = tprob; a.dprob = dprob; a.ratio = ratio; a.margin = margin;
  a.beta = beta;
  a.ws.cmax = reinterpret_cast<float*>(w + L.cmax);
  a.ws.carg = reinterpret_cast<int*>(w + L.carg);
  a.ws.csum = reinterpret_cast<double*>(w + L.csum);
  a.ws.ctv = reinterpret_cast<float*>(w + L.ctv);
  a.ws.cti = reinterpret_cast<int*>(w + L.cti);
  a.ws.rmax = reinterpret_cast<float*>(w + L.rmax);
  a.ws.rarg = reinterpret_cast<int*>(w + L.rarg);
  a.ws.rsum = reinterpret_cast<double*>(w + L.rsum);
  a.ws.rkn = reinterpret_cast<int*>(w + L.rkn);
  a.ws.rki = reinterpret_cast<int*>(w + L.rki);
  a.ws.rkp = reinterpret_cast<double*>(w + L.rkp);
  a.ws.job = reinterpret_cast<DrawJob*>(w + L.job);
  a.ws.jsum = reinterpret_cast<double*>(w + L.jsum);
  a.ws.jsub = reinterpret_cast<double*>(w + L.jsub);
  a.ws.jbeta = reinterpret_cast<double*>(w + L.jbeta);

  const bool vec = (V & 3) == 0;
  const long long work = (long long)a.n_rows * a.nch;
  if (k > 0) {
    // top-k (sampling only, so no sums are needed): persistent workgroups
    // with equal runs of chunks, as below
    long long cpw = (work + STATS_GRID - 1) / STATS_GRID;
    if (cpw < 1) cpw = 1;
    a.cpw = int(cpw);
    const unsigned grid = unsigned((work + cpw - 1) / cpw);
    if (vec) hipLaunchKernelGGL(vb_topk_stream<true>, dim3(grid), dim3(VT), 0, stream, a);
    else hipLaunchKernelGGL(vb_topk_stream<false>, dim3(grid), dim3(VT), 0, stream, a);
  } else {
    // at most STATS_GRID persistent workgroups with equal runs of chunks
    long long cpw = (work + STATS_GRID - 1) / STATS_GRID;
    if (cpw < 1) cpw = 1;
    a.cpw = int(cpw);
    const unsigned grid = unsigned((work + cpw - 1) / cpw);
    // the index of each row's maximum is needed by the greedy decision only
    if (greedy) {
      if (vec) hipLaunchKernelGGL((vb_stats_stream<true, true>), dim3(grid), dim3(VT), 0, stream, a);
      else hipLaunchKernelGGL((vb_stats_stream<false, true>), dim3(grid), dim3(VT), 0, stream, a);
    } else {
      if (vec) hipLaunchKernelGGL((vb_stats_stream<true, false>), dim3(grid), dim3(VT), 0, stream, a);
      else hipLaunchKernelGGL((vb_stats_stream<false, false>), dim3(grid), dim3(VT), 0, stream, a);
    }
  }
  if (!greedy && k == 0) {
    if (vec) hipLaunchKernelGGL(vb_decide_sums<true>, dim3(a.nch, B), dim3(VT), 0, stream, a);
    else hipLaunchKernelGGL(vb_decide_sums<false>, dim3(a.nch, B), dim3(VT), 0, stream, a);
    if (vec) hipLaunchKernelGGL(vb_draw_pick<true>, dim3(B), dim3(VT), 0, stream, a);
    else hipLaunchKernelGGL(vb_draw_pick<false>, dim3(B), dim3(VT), 0, stream, a);
  } else {
    if (k > 0) {
      // one wave per (request, row); LDS for a row's chunk lists (one record
      // per chunk with a top-k filter)
      const size_t lds = size_t(a.nch) * k * 8;
      hipLaunchKernelGGL(vb_merge_rows, dim3(B, 2 * a.G + 1), dim3(64), lds, stream, a);
    }
    hipLaunchKernelGGL(vb_decide, dim3(B), dim3(DT), 0, stream, a);
  }
  if (tprob || dprob)
    hipLaunchKernelGGL(vb_write_probs, dim3(unsigned(a.n_rows) * unsigned(a.nch)), dim3(VT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bd
