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
// Work item = (split, KV head g, request b).  Split 0 holds the K in-block
// keys; splits 1.. hold consecutive chunks of the visible context.  The
// item's query rows are the group's (n_q / n_kv) heads at all K block
// positions (row r = i * group + hh).  Each wave owns 16-row blocks; the key
// tile (64 keys) is staged once in LDS and shared by the four waves.
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
  int window, max_ctx, chunk, nsplit;  // nsplit includes the block split
  float sl2;                           // scale * log2(e)
  uint16_t* out;
  float* lse;
  float* wo;   // [B][n_kv][nsplit][R][HD]
  float* wml;  // [B][n_kv][nsplit][R][2]
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

template <int HD, int RB>
__global__ __launch_bounds__(AT) void attn_partial(AttnArgs a) {
  constexpr int LS = HD + 8;          // LDS row stride (elements)
  constexpr int PIECES = TK * HD / 8;  // 16-byte pieces per tile
  constexpr int PPT = PIECES / AT;     // per thread
  constexpr int NKS = HD / 32;         // k-steps of the score MFMA
  constexpr int NDB = HD / 16;         // dim blocks of the output MFMA
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TK * LS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[TK * LS];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lr = lane & 15, q4 = lane >> 4;

  int64_t cbase;
  int lo, hi;
  if (!visible(a, b, cbase, lo, hi)) return;

  const uint16_t* kp;
  const uint16_t* vp;
  int nkeys;
  const size_t kstride = size_t(a.n_kv) * HD;
  if (split == 0) {
    kp = a.kb + (size_t(b) * a.K * a.n_kv + g) * HD;
    vp = a.vb + (size_t(b) * a.K * a.n_kv + g) * HD;
    nkeys = a.K;
  } else {
    int s0 = lo + (split - 1) * a.chunk;
    if (s0 >= hi) return;
    nkeys = min(a.chunk, hi - s0);
    kp = a.kc + (size_t(cbase + s0) * a.n_kv + g) * HD;
    vp = a.vc + (size_t(cbase + s0) * a.n_kv + g) * HD;
  }

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

  const int ntiles = (nkeys + TK - 1) / TK;
  uint4 pk[PPT], pv[PPT];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int piece = t + p * AT;
      const int key = piece / (HD / 8), dc = piece - key * (HD / 8);
      const int kk = tile * TK + key;
      if (kk < nkeys) {
        pk[p] = *reinterpret_cast<const uint4*>(kp + size_t(kk) * kstride + dc * 8);
        pv[p] = *reinterpret_cast<const uint4*>(vp + size_t(kk) * kstride + dc * 8);
      } else {
        pk[p] = make_uint4(0, 0, 0, 0);
        pv[p] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  fetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int piece = t + p * AT;
      const int key = piece / (HD / 8), dc = piece - key * (HD / 8);
      *reinterpret_cast<uint4*>(&Ks[key * LS + dc * 8]) = pk[p];
      *reinterpret_cast<uint4*>(&Vs[key * LS + dc * 8]) = pv[p];
    }
    __syncthreads();
    if (tile + 1 < ntiles) fetch(tile + 1);
    const int nvalid = nkeys - tile * TK;

#pragma unroll
    for (int j = 0; j < RB; ++j) {
      if ((w + 4 * j) * 16 >= a.R) continue;
      // scores for 64 keys: 4 key blocks of 16
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
      // O^T += V^T P^T; V fragment: lane (dim = 16d + lr) gathers the same
      // 8 keys of the k-step that its P fragment holds
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pw[ks2 * 4], pw[ks2 * 4 + 1], pw[ks2 * 4 + 2], pw[ks2 * 4 + 3]));
        const int k0 = ks2 * 32 + q4 * 4;
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const int dim = d * 16 + lr;
          short8 vf;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            vf[r] = short(Vs[(k0 + r) * LS + dim]);
            vf[4 + r] = short(Vs[(k0 + 16 + r) * LS + dim]);
          }
          acc[j][d] = mfma16x16x32(__builtin_bit_cast(bf16x8, vf), pb, acc[j][d]);
        }
      }
    }
  }

  // partial results: unnormalised O, running max (exp2 domain), normaliser
  const size_t item = (size_t(b) * a.n_kv + g) * a.nsplit + split;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int row = (w + 4 * j) * 16 + lr;
    float l = l_run[j];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (row < a.R) {
      float* o = a.wo + (item * a.R + row) * HD;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
        *reinterpret_cast<floatx4*>(o + d * 16 + q4 * 4) = acc[j][d];
      if (q4 == 0) {
        a.wml[(item * a.R + row) * 2] = m_run[j];
        a.wml[(item * a.R + row) * 2 + 1] = l;
      }
    }
  }
}

template <int HD>
__global__ __launch_bounds__(AT) void attn_merge(AttnArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  int64_t cbase;
  int lo, hi;
  const bool ok = visible(a, b, cbase, lo, hi);
  const int nctx = ok ? (hi - lo + a.chunk - 1) / a.chunk : 0;
  const int ns = 1 + nctx;
  const size_t item0 = (size_t(b) * a.n_kv + g) * a.nsplit;
  for (int e = t; e < a.R * HD; e += AT) {
    const int row = e / HD, d = e - row * HD;
    const int i = row / a.group, hh = row - i * a.group;
    const size_t oidx = ((size_t(b) * a.K + i) * a.n_q + g * a.group + hh);
    if (!ok) {
      a.out[oidx * HD + d] = 0x7fc0;
      if (d == 0 && a.lse) a.lse[oidx] = NAN;
      continue;
    }
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.wml[((item0 + s) * a.R + row) * 2]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = a.wml[((item0 + s) * a.R + row) * 2];
      const float f = exp2f(ms - M);
      L += a.wml[((item0 + s) * a.R + row) * 2 + 1] * f;
      O += a.wo[((item0 + s) * a.R + row) * HD + d] * f;
    }
    a.out[oidx * HD + d] = f32_to_bf16(O / L);
    if (d == 0 && a.lse) a.lse[oidx] = (M + log2f(L)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------- host side
static inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

struct AttnPlan {
  int chunk, nsplit;
};

static AttnPlan attn_plan(int B, int n_kv, int max_ctx, int window) {
  const int vis = (window > 0 && max_ctx > window) ? window : max_ctx;
  const int tiles = (vis + TK - 1) / TK;
  const int items = B * n_kv;
  int target = (1536 + items - 1) / items;  // context splits per item
  if (target > 32) target = 32;
  if (target < 1) target = 1;
  int ct = (tiles + target - 1) / target;    // tiles per chunk
  if (ct < 2) ct = 2;
  AttnPlan p;
  p.chunk = ct * TK;
  p.nsplit = 1 + (vis + p.chunk - 1) / p.chunk;
  return p;
}

size_t attn_ws_bytes(int B, int K, int n_q, int n_kv, int hd, int max_ctx, int window) {
  if (B <= 0) return 0;
  AttnPlan p = attn_plan(B, n_kv, max_ctx, window);
  const size_t R = size_t(K) * (n_q / n_kv);
  const size_t items = size_t(B) * n_kv * p.nsplit;
  return al(items * R * hd * 4) + al(items * R * 2 * 4);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kb, const uint16_t* vb, const uint16_t* kc,
                       const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                       int64_t T_cap, int max_ctx, int B, int K, int n_q, int n_kv, int hd, int window,
                       float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  AttnPlan p = attn_plan(B, n_kv, max_ctx, window);
  AttnArgs a{};
  a.q = q; a.kb = kb; a.vb = vb; a.kc = kc; a.vc = vc;
  a.cache_base = cache_base; a.ctx_len = ctx_len; a.T_cap = T_cap;
  a.B = B; a.K = K; a.n_q = n_q; a.n_kv = n_kv; a.group = n_q / n_kv; a.R = K * a.group;
  a.window = window; a.max_ctx = max_ctx; a.chunk = p.chunk; a.nsplit = p.nsplit;
  const float sc = scale > 0.f ? scale : float(1.0 / sqrt(double(hd)));
  a.sl2 = float(double(sc) * 1.4426950408889634);
  a.out = out; a.lse = lse;
  const size_t R = size_t(a.R);
  const size_t items = size_t(B) * n_kv * p.nsplit;
  a.wo = static_cast<float*>(ws);
  a.wml = reinterpret_cast<float*>(static_cast<char*>(ws) + al(items * R * hd * 4));
  dim3 grid(p.nsplit, n_kv, B);
  const bool two = a.R > 64;
  if (hd == 128) {
    if (two) hipLaunchKernelGGL((attn_partial<128, 2>), grid, dim3(AT), 0, stream, a);
    else hipLaunchKernelGGL((attn_partial<128, 1>), grid, dim3(AT), 0, stream, a);
    hipLaunchKernelGGL(attn_merge<128>, dim3(n_kv, B), dim3(AT), 0, stream, a);
  } else {
    if (two) hipLaunchKernelGGL((attn_partial<64, 2>), grid, dim3(AT), 0, stream, a);
    else hipLaunchKernelGGL((attn_partial<64, 1>), grid, dim3(AT), 0, stream, a);
    hipLaunchKernelGGL(attn_merge<64>, dim3(n_kv, B), dim3(AT), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bd
