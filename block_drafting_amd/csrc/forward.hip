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
// The GEMMs are plain library GEMMs (rocBLAS, bf16 in, fp32 accumulate, the
// residual added in the same call with beta = 1); the norms, RoPE and the
// gate run in the small kernels below; attention is this library's kernel.
#include "bd_common.hpp"
#include "bd_launch.hpp"

#include <rocblas/rocblas.h>

#include <cmath>
#include <map>
#include <mutex>

namespace bd {

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

struct QkArgs {
  const uint16_t* qkv;  // [M, (n_q + 2 n_kv) hd]
  const uint16_t* gq;   // [hd]
  const uint16_t* gk;   // [hd]
  const int32_t* ctx_len;
  uint16_t* q;          // [M, n_q hd]
  uint16_t* kb;         // [M, n_kv hd]
  uint16_t* vb;         // [M, n_kv hd]
  int K, n_q, n_kv, hd;
  float eps;
  double inv_freq[64];
};

// Per row m = b K + i: RMSNorm of every Q and K head with its gain, RoPE
// (pairs d, d + hd/2) at position ctx_len[b] + i; V copied.  One thread per
// (head, dim pair).
__global__ __launch_bounds__(256) void fw_qk_norm_rope(QkArgs a) {
  const int m = blockIdx.x, t = threadIdx.x;
  const int b = m / a.K, i = m - b * a.K;
  const int pos = a.ctx_len[b] + i;
  const int hd = a.hd, half = hd >> 1;
  const int nh = a.n_q + a.n_kv;  // heads that get norm + RoPE
  const int ld = (a.n_q + 2 * a.n_kv) * hd;
  const uint16_t* row = a.qkv + size_t(m) * ld;
  // half / 64 threads per head when hd = 128 (a wave covers one head)
  for (int it = t; it < nh * half; it += 256) {
    const int head = it / half, d = it - head * half;
    const uint16_t* src = row + size_t(head) * hd;
    const float xa = bf16_to_f32(src[d]), xb = bf16_to_f32(src[half + d]);
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
  const uint16_t* vsrc = row + size_t(nh) * hd;
  for (int c = t; c < a.n_kv * hd; c += 256) a.vb[size_t(m) * a.n_kv * hd + c] = vsrc[c];
}

// h = silu(gate) * up, gu row = [gate (F) | up (F)]
__global__ __launch_bounds__(256) void fw_silu_mul(const uint16_t* gu, int F, uint16_t* h) {
  const int m = blockIdx.x;
  const uint16_t* row = gu + size_t(m) * 2 * F;
  for (int c = threadIdx.x; c < F; c += 256) {
    const float g = bf16_to_f32(row[c]), u = bf16_to_f32(row[F + c]);
    h[size_t(m) * F + c] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
  }
}

namespace {

std::mutex g_blas_mu;

rocblas_handle blas_handle() {
  static std::map<int, rocblas_handle> hs;
  int dev = 0;
  (void)hipGetDevice(&dev);
  auto it = hs.find(dev);
  if (it != hs.end()) return it->second;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
  hs[dev] = h;
  return h;
}

// row-major Y[M, N] = X[M, Kd] . W[N, Kd]^T + beta * C  (column-major: Y^T = W X^T)
bool gemm_rm(rocblas_handle h, int M, int N, int Kd, const uint16_t* X, const uint16_t* W, const void* C, void* Y,
             bool y_f32, float beta) {
  const float alpha = 1.0f;
  const rocblas_datatype yt = y_f32 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
  return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, M, Kd, &alpha, W,
                         rocblas_datatype_bf16_r, Kd, X, rocblas_datatype_bf16_r, Kd, &beta, C ? C : Y, yt, N, Y, yt,
                         N, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) == rocblas_status_success;
}

inline size_t al(size_t x) { return (x + 255) & ~size_t(255); }

struct FwLayout {
  size_t x, xn, qkv, q, kb, vb, att, gu, h, attn_ws, total;
};

FwLayout fw_layout(int B, int K, int d, int n_q, int n_kv, int hd, int ffn, int max_ctx, int window) {
  const size_t M = size_t(B) * K;
  FwLayout L{};
  size_t o = 0;
  L.x = o; o += al(M * d * 2);
  L.xn = o; o += al(M * d * 2);
  L.qkv = o; o += al(M * size_t(n_q + 2 * n_kv) * hd * 2);
  L.q = o; o += al(M * size_t(n_q) * hd * 2);
  L.kb = o; o += al(M * size_t(n_kv) * hd * 2);
  L.vb = o; o += al(M * size_t(n_kv) * hd * 2);
  L.att = o; o += al(M * size_t(n_q) * hd * 2);
  L.gu = o; o += al(M * size_t(2) * ffn * 2);
  L.h = o; o += al(M * size_t(ffn) * 2);
  L.attn_ws = o; o += al(attn_ws_bytes(B, K, n_q, n_kv, hd, max_ctx, window));
  L.total = o;
  return L;
}

}  // namespace

size_t forward_ws_bytes(int B, int K, int d, int n_q, int n_kv, int hd, int ffn, int max_ctx, int window) {
  return fw_layout(B, K, d, n_q, n_kv, hd, ffn, max_ctx, window).total;
}

// returns hipSuccess, or hipErrorUnknown when a library GEMM failed
hipError_t launch_forward(const uint16_t* x_in, int B, int K, int d, int L, int n_q, int n_kv, int hd, int ffn,
                          int V, const uint16_t* const* lw, const uint16_t* g_final, const uint16_t* w_lm,
                          const uint16_t* kc, const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                          int64_t T_cap, int max_ctx, int window, float rope_theta, float eps, float* logits,
                          void* ws, hipStream_t stream) {
  const int M = B * K;
  const FwLayout Lo = fw_layout(B, K, d, n_q, n_kv, hd, ffn, max_ctx, window);
  char* w = static_cast<char*>(ws);
  auto P = [&](size_t off) { return reinterpret_cast<uint16_t*>(w + off); };
  uint16_t *x = P(Lo.x), *xn = P(Lo.xn), *qkv = P(Lo.qkv), *q = P(Lo.q), *kb = P(Lo.kb), *vb = P(Lo.vb),
           *att = P(Lo.att), *gu = P(Lo.gu), *h = P(Lo.h);
  QkArgs qa{};
  qa.qkv = qkv; qa.ctx_len = ctx_len; qa.q = q; qa.kb = kb; qa.vb = vb;
  qa.K = K; qa.n_q = n_q; qa.n_kv = n_kv; qa.hd = hd; qa.eps = eps;
  for (int i = 0; i < hd / 2; ++i) qa.inv_freq[i] = pow(double(rope_theta), -2.0 * i / double(hd));
  const int n_qkv = (n_q + 2 * n_kv) * hd;
  const size_t layer_cache = size_t(T_cap) * n_kv * hd;

  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle bh = blas_handle();
  if (!bh || rocblas_set_stream(bh, stream) != rocblas_status_success) return hipErrorUnknown;
  for (int l = 0; l < L; ++l) {
    const uint16_t* g_attn = lw[8 * l + 0];
    const uint16_t* w_qkv = lw[8 * l + 1];
    const uint16_t* g_q = lw[8 * l + 2];
    const uint16_t* g_k = lw[8 * l + 3];
    const uint16_t* w_o = lw[8 * l + 4];
    const uint16_t* g_mlp = lw[8 * l + 5];
    const uint16_t* w_gu = lw[8 * l + 6];
    const uint16_t* w_dn = lw[8 * l + 7];
    const uint16_t* xr = l == 0 ? x_in : x;  // the residual stream
    hipLaunchKernelGGL(fw_rmsnorm, dim3(M), dim3(256), 0, stream, xr, g_attn, d, eps, xn);
    if (!gemm_rm(bh, M, n_qkv, d, xn, w_qkv, nullptr, qkv, false, 0.f)) return hipErrorUnknown;
    qa.gq = g_q; qa.gk = g_k;
    hipLaunchKernelGGL(fw_qk_norm_rope, dim3(M), dim3(256), 0, stream, qa);
    hipError_t e = launch_attn(q, kb, vb, kc + l * layer_cache, vc + l * layer_cache, cache_base, ctx_len, T_cap,
                               max_ctx, B, K, n_q, n_kv, hd, window, 0, 0.f, att, nullptr, w + Lo.attn_ws, stream);
    if (e != hipSuccess) return e;
    if (!gemm_rm(bh, M, d, n_q * hd, att, w_o, xr, x, false, 1.f)) return hipErrorUnknown;
    hipLaunchKernelGGL(fw_rmsnorm, dim3(M), dim3(256), 0, stream, x, g_mlp, d, eps, xn);
    if (!gemm_rm(bh, M, 2 * ffn, d, xn, w_gu, nullptr, gu, false, 0.f)) return hipErrorUnknown;
    hipLaunchKernelGGL(fw_silu_mul, dim3(M), dim3(256), 0, stream, gu, ffn, h);
    if (!gemm_rm(bh, M, d, ffn, h, w_dn, x, x, false, 1.f)) return hipErrorUnknown;
  }
  hipLaunchKernelGGL(fw_rmsnorm, dim3(M), dim3(256), 0, stream, L > 0 ? x : x_in, g_final, d, eps, xn);
  if (!gemm_rm(bh, M, V, d, xn, w_lm, nullptr, logits, true, 0.f)) return hipErrorUnknown;
  return hipGetLastError();
}

}  // namespace bd
