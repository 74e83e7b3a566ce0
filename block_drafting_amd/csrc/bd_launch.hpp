// Host launchers of the three kernel families (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

// the workspace every call with up to M rows fits in (the size reported to
// callers), and the part of it a call with exactly M rows uses
size_t inject_ws_bytes(int M, int d_in, int L, int n_kv, int hd);
size_t inject_ws_bytes_call(int M, int d_in, int L, int n_kv, int hd);
hipError_t launch_inject(const uint16_t* h, const uint16_t* w, const uint16_t* gain, const int32_t* row_cu,
                         const int32_t* row_pos0, const int64_t* cache_base, uint16_t* kc, uint16_t* vc,
                         int64_t T_cap, int B, int M, int d_in, int L, int n_kv, int hd, float theta,
                         float eps, void* ws, hipStream_t stream);

size_t attn_ws_bytes(int B, int K, int n_q, int n_kv, int hd, int max_ctx, int window);
hipError_t launch_attn(const uint16_t* q, const uint16_t* kb, const uint16_t* vb, const uint16_t* kc,
                       const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                       int64_t T_cap, int max_ctx, int B, int K, int n_q, int n_kv, int hd, int window,
                       int flags, float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream);

// n_trows target rows in all (B * (G + 1) without a row map); G is the
// largest drafted length; beta (labels) may be NULL
size_t verify_ws_bytes(int B, int n_trows, int V, int top_k, bool beta);
hipError_t launch_verify(const float* zt, const float* zd, const int* dtok, const float* uni,
                         const int* row_cu, int B, int n_trows, int G, int V, float temperature, int top_k,
                         float top_p, int* tau, int* out, float* tprob, float* dprob, float* ratio, float* margin,
                         float* beta, void* ws, hipStream_t stream);

hipError_t launch_commit(const int32_t* tau, int B, int K, int32_t* ctx_len, int32_t* row_pos0, const int32_t* cap,
                         int32_t* done, hipStream_t stream);

// Weight-streaming GEMM (forward.hip): P[s][m][n] = the d_in split s of X . W^T
// (X [M][Kd], W [N][Kd] bf16, Kd a multiple of 64; P fp32, S splits of
// steps_per_split 64-wide steps; with S = 1 the product itself).  fg_plan
// picks the tile shape, split and grid for a shape (split = false: S = 1).
struct FgPlan {
  int FN, WMW, S, steps_per_split, MT, G, nwg;
};
FgPlan fg_plan(int M, int N, int Kd, bool split = true);
hipError_t fg_run(const FgPlan& p, const uint16_t* X, const uint16_t* W, float* P, int M, int N, int Kd,
                  hipStream_t stream);

size_t forward_ws_bytes(int B, int K, int d, int n_q, int n_kv, int hd, int ffn, int max_ctx, int window);
hipError_t launch_forward(const uint16_t* x_in, int B, int K, int d, int L, int n_q, int n_kv, int hd, int ffn,
                          int V, const uint16_t* const* lw, const uint16_t* g_final, const uint16_t* w_lm,
                          const uint16_t* kc, const uint16_t* vc, const int64_t* cache_base, const int32_t* ctx_len,
                          int64_t T_cap, int max_ctx, int window, float rope_theta, float eps, float* logits,
                          void* ws, hipStream_t stream);

size_t select_ws_bytes(int B, int G, int V);
hipError_t launch_select(const float* z, const int32_t* anchor, const uint16_t* E, const uint16_t* F, int B, int G,
                         int V, int r, int32_t* tokens, float* scores, int32_t* cand, void* ws, hipStream_t stream);

// prefix scheduler (host)
int prefix_schedule(const float* surv, const int32_t* surv_cu, int R, const float* sps_b, const float* sps_v,
                    int n_sps, int32_t* ell, double* theta);

}  // namespace bd
