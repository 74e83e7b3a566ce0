// C ABI of the block-draft library: argument checks on the host, workspace
// sizing, and the launches (declared in include/blockdraft.h).
//
// Every check runs before any HIP call, so an invalid call returns without
// touching the device and leaves the outputs as they were.
#include "../../include/blockdraft.h"
#include "bd_launch.hpp"

#include <stdarg.h>
#include <stdio.h>

#include <mutex>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BD_E_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* blockdraft_last_error(void) { return g_err; }

// ------------------------------------------------------------------ inject_kv
size_t inject_kv_workspace_size(int32_t M, int32_t d_in, int32_t L, int32_t n_kv, int32_t hd) {
  if (M <= 0 || d_in <= 0 || L <= 0 || n_kv <= 0 || hd <= 0) return 0;
  return bd::inject_ws_bytes(M, d_in, L, n_kv, hd);
}

int inject_kv(const uint16_t* h_target, const uint16_t* w_kv, const uint16_t* k_norm_w,
              const int32_t* row_cu, const int32_t* row_pos0, const int64_t* cache_base,
              uint16_t* k_cache, uint16_t* v_cache, int64_t T_cap,
              int32_t B, int32_t M, int32_t d_in, int32_t L, int32_t n_kv, int32_t hd,
              float rope_theta, float rms_eps,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || M < 0 || d_in <= 0 || L <= 0 || n_kv <= 0 || hd <= 0 || T_cap < 0)
    return fail(BD_E_SHAPE, "inject_kv: need B >= 0, M >= 0, T_cap >= 0 and positive d_in, L, n_kv, hd "
                "(got B=%d M=%d d_in=%d L=%d n_kv=%d hd=%d T_cap=%lld)", B, M, d_in, L, n_kv, hd,
                (long long)T_cap);
  if (!(rope_theta > 0.f) || !(rms_eps >= 0.f))
    return fail(BD_E_SHAPE, "inject_kv: need rope_theta > 0 and rms_eps >= 0");
  if (hd != 64 && hd != 128) return fail(BD_E_UNSUPPORTED, "inject_kv: hd must be 64 or 128 (got %d)", hd);
  if (d_in % 64 != 0) return fail(BD_E_UNSUPPORTED, "inject_kv: d_in must be a multiple of 64 (got %d)", d_in);
  if (n_kv > 64) return fail(BD_E_UNSUPPORTED, "inject_kv: n_kv must be <= 64 (got %d)", n_kv);
  if ((long long)L * 2 * n_kv * hd > (1 << 24))
    return fail(BD_E_UNSUPPORTED, "inject_kv: L*2*n_kv*hd too large");
  if (!h_target || !w_kv || !row_cu || !row_pos0 || !cache_base || !k_cache || !v_cache)
    return fail(BD_E_NULL, "inject_kv: a required pointer is NULL");
  if (!aligned16(h_target) || !aligned16(w_kv) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(BD_E_UNSUPPORTED, "inject_kv: H, W and the caches must be 16-byte aligned");
  // the bytes this call uses (at most what inject_kv_workspace_size reports)
  const size_t need = bd::inject_ws_bytes_call(M, d_in, L, n_kv, hd);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BD_E_WORKSPACE, "inject_kv: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace)) return fail(BD_E_UNSUPPORTED, "inject_kv: workspace must be 16-byte aligned");
  if (M == 0 || B == 0) return ok();
  return launched(bd::launch_inject(h_target, w_kv, k_norm_w, row_cu, row_pos0, cache_base, k_cache, v_cache,
                                    T_cap, B, M, d_in, L, n_kv, hd, rope_theta, rms_eps, workspace, stream),
                  "inject_kv");
}

// ------------------------------------------------------------ draft_block_attn
size_t draft_block_attn_workspace_size(int32_t B, int32_t K, int32_t n_q, int32_t n_kv, int32_t hd,
                                       int32_t max_ctx, int32_t window) {
  if (B <= 0 || K <= 0 || n_q <= 0 || n_kv <= 0 || hd <= 0 || max_ctx < 0 || window < 0 || n_q % n_kv)
    return 0;
  return bd::attn_ws_bytes(B, K, n_q, n_kv, hd, max_ctx, window);
}

int draft_block_attn(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                     const uint16_t* k_cache, const uint16_t* v_cache,
                     const int64_t* cache_base, const int32_t* ctx_len,
                     int64_t T_cap, int32_t max_ctx,
                     int32_t B, int32_t K, int32_t n_q, int32_t n_kv, int32_t hd,
                     int32_t window, int32_t flags, float scale,
                     uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || K < 1 || n_q < 1 || n_kv < 1 || hd < 1 || max_ctx < 0 || window < 0 || T_cap < 0)
    return fail(BD_E_SHAPE, "draft_block_attn: need B >= 0, K, n_q, n_kv, hd >= 1 and max_ctx, window, "
                "T_cap >= 0 (got B=%d K=%d n_q=%d n_kv=%d hd=%d max_ctx=%d window=%d)",
                B, K, n_q, n_kv, hd, max_ctx, window);
  if (n_q % n_kv) return fail(BD_E_SHAPE, "draft_block_attn: n_q (%d) must be a multiple of n_kv (%d)", n_q, n_kv);
  if (scale != scale) return fail(BD_E_SHAPE, "draft_block_attn: scale is NaN");
  if (flags & ~(BD_ATTN_CAUSAL | BD_ATTN_QUERY_WINDOW))
    return fail(BD_E_UNSUPPORTED, "draft_block_attn: unknown flags 0x%x", unsigned(flags));
  if (hd != 64 && hd != 128) return fail(BD_E_UNSUPPORTED, "draft_block_attn: hd must be 64 or 128 (got %d)", hd);
  if (K > 64) return fail(BD_E_UNSUPPORTED, "draft_block_attn: K must be <= 64 (got %d)", K);
  if ((n_q / n_kv) * K > 128)
    return fail(BD_E_UNSUPPORTED, "draft_block_attn: (n_q/n_kv)*K must be <= 128 (got %d)", (n_q / n_kv) * K);
  if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !cache_base || !ctx_len || !out)
    return fail(BD_E_NULL, "draft_block_attn: a required pointer is NULL");
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(BD_E_UNSUPPORTED, "draft_block_attn: Q, block K/V and the caches must be 16-byte aligned");
  const size_t need = draft_block_attn_workspace_size(B, K, n_q, n_kv, hd, max_ctx, window);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BD_E_WORKSPACE, "draft_block_attn: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace))
    return fail(BD_E_UNSUPPORTED, "draft_block_attn: workspace must be 16-byte aligned");
  if (B == 0) return ok();
  return launched(bd::launch_attn(q, k_blk, v_blk, k_cache, v_cache, cache_base, ctx_len, T_cap, max_ctx, B, K,
                                  n_q, n_kv, hd, window, flags, scale, out, lse, workspace, stream),
                  "draft_block_attn");
}

// ---------------------------------------------------------------- verify_block
size_t verify_block_workspace_size(int32_t B, int32_t G, int32_t V, int32_t top_k) {
  if (B <= 0 || G < 0 || V <= 0 || top_k < 0) return 0;
  return bd::verify_ws_bytes(B, B * (G + 1), V, top_k, false);
}

}  // extern "C"

namespace {

// Host checks shared by verify_block and verify_block_noalloc (everything but
// the workspace).
int verify_checks(const char* who, const float* target_logits, const float* draft_logits,
                  const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t G, int32_t V,
                  float temperature, int32_t top_k, float top_p, int32_t* tau, int32_t* out_tokens,
                  float* draft_probs) {
  if (B < 0 || G < 0 || V < 1 || top_k < 0)
    return fail(BD_E_SHAPE, "%s: need B >= 0, G >= 0, V >= 1, top_k >= 0 (got B=%d G=%d V=%d top_k=%d)", who,
                B, G, V, top_k);
  if (!(temperature >= 0.f) || temperature == INFINITY || top_p != top_p)
    return fail(BD_E_SHAPE, "%s: temperature must be finite and >= 0, top_p not NaN", who);
  if (top_k > 64) return fail(BD_E_UNSUPPORTED, "%s: top_k must be <= 64 (got %d)", who, top_k);
  if (temperature > 0.f && top_p < 1.f && (top_k == 0 || top_k >= V))
    return fail(BD_E_UNSUPPORTED, "%s: a top-p filter needs a top-k filter with 0 < top_k < V "
                "(got top_k=%d, V=%d, top_p=%g)", who, top_k, V, double(top_p));
  if (G > 64) return fail(BD_E_UNSUPPORTED, "%s: G must be <= 64 (got %d)", who, G);
  if ((long long)B * (2 * G + 1) * ((V + 8191) / 8192) > 0x7fffffffLL)
    return fail(BD_E_UNSUPPORTED, "%s: too many (row, chunk) pairs", who);
  const bool greedy = temperature == 0.f;
  if (!target_logits || !tau || !out_tokens || (G > 0 && !draft_tokens))
    return fail(BD_E_NULL, "%s: target_logits, draft_tokens, tau and out_tokens are required", who);
  if (!greedy && (!uniforms || (G > 0 && !draft_logits)))
    return fail(BD_E_NULL, "%s: sampling needs draft_logits and uniforms", who);
  if (draft_probs && G > 0 && !draft_logits)
    return fail(BD_E_NULL, "%s: draft_probs needs draft_logits", who);
  if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits)))
    return fail(BD_E_UNSUPPORTED, "%s: logits must be 16-byte aligned", who);
  return BD_OK;
}

}  // namespace

extern "C" {

int verify_block(const float* target_logits, const float* draft_logits,
                 const int32_t* draft_tokens, const float* uniforms,
                 int32_t B, int32_t G, int32_t V,
                 float temperature, int32_t top_k, float top_p,
                 int32_t* tau, int32_t* out_tokens,
                 float* target_probs, float* draft_probs,
                 float* accept_ratio, float* sample_margin,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = verify_checks("verify_block", target_logits, draft_logits, draft_tokens, uniforms, B, G, V,
                               temperature, top_k, top_p, tau, out_tokens, draft_probs);
  if (st != BD_OK) return st;
  const size_t need = verify_block_workspace_size(B, G, V, top_k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BD_E_WORKSPACE, "verify_block: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace)) return fail(BD_E_UNSUPPORTED, "verify_block: workspace must be 16-byte aligned");
  if (B == 0) return ok();
  return launched(bd::launch_verify(target_logits, draft_logits, draft_tokens, uniforms, nullptr, B, B * (G + 1), G,
                                    V, temperature, top_k, top_p, tau, out_tokens, target_probs, draft_probs,
                                    accept_ratio, sample_margin, nullptr, workspace, stream),
                  "verify_block");
}

size_t verify_block_ragged_workspace_size(int32_t B, int32_t n_target_rows, int32_t G_max, int32_t V,
                                          int32_t top_k, int32_t want_beta) {
  if (B <= 0 || n_target_rows < B || G_max < 0 || V <= 0 || top_k < 0) return 0;
  return bd::verify_ws_bytes(B, n_target_rows, V, top_k, want_beta != 0);
}

int verify_block_ragged(const float* target_logits, const float* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms, const int32_t* row_cu,
                        int32_t B, int32_t n_target_rows, int32_t G_max, int32_t V,
                        float temperature, int32_t top_k, float top_p,
                        int32_t* tau, int32_t* out_tokens,
                        float* target_probs, float* draft_probs,
                        float* accept_ratio, float* sample_margin, float* beta,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || G_max < 0 || V < 1 || top_k < 0 || n_target_rows < B)
    return fail(BD_E_SHAPE, "verify_block_ragged: need B >= 0, n_target_rows >= B, G_max >= 0, V >= 1, top_k >= 0 "
                "(got B=%d n_target_rows=%d G_max=%d V=%d top_k=%d)", B, n_target_rows, G_max, V, top_k);
  if ((long long)n_target_rows > (long long)B * (G_max + 1))
    return fail(BD_E_SHAPE, "verify_block_ragged: n_target_rows (%d) exceeds B * (G_max + 1) (%lld)", n_target_rows,
                (long long)B * (G_max + 1));
  if (!(temperature >= 0.f) || temperature == INFINITY || top_p != top_p)
    return fail(BD_E_SHAPE, "verify_block_ragged: temperature must be finite and >= 0, top_p not NaN");
  if (top_k > 64) return fail(BD_E_UNSUPPORTED, "verify_block_ragged: top_k must be <= 64 (got %d)", top_k);
  if (temperature > 0.f && top_p < 1.f && (top_k == 0 || top_k >= V))
    return fail(BD_E_UNSUPPORTED, "verify_block_ragged: a top-p filter needs a top-k filter with 0 < top_k < V "
                "(got top_k=%d, V=%d, top_p=%g)", top_k, V, double(top_p));
  if (G_max > 64) return fail(BD_E_UNSUPPORTED, "verify_block_ragged: G_max must be <= 64 (got %d)", G_max);
  if ((2LL * n_target_rows - B) * ((V + 8191) / 8192) > 0x7fffffffLL)
    return fail(BD_E_UNSUPPORTED, "verify_block_ragged: too many (row, chunk) pairs");
  const bool greedy = temperature == 0.f;
  const bool drafts = n_target_rows > B;
  if (!target_logits || !tau || !out_tokens || (B > 0 && !row_cu) || (drafts && !draft_tokens))
    return fail(BD_E_NULL, "verify_block_ragged: target_logits, row_cu, draft_tokens, tau and out_tokens are required");
  if (!greedy && (!uniforms || (drafts && !draft_logits)))
    return fail(BD_E_NULL, "verify_block_ragged: sampling needs draft_logits and uniforms");
  if ((draft_probs || beta) && drafts && !draft_logits)
    return fail(BD_E_NULL, "verify_block_ragged: draft_probs and beta need draft_logits");
  if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits)))
    return fail(BD_E_UNSUPPORTED, "verify_block_ragged: logits must be 16-byte aligned");
  const size_t need = verify_block_ragged_workspace_size(B, n_target_rows, G_max, V, top_k, beta != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BD_E_WORKSPACE, "verify_block_ragged: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace))
    return fail(BD_E_UNSUPPORTED, "verify_block_ragged: workspace must be 16-byte aligned");
  if (B == 0) return ok();
  return launched(bd::launch_verify(target_logits, draft_logits, draft_tokens, uniforms, row_cu, B, n_target_rows,
                                    G_max, V, temperature, top_k, top_p, tau, out_tokens, target_probs, draft_probs,
                                    accept_ratio, sample_margin, beta, workspace, stream),
                  "verify_block_ragged");
}

// ---------------------------------------------------------------- draft_forward
size_t draft_forward_workspace_size(int32_t B, int32_t K, int32_t d_model, int32_t n_q, int32_t n_kv, int32_t hd,
                                    int32_t ffn, int32_t max_ctx, int32_t window) {
  if (B <= 0 || K <= 0 || d_model <= 0 || n_q <= 0 || n_kv <= 0 || hd <= 0 || ffn <= 0 || max_ctx < 0 || window < 0 ||
      n_q % n_kv)
    return 0;
  return bd::forward_ws_bytes(B, K, d_model, n_q, n_kv, hd, ffn, max_ctx, window);
}

int draft_forward(const uint16_t* x_in, int32_t B, int32_t K, int32_t d_model, int32_t L, int32_t n_q, int32_t n_kv,
                  int32_t hd, int32_t ffn, int32_t V, const uint16_t* const* layer_weights,
                  const uint16_t* final_norm, const uint16_t* lm_head, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int64_t* cache_base, const int32_t* ctx_len, int64_t T_cap,
                  int32_t max_ctx, int32_t window, float rope_theta, float rms_eps, float* logits, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || K < 1 || d_model < 1 || L < 0 || n_q < 1 || n_kv < 1 || ffn < 1 || V < 1 || max_ctx < 0 ||
      window < 0 || T_cap < 0)
    return fail(BD_E_SHAPE, "draft_forward: need B, L, max_ctx, window, T_cap >= 0 and K, d_model, n_q, n_kv, ffn, "
                "V >= 1");
  if (n_q % n_kv) return fail(BD_E_SHAPE, "draft_forward: n_q (%d) must be a multiple of n_kv (%d)", n_q, n_kv);
  if (!(rope_theta > 0.f) || !(rms_eps >= 0.f))
    return fail(BD_E_SHAPE, "draft_forward: need rope_theta > 0 and rms_eps >= 0");
  if (hd != 64 && hd != 128) return fail(BD_E_UNSUPPORTED, "draft_forward: hd must be 64 or 128 (got %d)", hd);
  if (K > 64 || (n_q / n_kv) * K > 128)
    return fail(BD_E_UNSUPPORTED, "draft_forward: need K <= 64 and (n_q/n_kv)*K <= 128");
  if (!x_in || !final_norm || !lm_head || !logits || !cache_base || !ctx_len || (L > 0 && (!layer_weights ||
      !k_cache || !v_cache)))
    return fail(BD_E_NULL, "draft_forward: a required pointer is NULL");
  for (int i = 0; i < 8 * L; ++i) {
    if (!layer_weights[i]) return fail(BD_E_NULL, "draft_forward: layer weight %d of layer %d is NULL", i % 8, i / 8);
    if (!aligned16(layer_weights[i]))
      return fail(BD_E_UNSUPPORTED, "draft_forward: layer weight %d of layer %d must be 16-byte aligned", i % 8, i / 8);
  }
  if (d_model % 64 || ffn % 64)
    return fail(BD_E_UNSUPPORTED, "draft_forward: d_model (%d) and ffn (%d) must be multiples of 64", d_model, ffn);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(x_in) || !aligned16(lm_head) || !aligned16(final_norm))
    return fail(BD_E_UNSUPPORTED, "draft_forward: x_in, final_norm, lm_head and the caches must be 16-byte aligned");
  if (V % 4 == 0 && !aligned16(logits))
    return fail(BD_E_UNSUPPORTED, "draft_forward: logits must be 16-byte aligned");
  const size_t need = draft_forward_workspace_size(B, K, d_model, n_q, n_kv, hd, ffn, max_ctx, window);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BD_E_WORKSPACE, "draft_forward: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && !aligned16(workspace)) return fail(BD_E_UNSUPPORTED, "draft_forward: workspace must be 16-byte aligned");
  if (B == 0) return ok();
  const hipError_t e = bd::launch_forward(x_in, B, K, d_model, L, n_q, n_kv, hd, ffn, V, layer_weights, final_norm,
                                          lm_head, k_cache, v_cache, cache_base, ctx_len, T_cap, max_ctx, window,
                                          rope_theta, rms_eps, logits, workspace, stream);
  return launched(e, "draft_forward");
}

// ------------------------------------------------------------------ select_block
size_t select_block_workspace_size(int32_t B, int32_t G, int32_t V) {
  if (B <= 0 || G <= 0 || V < 16) return 0;
  return bd::select_ws_bytes(B, G, V);
}

int select_block(const float* logits, const int32_t* anchor, const uint16_t* trans_prev, const uint16_t* trans_next,
                 int32_t B, int32_t G, int32_t V, int32_t r, int32_t* tokens, float* scores, int32_t* candidates,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || G < 0) return fail(BD_E_SHAPE, "select_block: need B >= 0 and G >= 0 (got B=%d G=%d)", B, G);
  if (V < 16 || V > 64 * 8192)
    return fail(BD_E_UNSUPPORTED, "select_block: need 16 <= V <= 524288 (got %d)", V);
  if (r < 8 || r > 256 || r % 8)
    return fail(BD_E_UNSUPPORTED, "select_block: the rank r must be a multiple of 8 in [8, 256] (got %d)", r);
  if (B == 0 || G == 0) return ok();
  if (!logits || !anchor || !trans_prev || !trans_next || !tokens)
    return fail(BD_E_NULL, "select_block: logits, anchor, trans_prev, trans_next and tokens are required");
  if (!aligned16(trans_prev) || !aligned16(trans_next))
    return fail(BD_E_UNSUPPORTED, "select_block: the transition tables must be 16-byte aligned");
  if ((V & 3) == 0 && !aligned16(logits))
    return fail(BD_E_UNSUPPORTED, "select_block: logits must be 16-byte aligned");
  const size_t need = select_block_workspace_size(B, G, V);
  if (!workspace || workspace_bytes < need)
    return fail(BD_E_WORKSPACE, "select_block: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(BD_E_UNSUPPORTED, "select_block: workspace must be 16-byte aligned");
  return launched(bd::launch_select(logits, anchor, trans_prev, trans_next, B, G, V, r, tokens, scores, candidates,
                                    workspace, stream),
                  "select_block");
}

// ---------------------------------------------------------------- commit_round
int commit_round(const int32_t* tau, int32_t B, int32_t K, int32_t* ctx_len, int32_t* row_pos0,
                 const int32_t* cap, int32_t* done, hipStream_t stream) {
  if (B < 0 || K < 0) return fail(BD_E_SHAPE, "commit_round: need B >= 0 and K >= 0 (got B=%d K=%d)", B, K);
  if (B > 0 && (!tau || !ctx_len)) return fail(BD_E_NULL, "commit_round: tau and ctx_len are required");
  if (B == 0) return ok();
  return launched(bd::launch_commit(tau, B, K, ctx_len, row_pos0, cap, done, stream), "commit_round");
}

// ---------------------------------------------------------------- prefix_schedule
int prefix_schedule(const float* survival, const int32_t* survival_cu, int32_t R, const float* sps_b,
                    const float* sps_v, int32_t n_sps, int32_t* ell, double* theta) {
  if (R < 0 || n_sps < 1) return fail(BD_E_SHAPE, "prefix_schedule: need R >= 0 and n_sps >= 1 (got R=%d n_sps=%d)",
                                      R, n_sps);
  if (!sps_b || !sps_v || (R > 0 && (!survival_cu || !ell)))
    return fail(BD_E_NULL, "prefix_schedule: sps_b, sps_v, survival_cu and ell are required");
  bd::prefix_schedule(survival, survival_cu, R, sps_b, sps_v, n_sps, ell, theta);
  return ok();
}

}  // extern "C"

// ----------------------------------------------------- verify_block_noalloc
// verify_block for callers that cannot allocate device memory: the records,
// kept lists and draw jobs live in a file-scope device array instead of a
// caller workspace.  Each device holds its own copy of the array from the
// first call on it until the process ends.  The host-side name `scratch` is
// only a stand-in for that array: its device address is looked up once per
// device (with the device current) and only that address reaches the kernels.
namespace bd {
__device__ __align__(256) uint8_t scratch[BD_NOALLOC_SCRATCH_BYTES];
}  // namespace bd

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BD_E_LAUNCH, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BD_E_UNSUPPORTED, "%s: device %d beyond %d", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(bd::scratch));
    if (e != hipSuccess || !p)
      return fail(BD_E_LAUNCH, "%s: hipGetSymbolAddress of the scratch array failed: %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BD_OK;
}

}  // namespace

extern "C" {

int verify_block_noalloc(const float* target_logits, const float* draft_logits,
                         const int32_t* draft_tokens, const float* uniforms,
                         int32_t B, int32_t G, int32_t V,
                         float temperature, int32_t top_k, float top_p,
                         int32_t* tau, int32_t* out_tokens,
                         float* target_probs, float* draft_probs,
                         float* accept_ratio, float* sample_margin, hipStream_t stream) {
  const int st = verify_checks("verify_block_noalloc", target_logits, draft_logits, draft_tokens, uniforms, B, G, V,
                               temperature, top_k, top_p, tau, out_tokens, draft_probs);
  if (st != BD_OK) return st;
  const size_t need = verify_block_workspace_size(B, G, V, top_k);
  if (need > BD_NOALLOC_SCRATCH_BYTES)
    return fail(BD_E_WORKSPACE, "verify_block_noalloc: this call needs %zu bytes of scratch, more than the "
                "%zu of the static array", need, (size_t)BD_NOALLOC_SCRATCH_BYTES);
  if (B == 0) return ok();
  void* ws = nullptr;
  const int sa = scratch_address("verify_block_noalloc", &ws);
  if (sa != BD_OK) return sa;
  return launched(bd::launch_verify(target_logits, draft_logits, draft_tokens, uniforms, nullptr, B, B * (G + 1), G,
                                    V, temperature, top_k, top_p, tau, out_tokens, target_probs, draft_probs,
                                    accept_ratio, sample_margin, nullptr, ws, stream),
                  "verify_block_noalloc");
}

}  // extern "C"
