/*
 * blockdraft.h -- C ABI of the block-draft round on one MI355X (gfx950).
 *
 * Three calls make one round of block-parallel speculative decoding:
 *   inject_kv         project the target's concatenated multi-layer hidden
 *                     states into every draft layer's K/V cache;
 *   draft_block_attn  attention of the K block positions over the injected
 *                     context K/V plus the block's own K/V (one layer);
 *   verify_block      greedy prefix matching or lossless rejection sampling
 *                     of the drafted tokens against the target's logits.
 *
 * Sources (cited by page title and section):
 *   "The Next Generation of Speculative Decoding: DFlash and Spec V2"
 *     (lmsys.org blog; "DFlash/Spec V2 blog"): summary and A2 give the KV
 *     injection KV_draft^(l) = Projection^(l)(H_target) into every draft
 *     layer; A7 gives immediate materialization through one layer-batched
 *     projection with fused Norm + RoPE post-processing.
 *   "Tencent open-sources DSpine" ("DSpine article"): block 16 = 1 anchor +
 *     15 drafted positions, 8192-token sliding window ("what these weights
 *     are"); DFlash's in-block attention is bidirectional ("principle").
 *   DeepSeek DSpark tutorial ("DSpark tutorial"), "speculative decoding
 *     basics": prefix acceptance, a replacement token at the first
 *     disagreement, one extra token per round, and losslessness.
 *   "Didi EAGLE-3 training/inference practice", 5.3: partial attention
 *     results merge exactly through their log-sum-exp.
 *
 * Conventions shared by every call
 *   - Pointers named as device memory are owned by the caller; the library
 *     never allocates, frees or keeps them.  Scratch space comes in through
 *     (workspace, workspace_bytes); the *_workspace_size functions give the
 *     size needed.
 *   - Calls are asynchronous on the caller's stream and never synchronise.
 *   - Arrays are dense and row-major; bf16 values are passed as uint16_t bit
 *     patterns; bf16 results are rounded to nearest, ties to even.
 *   - Every call checks its arguments on the host first and returns a status
 *     without launching anything (outputs untouched) when they are invalid;
 *     blockdraft_last_error() then gives a text for the calling thread.
 *     Per-request values that live on the device (context lengths, slots,
 *     token ids) cannot be checked on the host: the kernels never read or
 *     write outside [0, T_cap) or [0, V) because of them, and the affected
 *     request's outputs are undefined (attention writes NaN).
 *   - Results are deterministic: fixed reduction orders, no float atomics.
 *   - NaN inputs give undefined results.
 */
#ifndef BLOCKDRAFT_H
#define BLOCKDRAFT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BD_OK = 0,
  BD_E_NULL = -1,        /* a required pointer is NULL                      */
  BD_E_SHAPE = -2,       /* inconsistent or negative sizes                  */
  BD_E_UNSUPPORTED = -3, /* valid but outside the supported shapes          */
  BD_E_WORKSPACE = -4,   /* workspace smaller than *_workspace_size says    */
  BD_E_LAUNCH = -5       /* the HIP runtime reported an error at launch     */
};

/* Text of the last error raised on the calling thread ("" if none). */
const char* blockdraft_last_error(void);

/* ------------------------------------------------------------------------
 * inject_kv -- KV injection (DFlash/Spec V2 blog, summary, A2 and A7).
 *
 * For every row m of H (one token) and every draft layer l:
 *   y = H[m] . W^T  (fp32 accumulation of bf16 products), all layers at once;
 *   K head g = y[l][K][g] / sqrt(mean over hd of y^2 + rms_eps) * k_norm_w[l],
 *   then the half-split rotary embedding at the row's absolute position:
 *   dims (i, i + hd/2) turn by pos * rope_theta^(-2i/hd);
 *   V head g = y[l][V][g] unchanged;
 *   both rounded to bf16 and written to slot cache_base[b] + row_pos0[b] + j,
 *   where row m is the j-th row of request b (row_cu[b] <= m < row_cu[b+1]).
 *
 * h_target    device bf16 [M, d_in]: concatenated target-layer hidden states.
 * w_kv        device bf16 [L*2*n_kv*hd, d_in]: rows ordered [l][K|V][head][dim].
 * k_norm_w    device bf16 [L, hd] RMSNorm gains of K, or NULL for ones.
 * row_cu      device int32 [B+1]: request row offsets, row_cu[0] = 0,
 *             nondecreasing, row_cu[B] <= M (rows past row_cu[B] are not
 *             written).
 * row_pos0    device int32 [B]: absolute position of each request's first row.
 * cache_base  device int64 [B]: slot of position 0 of each request.
 * k_cache, v_cache  device bf16 [L, T_cap, n_kv, hd], updated in place; a row
 *             whose slot falls outside [0, T_cap) is skipped.
 * Supported: hd in {64, 128}; d_in a positive multiple of 64; 1 <= n_kv <= 64.
 * Workspace: inject_kv_workspace_size(M, ...) bytes, 16-byte aligned, serve
 * every call with up to M rows; a call returns BD_E_WORKSPACE only when the
 * workspace is smaller than the part of it that call uses.
 * ------------------------------------------------------------------------ */
size_t inject_kv_workspace_size(int32_t M, int32_t d_in, int32_t L, int32_t n_kv, int32_t hd);

int inject_kv(const uint16_t* h_target, const uint16_t* w_kv, const uint16_t* k_norm_w,
              const int32_t* row_cu, const int32_t* row_pos0, const int64_t* cache_base,
              uint16_t* k_cache, uint16_t* v_cache, int64_t T_cap,
              int32_t B, int32_t M, int32_t d_in, int32_t L, int32_t n_kv, int32_t hd,
              float rope_theta, float rms_eps,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * draft_block_attn -- block-draft attention of one layer (DFlash/Spec V2
 * blog, A2; DSpine article, "principle" and "what these weights are";
 * Didi EAGLE-3 article, 5.3 for the exact split-and-merge).
 *
 * For request b, query head h (KV head g = h / (n_q / n_kv)) and block
 * position i, the keys are the context positions [lo, ctx_len[b]) with
 * lo = max(0, ctx_len[b] - window) (lo = 0 when window == 0), read from slots
 * cache_base[b] + p, followed by the K in-block keys k_blk[b, :, g]; by
 * default every block position sees all of them (DFlash: no mask).
 *   out[b, i, h] = softmax(q . keys^T * scale) . values   (bf16)
 *   lse[b, i, h] = log sum exp(q . keys^T * scale)          (fp32, natural log)
 * flags (bit set):
 *   BD_ATTN_CAUSAL        DSpine's causal in-block attention ("principle"):
 *                         block position i sees block keys j <= i only.
 *   BD_ATTN_QUERY_WINDOW  with window W > 0, a per-query sliding window: the
 *                         query at block position i (absolute position
 *                         ctx + i) sees the keys at absolute positions p with
 *                         ctx + i - p < W, i.e. context [max(0, ctx + i + 1 - W),
 *                         ctx) and block keys j > i - W; without the flag the
 *                         window is block-uniform as above.
 *
 * q           device bf16 [B, K, n_q, hd] (already normalised / rotated).
 * k_blk, v_blk device bf16 [B, K, n_kv, hd].
 * k_cache, v_cache device bf16 [T_cap, n_kv, hd]: this layer's caches.
 * cache_base  device int64 [B]; ctx_len device int32 [B], 0 <= ctx_len <= max_ctx.
 * max_ctx     host upper bound of ctx_len (sizes the grid).
 * window      0 = whole context, else the sliding-window length.
 * flags       0 or an or of BD_ATTN_CAUSAL, BD_ATTN_QUERY_WINDOW; other bits
 *             give BD_E_UNSUPPORTED.
 * scale       <= 0 selects 1/sqrt(hd).
 * out         device bf16 [B, K, n_q, hd]; lse device fp32 [B, K, n_q] or NULL.
 * Supported: hd in {64, 128}; 1 <= K <= 64; (n_q / n_kv) * K <= 128.
 * ------------------------------------------------------------------------ */
enum { BD_ATTN_CAUSAL = 1, BD_ATTN_QUERY_WINDOW = 2 };

size_t draft_block_attn_workspace_size(int32_t B, int32_t K, int32_t n_q, int32_t n_kv, int32_t hd,
                                       int32_t max_ctx, int32_t window);

int draft_block_attn(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                     const uint16_t* k_cache, const uint16_t* v_cache,
                     const int64_t* cache_base, const int32_t* ctx_len,
                     int64_t T_cap, int32_t max_ctx,
                     int32_t B, int32_t K, int32_t n_q, int32_t n_kv, int32_t hd,
                     int32_t window, int32_t flags, float scale,
                     uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * verify_block -- verification of G drafted tokens per request (DSpark
 * tutorial, "speculative decoding basics"; DSpine article, "principle" for
 * greedy matching and "speed-up" for the sampling filters).
 *
 * Greedy (temperature == 0): d_i is kept while it equals the lowest-index
 * maximum of the target's raw logits at position i; the emitted token at the
 * first mismatch (or after G matches) is that maximum.
 * Sampling (temperature > 0): P_i = filt(softmax(z_t,i / T)),
 * Q_i = filt(softmax(z_d,i / T)); filt = keep the top_k largest raw logits
 * (value desc, index asc; off when top_k == 0), softmax over them, keep the
 * shortest prefix in probability order whose mass reaches top_p (off when
 * top_p >= 1), renormalise.  d_i is kept while u_i < fp32(P_i(d_i)) /
 * fp32(Q_i(d_i)) (IEEE fp32 division).  At the first rejection i the token is
 * the smallest x (vocab order) whose running sum of max(0, P_i - Q_i) exceeds
 * u'_i times its total (P_i itself if that total is 0); with every draft kept
 * the same draw runs over P_{G+1} with u'_{G+1}.
 *
 * target_logits device fp32 [B, G+1, V]; draft_logits device fp32 [B, G, V]
 *             (may be NULL when greedy and draft_probs is NULL).
 * draft_tokens device int32 [B, G]; a token outside [0, V) is rejected.
 * uniforms    device fp32 [B, G+1, 2] in [0, 1): [b, i, 0] accepts position i,
 *             [b, i, 1] draws the replacement / extra token at position i;
 *             may be NULL when greedy.
 * tau         device int32 [B]: accepted drafted tokens, 0..G.
 * out_tokens  device int32 [B, G+1]: d_1..d_tau, then the replacement or
 *             extra token, then -1.
 * target_probs, draft_probs  optional device fp32 [B, G+1, V] / [B, G, V]:
 *             the (filtered) P and Q; with temperature 0 the plain softmax.
 * accept_ratio optional device fp32 [B, G]: the ratio each accept test used
 *             (greedy: 1 on a match, else 0).
 * sample_margin optional device fp32 [B]: distance of u' * total to the
 *             nearer running-sum boundary of the drawn token (greedy: +inf).
 * Supported: 0 <= top_k <= 64; G <= 64; V >= 1.  A top-p filter (top_p < 1
 * with temperature > 0) is supported only together with a top-k filter
 * (0 < top_k < V), whose kept set bounds the tokens top-p sorts; without one
 * the call returns BD_E_UNSUPPORTED (there is no full-vocabulary top-p).
 * ------------------------------------------------------------------------ */
size_t verify_block_workspace_size(int32_t B, int32_t G, int32_t V, int32_t top_k);

int verify_block(const float* target_logits, const float* draft_logits,
                 const int32_t* draft_tokens, const float* uniforms,
                 int32_t B, int32_t G, int32_t V,
                 float temperature, int32_t top_k, float top_p,
                 int32_t* tau, int32_t* out_tokens,
                 float* target_probs, float* draft_probs,
                 float* accept_ratio, float* sample_margin,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * verify_block_noalloc -- verify_block for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * outputs as verify_block, without the workspace.  Its scratch space is a
 * static device array of BD_NOALLOC_SCRATCH_BYTES bytes per GPU, held from
 * the first call on a GPU until the process ends; the call itself allocates
 * nothing.  A call whose verify_block_workspace_size(B, G, V, top_k) exceeds
 * that size returns BD_E_WORKSPACE without launching.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (several streams or
 * host threads at once) race and give undefined results; calls ordered on
 * one stream are safe.  Nothing in the array needs to start at zero.
 * ------------------------------------------------------------------------ */
#define BD_NOALLOC_SCRATCH_BYTES (32u << 20)

int verify_block_noalloc(const float* target_logits, const float* draft_logits,
                         const int32_t* draft_tokens, const float* uniforms,
                         int32_t B, int32_t G, int32_t V,
                         float temperature, int32_t top_k, float top_p,
                         int32_t* tau, int32_t* out_tokens,
                         float* target_probs, float* draft_probs,
                         float* accept_ratio, float* sample_margin, hipStream_t stream);

/* ------------------------------------------------------------------------
 * verify_block_ragged -- verify_block with a drafted length per request and
 * the confidence label of every drafted position (DSpark tutorial,
 * confidence-scheduled verification: the prefix scheduler picks a verify
 * length per request; the label of a position is 1 - 1/2 |P - Q|_1, which
 * equals sum_x min(P(x), Q(x))).
 *
 * Rows are packed: request b owns target rows row_cu[b] .. row_cu[b+1] - 1
 * (G_b + 1 of them) and draft rows row_cu[b] - b .. row_cu[b+1] - b - 2
 * (G_b), with 0 <= G_b <= G_max.  Each request is decided exactly as
 * verify_block decides one request with G = G_b.
 *
 * target_logits device fp32 [n_target_rows, V]; draft_logits device fp32
 *             [n_target_rows - B, V] (may be NULL when greedy and neither
 *             draft_probs nor beta is asked for).
 * row_cu      device int32 [B + 1], row_cu[0] = 0, nondecreasing by at least
 *             one per request, row_cu[B] = n_target_rows; a request whose
 *             entries break this (rows outside the arrays, G_b outside
 *             [0, G_max]) gets tau = -1 and no other output.
 * draft_tokens device int32 [n_target_rows - B]; uniforms device fp32
 *             [n_target_rows, 2] (row-wise as in verify_block).
 * tau         device int32 [B]; out_tokens device int32 [n_target_rows]:
 *             per request d_1..d_tau, the replacement or extra token, -1.
 * target_probs, draft_probs, accept_ratio, sample_margin: as verify_block,
 *             on the packed rows; optional.
 * beta        optional device fp32 [n_target_rows - B]: sum_x min(P, Q) of
 *             each drafted position under the verification distributions
 *             (greedy: 1 when the two lowest-index maxima agree, else 0).
 * n_target_rows, G_max: host values; n_target_rows <= B * (G_max + 1).
 * Supported: 0 <= top_k <= 64; G_max <= 64; V >= 1; top-p only with a top-k
 * filter, as verify_block.
 * ------------------------------------------------------------------------ */
size_t verify_block_ragged_workspace_size(int32_t B, int32_t n_target_rows, int32_t G_max, int32_t V,
                                          int32_t top_k, int32_t want_beta);

int verify_block_ragged(const float* target_logits, const float* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms, const int32_t* row_cu,
                        int32_t B, int32_t n_target_rows, int32_t G_max, int32_t V,
                        float temperature, int32_t top_k, float top_p,
                        int32_t* tau, int32_t* out_tokens,
                        float* target_probs, float* draft_probs,
                        float* accept_ratio, float* sample_margin, float* beta,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * draft_forward -- one drafter forward over the block (DFlash/Spec V2 blog,
 * A2: the drafter's layers attend to the injected context plus the block,
 * and one forward yields every block position).  Qwen3-style layers with any
 * (e.g. random-init) weights, to measure a whole draft pass.
 *
 * Per layer l (layer_weights[8 l + 0..7], device bf16):
 *   g_attn [d]; w_qkv [(n_q + 2 n_kv) hd, d] (rows: Q heads, K heads, V
 *   heads); g_q [hd], g_k [hd] (per-head RMSNorm gains of Q and K);
 *   w_o [d, n_q hd]; g_mlp [d]; w_gu [2 ffn, d] (gate rows, then up rows);
 *   w_down [d, ffn].
 *   xn = RMSNorm(x, g_attn); q, k, v = xn W_qkv^T; q, k per-head RMSNorm and
 *   RoPE (pairs d, d + hd/2, angle (ctx_len[b] + i) theta^(-2d/hd)) at block
 *   position i; a = draft_block_attn(q, k, v, layer l's caches) (no flags);
 *   x += a W_o^T; xn = RMSNorm(x, g_mlp); x += (SiLU(gate) * up) W_down^T.
 * logits = RMSNorm(x, final_norm) lm_head^T, fp32.  Intermediates and the
 * residual stream are bf16 (fp32 arithmetic inside each step).  Every step
 * runs in this library's kernels; the projections in a weight-streaming GEMM
 * whose d_in splits are added, in a fixed order, by the kernel that consumes
 * them, so the result is deterministic.
 *
 * x_in        device bf16 [B K, d]: the block rows' input hidden states.
 * layer_weights host array of 8 L device pointers (may be NULL when L = 0).
 * final_norm  device bf16 [d]; lm_head device bf16 [V, d].
 * k_cache, v_cache device bf16 [L, T_cap, n_kv, hd] (filled by inject_kv);
 * cache_base, ctx_len, max_ctx, window: as draft_block_attn.
 * logits      device fp32 [B K, V].
 * Supported: hd in {64, 128}; K <= 64; (n_q / n_kv) K <= 128; d and ffn
 * multiples of 64; x_in, final_norm, lm_head, every layer weight and the
 * caches 16-byte aligned (logits too when V % 4 == 0).
 * ------------------------------------------------------------------------ */
size_t draft_forward_workspace_size(int32_t B, int32_t K, int32_t d_model, int32_t n_q, int32_t n_kv, int32_t hd,
                                    int32_t ffn, int32_t max_ctx, int32_t window);

int draft_forward(const uint16_t* x_in, int32_t B, int32_t K, int32_t d_model, int32_t L,
                  int32_t n_q, int32_t n_kv, int32_t hd, int32_t ffn, int32_t V,
                  const uint16_t* const* layer_weights, const uint16_t* final_norm, const uint16_t* lm_head,
                  const uint16_t* k_cache, const uint16_t* v_cache, const int64_t* cache_base,
                  const int32_t* ctx_len, int64_t T_cap, int32_t max_ctx, int32_t window,
                  float rope_theta, float rms_eps, float* logits,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * select_block -- the drafted tokens of a block chosen through a transition
 * cache (DSpine article, "principle": 16 candidates per position, every
 * pairing of adjacent positions' candidates scored at once into 16 x 16
 * tables, then a left-to-right walk through the tables; DSpark tutorial,
 * "semi-autoregressive generation": the previous token's influence is a
 * low-rank offset to the position's logits).
 *
 * Score of token b at drafted position t after token a:
 *   s_t(a, b) = logits[t][b] + sum_k trans_prev[a][k] * trans_next[b][k]
 * (bf16 products added in fp32).  Candidates c_t: the 16 largest logits of
 * position t (value desc, index asc).  Position 0's predecessor is anchor[b];
 * table T_t[i][j] = s_t(c_{t-1}[i], c_t[j]).  Walk: j_0 = argmax_j s_0(anchor,
 * c_0[j]), j_t = argmax_j T_t[j_{t-1}][j] (the lowest j on ties), token t =
 * c_t[j_t].
 *
 * logits      device fp32 [B, G, V]: the drafter's base logits of the G
 *             drafted positions (16-byte aligned when V % 4 == 0).
 * anchor      device int32 [B]: the token before position 0 (an anchor
 *             outside [0, V) gives that request tokens -1 and scores NaN).
 * trans_prev, trans_next device bf16 [V, r], 16-byte aligned.
 * tokens      device int32 [B, G] (out).
 * scores      device fp32 [B, G] or NULL: the chosen table entries.
 * candidates  device int32 [B, G, 16] or NULL: c_t.
 * Workspace: select_block_workspace_size(B, G, V) bytes, 16-byte aligned.
 * Supported: 16 <= V <= 524288; r a multiple of 8 in [8, 256].  NaN logits
 * are undefined behaviour.
 * Errors: BD_E_SHAPE (B, G < 0), BD_E_UNSUPPORTED (V, r, alignment), BD_E_NULL,
 * BD_E_WORKSPACE, BD_E_LAUNCH.
 * ------------------------------------------------------------------------ */
size_t select_block_workspace_size(int32_t B, int32_t G, int32_t V);

int select_block(const float* logits, const int32_t* anchor, const uint16_t* trans_prev, const uint16_t* trans_next,
                 int32_t B, int32_t G, int32_t V, int32_t r, int32_t* tokens, float* scores, int32_t* candidates,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * commit_round -- the bookkeeping between two rounds, on the device
 * (DFlash/Spec V2 blog, A7: overlap scheduling, so the host never waits for
 * the device between rounds).
 *
 * For each request b with tau[b] >= 0: ctx_len[b] += tau[b] + 1 (the
 * accepted drafts plus the replacement / extra token are committed) and
 * row_pos0[b] = ctx_len[b] before the update: the next round materializes the K
 * rows this round verified at the block's positions (DFlash/Spec V2 blog, A7,
 * immediate materialization), so the committed ones lie inside the context
 * the next round's attention reads.  tau[b] < 0 leaves ctx_len[b] as it is.  done[b] = 1 when
 * tau[b] < 0 or when the next K rows would pass cap[b] (ctx_len + K > cap),
 * else 0.
 *
 * tau device int32 [B]; ctx_len device int32 [B], updated in place;
 * row_pos0, cap, done device int32 [B] or NULL (cap NULL: no limit).
 * Errors: BD_E_SHAPE for B < 0 or K < 0, BD_E_NULL without tau / ctx_len.
 * ------------------------------------------------------------------------ */
int commit_round(const int32_t* tau, int32_t B, int32_t K, int32_t* ctx_len, int32_t* row_pos0,
                 const int32_t* cap, int32_t* done, hipStream_t stream);

/* ------------------------------------------------------------------------
 * prefix_schedule -- the hardware-aware prefix scheduler (DSpark tutorial,
 * confidence-scheduled verification), host code.
 *
 * Request r has L_r candidate drafted positions with conditional survival
 * probabilities survival[survival_cu[r] .. survival_cu[r+1] - 1] (values in
 * [0, 1]).  The scheduler chooses verify lengths ell[r] in [0, L_r] that
 * maximise Theta = tau * SPS(B) greedily: candidates in order of cumulative
 * survival (highest first; ties to the lower request, then position), each
 * extending its request's length by one, until the first one that does not
 * raise Theta.  B = sum_r (ell[r] + 1) tokens; tau = sum_r (1 + sum over the
 * verified positions of their cumulative survival); SPS is the linear
 * interpolation of the table (sps_b[j], sps_v[j]) (any order; clamped to the
 * end values outside it).
 *
 * survival, survival_cu [R + 1], sps_b, sps_v [n_sps], ell [R]: host memory,
 * owned by the caller.  theta (host, may be NULL) receives Theta.
 * Errors: BD_E_SHAPE for R < 0 or n_sps < 1, BD_E_NULL for missing arrays.
 * ------------------------------------------------------------------------ */
int prefix_schedule(const float* survival, const int32_t* survival_cu, int32_t R,
                    const float* sps_b, const float* sps_v, int32_t n_sps,
                    int32_t* ell, double* theta);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKDRAFT_H */
