// Round commit on the device: the bookkeeping between two drafting rounds.
//
// DFlash/Spec V2 blog, A7 (overlap scheduling): the host-side clean-up of
// batch N-1 (checking stop conditions, updating request metadata) runs while
// the GPU executes batch N, and batch N's KV allocation runs while the GPU
// executes batch N-1, so the host never waits for the device between rounds.
// Keeping the per-request update itself on the device removes the wait
// altogether: round N+1 reads the context lengths round N committed from
// device memory, and the host only reads the committed tokens when it wants
// them, one round late, from an asynchronous copy.
//
// Per request: tau + 1 tokens are committed (the accepted drafts and the
// replacement / extra token), so ctx_len += tau + 1.  The next round first
// materializes the K rows this round verified (the target's hidden states of
// the block) at the block's positions, old ctx_len .. + K - 1, so row_pos0
// takes the old ctx_len; the committed ones are then inside the context the
// next round's attention reads, the others are overwritten a round later.  A request
// whose verify reported tau = -1 (invalid metadata) is left unchanged and
// flagged done, as is one whose next K rows would not fit its slots.
#include "bd_common.hpp"
#include "bd_launch.hpp"

namespace bd {

__global__ __launch_bounds__(256) void commit_kernel(const int32_t* tau, int B, int K, int32_t* ctx_len,
                                                     int32_t* row_pos0, const int32_t* cap, int32_t* done) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int t = tau[b];
  const int c0 = ctx_len[b];
  const bool ok = t >= 0;
  const int c = ok ? c0 + t + 1 : c0;
  ctx_len[b] = c;
  if (row_pos0) row_pos0[b] = c0;
  if (done) done[b] = (!ok || (cap && (long long)c + K > (long long)cap[b])) ? 1 : 0;
}

hipError_t launch_commit(const int32_t* tau, int B, int K, int32_t* ctx_len, int32_t* row_pos0, const int32_t* cap,
                         int32_t* done, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(commit_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, tau, B, K, ctx_len, row_pos0, cap,
                     done);
  return hipGetLastError();
}

}  // namespace bd
