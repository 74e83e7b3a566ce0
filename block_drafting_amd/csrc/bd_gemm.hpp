// The generic split-K bf16 GEMM of the library: P[s][m][n] = sum over the d_in
// range of split s of A[m][k] W[n][k] (fp32 accumulation on the gfx950
// 32x32x16 bf16 MFMA), tiles of BM x BN staged through LDS by way of
// registers, the next step's tile loaded while the current one is consumed.
// Rows past M read row M - 1 and are zeroed before use; weight rows past N
// read row N - 1 and are not stored.  Used for the projection's small-M path
// and the drafter's GEMMs.
#pragma once

#include "bd_common.hpp"

namespace bd {

constexpr int GT = 256;  // threads per GEMM workgroup (2 x 2 waves)
constexpr int KALIGN = 64;  // d_in must be a multiple of this

struct GemmArgs {
  const uint16_t* A;  // [M, Kd]
  const uint16_t* Bw; // [N, Kd]
  float* P;           // [S][M][N]
  int M, N, Kd, S, steps_per_split, tiles_n;
};

template <int BM, int BN, int BK>
__global__ __launch_bounds__(GT) void ik_gemm(GemmArgs g) {
  constexpr int GLS = BK + 8;               // LDS row stride (elements)
  constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
  constexpr int FM = WM / 32, FN = WN / 32; // 32x32 blocks per wave
  constexpr int APT = BM * BK / 8 / GT;     // 16-byte pieces per thread
  constexpr int BPT = BN * BK / 8 / GT;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * GLS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * GLS];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int tm = tile / g.tiles_n, tn = tile - tm * g.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int step0 = split * g.steps_per_split;
  const int nsteps_all = g.Kd / BK;
  const int nsteps = min(g.steps_per_split, nsteps_all - step0);

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[APT], rb[BPT];
  auto fetch = [&](int step) {
    const int k0 = (step0 + step) * BK;
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int piece = t + p * GT;
      const int row = piece / (BK / 8), kc = piece - row * (BK / 8);
      const int m = m0 + row;
      ra[p] = *reinterpret_cast<const u32x4*>(g.A + size_t(m < g.M ? m : g.M - 1) * g.Kd + k0 + kc * 8);
    }
#pragma unroll
    for (int p = 0; p < BPT; ++p) {
      const int piece = t + p * GT;
      const int row = piece / (BK / 8), kc = piece - row * (BK / 8);
      // weight rows past N re-read row N - 1 (their columns are never stored)
      const int n = n0 + row;
      rb[p] = *reinterpret_cast<const u32x4*>(g.Bw + size_t(n < g.N ? n : g.N - 1) * g.Kd + k0 + kc * 8);
    }
  };

  if (nsteps > 0) fetch(0);
  for (int step = 0; step < nsteps; ++step) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      // rows past M were loaded from row M - 1 (unconditional loads); they
      // are zeroed here, where the data is consumed
      const int piece = t + p * GT;
      const int row = piece / (BK / 8), kc = piece - row * (BK / 8);
      const u32x4 z4 = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&As[row * GLS + kc * 8]) = m0 + row < g.M ? ra[p] : z4;
    }
#pragma unroll
    for (int p = 0; p < BPT; ++p) {
      const int piece = t + p * GT;
      const int row = piece / (BK / 8), kc = piece - row * (BK / 8);
      *reinterpret_cast<u32x4*>(&Bs[row * GLS + kc * 8]) = rb[p];
    }
    __syncthreads();
    if (step + 1 < nsteps) fetch(step + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &As[(wm * WM + i * 32 + (lane & 31)) * GLS + kk * 16 + (lane >> 5) * 8]));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &Bs[(wn * WN + j * 32 + (lane & 31)) * GLS + kk * 16 + (lane >> 5) * 8]));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
  }

  // C block layout: lane holds column (lane & 31), rows 8*jj + 4*(lane >> 5) + r
  float* P = g.P + size_t(split) * g.M * g.N;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * WM + i * 32 + jj * 8 + (lane >> 5) * 4 + r;
          if (m < g.M && n < g.N) P[size_t(m) * g.N + n] = acc[i][j][jj * 4 + r];
        }
    }
}

}  // namespace bd
