// Stand-alone ceilings of one MI355X (gfx950) that the kernels' rooflines are
// read against: how fast plain streaming reads, LDS-direct tile rings in the
// access patterns of the attention and projection kernels, and back-to-back
// bf16 matrix instructions can run on this part.  No arithmetic on the data:
// each test moves (or multiplies) and keeps only what stops the compiler from
// dropping the work.  Built and run by bench_ceilings.py; one line per test.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "block_drafting_amd/csrc/bd_common.hpp"

using namespace bd;

#define CHECK(x)                                                                     \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

// ------------------------------------------------------------ plain streaming
// Workgroup w reads float4 elements [w * per, (w + 1) * per) of the buffer,
// four loads per thread in flight; per is a multiple of 4 * 256.
template <bool NT>
__global__ __launch_bounds__(256) void read_stream(const float4* __restrict__ buf, long long per, float* sink) {
  const int t = threadIdx.x;
  const float4* p = buf + per * blockIdx.x;
  float acc = 0.f;
  for (long long i = 0; i < per; i += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4* q = p + i + u * 256 + t;
      v[u] = NT ? ld_stream(reinterpret_cast<const float*>(q)) : *q;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  if (acc == -1.25e-30f) sink[0] = acc;  // never true for the data written below
}

// The same loads, every workgroup reading the first `span` float4 (2 MB, held in
// each XCD's L2) over and over: the rate an L2-resident operand reaches
// registers, against the LDS-direct rate of the rings below.
__global__ __launch_bounds__(256) void read_l2(const float4* __restrict__ buf, int span, int iters, float* sink) {
  const int t = threadIdx.x;
  const int off = (blockIdx.x * 4096) % span;  // spread the workgroups' starting points
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = buf[(off + it * 1024 + u * 256 + t) % span];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  if (acc == -1.25e-30f) sink[0] = acc;
}

// ------------------------------------------------------------ LDS-direct tile rings
// One wave per workgroup streams tiles of 16 KB (8 KB of K, 8 KB of V, 16 loads
// of 1 KB) into an S-stage LDS ring with global_load_lds, as the attention
// kernel does; nothing reads the ring.  The buffers hold T rows of 2 KB (eight
// heads of 256 B, the cache row of one position).  MODE 0: tile j is the 8 KB
// at j * 8 KB (contiguous); MODE 1: one head's 256 B of 32 consecutive rows,
// tiles head-major (the attention kernel's items); MODE 2: the same tiles with
// the heads interleaved (tile j: row block j / 8, head j % 8); MODE 3: tile j
// is the 8 KB at (j mod 256) * 8 KB, so every tile comes from the same 2 MB,
// which stays in each XCD's L2 (the rate an L2-resident operand reaches LDS);
// MODE 4: workgroup w streams head w mod 8 of its group's rows (groups of 8
// workgroups cut the 32-row blocks into equal runs: the attention kernel's
// head-synchronous schedule); MODE 5: two adjacent heads (512 B) of 16 rows per
// tile, groups of 4 workgroups.
template <int L, int A>
__device__ __forceinline__ void wait_ring(int ahead) {
  if constexpr (A == 0) {
    vm_wait<0>();
  } else {
    if (ahead >= A) vm_wait<A * L>();
    else wait_ring<L, A - 1>(ahead);
  }
}

template <int MODE, int S>
__global__ __launch_bounds__(64) void tile_ring(const uint8_t* K, const uint8_t* V, int T, int ntiles) {
  static_assert(S >= 2 && (S - 2) * 16 < 64, "ring depth");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * 16384];
  const int lane = threadIdx.x, G = gridDim.x, w = blockIdx.x;
  // modes 4 / 5: groups of 8 (4) workgroups share one range of key tiles
  const int gs = MODE == 4 ? 8 : MODE == 5 ? 4 : 1;
  const int nt = MODE == 4 ? T / 32 : MODE == 5 ? T / 16 : ntiles;
  const int q = w / gs, Q = G / gs;
  const int j0 = int((long long)nt * q / Q), j1 = int((long long)nt * (q + 1) / Q);
  const uint32_t r0 = __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t(ring)));
  const int nkt = T / 32;
  auto issue = [&](int j, int st) {
    size_t base;
    if (MODE == 4) {
      // head-synchronous: workgroup w streams head w % 8; groups of 8 cut the key tiles
      base = size_t(j) * 32 * 2048 + size_t(w % 8) * 256;
    } else if (MODE == 5) {
      // two heads per workgroup: 16 keys x 512 B per tile buffer
      base = size_t(j) * 16 * 2048 + size_t(w % 4) * 512;
    } else if (MODE == 0) {
      base = size_t(j) * 8192;
    } else if (MODE == 3) {
      base = size_t(j % 256) * 8192;
    } else {
      const int g = MODE == 1 ? j / nkt : j % 8, kt = MODE == 1 ? j % nkt : j / 8;
      base = size_t(kt) * 32 * 2048 + size_t(g) * 256;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // MODE 0: 1 KB contiguous; else rows 4 i .. 4 i + 3 of the head, 16 lanes each
      const uint32_t vo = MODE == 0 || MODE == 3 ? uint32_t(i * 1024 + lane * 16)
                        : MODE == 5 ? uint32_t((2 * i + lane / 32) * 2048 + (lane % 32) * 16)
                                    : uint32_t((4 * i + lane / 16) * 2048 + (lane % 16) * 16);
      dma16(K + base, vo, r0 + st * 16384 + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t vo = MODE == 0 || MODE == 3 ? uint32_t(i * 1024 + lane * 16)
                        : MODE == 5 ? uint32_t((2 * i + lane / 32) * 2048 + (lane % 32) * 16)
                                    : uint32_t((4 * i + lane / 16) * 2048 + (lane % 16) * 16);
      dma16(V + base, vo, r0 + st * 16384 + 8192 + i * 1024);
    }
  };
  for (int s = 0; s < S - 1; ++s)
    if (j0 + s < j1) issue(j0 + s, s);
  int st = 0;
  for (int j = j0; j < j1; ++j) {
    wait_ring<16, S - 2>(min(S - 2, j1 - 1 - j));  // tile j has landed
    if (j + S - 1 < j1) issue(j + S - 1, st == 0 ? S - 1 : st - 1);
    st = st == S - 1 ? 0 : st + 1;
  }
  vm_wait<0>();
}

// ------------------------------------------------------------ matrix instructions
// Each wave runs `iters` rounds of NACC independent 32x32x16 bf16 MFMAs (NACC
// accumulators, so the matrix pipe never waits on a result).
template <int NACC>
__global__ __launch_bounds__(256) void mfma_rate(int iters, float* sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __bf16(float((t + e) & 7) * 0.125f);
    b[e] = __bf16(float((t * 3 + e) & 7) * 0.0625f);
  }
  floatx16 acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) acc[k] = floatx16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = mfma32x32x16(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k) s += acc[k][0] + acc[k][15];
  if (s == -1.25e-30f) sink[t] = s;
}

// ------------------------------------------------------------ driver
template <typename F>
static double time_us(F launch, int reps = 10, int warm = 3) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int i = 0; i < warm; ++i) launch();
  CHECK(hipEventRecord(e0));
  for (int i = 0; i < reps; ++i) launch();
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return ms * 1e3 / reps;
}

__global__ void fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x) p[i] = v;
}

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  std::printf("# compute units %d\n", cus);
  float* sink;
  CHECK(hipMalloc(&sink, 1024 * sizeof(float)));

  // plain streaming: 1 GiB read once per launch, four workgroups per CU
  {
    const int G = 4 * cus;
    const long long per = (1LL << 26) / G / 1024 * 1024;  // float4 per workgroup
    const size_t n4 = size_t(per) * G;
    float4* buf;
    CHECK(hipMalloc(&buf, n4 * sizeof(float4)));
    hipLaunchKernelGGL(fill_u32, dim3(4096), dim3(256), 0, 0, reinterpret_cast<uint32_t*>(buf), n4 * 4, 0x3c000000u);
    CHECK(hipDeviceSynchronize());
    const double bytes = double(n4) * 16;
    const double tn = time_us([&] { hipLaunchKernelGGL(read_stream<true>, dim3(G), dim3(256), 0, 0, buf, per, sink); });
    const double tp = time_us([&] { hipLaunchKernelGGL(read_stream<false>, dim3(G), dim3(256), 0, 0, buf, per, sink); });
    CHECK(hipGetLastError());
    std::printf("read_stream_nt      bytes %.0f  us %.1f  TB/s %.2f\n", bytes, tn, bytes / tn / 1e6);
    std::printf("read_stream_plain   bytes %.0f  us %.1f  TB/s %.2f\n", bytes, tp, bytes / tp / 1e6);
    for (int wpc : {4, 8}) {
      const int G2 = wpc * cus / 4, span = 1 << 17, iters = 2048;  // 2 MB; 8 MB per workgroup
      const double b2 = double(G2) * iters * 1024 * 16;
      const double t2 = time_us([&] { hipLaunchKernelGGL(read_l2, dim3(G2), dim3(256), 0, 0, buf, span, iters, sink); });
      CHECK(hipGetLastError());
      std::printf("read_l2_w%-10d bytes %.0f  us %.1f  TB/s %.2f  GB/s per CU %.1f\n", wpc, b2, t2, b2 / t2 / 1e6,
                  b2 / t2 / 1e3 / cus);
    }
    CHECK(hipFree(buf));
  }

  // LDS-direct tile rings over K and V of 73 728 rows of 2 KB (302 MB, the 8B
  // round's context cache of one layer), one tile of one head per 16 KB stage
  {
    const int T = 73728, ntiles = T / 4;  // 8 KB tiles per buffer
    uint8_t *K, *V;
    CHECK(hipMalloc(&K, size_t(T) * 2048));
    CHECK(hipMalloc(&V, size_t(T) * 2048));
    hipLaunchKernelGGL(fill_u32, dim3(4096), dim3(256), 0, 0, reinterpret_cast<uint32_t*>(K), size_t(T) * 512, 1u);
    hipLaunchKernelGGL(fill_u32, dim3(4096), dim3(256), 0, 0, reinterpret_cast<uint32_t*>(V), size_t(T) * 512, 1u);
    CHECK(hipDeviceSynchronize());
    const double bytes = 2.0 * T * 2048;
    auto run = [&](auto kern, int G, const char* name) {
      const double us = time_us([&] { hipLaunchKernelGGL(kern, dim3(G), dim3(64), 0, 0, K, V, T, ntiles); });
      CHECK(hipGetLastError());
      std::printf("%-19s bytes %.0f  us %.1f  TB/s %.2f  (grid %d)\n", name, bytes, us, bytes / us / 1e6, G);
    };
    run(tile_ring<0, 5>, cus, "ring_contiguous");
    run(tile_ring<1, 5>, cus, "ring_head_256B");
    run(tile_ring<2, 5>, cus, "ring_head_cycle");
    run(tile_ring<1, 3>, 3 * cus, "ring_head_256B_x3");
    run(tile_ring<4, 5>, cus, "ring_headsync");
    run(tile_ring<4, 3>, 3 * cus, "ring_headsync_x3");
    run(tile_ring<5, 5>, cus, "ring_2heads_512B");
    run(tile_ring<5, 3>, 3 * cus, "ring_2heads_512B_x3");
    // L2-resident tiles: 512 tiles of 16 KB per workgroup from the first 2 MB
    auto run_l2 = [&](auto kern, int G, const char* name) {
      const int nt = 512 * G;
      const double b = double(nt) * 16384;
      const double us = time_us([&] { hipLaunchKernelGGL(kern, dim3(G), dim3(64), 0, 0, K, V, T, nt); });
      CHECK(hipGetLastError());
      std::printf("%-19s bytes %.0f  us %.1f  TB/s %.2f  GB/s per CU %.1f  (grid %d)\n", name, b, us, b / us / 1e6,
                  b / us / 1e3 / cus, G);
    };
    run_l2(tile_ring<3, 5>, cus, "ring_l2_1wave");
    run_l2(tile_ring<3, 3>, 3 * cus, "ring_l2_3waves");
    CHECK(hipFree(K));
    CHECK(hipFree(V));
  }

  // back-to-back 32x32x16 bf16 MFMAs: one wave per SIMD with 16 chains, two
  // waves per SIMD with 8 chains each (their accumulators fit the registers)
  {
    const int iters = 4096;
    auto run = [&](auto kern, int nacc, int G, const char* name) {
      const double flops = double(G) * 4 * iters * nacc * 2.0 * 32 * 32 * 16;
      const double us = time_us([&] { hipLaunchKernelGGL(kern, dim3(G), dim3(256), 0, 0, iters, sink); });
      CHECK(hipGetLastError());
      std::printf("%-19s flops %.0f  us %.1f  TFLOP/s %.1f\n", name, flops, us, flops / us / 1e6);
    };
    run(mfma_rate<16>, 16, cus, "mfma_bf16_1wave");
    run(mfma_rate<8>, 8, 2 * cus, "mfma_bf16_2waves");
  }
  CHECK(hipFree(sink));
  return 0;
}
