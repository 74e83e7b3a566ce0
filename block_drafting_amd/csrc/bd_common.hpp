// Shared device helpers of the block-draft library (gfx950, wave64).
#pragma once

#include <stddef.h>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// Round to nearest, ties to even; NaN maps to a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- streaming loads
// Non-temporal 16-byte loads for data read once per call (logits, K/V tiles,
// projection weights): they stream through the caches at low priority.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ u32x4 ld_stream_v(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ float4 ld_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- global -> LDS
// 16 bytes from global address base + voff (base the same for the whole wave)
// to LDS byte address lds_base + 16 * lane; NT marks data read once (streamed
// past the caches at low priority).  Issued as inline assembly so the compiler
// inserts no wait of its own for these loads: callers track them with
// explicit vmcnt waits and a barrier.
template <bool NT = true>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Element i of an array member (at byte offset member_offset) of the argument
// struct of a kernel whose only argument is that struct, read straight from
// the kernel-argument segment, where the struct sits at offset 0.  For a
// per-lane index: indexing the by-value argument itself would make the
// compiler copy the whole struct to private memory.
template <typename T>
__device__ __forceinline__ T kernarg_elem(size_t member_offset, int i) {
  const char* base = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  return reinterpret_cast<const T*>(base + member_offset)[i];
}

// wait until at most min(n, N) vector memory operations are outstanding (n
// known only at run time, N its compile-time bound)
template <int N>
__device__ __forceinline__ void vm_wait_le(int n) {
  if constexpr (N == 0) {
    vm_wait<0>();
  } else {
    if (n >= N) vm_wait<N>();
    else vm_wait_le<N - 1>(n);
  }
}

// sin and cos of a rotary angle given in fp64 (any size, e.g. position x
// frequency): Cody-Waite reduction by pi/2 in fp64 with a two-term pi/2, so the
// reduced |y| <= pi/4 keeps the angle's accuracy at positions in the tens of
// thousands; then the Taylor polynomials of sin (to y^9) and cos (to y^10) in
// fp32, whose truncation is below 2e-9 on |y| <= pi/4; then the quadrant's
// swap and signs.  Absolute error below 1e-7 (checked against libm in fp64).
__device__ __forceinline__ void sincos_angle(double ang, float* s_out, float* c_out) {
  const double q = rint(ang * 0.63661977236758134);  // 2 / pi
  double y = fma(-q, 1.5707963267948966, ang);
  y = fma(-q, 6.123233995736766e-17, y);
  const float x = float(y), x2 = x * x;
  float s = fmaf(x2, 1.f / 362880.f, -1.f / 5040.f);
  s = fmaf(x2, s, 1.f / 120.f);
  s = fmaf(x2, s, -1.f / 6.f);
  s = fmaf(x2 * x, s, x);
  float c = fmaf(x2, -1.f / 3628800.f, 1.f / 40320.f);
  c = fmaf(x2, c, -1.f / 720.f);
  c = fmaf(x2, c, 1.f / 24.f);
  c = fmaf(x2, c, -0.5f);
  c = fmaf(x2, c, 1.f);
  const int quad = int(q - 4.0 * floor(q * 0.25));  // q mod 4
  const float ss = (quad & 1) ? c : s, cc = (quad & 1) ? s : c;
  *s_out = (quad & 2) ? -ss : ss;
  *c_out = ((quad + 1) & 2) ? -cc : cc;
}

// 2^x with the hardware instruction (no denormal-result handling): used for
// softmax terms exp((z - max) / T), where a result below 2^-126 is negligible
// next to the term 1 of the maximum itself.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- MFMA
// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulators (gfx950).
__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D = A(16x32) * B(32x16) + C.
__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// (value, index) ordering used for argmax and top-k: larger value first,
// lower index first among equal values; index INT32_MAX marks "no element".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  if (ia == INT32_MAX) return false;
  if (ib == INT32_MAX) return true;
  if (va > vb) return true;
  if (va < vb) return false;
  return ia < ib;
}

// Value of lane l ^ J, for every lane, without the LDS permute: DPP row
// moves within rows of 16 lanes, the gfx950 permlane swaps across them.
template <int J>
__device__ __forceinline__ int xor_lane(int x) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (J == 4) {
    const int y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // row_half_mirror: l ^ 7
    return __builtin_amdgcn_mov_dpp(y, 0x1B, 0xF, 0xF, false);          // quad_perm [3, 2, 1, 0]: ^ 3
  } else if constexpr (J == 8) {
    const int y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // row_mirror: l ^ 15
    return __builtin_amdgcn_mov_dpp(y, 0x141, 0xF, 0xF, false);         // row_half_mirror: ^ 7
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return ((threadIdx.x >> 4) & 1) ? int(r[0]) : int(r[1]);
  } else {
    static_assert(J == 32, "xor distance");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? int(r[0]) : int(r[1]);
  }
}
template <int J>
__device__ __forceinline__ float xor_lane(float x) {
  return __int_as_float(xor_lane<J>(__float_as_int(x)));
}

// Lane s's value (s the same in every lane).
__device__ __forceinline__ int lane_value(int x, int s) { return __builtin_amdgcn_readlane(x, s); }
__device__ __forceinline__ float lane_value(float x, int s) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), s));
}
__device__ __forceinline__ double lane_value(double x, int s) {
  const long long u = __double_as_longlong(x);
  const unsigned lo = unsigned(__builtin_amdgcn_readlane(int(u), s));
  const unsigned hi = unsigned(__builtin_amdgcn_readlane(int(u >> 32), s));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// (value desc, index asc) order without branches
__device__ __forceinline__ bool sel_better(float v, int i, float w, int j) {
  return (v > w) | ((v == w) & (i < j));
}

// Wave-wide bitonic sort of one (value, index) pair per lane, best first:
// lane 0 ends with the best.
template <int K, int J>
__device__ __forceinline__ void bitonic_step(float& sv, int& si) {
  const int lane = threadIdx.x & 63;
  const float ov = xor_lane<J>(sv);
  const int oi = xor_lane<J>(si);
  const bool lower = (lane & J) == 0, desc = (lane & K) == 0;
  // in a descending run the lower lane keeps the better of the pair
  const bool take = (lower == desc) ? sel_better(ov, oi, sv, si) : sel_better(sv, si, ov, oi);
  sv = take ? ov : sv;
  si = take ? oi : si;
}
template <int K, int J>
__device__ __forceinline__ void bitonic_merge(float& sv, int& si) {
  bitonic_step<K, J>(sv, si);
  if constexpr (J > 1) bitonic_merge<K, J / 2>(sv, si);
}
template <int K>
__device__ __forceinline__ void bitonic_sort(float& sv, int& si) {
  if constexpr (K > 2) bitonic_sort<K / 2>(sv, si);
  bitonic_merge<K, K / 2>(sv, si);
}
__device__ __forceinline__ void wave_sort_best_first(float& sv, int& si) { bitonic_sort<64>(sv, si); }

// Order-preserving 32-bit keys of finite or infinite floats: a < b exactly
// when key(a) < key(b), with -0 taken as +0 so that equal values get equal
// keys.  key_value inverts it (giving +0 for either zero).
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The n-th largest (1 <= n <= 64) of the wave's 64 keys (one per lane),
// found bit by bit from the top: the largest T with at least n keys >= T,
// which is always one of the keys.  One compare and one ballot count per bit.
__device__ __forceinline__ uint32_t wave_nth_key(uint32_t k, int n) {
  uint32_t T = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    if (__popcll(__ballot(k >= c)) >= n) T = c;
  }
  return T;
}

// every lane gets the wave's best (value, index) pair (lowest index on ties)
template <int J>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = xor_lane<J>(v);
  const int oi = xor_lane<J>(i);
  if (better(ov, oi, v, i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<32>(v, i);
  argmax_step<16>(v, i);
  argmax_step<8>(v, i);
  argmax_step<4>(v, i);
  argmax_step<2>(v, i);
  argmax_step<1>(v, i);
}

}  // namespace bd
