// Device-side helpers shared by the kvsel kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;       // the only head dimension the kernels take
constexpr int kRowBytes = kHeadDim * 2;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- MFMA ----
//
// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32], one wave.
// Lane l supplies A[m = l%32][kk = 8*(l/32) + j] and B[kk = 8*(l/32)+j]
// [n = l%32] for j < 8; accumulator register i of lane l holds
// C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32].
//
// Head-dim order: the contraction runs over d = 128 in 8 steps. At step s,
// lane half hf = l/32 supplies elements [64*hf + 8*s, 64*hf + 8*s + 8) of
// its row. A and B use the same order, so the sum covers every d once, and
// each lane reads one contiguous 128-byte half-row for the whole product.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (M index) of accumulator register i for this lane.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

__device__ __forceinline__ bf16x8 ld16(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// The 8 per-step operands of one lane: row base pointer (bytes), half hf.
__device__ __forceinline__ void load_half_row(const void* row, int hf, bf16x8 (&x)[8]) {
  const char* p = reinterpret_cast<const char*>(row) + hf * 128;
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = ld16(p + 16 * s);
}

// Same, for data read exactly once (non-temporal: not kept in the caches).
__device__ __forceinline__ void load_half_row_stream(const void* row, int hf, bf16x8 (&x)[8]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(row) + hf * 128);
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(p + s));
}

__device__ __forceinline__ void zero_ops(bf16x8 (&x)[8]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ----------------------------------------------------------- dispatch ----
//
// The command processor hands workgroup w of a 1-D grid to XCD w % 8, and
// each XCD has its own L2. Workgroups that re-read the same operand should
// share an L2, so a kernel works on the logical index returned here: the
// workgroups of one XCD take one contiguous logical range (a bijection on
// [0, total)).
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total / kXcds, r = total % kXcds, x = w % kXcds;
  return x * q + min(x, r) + w / kXcds;
}

// ---------------------------------------------------------------- math ----

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of the lane 32 away (lane l ^ 32) by one v_permlane32_swap, which
// swaps the upper half of its first operand with the lower half of its
// second: no LDS round trip (a ds_bpermute's) on the way.
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Merge two (max, sum-of-exp2) pairs; max may be -inf with sum 0.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float mm = fmaxf(m, m2);
  if (mm == neg_inf()) return;
  s = s * fast_exp2(m - mm) + s2 * fast_exp2(m2 - mm);
  m = mm;
}

}  // namespace kvsel
