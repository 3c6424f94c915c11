// Shared device/host helpers for the gfx950 kernels of libmt.
//
// Conventions used by every kernel:
//  - bf16 values travel as uint16_t bit patterns (RNE from fp32); math is fp32.
//  - MFMA: v_mfma_f32_32x32x16_bf16.  Operand fragments are 8 bf16 per lane.
//    For an M x K operand tile A (32 x 16), lane l supplies row (l % 32) and
//    the 8 k-slots 8*(l/32) .. 8*(l/32)+7; the N x K operand B likewise
//    supplies column (l % 32).  Any fixed assignment of k-slots to actual k
//    indices is valid as long as A and B use the same one (the product sums
//    over k).  The 32 x 32 fp32 result: lane l holds column (l % 32) and, in
//    accumulator element 4*j + i, row 8*j + 4*(l/32) + i (j, i in 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline float bf2f(uint16_t b) {
  union { uint32_t u; float f; } c;
  c.u = ((uint32_t)b) << 16;
  return c.f;
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN keeping the sign.
__host__ __device__ inline uint16_t f2bf(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  uint32_t u = c.u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

__device__ inline float lo_bf(uint32_t w) { return bf2f((uint16_t)(w & 0xFFFFu)); }
__device__ inline float hi_bf(uint32_t w) { return bf2f((uint16_t)(w >> 16)); }
__device__ inline uint32_t pack_bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// 8 bf16 in four dwords <-> the MFMA operand vector type.
__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ inline f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Wave-level reductions over all 64 lanes (butterfly via ds_swizzle-free shuffles).
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace mt
