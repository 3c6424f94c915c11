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

// fp32 -> bf16 by gfx950's packed conversion (v_cvt_pk_bf16_f32): round to
// nearest even, identical to rounding the fp32 bit pattern for every finite
// value and infinity (checked over all 2^32 patterns); NaN stays NaN.  One
// instruction instead of the bit arithmetic and its NaN branch.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ inline uint16_t f2bf(float f) { return (uint16_t)pack_bf(f, 0.f); }

__device__ inline float lo_bf(uint32_t w) { return bf2f((uint16_t)(w & 0xFFFFu)); }
__device__ inline float hi_bf(uint32_t w) { return bf2f((uint16_t)(w >> 16)); }

// 8 bf16 in four dwords <-> the MFMA operand vector type.
__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ inline f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: lane l supplies row (column) l % 16 of A (B)
// at k-slots 8 (l / 16) .. + 7; the 16 x 16 fp32 result: lane l holds
// column l % 16, rows 4 (l / 16) .. + 3.
__device__ inline f32x4_t mfma16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// LDS byte address of a pointer into shared memory.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One direct global -> LDS copy (gfx950 global_load_lds_dwordx4): lane l's
// 16 bytes at g land at lds + 16 l (lds wave-uniform, through M0).  Issued
// as asm so that the compiler's wait insertion does not track it: seeing an
// LDS store in flight, it would drain every outstanding global load
// (vmcnt(0)) before each LDS read that follows, including the reads of a
// stage that an earlier wait and barrier already made complete, and so
// serialize a load ring.  Kernels that use it order the copies themselves:
// a vmcnt wait and a workgroup barrier before any wave reads the stage.
// The instruction has no register result; the s_nop covers the one wait
// state that a write of M0 needs before an LDS DMA.
__device__ inline void lds_dma16(const void* g, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives 16-bit element i & 3 of the 8-byte pieces that
// lanes 4 j + (i >> 2), j = 0..3, address.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ inline u32x2_t lds_tr16(const void* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) i16x4_t*)(const __attribute__((address_space(3))) char*)p));
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
