// Device-side helpers shared by the gfx950 MSA kernels: vector types, the
// 16x16x32 bf16 MFMA, bf16 conversion and wavefront (64-lane) reductions.
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_bf16, wave64,
// lane l, q = l / 16, c = l % 16):
//   A (16 x 32): lane holds A[c][8q .. 8q+7]       (8 bf16)
//   B (32 x 16): lane holds B[8q .. 8q+7][c]       (8 bf16)
//   D (16 x 16): lane holds D[4q + r][c], r = 0..3 (4 fp32)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_launch.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Cross-lane exchange within a wave (ds_bpermute based).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Order-preserving map of fp32 onto uint32 (larger float -> larger uint).
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace msa
