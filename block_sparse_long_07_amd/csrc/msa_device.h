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

typedef __attribute__((address_space(3))) char lds_char;

// Direct global -> LDS loads (no registers): lane L's SIZE bytes from src land
// at lds + SIZE*L, lds being the same for the whole wave. They are written as
// inline assembly because the compiler, unable to tell which LDS bytes such a
// load writes, would otherwise wait for every one of them before any later
// LDS read, which serialises double buffering. The caller therefore waits
// itself (s_waitcnt vmcnt, plus a barrier when other waves read the data).
// Every wait on them must be an s_waitcnt the compiler sees (the builtins
// below): a wait the compiler cannot see leaves it assuming older loads are
// still in flight, and its own vmcnt(0) before their first use would then
// also wait for the LDS loads.
__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
// s_waitcnt through the builtin (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8), so that the compiler's own wait tracking knows
// about it.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_vmcnt5() { __builtin_amdgcn_s_waitcnt(0x0F75); }
__device__ __forceinline__ void wait_vmcnt10() { __builtin_amdgcn_s_waitcnt(0x0F7A); }
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// vmcnt(min(n, 31)) for a wave-uniform n: at most n vector memory operations
// (those issued last) may still be in flight; a smaller count only waits more
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n < 31 ? n : 31) {
#define MSA_VMCNT_CASE(N) \
  case N:                 \
    __builtin_amdgcn_s_waitcnt(0x0F70 | N); break;
    MSA_VMCNT_CASE(0) MSA_VMCNT_CASE(1) MSA_VMCNT_CASE(2) MSA_VMCNT_CASE(3) MSA_VMCNT_CASE(4) MSA_VMCNT_CASE(5)
    MSA_VMCNT_CASE(6) MSA_VMCNT_CASE(7) MSA_VMCNT_CASE(8) MSA_VMCNT_CASE(9) MSA_VMCNT_CASE(10) MSA_VMCNT_CASE(11)
    MSA_VMCNT_CASE(12) MSA_VMCNT_CASE(13) MSA_VMCNT_CASE(14) MSA_VMCNT_CASE(15)
#undef MSA_VMCNT_CASE
    default:
      if (n >= 31) __builtin_amdgcn_s_waitcnt(0x4F7F);  // vmcnt(31)
      else if (n >= 24) __builtin_amdgcn_s_waitcnt(0x4F78);  // vmcnt(24)
      else __builtin_amdgcn_s_waitcnt(0x0F7F);  // vmcnt(15)
      break;
  }
}

// Workgroup barrier for LDS data: this wave's LDS operations complete, then
// s_barrier. Unlike __syncthreads it does not wait for outstanding global
// loads, so loads in flight (into registers or direct to LDS) stay in flight
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void lds_dma16(const void* src, const lds_char* lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr(lds))
               : "memory", "m0");
}
// The same load addressed as an SGPR base (wave-uniform; taken from the first
// lane) plus a 32-bit per-lane byte offset: no per-lane 64-bit address
// arithmetic.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t voff, const lds_char* lds) {
  // readfirstlane returns int: both halves are widened from uint32_t (a sign
  // extension of the low half would corrupt the high half)
  const uint64_t u = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint64_t b = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(b), "s"(lds_addr(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* src, const lds_char* lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(lds_addr(lds))
               : "memory", "m0");
}

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

// Work item of workgroup w in a one-dimensional grid of n workgroups, so that
// each XCD runs a contiguous run of items: the dispatcher hands workgroups to
// the kXcd XCDs in turn (w mod kXcd), and XCD x is given the items after those
// of XCDs 0 .. x-1 (each holds n/kXcd of them, the first n mod kXcd one more).
// Neighbouring items, which read the same K/V blocks, then share one L2.
// A bijection of [0, n) for any n.
constexpr int kXcd = 8;
__device__ __forceinline__ int xcd_item(int w, int n) {
  const int x = w % kXcd, k = w / kXcd;
  const int q = n / kXcd, r = n % kXcd;
  return x * q + min(x, r) + k;
}

// max over the four lanes l ^ {0, 16, 32, 48} (the four lane groups of an
// MFMA 16x16 fragment column): v_permlane32_swap then v_permlane16_swap with
// both operands x return x of the partner half / row in one of the two
// results, so each step is one VALU swap and a max, with no LDS traffic.
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger uint).
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace msa
