// Device helpers for the gfx950 kernels (vector types, LDS access, MFMA,
// FP8 conversion, wave reductions, waitcnt).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;

#define DCP_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// The global->LDS copies of the decode pipeline are issued from inline asm
// on purpose: the compiler cannot prove that later LDS reads of other stages
// do not alias them and would otherwise drain every copy (vmcnt(0)) before
// each LDS read, serialising the pipeline.  Their completion is tracked by
// hand with wait_vmcnt<>, counted per wave; the "memory" clobbers keep the
// compiler from moving LDS or global accesses across these statements.

// Wait until at most VM vector-memory operations of this wave are in flight.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM) : "memory");
}

// Workgroup barrier that drains this wave's LDS operations but leaves its
// in-flight global->LDS copies running.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct global -> LDS copies: lane l's bytes land at lds_base + l * size.
// lds_base must be the same for the whole wave (it is read from lane 0).
// (The instruction's immediate offset field would be added to the LDS
// address as well as to the global one, so these helpers never use it.)
__device__ __forceinline__ void dma16(const void* src, DCP_LDS void* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, DCP_LDS void* lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// Forces a value to be materialised here (its loads completed) without
// emitting any instruction.
template <typename V>
__device__ __forceinline__ void touch(const V& v) {
  asm volatile("" ::"v"(v));
}

// FP8 E4M3FN -> bf16 / f16, exact (scale 1).  Eight codes in two dwords, in
// byte order.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(int lo, int hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ f16x8 e4m3x8_to_f16(int lo, int hi) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)lo, 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)hi, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
__device__ __forceinline__ __bf16 f32_to_bf16(float f) {
  unsigned short b = f32_to_bf16_bits(f);
  return __builtin_bit_cast(__bf16, b);
}
__device__ __forceinline__ float bf16_to_f32(__bf16 h) {
  return __uint_as_float(((unsigned)__builtin_bit_cast(unsigned short, h)) << 16);
}

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace dcp
