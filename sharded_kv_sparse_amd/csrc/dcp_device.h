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

// Max with the value of lane ^ 16 and of lane ^ 32, through the gfx950 row
// swaps (VALU only, no LDS round trip).  permlane16_swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second, so
// with both operands = v the pair holds {v[lane], v[lane ^ 16]} in some
// order; permlane32_swap does the same for the two 32-lane halves.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^e as a float, for -126 <= e <= 127.
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((unsigned)(e + 127) << 23); }

// Largest e with x * 2^e <= 448 (the E4M3 maximum 1.75 * 2^8), clamped to
// [-120, 120]; 0 when x is not positive.  From the bits of x = 1.m * 2^E:
// e = 8 - E when 1.m <= 1.75 (mantissa field <= 0x600000), else 7 - E.
__device__ __forceinline__ int e4m3_exponent(float x) {
  const unsigned u = __float_as_uint(x);
  const int E = (int)(u >> 23) - 127;
  const int e = 8 - E - ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return x > 0.f ? min(max(e, -120), 120) : 0;
}

// Device-scope coherent global accesses.  Buffer loads and stores with the
// SC1 cache-policy bit are the agent-scope forms of the gfx950 memory model
// (those of relaxed agent-scope atomics), so data written this way by one
// block is seen by a block on another XCD that reads it the same way after
// an agent-scope atomic has ordered the two, with no L2 write-back or
// invalidate.  A resource covers `bytes` bytes from `base`; offsets are in
// bytes and out-of-range accesses read 0 / are dropped.
constexpr int kCachePolicySc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 load_coherent4(__amdgpu_buffer_rsrc_t r, unsigned off) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicySc1));
}
__device__ __forceinline__ float load_coherent(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCachePolicySc1));
}
__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, unsigned off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, kCachePolicySc1);
}

// Eight-byte coherent accesses (four fp16 values).
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
__device__ __forceinline__ u32x2 load_coherent2(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCachePolicySc1));
}
__device__ __forceinline__ void store_coherent2(__amdgpu_buffer_rsrc_t r, unsigned off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCachePolicySc1);
}
// Four floats as fp16 (round to nearest even) and back.  (Whole-vector bit
// casts only: a bit cast of a single vector element has been seen to lose
// the other element.)
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 pack_f16x4(f32x4 v) {
  const f16x4 h = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  return __builtin_bit_cast(u32x2, h);
}
__device__ __forceinline__ f32x4 unpack_f16x4(u32x2 u) {
  const f16x4 h = __builtin_bit_cast(f16x4, u);
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// Plain buffer reads of a bounded table: offsets in bytes, reads past the
// `bytes` the resource covers return 0 without touching memory.
__device__ __forceinline__ int load_bounded(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

}  // namespace dcp
