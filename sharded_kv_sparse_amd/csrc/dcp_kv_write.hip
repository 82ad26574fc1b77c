// Interleaved KV-cache write with FP8 quantisation: the new tokens' key rows
// go to the shard that owns their slot, quantised to E4M3FN with one fp32
// scale per token when the pool is FP8.
//
// Pages: [P1] "feat: support decode context parallelism for PyTorch MLA",
// File summaries (the KV-cache fill kernel writes new tokens interleaved over
// the DCP ranks); [P2] "Feat[DCP] Support decode context parallelism for DSA
// models with the flashmla_kv backend", summary (FP8 caches hold packed FP8)
// and the review of the gathered buffer (rows are quantised when written to
// the persistent cache).  Slot g of the DCP-wide pool is row g div N of shard
// g mod N (interleave 1).  The pages give no scale rule; the one used: scale =
// amax / 448 with amax the largest |x| of the token's 576 values, inverse
// scale 448 / amax (both 1 for an all-zero token), and code = E4M3FN(x *
// inverse scale), round to nearest even, the fp32 product clamped to +-448.
// The two divisions are IEEE fp32 divisions, once per token.
//
// One wave per token: lane l holds latent values 8l .. 8l + 7 (16 bytes of
// the bf16 row), lanes 0..7 also RoPE values 512 + 8l .. + 7; the largest
// magnitude is reduced across the wave.  FP8 rows are stored as 8-byte code
// groups, the scale by lane 0; BF16 rows as 16-byte groups.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kWriteThreads = 256;                 // four tokens per block

template <bool FP8>
__global__ __launch_bounds__(kWriteThreads) void kv_write_kernel(KvWriteParams p) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * (kWriteThreads / 64) + (threadIdx.x >> 6);
  if (t >= p.tokens) return;
  const int g = p.slots[t];
  if (g < 0) return;                                 // skipped token
  const int r = g % p.num_shards;
  const long long row = g / p.num_shards;
  const ShardArg sh = p.shard[r];
  if (row >= sh.pool_rows) return;                   // beyond the shard's pool: skipped
  const bool rope = lane < 8;
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const char* src = static_cast<const char*>(p.kv_new) + t * (kHeadDim * 2);
  const u32x4 lat = *reinterpret_cast<const u32x4*>(src + 16 * lane);
  const u32x4 rp = rope ? *reinterpret_cast<const u32x4*>(src + 1024 + 16 * lane) : u32x4{0, 0, 0, 0};
  char* dst = static_cast<char*>(const_cast<void*>(sh.kv)) + row * sh.row_stride;
  if constexpr (!FP8) {
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = lat;
    if (rope) *reinterpret_cast<u32x4*>(dst + 1024 + 16 * lane) = rp;
  } else {
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(lat[i] << 16);
      x[2 * i + 1] = __uint_as_float(lat[i] & 0xffff0000u);
      x[8 + 2 * i] = __uint_as_float(rp[i] << 16);
      x[8 + 2 * i + 1] = __uint_as_float(rp[i] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));   // RoPE slots are 0 off lanes 0..7
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 1.0f;
    auto code8 = [&](int base) -> uint2 {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(x[base + i] * inv, -448.0f), 448.0f);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
      return make_uint2((unsigned)lo, (unsigned)hi);
    };
    *reinterpret_cast<uint2*>(dst + 8 * lane) = code8(0);
    if (rope) *reinterpret_cast<uint2*>(dst + 512 + 8 * lane) = code8(8);
    if (lane == 0)
      *reinterpret_cast<float*>(reinterpret_cast<char*>(const_cast<float*>(sh.scale)) + row * sh.scale_stride) =
          scale;
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteParams& p, bool fp8, hipStream_t stream) {
  const long long blocks = (p.tokens + kWriteThreads / 64 - 1) / (kWriteThreads / 64);
  void* args[] = {(void*)&p};
  const void* fn = fp8 ? (const void*)kv_write_kernel<true> : (const void*)kv_write_kernel<false>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kWriteThreads), args, 0, stream);
}

}  // namespace dcp
