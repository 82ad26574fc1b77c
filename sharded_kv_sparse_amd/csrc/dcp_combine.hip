// Step 3 standalone: LSE-weighted merge of per-shard partials ([P1] "feat:
// support decode context parallelism for PyTorch MLA", Summary, decode bullet;
// [P3] "[DSA] Fix decode context parallelism for RoPE sparse attention on
// Blackwell", Modifications, Fixes in shared code: zero output when every
// shard is empty; [P2] "Feat[DCP] Support decode context parallelism for DSA
// models with the flashmla_kv backend", review of the LSE combine: safe
// denominator and a -inf global LSE).
//
// One wave per (row, head): every lane reads the N LSEs (broadcast loads),
// forms M = max over the shards with LSE > -inf and the weights
// e^(LSE_r - M) / sum, and merges dv/4 float4 columns of the partial outputs.
// Shards with LSE = -inf are skipped, never read, so garbage there is inert.
// Memory-bound: N*dv*4 bytes in, dv*4 (or dv*2) bytes out per (row, head).
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int num_shards,
    long long pairs, int dv, void* __restrict__ o, float* __restrict__ lse, int out_bf16) {
  const long long pair = (long long)blockIdx.x * (kCombineThreads / 64) + (threadIdx.x >> 6);
  if (pair >= pairs) return;
  const int lane = threadIdx.x & 63;
  const int chunks = dv / 4;

  float m = kNegInf;
  for (int r = 0; r < num_shards; ++r) {
    float l = lse_part[(long long)r * pairs + pair];
    m = (l > m) ? l : m;
  }
  if (m == kNegInf) {
    for (int c = lane; c < chunks; c += 64) {
      if (out_bf16) {
        reinterpret_cast<uint2*>(o)[pair * chunks + c] = make_uint2(0u, 0u);
      } else {
        reinterpret_cast<float4*>(o)[pair * chunks + c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (lane == 0) lse[pair] = kNegInf;
    return;
  }
  float wsum = 0.f;
  for (int r = 0; r < num_shards; ++r) {
    float l = lse_part[(long long)r * pairs + pair];
    if (l > kNegInf) wsum += fast_exp2((l - m) * kLog2e);
  }
  const float inv = 1.0f / wsum;
  for (int c = lane; c < chunks; c += 64) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < num_shards; ++r) {
      float l = lse_part[(long long)r * pairs + pair];
      if (l > kNegInf) {
        float w = fast_exp2((l - m) * kLog2e) * inv;
        float4 v = reinterpret_cast<const float4*>(o_part)[((long long)r * pairs + pair) * chunks + c];
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
    }
    if (out_bf16) {
      unsigned lo = f32_to_bf16_bits(acc.x) | ((unsigned)f32_to_bf16_bits(acc.y) << 16);
      unsigned hi = f32_to_bf16_bits(acc.z) | ((unsigned)f32_to_bf16_bits(acc.w) << 16);
      reinterpret_cast<uint2*>(o)[pair * chunks + c] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<float4*>(o)[pair * chunks + c] = acc;
    }
  }
  if (lane == 0) lse[pair] = m + logf(wsum);
}

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part, int num_shards,
                          long long rows, int heads, int dv, void* o, float* lse, int out_bf16,
                          hipStream_t stream) {
  long long pairs = rows * heads;
  long long blocks = (pairs + (kCombineThreads / 64) - 1) / (kCombineThreads / 64);
  void* args[] = {(void*)&o_part, (void*)&lse_part, (void*)&num_shards, (void*)&pairs,
                  (void*)&dv, (void*)&o, (void*)&lse, (void*)&out_bf16};
  return hipLaunchKernel((const void*)combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads),
                         args, 0, stream);
}

}  // namespace dcp
