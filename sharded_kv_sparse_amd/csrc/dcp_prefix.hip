// Prefill over a cached prefix: the prefix's KV is gathered from the shards
// in bounded chunks, each chunk is attended with its LSE (the dense decode
// kernels, see dcp_api.cpp), and the chunks' partials are merged into a
// running result.
//
// Pages: [P1] "feat: support decode context parallelism for PyTorch MLA",
// Summary (prefill gathers the cached-prefix KV in bounded chunks) and the
// review exchange on prefix_output (the merge arithmetic is fp32, the
// running output is stored in BF16); [P2] "Feat[DCP] Support decode context
// parallelism for DSA models with the flashmla_kv backend", summary (with an
// FP8 cache the gathered temporary buffer keeps the packed FP8 format, so
// nothing is dequantised or quantised again).
//
// Gather: position t of a sequence has slot g = BT[t div (page*N)] * page*N
// + t mod (page*N), i.e. row g div N of shard g mod N.  One wave copies one
// token's row (36 x 16 bytes FP8 plus the 4-byte scale, or 72 x 16 bytes
// BF16) into the chunk buffer; memory-bound: 2 x 580 (FP8) or 2 x 1152
// (BF16) bytes per token.
//
// Running merge: one wave per (row, head): weights from the two LSEs (a side
// with LSE = -inf is skipped, never read), O and LSE of the merge written over
// the accumulator, which is fp32 or bf16.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kPrefixThreads = 256;   // four waves, one token (gather) or one (row, head) (merge) each

template <bool FP8>
__global__ __launch_bounds__(kPrefixThreads) void gather_prefix_kernel(GatherParams p) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int j = blockIdx.x * (kPrefixThreads / 64) + (threadIdx.x >> 6);
  const int o0 = p.out_offset[b];
  const int len = p.out_offset[b + 1] - o0;
  if (j >= len) return;
  const long long t = (long long)p.pos_begin[b] + j;
  const long long span = (long long)p.page_size * p.num_shards;
  const long long lp = t / span;
  // pages beyond the block table, and rows beyond a pool, are clamped into
  // range (the result is then unspecified, but nothing is read out of bounds)
  const int page_id = p.block_table[(long long)b * p.max_pages + min(max(lp, 0LL), (long long)p.max_pages - 1)];
  const long long g = (long long)page_id * span + (t - lp * span);
  const int r = (int)(g % p.num_shards);
  const ShardArg sh = p.shard[r];
  const long long row = min(max(g / p.num_shards, 0LL), sh.pool_rows - 1);
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const char* src = static_cast<const char*>(sh.kv) + row * sh.row_stride;
  char* dst = static_cast<char*>(p.out_kv) + (long long)(o0 + j) * (FP8 ? kHeadDim : 2 * kHeadDim);
  if constexpr (FP8) {
    if (lane < kHeadDim / 16)
      *reinterpret_cast<u32x4*>(dst + 16 * lane) = *reinterpret_cast<const u32x4*>(src + 16 * lane);
    if (lane == kHeadDim / 16)
      p.out_scale[o0 + j] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sh.scale) +
                                                            row * sh.scale_stride);
  } else {
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = *reinterpret_cast<const u32x4*>(src + 16 * lane);
    if (lane < 2 * kHeadDim / 16 - 64)
      *reinterpret_cast<u32x4*>(dst + 1024 + 16 * lane) = *reinterpret_cast<const u32x4*>(src + 1024 + 16 * lane);
  }
}

__global__ __launch_bounds__(kPrefixThreads) void merge_into_kernel(
    void* __restrict__ o_acc, float* __restrict__ lse_acc, const float* __restrict__ o_new,
    const float* __restrict__ lse_new, long long pairs, int dv, int acc_bf16) {
  const long long pair = (long long)blockIdx.x * (kPrefixThreads / 64) + (threadIdx.x >> 6);
  if (pair >= pairs) return;
  const int lane = threadIdx.x & 63;
  const int chunks = dv / 4;
  const float la = lse_acc[pair], ln = lse_new[pair];
  const float m = fmaxf(la, ln);
  const bool va = la > kNegInf, vn = ln > kNegInf;
  const float wa = va ? fast_exp2((la - m) * kLog2e) : 0.f;
  const float wn = vn ? fast_exp2((ln - m) * kLog2e) : 0.f;
  const float sum = wa + wn;
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  const float ca = wa * inv, cn = wn * inv;
  for (int c = lane; c < chunks; c += 64) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (va) {
      if (acc_bf16) {
        const uint2 u = reinterpret_cast<const uint2*>(o_acc)[pair * chunks + c];
        acc = ca * f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                         __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
      } else {
        acc = ca * reinterpret_cast<const f32x4*>(o_acc)[pair * chunks + c];
      }
    }
    if (vn) acc += cn * reinterpret_cast<const f32x4*>(o_new)[pair * chunks + c];
    if (acc_bf16) {
      const unsigned lo = f32_to_bf16_bits(acc[0]) | ((unsigned)f32_to_bf16_bits(acc[1]) << 16);
      const unsigned hi = f32_to_bf16_bits(acc[2]) | ((unsigned)f32_to_bf16_bits(acc[3]) << 16);
      reinterpret_cast<uint2*>(o_acc)[pair * chunks + c] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<f32x4*>(o_acc)[pair * chunks + c] = acc;
    }
  }
  if (lane == 0) lse_acc[pair] = sum > 0.f ? m + logf(sum) : kNegInf;
}

}  // namespace

hipError_t launch_gather_prefix(const GatherParams& p, bool fp8, int max_len, hipStream_t stream) {
  const dim3 grid((unsigned)((max_len + kPrefixThreads / 64 - 1) / (kPrefixThreads / 64)),
                  (unsigned)p.num_seqs);
  void* args[] = {(void*)&p};
  const void* fn = fp8 ? (const void*)gather_prefix_kernel<true> : (const void*)gather_prefix_kernel<false>;
  return hipLaunchKernel(fn, grid, dim3(kPrefixThreads), args, 0, stream);
}

hipError_t launch_merge_into(void* o_acc, float* lse_acc, const float* o_new, const float* lse_new,
                             long long rows, int heads, int dv, int acc_bf16, hipStream_t stream) {
  long long pairs = rows * heads;
  const long long blocks = (pairs + kPrefixThreads / 64 - 1) / (kPrefixThreads / 64);
  void* args[] = {(void*)&o_acc, (void*)&lse_acc, (void*)&o_new, (void*)&lse_new, (void*)&pairs,
                  (void*)&dv, (void*)&acc_bf16};
  return hipLaunchKernel((const void*)merge_into_kernel, dim3((unsigned)blocks), dim3(kPrefixThreads),
                         args, 0, stream);
}

}  // namespace dcp
