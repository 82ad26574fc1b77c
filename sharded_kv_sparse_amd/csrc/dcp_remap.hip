// Step 1: index remap of a global top-k slot table into per-shard compacted
// local slot ids ([P3] "[DSA] Fix decode context parallelism for RoPE sparse
// attention on Blackwell", Modifications, Index remap).
//
// One block of four waves per row, over segments of 2048 entries.  In a
// segment wave w owns a contiguous quarter; every lane loads its eight
// entries before any is used.  Pass 1 counts, per shard, the entries of each
// 64-entry chunk with a wave ballot; the per-wave totals are exchanged
// through LDS.  Pass 2 places every kept entry at
//   (kept entries of earlier segments) + (of earlier waves)
//   + (of earlier chunks of this wave) + (lower lanes with the same shard)
// which is exactly its rank among the row's entries for that shard, so the
// order of the input row is preserved and the result is deterministic.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kRemapThreads = 256;

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

constexpr int kPerLane = 8;                       // entries a lane holds per segment
constexpr int kSegment = kRemapThreads * kPerLane;  // 2048 entries per segment

__global__ __launch_bounds__(kRemapThreads) void remap_kernel(
    const int* __restrict__ topk_global, int rows, int k, int num_shards, int shard_sel,
    int* __restrict__ topk_local, int* __restrict__ counts) {
  __shared__ int wave_count[4][kMaxShards];
  __shared__ int seg_base[kMaxShards];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int out_shards = shard_sel < 0 ? num_shards : 1;
  const int* in = topk_global + (size_t)row * k;
  const bool pow2 = (num_shards & (num_shards - 1)) == 0;
  const int shift = __builtin_ctz(num_shards);
  if (threadIdx.x < kMaxShards) seg_base[threadIdx.x] = 0;

  for (int seg = 0; seg < k; seg += kSegment) {
    // Wave w owns entries [seg + w*512, seg + (w+1)*512): chunk j of 64
    // entries is held by the wave's lanes in order.  All loads first.
    int slot[kPerLane], local[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int idx = seg + wave * (64 * kPerLane) + j * 64 + lane;
      slot[j] = idx < k ? in[idx] : -1;
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int g = slot[j];
      int s = -1, l = 0;
      if (g >= 0) {
        const int r = pow2 ? (g & (num_shards - 1)) : g % num_shards;
        l = pow2 ? (g >> shift) : g / num_shards;
        s = shard_sel < 0 ? r : (r == shard_sel ? 0 : -1);
      }
      slot[j] = s;
      local[j] = l;
    }
    // Pass 1: per-shard counts of this wave's part of the segment.
    int cnt[kMaxShards];
#pragma unroll
    for (int s = 0; s < kMaxShards; ++s) {
      cnt[s] = 0;
      if (s < out_shards) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) cnt[s] += __popcll(__ballot(slot[j] == s));
      }
    }
    __syncthreads();   // previous segment's readers of wave_count are done
    if (lane == 0) {
#pragma unroll
      for (int s = 0; s < kMaxShards; ++s)
        if (s < out_shards) wave_count[wave][s] = cnt[s];
    }
    __syncthreads();
    // Pass 2: scatter every kept entry to its rank among the row's entries
    // of that shard: segment base + earlier waves + earlier chunks + lower lanes.
#pragma unroll
    for (int s = 0; s < kMaxShards; ++s) {
      if (s < out_shards) {
        int pos = seg_base[s];
        for (int w = 0; w < wave; ++w) pos += wave_count[w][s];
        int* out = topk_local + ((size_t)s * rows + row) * k;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
          const unsigned long long m = __ballot(slot[j] == s);
          if (slot[j] == s) out[pos + lanes_below(m)] = local[j];
          pos += __popcll(m);
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < out_shards) {
      const int s = threadIdx.x;
      seg_base[s] += wave_count[0][s] + wave_count[1][s] + wave_count[2][s] + wave_count[3][s];
    }
  }
  __syncthreads();

  // Counts and the -1 tail.
  for (int s = 0; s < out_shards; ++s) {
    const int total = seg_base[s];
    int* out = topk_local + ((size_t)s * rows + row) * k;
    for (int j = total + threadIdx.x; j < k; j += kRemapThreads) out[j] = -1;
    if (threadIdx.x == 0) counts[(size_t)s * rows + row] = total;
  }
}

}  // namespace

hipError_t launch_remap(const int* topk_global, long long rows, int k, int num_shards, int shard,
                        int* topk_local, int* counts, hipStream_t stream) {
  int r = (int)rows;
  void* args[] = {(void*)&topk_global, (void*)&r, (void*)&k, (void*)&num_shards, (void*)&shard,
                  (void*)&topk_local, (void*)&counts};
  return hipLaunchKernel((const void*)remap_kernel, dim3((unsigned)rows), dim3(kRemapThreads),
                         args, 0, stream);
}

}  // namespace dcp
