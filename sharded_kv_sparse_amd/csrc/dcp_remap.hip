// Step 1: index remap of a global top-k slot table into per-shard compacted
// local slot ids ([P3] "[DSA] Fix decode context parallelism for RoPE sparse
// attention on Blackwell", Modifications, Index remap).
//
// One block of four waves per row.  Wave w owns a contiguous quarter of the
// row.  Pass 1 counts, per shard, the entries of each 64-entry chunk with a
// wave ballot; the per-wave totals are exchanged through LDS.  Pass 2 walks
// the same chunks again and places every kept entry at
//   (kept entries of earlier waves) + (earlier chunks of this wave)
//   + (lower lanes of this chunk with the same shard)       [mbcnt prefix]
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

__global__ __launch_bounds__(kRemapThreads) void remap_kernel(
    const int* __restrict__ topk_global, int rows, int k, int num_shards, int shard_sel,
    int* __restrict__ topk_local, int* __restrict__ counts) {
  __shared__ int wave_count[4][kMaxShards];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int out_shards = shard_sel < 0 ? num_shards : 1;
  const int* in = topk_global + (size_t)row * k;

  const int per_wave = (((k + 3) / 4) + 63) / 64 * 64;
  const int lo = min(k, wave * per_wave);
  const int hi = min(k, lo + per_wave);

  // Output shard slot of an entry (-1: padding or another shard) and its local id.
  auto classify = [&](int idx, int& slot, int& local) {
    int g = idx < hi ? in[idx] : -1;
    slot = -1;
    local = 0;
    if (g >= 0) {
      int r = g % num_shards;
      local = g / num_shards;
      if (shard_sel < 0) slot = r;
      else if (r == shard_sel) slot = 0;
    }
  };

  // Pass 1: per-shard counts of this wave's quarter.
  int cnt[kMaxShards];
#pragma unroll
  for (int s = 0; s < kMaxShards; ++s) cnt[s] = 0;
  for (int base = lo; base < hi; base += 64) {
    int slot, local;
    classify(base + lane, slot, local);
#pragma unroll
    for (int s = 0; s < kMaxShards; ++s)
      if (s < out_shards) cnt[s] += __popcll(__ballot(slot == s));
  }
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < kMaxShards; ++s)
      if (s < out_shards) wave_count[wave][s] = cnt[s];
  }
  __syncthreads();

  // Pass 2: scatter to the exclusive prefix.
  int pos[kMaxShards];
#pragma unroll
  for (int s = 0; s < kMaxShards; ++s) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += (s < out_shards) ? wave_count[w][s] : 0;
    pos[s] = before;
  }
  for (int base = lo; base < hi; base += 64) {
    int slot, local;
    classify(base + lane, slot, local);
#pragma unroll
    for (int s = 0; s < kMaxShards; ++s) {
      if (s < out_shards) {
        unsigned long long m = __ballot(slot == s);
        if (slot == s)
          topk_local[((size_t)s * rows + row) * k + pos[s] + lanes_below(m)] = local;
        pos[s] += __popcll(m);
      }
    }
  }

  // Counts and the -1 tail.
  for (int s = 0; s < out_shards; ++s) {
    int total = wave_count[0][s] + wave_count[1][s] + wave_count[2][s] + wave_count[3][s];
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
