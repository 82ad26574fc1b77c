// Step 1: index remap of a global top-k slot table into per-shard compacted
// local slot ids ([P3] "[DSA] Fix decode context parallelism for RoPE sparse
// attention on Blackwell", Modifications, Index remap).
//
// One block of four waves per (row, output shard), over segments of 2048
// entries.  In a segment wave w owns a contiguous quarter; every lane loads
// its eight entries before any is used (the blocks of a row read the same
// entries, mostly from L2).  The kept entries of each 64-entry chunk are
// counted with a wave ballot and the per-wave totals exchanged through LDS;
// every kept entry is then placed at
//   (kept entries of earlier segments) + (of earlier waves)
//   + (of earlier chunks of this wave) + (lower lanes that keep theirs)
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
  __shared__ int wave_count[2][4];
  const int row = blockIdx.x;
  const int os = blockIdx.y;                       // output shard index
  const int shard = shard_sel < 0 ? os : shard_sel;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int* in = topk_global + (size_t)row * k;
  int* out = topk_local + ((size_t)os * rows + row) * k;
  const bool pow2 = (num_shards & (num_shards - 1)) == 0;
  const int shift = __builtin_ctz(num_shards);

  int base = 0;                                    // kept entries of earlier segments
  for (int seg = 0, parity = 0; seg < k; seg += kSegment, parity ^= 1) {
    // Wave w owns entries [seg + w*512, seg + (w+1)*512): chunk j of 64
    // entries is held by the wave's lanes in order.  All loads first.
    int g[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int idx = seg + wave * (64 * kPerLane) + j * 64 + lane;
      g[j] = idx < k ? in[idx] : -1;
    }
    unsigned long long keep[kPerLane];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int r = pow2 ? (g[j] & (num_shards - 1)) : g[j] % num_shards;
      keep[j] = __ballot(g[j] >= 0 && r == shard);
      cnt += __popcll(keep[j]);
    }
    // Two copies of the per-wave counts alternate between segments, so one
    // barrier per segment suffices.
    if (lane == 0) wave_count[parity][wave] = cnt;
    __syncthreads();
    int pos = base;
    for (int w = 0; w < wave; ++w) pos += wave_count[parity][w];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      if ((keep[j] >> lane) & 1ull) {
        const int l = pow2 ? (g[j] >> shift) : g[j] / num_shards;
        out[pos + lanes_below(keep[j])] = l;
      }
      pos += __popcll(keep[j]);
    }
    base += wave_count[parity][0] + wave_count[parity][1] + wave_count[parity][2] +
            wave_count[parity][3];
  }

  // The -1 tail and the count.
  for (int j = base + threadIdx.x; j < k; j += kRemapThreads) out[j] = -1;
  if (threadIdx.x == 0) counts[(size_t)os * rows + row] = base;
}

}  // namespace

hipError_t launch_remap(const int* topk_global, long long rows, int k, int num_shards, int shard,
                        int* topk_local, int* counts, hipStream_t stream) {
  int r = (int)rows;
  void* args[] = {(void*)&topk_global, (void*)&r, (void*)&k, (void*)&num_shards, (void*)&shard,
                  (void*)&topk_local, (void*)&counts};
  const unsigned out_shards = shard < 0 ? (unsigned)num_shards : 1u;
  return hipLaunchKernel((const void*)remap_kernel, dim3((unsigned)rows, out_shards),
                         dim3(kRemapThreads), args, 0, stream);
}

}  // namespace dcp
