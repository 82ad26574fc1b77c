// Epilogue shared by the decode kernels: per-block partial output, arrival
// counters and the LSE merge done by the last block of a row (the pack and
// combine steps fused into the attention kernel).
//
// Merge ([P1] "feat: support decode context parallelism for PyTorch MLA",
// Summary; [P3] "[DSA] Fix decode context parallelism for RoPE sparse
// attention on Blackwell", Modifications, Fixes in shared code; [P2]
// "Feat[DCP] Support decode context parallelism for DSA models with the
// flashmla_kv backend", review of the LSE combine): M = max LSE_r over
// partials with LSE_r > -inf, O = sum_r e^(LSE_r - M) O_r / sum_r e^(LSE_r - M),
// LSE = M + ln sum; O = 0 and LSE = -inf when every partial is empty.
#pragma once

#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {

// Block-wide LSE merge of n_in partials [n_in][H][512] + [n_in][H] into one
// [H][512] output (fp32 or bf16) + [H] LSE.  Weights go to LDS first; then
// every thread merges float4 columns with all of its loads for a batch of
// inputs issued before any is consumed, so the merge is bandwidth- rather
// than latency-bound.  A partial whose weight is 0 (empty shard) is loaded
// but never multiplied: the select keeps NaN garbage out.
template <int NT>
__device__ inline void merge_partials(const float* __restrict__ in_o, const float* __restrict__ in_lse,
                               int n_in, int H, void* __restrict__ out_o, int out_bf16,
                               float* __restrict__ out_lse, DCP_LDS float* wts) {
  const int tid = threadIdx.x;
  for (int h = tid; h < H; h += NT) {
    float m = kNegInf;
    for (int i = 0; i < n_in; ++i) {
      float l = __builtin_nontemporal_load(in_lse + (size_t)i * H + h);
      m = (l > m) ? l : m;
    }
    float wsum = 0.f;
    for (int i = 0; i < n_in; ++i) {
      float l = __builtin_nontemporal_load(in_lse + (size_t)i * H + h);
      float w = (m > kNegInf && l > kNegInf) ? fast_exp2((l - m) * kLog2e) : 0.f;
      wts[i * H + h] = w;
      wsum += w;
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    for (int i = 0; i < n_in; ++i) wts[i * H + h] *= inv;
    out_lse[h] = wsum > 0.f ? m + logf(wsum) : kNegInf;
  }
  __syncthreads();
  constexpr int C = kVDim / 4;
  constexpr int B = 8;                 // inputs loaded per batch
  constexpr int CH = 2;                // columns per thread per pass
  const f32x4* src = reinterpret_cast<const f32x4*>(in_o);
  for (int base = tid; base < H * C; base += NT * CH) {
    f32x4 acc[CH];
    int hh[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      hh[u] = min(base + u * NT, H * C - 1) / C;
    }
    for (int i0 = 0; i0 < n_in; i0 += B) {
      f32x4 v[CH][B];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int idx = min(base + u * NT, H * C - 1);
#pragma unroll
        for (int j = 0; j < B; ++j) {
          const int i = min(i0 + j, n_in - 1);
          v[u][j] = __builtin_nontemporal_load(src + (size_t)i * H * C + idx);
        }
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
#pragma unroll
        for (int j = 0; j < B; ++j) {
          const float w = (i0 + j < n_in) ? wts[(i0 + j) * H + hh[u]] : 0.f;
          acc[u] += (w != 0.f) ? w * v[u][j] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = base + u * NT;
      if (idx >= H * C) break;
      if (out_bf16) {
        unsigned lo = f32_to_bf16_bits(acc[u][0]) | ((unsigned)f32_to_bf16_bits(acc[u][1]) << 16);
        unsigned hi = f32_to_bf16_bits(acc[u][2]) | ((unsigned)f32_to_bf16_bits(acc[u][3]) << 16);
        reinterpret_cast<uint2*>(out_o)[idx] = make_uint2(lo, hi);
      } else {
        reinterpret_cast<f32x4*>(out_o)[idx] = acc[u];
      }
    }
  }
}

// Writes this block's normalised partial (O / l and LSE = ln l + max) for
// its heads to the workspace and/or o_part, then elects the last block of
// the (row, shard) and of the row with arrival counters and merges there.
// Release: all stores issued, workgroup barrier, device fence, count.
// Acquire: the winner fences again before reading the others' partials.
// The winner resets the counter, so the workspace needs zeroing only once.
// oacc[d][i] holds O^T for dim 16d + 4g + i of `head`; m_run / l_tot are the
// head's base-2 reference max and its sum of 2^(z - m_run).
template <int NT>
__device__ inline void finish_block(const DecodeParams& p, long long row, int shard, int split,
                                    int head, int g, bool writer, const f32x4 (&oacc)[32],
                                    float m_run, float l_tot, DCP_LDS char* smem, int* s_flag) {
  const int tid = threadIdx.x;
  const int N = p.num_shards, S = p.num_splits, HB = p.head_blocks, H = p.heads;
  const bool need_shard_merge = p.o_part != nullptr && S > 1;
  const bool fused = p.o != nullptr;
  const bool to_ws = fused || need_shard_merge;
  const bool to_part = p.o_part != nullptr && S == 1;
  if (writer) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    const long long blk_part = ((row * N + shard) * S + split);
    float* wo = to_ws ? p.ws_o + (blk_part * H + head) * kVDim : nullptr;
    float* po = to_part ? p.o_part + (((long long)shard * p.rows + row) * H + head) * kVDim : nullptr;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const f32x4 v = oacc[d] * inv;
      const int dim = 16 * d + 4 * g;
      if (to_ws) *reinterpret_cast<f32x4*>(wo + dim) = v;
      if (to_part) *reinterpret_cast<f32x4*>(po + dim) = v;
    }
    if (g == 0) {
      if (to_ws) p.ws_lse[blk_part * H + head] = lse_v;
      if (to_part) p.lse_part[((long long)shard * p.rows + row) * H + head] = lse_v;
    }
  }
  if (!to_ws) return;

  __syncthreads();
  DCP_LDS float* wts = (DCP_LDS float*)smem;
  if (need_shard_merge) {
    if (tid == 0) {
      __threadfence();
      const int old = atomicAdd(p.cnt_shard + row * N + shard, 1);
      *s_flag = (old == S * HB - 1);
    }
    __syncthreads();
    if (*s_flag) {
      __threadfence();
      const long long base = (row * N + shard) * S;
      merge_partials<NT>(p.ws_o + base * H * kVDim, p.ws_lse + base * H, S, H,
                         p.o_part + ((long long)shard * p.rows + row) * H * kVDim, 0,
                         p.lse_part + ((long long)shard * p.rows + row) * H, wts);
      if (tid == 0) p.cnt_shard[row * N + shard] = 0;
    }
    __syncthreads();
  }
  if (fused) {
    if (tid == 0) {
      __threadfence();
      const int old = atomicAdd(p.cnt_row + row, 1);
      *s_flag = (old == N * S * HB - 1);
    }
    __syncthreads();
    if (*s_flag) {
      __threadfence();
      const long long base = row * N * S;
      void* out = p.out_bf16 ? (void*)(static_cast<unsigned short*>(p.o) + row * H * kVDim)
                             : (void*)(static_cast<float*>(p.o) + row * H * kVDim);
      merge_partials<NT>(p.ws_o + base * H * kVDim, p.ws_lse + base * H, N * S, H, out,
                         p.out_bf16, p.lse + row * H, wts);
      if (tid == 0) p.cnt_row[row] = 0;
    }
  }
}

}  // namespace dcp
