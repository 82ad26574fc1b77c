// Epilogue shared by the decode kernels: per-block partial output, arrival
// counters and the LSE merge of a (row, head block)'s partials (the pack and
// combine steps fused into the attention kernel).
//
// Merge ([P1] "feat: support decode context parallelism for PyTorch MLA",
// Summary; [P3] "[DSA] Fix decode context parallelism for RoPE sparse
// attention on Blackwell", Modifications, Fixes in shared code; [P2]
// "Feat[DCP] Support decode context parallelism for DSA models with the
// flashmla_kv backend", review of the LSE combine): M = max LSE_r over
// partials with LSE_r > -inf, O = sum_r e^(LSE_r - M) O_r / sum_r e^(LSE_r - M),
// LSE = M + ln sum; O = 0 and LSE = -inf when every partial is empty.
//
// Hand-off between blocks.  Every block stores its normalised partial with
// device-scope coherent stores (agent-scope relaxed-atomic form of the
// gfx950 memory model: written through to memory, so no L2 write-back is
// needed), waits for them, and then counts itself on the agent-scope
// arrival word of its (row, head block).  The workspace copy of a partial
// is laid out [dim tile d][head][lane group g][4 dims], so that the 64 lanes
// of a wave store -- and a merger loads -- 1 KB contiguous per instruction.
//
// The merge is split into n_in parts of the head block's elements, one per
// member (partial).  When the grid fits on the GPU at once, a block that is
// not the last to arrive waits (bounded in time) for the others and then
// merges its own part, so the merge of a row runs on all its blocks in
// parallel.  A block that gives up first marks its part abandoned, with a
// compare-and-swap that can only succeed before the last arrival; the last
// arriver merges its own part plus every abandoned one.  Without waiting
// (large grids, many partials, or a zero time limit) every block arrives
// with its part marked abandoned, and the last arriver merges everything.
// Partials are added in index order, so the result does not depend on
// which block merges.  The last arriver starts the arrival word's next
// generation (count and abandon bits cleared) as soon as it has read it, and
// the blocks that wait watch for that generation change: the workspace needs
// zeroing only once, and no block waits for the others to finish merging.
#pragma once

#include <type_traits>

#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {

constexpr int kMaxWaitMembers = 48;         // abandon bits 8..55 of the 64-bit arrival word

// Weights of the n_in partials of a head block, from their LSEs: w[i][hl]
// (normalised), and the merged LSE of each head written to out_lse when
// asked.  With fp16 partials (wx non-null) every weight also carries the
// partial's power of two 2^wx[i][hl], so that the stored values need no
// rescaling.  Whole block; leaves w in LDS.
template <int NT>
__device__ __forceinline__ void merge_weights_from_lds(int n_in, int h0, int nh, float* out_lse,
                                              bool write_lse, DCP_LDS float* w, DCP_LDS int* wx);
template <int NT>
__device__ __forceinline__ void merge_weights(const DecodeParams& p, long long part0, int n_in, int h0, int nh,
                                     float* out_lse, bool write_lse, DCP_LDS float* w,
                                     DCP_LDS int* wx) {
  const int H = p.heads, tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(p.ws_lse + part0 * H, (unsigned)(n_in * H) * 4u);
  const __amdgpu_buffer_rsrc_t rx = coherent_rsrc(p.ws_exp + part0 * H, wx ? (unsigned)(n_in * H) * 4u : 0u);
  // All loads of a round are issued before any is used: one memory round
  // trip per round instead of one per value.
  constexpr int R = 8;                        // values per thread per round
  constexpr unsigned kNowhere = 0x80000000u;  // beyond every resource: reads 0, no traffic
  for (int base = 0; base < n_in * nh; base += NT * R) {
    float lv[R];
    int xv[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = base + k * NT + tid, pi = i / nh, hl = i - pi * nh;
      const unsigned off = i < n_in * nh ? (unsigned)(pi * H + h0 + hl) * 4u : kNowhere;
      lv[k] = load_coherent(rl, off);
      xv[k] = wx ? __float_as_int(load_coherent(rx, off)) : 0;
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = base + k * NT + tid, pi = i / nh, hl = i - pi * nh;
      if (i < n_in * nh) {
        w[pi * kHeadsPerBlock + hl] = lv[k];
        if (wx) wx[pi * kHeadsPerBlock + hl] = xv[k];
      }
    }
  }
  merge_weights_from_lds<NT>(n_in, h0, nh, out_lse, write_lse, w, wx);
}

// The second half of merge_weights: w[i][hl] holds the LSEs (and wx[i][hl]
// the powers of two of fp16 partials).
template <int NT>
__device__ __forceinline__ void merge_weights_from_lds(int n_in, int h0, int nh, float* out_lse,
                                              bool write_lse, DCP_LDS float* w, DCP_LDS int* wx) {
  const int tid = threadIdx.x;
  __syncthreads();
  for (int hl = tid; hl < nh; hl += NT) {
    float M = kNegInf;
    for (int i = 0; i < n_in; ++i) M = fmaxf(M, w[i * kHeadsPerBlock + hl]);
    float sum = 0.f;
    for (int i = 0; i < n_in; ++i) {
      const float l = w[i * kHeadsPerBlock + hl];
      const float e = (M > kNegInf && l > kNegInf) ? fast_exp2((l - M) * kLog2e) : 0.f;
      w[i * kHeadsPerBlock + hl] = e;
      sum += e;
    }
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
    for (int i = 0; i < n_in; ++i)
      w[i * kHeadsPerBlock + hl] *= wx ? inv * pow2i(wx[i * kHeadsPerBlock + hl]) : inv;
    if (write_lse) out_lse[h0 + hl] = sum > 0.f ? M + logf(sum) : kNegInf;
  }
  __syncthreads();
}

// The workspace partials of a row: fp32, or (HALF) fp16 scaled by a power
// of two per (partial, head); element e of a head block (dim tile e / 4nh,
// head (e / 4) % nh, lane group e % 4) holds four consecutive dims.
template <bool HALF>
struct WsPartials {
  static constexpr unsigned kElem = HALF ? 8u : 16u;   // bytes per element
  __amdgpu_buffer_rsrc_t r;
  unsigned part_bytes;
  __device__ WsPartials(const DecodeParams& p, long long part0, int n_in) {
    part_bytes = (unsigned)p.heads * kVDim * (kElem / 4u);
    r = coherent_rsrc(reinterpret_cast<const char*>(p.ws_o) + (size_t)part0 * part_bytes,
                      (unsigned)n_in * part_bytes);
  }
  __device__ f32x4 load(unsigned off) const {
    if constexpr (HALF) return unpack_f16x4(load_coherent2(r, off));
    else return load_coherent4(r, off);
  }
};

// Element range of parts [m0, m1) of n_parts of a head block's 128 * nh
// float4 elements.
__device__ __forceinline__ int2 part_range(int m0, int m1, int n_parts, int nh) {
  const long long T = 128LL * nh;
  return make_int2((int)(m0 * T / n_parts), (int)(m1 * T / n_parts));
}

// Merges the head block's float4 elements [e0, e1) (element e: dim tile
// e / 4nh, head (e / 4) % nh, lane group e % 4) over the partials part0 ..
// part0 + n_in - 1 into out (the output row's [H][512] values, fp32 or
// bf16).  Whole block.
template <int NT, bool HALF, int K, int G>
__device__ __forceinline__ void merge_part_kg(const DecodeParams& p, long long part0, int n_in, int h0, int nh,
                                     int e0, int e1, const DCP_LDS float* w, void* out,
                                     int out_bf16) {
  const int tid = threadIdx.x;
  const WsPartials<HALF> ws(p, part0, n_in);
  const unsigned part_bytes = ws.part_bytes;
  const unsigned blk_off = (unsigned)h0 * 128u * ws.kElem;
  constexpr unsigned kNowhere = 0x80000000u;      // beyond every resource: reads 0, no traffic
  for (int eb = e0; eb < e1; eb += NT * K) {
    f32x4 acc[K];
    int hl[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int e = min(eb + k * NT + tid, e1 - 1);
      hl[k] = (e >> 2) % nh;
    }
    for (int i0 = 0; i0 < n_in; i0 += G) {
      // raw loads (packed fp16 stay packed until used)
      typedef typename std::conditional<HALF, u32x2, f32x4>::type Raw;
      Raw v[G][K];
#pragma unroll
      for (int u = 0; u < G; ++u)
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int e = eb + k * NT + tid;
          const bool live = i0 + u < n_in && e < e1;
          const unsigned off = live ? (unsigned)(i0 + u) * part_bytes + blk_off + ws.kElem * e : kNowhere;
          if constexpr (HALF) v[u][k] = load_coherent2(ws.r, off);
          else v[u][k] = load_coherent4(ws.r, off);
        }
#pragma unroll
      for (int u = 0; u < G; ++u)
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float wt = i0 + u < n_in ? w[(i0 + u) * kHeadsPerBlock + hl[k]] : 0.f;
          f32x4 x;
          if constexpr (HALF) x = unpack_f16x4(v[u][k]);
          else x = v[u][k];
          acc[k] += (wt != 0.f) ? wt * x : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = eb + k * NT + tid;
      if (e >= e1) break;
      const int d = e / (4 * nh), g = e & 3;
      const size_t idx = (size_t)(h0 + hl[k]) * kVDim + 16 * d + 4 * g;
      if (out_bf16) {
        const unsigned lo = f32_to_bf16_bits(acc[k][0]) | ((unsigned)f32_to_bf16_bits(acc[k][1]) << 16);
        const unsigned hi = f32_to_bf16_bits(acc[k][2]) | ((unsigned)f32_to_bf16_bits(acc[k][3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<unsigned short*>(out) + idx) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = acc[k];
      }
    }
  }
}

// merge_part_kg with more of a pass's loads in flight when there are many
// members: up to 16 members, 2 elements per thread and 16 members' loads
// together; beyond, 1 element and 32 members (one memory round trip per
// pass while they cover n_in).  A function of its own, so that its loads'
// registers do not add to the calling kernel's.
template <int NT, bool HALF>
__device__ __attribute__((noinline)) void merge_part_many(const DecodeParams& p, long long part0,
                                                          int n_in, int h0, int nh, int e0, int e1,
                                                          const DCP_LDS float* w, void* out,
                                                          int out_bf16) {
  if (n_in <= 16) merge_part_kg<NT, HALF, 2, 16>(p, part0, n_in, h0, nh, e0, e1, w, out, out_bf16);
  else merge_part_kg<NT, HALF, 1, 32>(p, part0, n_in, h0, nh, e0, e1, w, out, out_bf16);
}

// Up to 4 members: 8 elements per thread, the members' loads together.
template <int NT, bool HALF>
__device__ __forceinline__ void merge_part(const DecodeParams& p, long long part0, int n_in, int h0, int nh,
                                  int e0, int e1, const DCP_LDS float* w, void* out, int out_bf16) {
  if (n_in <= 4) merge_part_kg<NT, HALF, 8, 4>(p, part0, n_in, h0, nh, e0, e1, w, out, out_bf16);
  else merge_part_many<NT, HALF>(p, part0, n_in, h0, nh, e0, e1, w, out, out_bf16);
}

// Merges this block's own part (member `member` of NIN = 4 or 8: dim tiles
// [d0, d0 + 32 / NIN) of every head of the block, d0 = member * 32 / NIN)
// with its own normalised values own[j] (dim tile d0 + j) taken from
// registers instead of the workspace.  Thread (wave w, lane 16g + i16)
// handles head 16w + i16 and lane group g, the elements it holds.  The other
// members' values are loaded first and `weights` (which fills w) runs while
// they are in flight.  Partials are added in index order with the same
// arithmetic as merge_part, so the result is bit-identical.
template <int NT, int NIN, bool HALF>
__device__ __forceinline__ void merge_own_part(const DecodeParams& p, long long part0, int member, int h0,
                                      int nh, int hl, int g, const f32x4 (&own)[8],
                                      DCP_LDS float* w, DCP_LDS int* wx, float* out_lse,
                                      bool write_lse, void* out, int out_bf16) {
  constexpr int ND = 32 / NIN;
  constexpr int NL = (NIN * kHeadsPerBlock + NT - 1) / NT;   // LSE loads per thread
  const int H = p.heads, tid = threadIdx.x;
  const int d0 = member * ND;
  // The LSEs first: vmcnt drains in issue order, so they can be waited for
  // while the partials are still in flight.
  const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(p.ws_lse + part0 * H, (unsigned)(NIN * H) * 4u);
  const __amdgpu_buffer_rsrc_t rx = coherent_rsrc(p.ws_exp + part0 * H, HALF ? (unsigned)(NIN * H) * 4u : 0u);
  float lse_in[NL];
  int exp_in[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int i = tid + k * NT, pi = i / nh, hi = i - pi * nh;
    const unsigned off = (unsigned)(pi * H + h0 + hi) * 4u;
    lse_in[k] = i < NIN * nh ? load_coherent(rl, off) : 0.f;
    exp_in[k] = HALF && i < NIN * nh ? __float_as_int(load_coherent(rx, off)) : 0;
  }
  const WsPartials<HALF> ws(p, part0, NIN);
  const unsigned part_bytes = ws.part_bytes;
  const unsigned blk_off = (unsigned)h0 * 128u * ws.kElem;
  constexpr unsigned kNowhere = 0x80000000u;      // beyond every resource: reads 0, no traffic
  f32x4 v[NIN][ND];
#pragma unroll
  for (int i = 0; i < NIN; ++i)
#pragma unroll
    for (int j = 0; j < ND; ++j)
      v[i][j] = ws.load(i != member ? (unsigned)i * part_bytes + blk_off +
                                          ws.kElem * (unsigned)(((d0 + j) * nh + hl) * 4 + g)
                                    : kNowhere);
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int i = tid + k * NT, pi = i / nh, hi = i - pi * nh;
    if (i < NIN * nh) {
      w[pi * kHeadsPerBlock + hi] = lse_in[k];
      if (HALF) wx[pi * kHeadsPerBlock + hi] = exp_in[k];
    }
  }
  merge_weights_from_lds<NT>(NIN, h0, nh, out_lse, write_lse, w, HALF ? wx : nullptr);
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NIN; ++i) {
      const float wt = w[i * kHeadsPerBlock + hl];
      const f32x4 x = i == member ? own[j] : v[i][j];
      acc += (wt != 0.f) ? wt * x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const size_t idx = (size_t)(h0 + hl) * kVDim + 16 * (d0 + j) + 4 * g;
    if (out_bf16) {
      const unsigned lo = f32_to_bf16_bits(acc[0]) | ((unsigned)f32_to_bf16_bits(acc[1]) << 16);
      const unsigned hi = f32_to_bf16_bits(acc[2]) | ((unsigned)f32_to_bf16_bits(acc[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<unsigned short*>(out) + idx) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = acc;
    }
  }
}

// Power of two of a block's fp16 row-merge partial: ex with every |value| *
// 2^-ex below 2^15, from a bound on the values (their largest magnitude, or
// any larger bound): the bound lands in [2^14, 2^15).
__device__ __forceinline__ int half_exponent(float bound) {
  const int F = (int)((__float_as_uint(bound) >> 23) & 0xffu);
  return bound > 0.f ? min(max(F - 141, -100), 100) : 0;
}
constexpr int kExFromValues = -1000;         // finish_block: exponent from the values

// Where and how a block's workspace partial is stored: fp16 scaled by
// 2^-ex for the row merge when HALF_X, else fp32 (always fp32 for the merge
// of one shard's splits); the own dim tiles [od0, od1) of a block that
// merges its own part in parallel stay in registers.  Element (d, head, lane
// group g) holds dims 16d + 4g..
template <int NT, bool OWN, bool HALF_X>
struct WsPartial {
  bool half;
  int od0, od1, nh, hl, g, ex;
  float scale;                               // O -> stored value
  unsigned elem;                             // bytes per element
  __amdgpu_buffer_rsrc_t r;
  __device__ WsPartial(const DecodeParams& p, long long row, int shard, int split, int head,
                       int g_, float inv, int ex_) {
    const int N = p.num_shards, S = p.num_splits, H = p.heads;
    const int h0 = head / kHeadsPerBlock * kHeadsPerBlock;
    nh = min(kHeadsPerBlock, H - h0);
    hl = head - h0;
    g = g_;
    const bool need_shard_merge = p.o_part != nullptr && S > 1;
    const bool fused = p.o != nullptr;
    const int n_in = N * S, member = shard * S + split;
    const bool may_wait = fused && p.merge_wait_ticks > 0 && n_in <= kMaxWaitMembers;
    const bool own = OWN && may_wait && !need_shard_merge && n_in == 4 && nh * 4 == NT;
    od0 = own ? member * (32 / n_in) : 0;
    od1 = own ? od0 + 32 / n_in : 0;
    half = HALF_X && fused && !need_shard_merge;
    ex = half ? ex_ : 0;
    scale = half ? inv * pow2i(-ex) : inv;
    elem = half ? 8u : 16u;
    const long long blk_part = (row * N + shard) * S + split;
    r = coherent_rsrc(reinterpret_cast<const char*>(p.ws_o) + (size_t)(blk_part * H + h0) * 128u * elem,
                      (unsigned)nh * 128u * elem);
  }
  __device__ bool is_own(int d) const { return d >= od0 && d < od1; }
  // The value as the merge sees it (fp16 image back in fp32).
  __device__ f32x4 value(const f32x4& o) const {
    return half ? unpack_f16x4(pack_f16x4(o * scale)) : o * scale;
  }
  __device__ void store(int d, const f32x4& o) const {
    const unsigned off = (unsigned)((d * nh + hl) * 4 + g) * elem;
    if (half) store_coherent2(r, off, pack_f16x4(o * scale));
    else store_coherent4(r, off, o * scale);
  }
  // The fp16 store without a branch (for a partial known to be fp16): when
  // !keep it goes to an offset past the resource, where it is dropped.
  __device__ void store_half(int d, const f32x4& o, bool keep) const {
    const unsigned off = keep ? (unsigned)((d * nh + hl) * 4 + g) * 8u : 0x80000000u;
    store_coherent2(r, off, pack_f16x4(o * scale));
  }
};

// Writes this block's normalised partial (O / l and LSE = ln l + max) for
// its heads to the workspace and/or o_part, then takes part in the merges of
// its (row, shard, head block) (splits -> o_part) and (row, head block)
// (everything -> o).  oacc[d][i] holds O^T for dim 16d + 4g + i of `head`;
// m_run / l_tot are the head's base-2 reference max and its sum of
// 2^(z - m_run).  OWN: every thread is a writer of its own (head, lane
// group), heads 16 * wave + lane % 16, so a block that merges its own part
// in parallel with the others can take its own values from registers and
// leaves them out of the workspace unless it gives its part up.
// ex_given: the fp16 exponent when the caller has a bound (else it comes
// from the values); pre_stored: the caller already stored the non-own dim
// tiles of its workspace partial (with that exponent).
template <int NT, bool OWN = false, bool HALF_X = false>
__device__ __forceinline__ void finish_block(const DecodeParams& p, long long row, int shard, int split,
                                    int head, int g, bool writer, const f32x4 (&oacc)[32],
                                    float m_run, float l_tot, DCP_LDS char* smem, int* s_flag,
                                    int ex_given = kExFromValues, bool pre_stored = false) {
  const int tid = threadIdx.x;
  const int N = p.num_shards, S = p.num_splits, HB = p.head_blocks, H = p.heads;
  const int hblk = head / kHeadsPerBlock;
  const int h0 = hblk * kHeadsPerBlock, nh = min(kHeadsPerBlock, H - h0), hl = head - h0;
  const bool need_shard_merge = p.o_part != nullptr && S > 1;
  const bool fused = p.o != nullptr;
  const bool to_ws = fused || need_shard_merge;
  const bool to_part = p.o_part != nullptr && S == 1;

  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  const long long blk_part = (row * N + shard) * S + split;
  const int n_in = N * S, member = shard * S + split;
  const bool may_wait = fused && p.merge_wait_ticks > 0 && n_in <= kMaxWaitMembers;
  // With HALF_X the row merge exchanges fp16 partials (the merge of one
  // shard's splits into o_part keeps fp32): each (partial, head) is scaled
  // by a power of two 2^-ex that keeps every |value| below 2^15, so every
  // value keeps 11 significant bits (the merge weights carry the 2^ex back)
  // and the merged O is within |O| * 2^-11 of the fp32 merge.  Without it
  // (the generic kernel: more partials per row and a larger error of its
  // own) the exchange is fp32.
  const bool half_ws = HALF_X && fused && !need_shard_merge;
  int ex = 0;
  if (half_ws && writer) {
    if (ex_given != kExFromValues) {
      ex = ex_given;
    } else {
      float amax = 0.f;
#pragma unroll
      for (int d = 0; d < 32; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(oacc[d][i]));
      ex = half_exponent(max_xor32(max_xor16(amax * inv)));
    }
  }
  const WsPartial<NT, OWN, HALF_X> wsp(p, row, shard, split, head, g, inv, ex);
  // Own part from registers: dim tiles [od0, od1) of this block's partial are
  // not stored unless the block gives its part up.
  const bool own = wsp.od1 > wsp.od0;
  const int od0 = wsp.od0, od1 = wsp.od1;
  // The own dim tiles, as stored, in eight registers (a uniform switch, so
  // that only these stay live through the wait).
  f32x4 own_v[8];
  if (own) {
    switch (od0 >> 2) {
#define DCP_OWN_CASE(c) \
      case c: { _Pragma("unroll") for (int j = 0; j < 8; ++j) own_v[j] = wsp.value(oacc[min(4 * c + j, 31)]); } break;
      DCP_OWN_CASE(0) DCP_OWN_CASE(1) DCP_OWN_CASE(2) DCP_OWN_CASE(3)
      DCP_OWN_CASE(4) DCP_OWN_CASE(5) DCP_OWN_CASE(6) DCP_OWN_CASE(7)
#undef DCP_OWN_CASE
      default: break;
    }
  }
  if (writer) {
    if (to_part) {
      float* po = p.o_part + (((long long)shard * p.rows + row) * H + head) * kVDim;
#pragma unroll
      for (int d = 0; d < 32; ++d) *reinterpret_cast<f32x4*>(po + 16 * d + 4 * g) = oacc[d] * inv;
      if (g == 0) p.lse_part[((long long)shard * p.rows + row) * H + head] = lse_v;
    }
    if (to_ws && !pre_stored) {
#pragma unroll
      for (int d = 0; d < 32; ++d)
        if (!wsp.is_own(d)) wsp.store(d, oacc[d]);
    }
    if (to_ws) {
      if (g == 0) {
        store_coherent(coherent_rsrc(p.ws_lse + blk_part * H, (unsigned)H * 4u),
                       (unsigned)head * 4u, lse_v);
        if (half_ws)
          store_coherent(coherent_rsrc(p.ws_exp + blk_part * H, (unsigned)H * 4u),
                         (unsigned)head * 4u, __int_as_float(ex));
      }
    }
  }
  if (!to_ws) return;

  wait_vmcnt<0>();       // this thread's coherent stores have completed ...
  __syncthreads();       // ... and so have those of every thread of the block
  DCP_LDS float* w = (DCP_LDS float*)smem;                    // [kMaxMergeInputs][64]
  DCP_LDS unsigned* s_word = (DCP_LDS unsigned*)(w + kMaxMergeInputs * kHeadsPerBlock);
  DCP_LDS unsigned long long* s_seen = (DCP_LDS unsigned long long*)(s_word + 2);  // arrival word read
  DCP_LDS int* wx = (DCP_LDS int*)(s_word + 64);              // [kMaxMergeInputs][64]

  if (need_shard_merge) {
    // splits of one shard -> o_part: the last of the S blocks merges
    int* cnt = p.cnt_shard + (row * N + shard) * HB + hblk;
    if (tid == 0)
      *s_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (*s_flag) {
      const long long part0 = (row * N + shard) * S;
      merge_weights<NT>(p, part0, S, h0, nh, p.lse_part + ((long long)shard * p.rows + row) * H, true, w,
                        nullptr);
      const int2 er = part_range(0, 1, 1, nh);
      merge_part<NT, false>(p, part0, S, h0, nh, er.x, er.y, w,
                            p.o_part + ((long long)shard * p.rows + row) * H * kVDim, 0);
      if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
  if (!fused) return;

  // ---- all partials of the row -> o.  Arrival word (64 bits): count in
  // bits 0..7, abandoned parts in bits 8 + member, generation in bits
  // 56..63.  Four 32-bit counter words per (row, head block), the first two
  // used.  Every member has arrived once the generation differs from the
  // one its own arrival saw (or, before the last arriver has moved it on,
  // the count has reached n_in).
  unsigned long long* arrive = reinterpret_cast<unsigned long long*>(p.cnt_row + (row * HB + hblk) * 4);
  unsigned long long gen0 = 0;           // (thread 0) generation at this block's arrival
  auto all_in = [&](unsigned long long now) {
    return (now >> 56) != gen0 || (now & 0xffull) == (unsigned long long)n_in;
  };
  // Abandons this block's part: with an own part kept in registers, that
  // part is stored (and waited for) first.  Returns the parts to merge.
  auto give_up = [&](unsigned long long now) -> unsigned {
    for (;;) {
      if (all_in(now)) return 1u;
      unsigned long long expect = now;
      if (__hip_atomic_compare_exchange_strong(arrive, &expect, now | (1ull << (8 + member)),
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        return 0u;                       // abandoned: the last arriver merges this part
      now = expect;                      // the word moved; look again
    }
  };
  if (tid == 0) {
    const unsigned long long add =
        1ull + (!may_wait && n_in <= kMaxWaitMembers ? 1ull << (8 + member) : 0ull);
    const unsigned long long old =
        __hip_atomic_fetch_add(arrive, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    gen0 = old >> 56;
    unsigned parts = 0u;                 // bit 0: own part; bit 1: last arriver
    if ((old & 0xffull) == (unsigned long long)n_in - 1) {
      parts = 3u;
      *s_seen = old;
      // every member is in and the abandon bits are read: next generation
      __hip_atomic_store(arrive, ((gen0 + 1ull) & 0xffull) << 56, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    } else if (may_wait) {
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        const unsigned long long now =
            __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (all_in(now)) { parts = 1u; break; }
        if (__builtin_amdgcn_s_memrealtime() - t0 > (unsigned long long)p.merge_wait_ticks) {
          if (own) {
            parts = 4u;                  // timed out: store the own part first
            *s_seen = now;
          } else {
            parts = give_up(now);
          }
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
    s_word[0] = parts;
  }
  __syncthreads();
  unsigned parts = s_word[0];
  if (parts == 4u) {
    if (writer) {
#pragma unroll
      for (int j = 0; j < 8; ++j)    // own_v holds the fp16 image: re-packing is exact
        if (od0 + j < od1)
          store_coherent2(wsp.r, (unsigned)(((od0 + j) * nh + hl) * 4 + g) * 8u, pack_f16x4(own_v[j]));
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) s_word[0] = give_up(*s_seen);
    __syncthreads();
    parts = s_word[0];
  }
  if (parts == 0u) return;
  // The last arriver merges every part whose member gave up (all parts
  // when there are too many members for abandon bits).
  const bool all = (parts & 2u) && n_in > kMaxWaitMembers;
  const unsigned long long abandoned = (parts & 2u) ? (*s_seen >> 8) & ((1ull << kMaxWaitMembers) - 1) : 0ull;

  void* out = p.out_bf16 ? (void*)(static_cast<unsigned short*>(p.o) + row * H * kVDim)
                         : (void*)(static_cast<float*>(p.o) + row * H * kVDim);
  const long long part0 = row * N * S;
  float* out_lse = p.lse + row * H;
  const bool last = (parts & 2u) != 0u;
  if (own && (parts & 1u)) {       // (own implies the fp16 workspace)
    merge_own_part<NT, 4, true>(p, part0, member, h0, nh, hl, g, own_v, w, wx, out_lse, last, out,
                                p.out_bf16);
  } else {
    merge_weights<NT>(p, part0, n_in, h0, nh, out_lse, last, w, half_ws ? wx : nullptr);
  }
  // Runs of consecutive parts go through the merge as one element range, so
  // that a block merging many parts keeps all its threads' loads in flight.
  auto want = [&](int m) {
    return !(own && m == member) &&
           (all || m == member || (m < kMaxWaitMembers && ((abandoned >> m) & 1ull)));
  };
  for (int m = 0; m < n_in;) {
    if (!want(m)) { ++m; continue; }
    int m1 = m + 1;
    while (m1 < n_in && want(m1)) ++m1;
    const int2 er = part_range(m, m1, n_in, nh);
    if (half_ws) merge_part<NT, true>(p, part0, n_in, h0, nh, er.x, er.y, w, out, p.out_bf16);
    else merge_part<NT, false>(p, part0, n_in, h0, nh, er.x, er.y, w, out, p.out_bf16);
    m = m1;
  }
}

}  // namespace dcp
