// Step 2 (+ step 3 fused): absorbed-weight MLA decode with LSE over one DCP
// shard's paged latent KV, for all gathered heads of the DCP group, with the
// LSE merge of the shards done in the epilogue of the last block to finish.
//
// Pages: [P3] "[DSA] Fix decode context parallelism for RoPE sparse attention
// on Blackwell" -- Motivation (the backend must return output and LSE; every
// rank runs the heads of the whole DCP group; counters sized by those heads),
// Modifications (Backend: return_lse, rows with no local KV fixed up, partials
// merged), Fixes in shared code (zero when every shard is empty), Follow-ups
// item 1 (pack, exchange and combine fused into one kernel).
// [P1] "feat: support decode context parallelism for PyTorch MLA", Summary
// (gather query heads, attend local KV, merge with LSE weights; dense and
// sparse FlashMLA, BF16 KV and sparse FP8 KV).
//
// Work decomposition.  One block per (row, shard, split, head block of 64).
// Blocks are numbered so that the blocks of one row are consecutive inside
// one XCD's share of the grid (the hardware deals blocks round-robin over the
// 8 XCDs), which keeps the row's query and partials in one L2.
//
// Inside a block, wave w owns 16 heads (head group hg) and, when the block
// has fewer than four head groups, a share of each tile's tokens (token
// group ts).  Per tile:
//   * the KV rows of T tokens (T = 64 FP8 / 32 BF16: 36 KB either way) are
//     copied straight from HBM into LDS with global->LDS DMA, three stages
//     deep, rows stored 16-byte-chunk-swizzled against bank conflicts;
//   * S^T = K Q^T on bf16 MFMA 16x16x32 (K codes converted to bf16 after the
//     LDS read -- E4M3 is exact in bf16; Q stays in registers for the block);
//   * online softmax in base 2, row statistics kept per head = per lane
//     column, reductions over the four lanes of a head with shuffles;
//   * O^T += V^T P^T: V^T operands come straight out of the row-major tile
//     with the gfx950 transposing LDS reads (ds_read_b64_tr_b8 / _b16).  FP8:
//     fp16 MFMA with P' = p * per-token scale in fp16 (V codes exact in fp16).
//     BF16: bf16 MFMA twice, P split into bf16 hi + lo.
// Epilogue: O / l and LSE = ln(sum) per head; partials go to o_part and/or
// the workspace; an arrival counter per (row) [and per (row, shard) when a
// shard is split] elects the last block, which merges the partials with LSE
// weights and resets the counter for the next call.
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

template <bool FP8> struct Tile;
template <> struct Tile<true> {
  static constexpr int T = 64;       // tokens per tile
  static constexpr int RB = 576;     // bytes per KV row
  static constexpr int CPR = 36;     // 16-byte chunks per row
};
template <> struct Tile<false> {
  static constexpr int T = 32;
  static constexpr int RB = 1152;
  static constexpr int CPR = 72;
};

// Chunk swizzle of token t's row: logical chunk c sits at position c ^ swz(t).
// The XOR stays inside an aligned group of 4 (FP8) or 8 (BF16) chunks, and
// 36 and 72 are multiples of those.
template <bool FP8>
__device__ __forceinline__ int swz(int t) {
  if constexpr (FP8) return ((t >> 2) ^ (t >> 4)) & 3;
  else return (t >> 1) & 7;
}

constexpr int kTileBytes = 36864;
constexpr int kStages = 3;
constexpr int kStageBytes = kTileBytes + 256;            // + 64 fp32 scales (FP8)
constexpr int kListOff = kStages * kStageBytes;
constexpr int kSmemBytes = kListOff + kMaxList * 4;

// Block-wide LSE merge of n_in partials [n_in][H][512] + [n_in][H] into one
// [H][512] output (fp32 or bf16) + [H] LSE.  Weights in LDS.
template <int NT>
__device__ void merge_partials(const float* __restrict__ in_o, const float* __restrict__ in_lse,
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
  for (int idx = tid; idx < H * C; idx += NT) {
    const int h = idx / C;
    const int c = idx - h * C;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n_in; ++i) {
      const float w = wts[i * H + h];
      if (w != 0.f) {
        const f32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(in_o + ((size_t)i * H + h) * kVDim) + c);
        acc += w * v;
      }
    }
    if (out_bf16) {
      unsigned lo = f32_to_bf16_bits(acc[0]) | ((unsigned)f32_to_bf16_bits(acc[1]) << 16);
      unsigned hi = f32_to_bf16_bits(acc[2]) | ((unsigned)f32_to_bf16_bits(acc[3]) << 16);
      reinterpret_cast<uint2*>(out_o)[(size_t)h * C + c] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<f32x4*>(out_o)[(size_t)h * C + c] = acc;
    }
  }
}

template <bool FP8, bool DENSE, int NW, int TS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const DecodeParams p) {
  using TL = Tile<FP8>;
  constexpr int T = TL::T, RB = TL::RB, CPR = TL::CPR;
  constexpr int NT = NW * 64;
  constexpr int HG = NW / TS;          // head groups of 16 in this block
  constexpr int TSUB = T / TS;         // tokens of a tile per token group
  constexpr int NST = TSUB / 16;       // 16-token S tiles per wave per tile
  constexpr int NKB = TSUB / 32;       // 32-token PV blocks per wave per tile
  constexpr int IPW = (kTileBytes / 1024) / NW;   // DMA instructions per wave per tile
  static_assert(NKB >= 1 && IPW * NW * 1024 == kTileBytes, "tile split");

  __shared__ __attribute__((aligned(16))) char smem_raw[kSmemBytes];
  __shared__ int s_flag;
  DCP_LDS char* smem = (DCP_LDS char*)smem_raw;
  DCP_LDS int* list = (DCP_LDS int*)(smem + kListOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave % HG;
  const int ts = wave / HG;
  const int g = lane >> 4;             // 16-lane group of the MFMA layouts
  const int i16 = lane & 15;

  // ---- block -> (row, shard, split, head block)
  long long b = blockIdx.x;
  if (p.xcd_swizzle) {
    const long long per_xcd = (long long)gridDim.x >> 3;
    b = (b & 7) * per_xcd + (b >> 3);
  }
  const int HB = p.head_blocks, S = p.num_splits, N = p.num_shards;
  const int hblk = (int)(b % HB); b /= HB;
  const int split = (int)(b % S); b /= S;
  const int shard = (int)(b % N);
  const long long row = b / N;
  const int H = p.heads;

  const ShardArg sh = p.shard[shard];
  const char* kvbase = static_cast<const char*>(sh.kv);
  const long long max_prow = sh.pool_rows - 1;

  // ---- this block's token range [start, end) of the shard's local tokens
  int n_tok;
  if constexpr (DENSE) {
    n_tok = (int)min((long long)sh.local_len[row], (long long)p.max_pages * p.page_size);
  } else {
    n_tok = min(p.counts[(long long)shard * p.rows + row], p.k);
  }
  n_tok = max(n_tok, 0);
  const int chunk = ((n_tok + S - 1) / S + T - 1) / T * T;
  const int start = min(n_tok, split * chunk);
  const int end = min(n_tok, start + chunk);
  const int ntiles = (end - start + T - 1) / T;

  // ---- stage the block's slot ids (sparse) or page ids (dense) in LDS
  const int page = DENSE ? p.page_size : 1;
  const int pg0 = DENSE ? start / page : 0;
  if constexpr (DENSE) {
    const int npg = end > start ? (end - 1) / page - pg0 + 1 : 0;
    const int* bt = p.block_table + row * p.max_pages + pg0;
    for (int i = tid; i < min(npg, kMaxList); i += NT) list[i] = bt[i];
  } else {
    const int* src = p.topk_local + ((long long)shard * p.rows + row) * p.k + start;
    for (int i = tid; i < min(end - start, kMaxList); i += NT) list[i] = src[i];
  }

  // Pool row of local token j (start <= j < end), clamped into the pool.
  auto pool_row = [&](int j) -> long long {
    long long r;
    if constexpr (DENSE) {
      const int pg = j / page;
      const int li = min(max(pg - pg0, 0), kMaxList - 1);
      r = (long long)list[li] * page + (j - pg * page);
    } else {
      r = list[min(max(j - start, 0), kMaxList - 1)];
    }
    return min(max(r, 0LL), max_prow);
  };

  // ---- query fragments (B operand of S^T = K Q^T), kept for the whole block
  const int head = hblk * kHeadsPerBlock + hg * 16 + i16;
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((size_t)row * H + head) * kHeadDim;
  bf16x8 qf[18];
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    const int dim = FP8 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
    qf[s] = *reinterpret_cast<const bf16x8*>(qrow + dim);
  }
  // Complete the query loads here, so that no wait for them lands inside the
  // tile loop (where it would also drain the in-flight KV copies).
#pragma unroll
  for (int s = 0; s < 18; ++s) touch(qf[s]);
  __syncthreads();   // list visible

  auto issue_tile = [&](int it) {
    DCP_LDS char* sbase = smem + (it % kStages) * kStageBytes;
    const int tok0 = start + it * T;
    const int nval = min(T, end - tok0);
#pragma unroll 3
    for (int ii = 0; ii < IPW; ++ii) {
      const int blk = wave * IPW + ii;
      const int lc = blk * 64 + lane;
      const int t = lc / CPR;
      const int pch = lc - t * CPR;
      const long long prow = pool_row(tok0 + (t < nval ? t : 0));
      const int c = pch ^ swz<FP8>(t);
      dma16(kvbase + prow * RB + c * 16, sbase + blk * 1024);
    }
    if constexpr (FP8) {
      if (wave == 0) {
        const long long prow = pool_row(tok0 + (lane < nval ? lane : 0));
        dma4(sh.scale + prow, sbase + kTileBytes);
      }
    }
  };

  // ---- online-softmax state: per lane, head = hg*16 + i16; O^T tiles
  float m_run = kNegInf;    // running max, base-2 logits
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 oacc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < kStages - 1 && it < ntiles; ++it) issue_tile(it);

  for (int it = 0; it < ntiles; ++it) {
    // Tile `it` has landed once at most one later tile's copies are in flight.
    if (it + 1 < ntiles) {
      if (FP8 && wave == 0) wait_vmcnt<IPW + 1>();
      else wait_vmcnt<IPW>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (it + kStages - 1 < ntiles) issue_tile(it + kStages - 1);

    const DCP_LDS char* sbase = smem + (it % kStages) * kStageBytes;
    const int tok0 = start + it * T;
    const int sub0 = ts * TSUB;

    // S^T = K Q^T for this wave's NST 16-token tiles
    f32x4 sacc[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int t = sub0 + st * 16 + i16;
      const DCP_LDS char* rp = sbase + t * RB;
      const int sw = swz<FP8>(t);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
#pragma unroll
        for (int s2 = 0; s2 < 9; ++s2) {
          const i32x4 raw = *reinterpret_cast<const DCP_LDS i32x4*>(rp + 16 * ((4 * s2 + g) ^ sw));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(raw.x, raw.y), qf[2 * s2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(raw.z, raw.w), qf[2 * s2 + 1], acc, 0, 0, 0);
          if (s2 % 3 == 2) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const bf16x8 a = *reinterpret_cast<const DCP_LDS bf16x8*>(rp + 16 * ((4 * s + g) ^ sw));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], acc, 0, 0, 0);
          if (s % 6 == 5) __builtin_amdgcn_sched_barrier(0);
        }
      }
      sacc[st] = acc;
    }

    // online softmax (lane: head column, tokens 4g..4g+3 of each S tile)
    float z[NST][4];
    float sc[NST][4];
    float tmax = kNegInf;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int tk = sub0 + st * 16 + 4 * g;
      if constexpr (FP8) {
        const f32x4 s4 = *reinterpret_cast<const DCP_LDS f32x4*>(sbase + kTileBytes + 4 * tk);
        sc[st][0] = s4[0]; sc[st][1] = s4[1]; sc[st][2] = s4[2]; sc[st][3] = s4[3];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sacc[st][i] * p.sm_scale_log2;
        if constexpr (FP8) v *= sc[st][i];
        v = (tok0 + tk + i < end) ? v : kNegInf;
        z[st][i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = wave_xor_max(tmax, 16);
    tmax = wave_xor_max(tmax, 32);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int d = 0; d < 32; ++d) oacc[d] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;
    float pr[NST][4];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(z[st][i] - m_use);
        l_run += e;
        pr[st][i] = FP8 ? e * sc[st][i] : e;
      }
    }

    // O^T += V^T P^T, one 32-token block at a time.  k-slot j of lane group g
    // is token 4g+j (j < 4) or 16+4g+(j-4) (j >= 4) of the block: exactly the
    // tokens this lane holds in the two S tiles, so P needs no shuffle.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int blk0 = sub0 + 32 * kb;
      if constexpr (FP8) {
        const f16x8 bp = f16x8{(_Float16)pr[2 * kb][0], (_Float16)pr[2 * kb][1],
                               (_Float16)pr[2 * kb][2], (_Float16)pr[2 * kb][3],
                               (_Float16)pr[2 * kb + 1][0], (_Float16)pr[2 * kb + 1][1],
                               (_Float16)pr[2 * kb + 1][2], (_Float16)pr[2 * kb + 1][3]};
        // tr8: lane i of a 16-lane group receives byte i%8 from the lanes
        // (i/8) + 2j; lane L therefore points at token slot L/2, bytes
        // [16d + 8(L%2), +8) -- lane i ends up with dim 16d + i of 8 tokens.
        const int jj = i16 >> 1;
        const int tk = blk0 + (jj < 4 ? 4 * g + jj : 16 + 4 * g + (jj - 4));
        const DCP_LDS char* vp = sbase + tk * RB + 8 * (i16 & 1);
        const int sw = swz<FP8>(tk);
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (DCP_LDS i32x2*)(vp + 16 * (d ^ sw)));
          oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(raw.x, raw.y), bp, oacc[d], 0, 0, 0);
          if (d % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        bf16x8 bh, bl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = pr[2 * kb + (j >> 2)][j & 3];
          const __bf16 hi = f32_to_bf16(v);
          bh[j] = hi;
          bl[j] = f32_to_bf16(v - bf16_to_f32(hi));
        }
        // tr16: lane i receives element i%4 from the lanes (i/4) + 4j; lane L
        // points at token slot L/4 (+4 for the second read), elements
        // [16d + 4(L%4), +4) -- lane i ends up with dim 16d + i of 4 tokens.
        const int tka = blk0 + 4 * g + (i16 >> 2);
        const int tkb = blk0 + 16 + 4 * g + (i16 >> 2);
        const int swa = swz<FP8>(tka), swb = swz<FP8>(tkb);
        const int half = (i16 & 3) >> 1;
        const DCP_LDS char* va = sbase + tka * RB + 8 * (i16 & 1);
        const DCP_LDS char* vb = sbase + tkb * RB + 8 * (i16 & 1);
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          const i16x4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (DCP_LDS i16x4*)(va + 16 * ((2 * d + half) ^ swa)));
          const i16x4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (DCP_LDS i16x4*)(vb + 16 * ((2 * d + half) ^ swb)));
          const i32x2 ra2 = __builtin_bit_cast(i32x2, ra);
          const i32x2 rb2 = __builtin_bit_cast(i32x2, rb);
          const bf16x8 a = __builtin_bit_cast(bf16x8, i32x4{ra2.x, ra2.y, rb2.x, rb2.y});
          oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, oacc[d], 0, 0, 0);
          oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, oacc[d], 0, 0, 0);
          if (d % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // ---- per-head totals; merge token groups inside the block
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if constexpr (TS > 1) {
    __syncthreads();   // every wave is done with the stage buffers
    DCP_LDS float* red = (DCP_LDS float*)smem;
    constexpr int SLOT = 64 * (128 + 2);
    if (ts > 0) {
      DCP_LDS float* my = red + ((ts - 1) * HG + hg) * SLOT;
#pragma unroll
      for (int d = 0; d < 32; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) my[(d * 4 + i) * 64 + lane] = oacc[d][i];
      my[128 * 64 + lane] = m_run;
      my[129 * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (ts == 0) {
      for (int o = 1; o < TS; ++o) {
        const DCP_LDS float* ot = red + ((o - 1) * HG + hg) * SLOT;
        const float mo = ot[128 * 64 + lane];
        const float lo = ot[129 * 64 + lane];
        const float mm = fmaxf(m_run, mo);
        const float mu = (mm == kNegInf) ? 0.f : mm;
        const float a = fast_exp2(m_run - mu), bsc = fast_exp2(mo - mu);
#pragma unroll
        for (int d = 0; d < 32; ++d)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[d][i] = oacc[d][i] * a + ot[(d * 4 + i) * 64 + lane] * bsc;
        l_tot = l_tot * a + lo * bsc;
        m_run = mm;
      }
    }
  }

  const bool need_shard_merge = p.o_part != nullptr && S > 1;
  const bool fused = p.o != nullptr;
  const bool to_ws = fused || need_shard_merge;
  const bool to_part = p.o_part != nullptr && S == 1;
  if (ts == 0) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    const long long blk_part = ((row * N + shard) * S + split);
    float* wo = to_ws ? p.ws_o + (blk_part * H + head) * kVDim : nullptr;
    float* po = to_part ? p.o_part + (((long long)shard * p.rows + row) * H + head) * kVDim : nullptr;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const float4 v = make_float4(oacc[d][0] * inv, oacc[d][1] * inv, oacc[d][2] * inv, oacc[d][3] * inv);
      const int dim = 16 * d + 4 * g;
      if (to_ws) *reinterpret_cast<float4*>(wo + dim) = v;
      if (to_part) *reinterpret_cast<float4*>(po + dim) = v;
    }
    if (g == 0) {
      if (to_ws) p.ws_lse[blk_part * H + head] = lse_v;
      if (to_part) p.lse_part[((long long)shard * p.rows + row) * H + head] = lse_v;
    }
  }
  if (!to_ws) return;

  // ---- elect the last block and merge (release: fence then count;
  // acquire: fence after winning)
  __syncthreads();
  DCP_LDS float* wts = (DCP_LDS float*)smem;
  if (need_shard_merge) {
    if (tid == 0) {
      __threadfence();
      const int old = atomicAdd(p.cnt_shard + row * N + shard, 1);
      s_flag = (old == S * HB - 1);
    }
    __syncthreads();
    if (s_flag) {
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
      s_flag = (old == N * S * HB - 1);
    }
    __syncthreads();
    if (s_flag) {
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

template <bool FP8, bool DENSE, int NW, int TS>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const long long blocks = p.rows * p.num_shards * (long long)p.num_splits * p.head_blocks;
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)decode_kernel<FP8, DENSE, NW, TS>, dim3((unsigned)blocks),
                         dim3(NW * 64), args, 0, stream);
}

template <bool FP8, bool DENSE>
hipError_t launch_heads(const DecodeParams& p, hipStream_t stream) {
  // heads per block = min(H, 64): four 16-head groups, or fewer groups with
  // the tile's tokens shared between waves (FP8 tiles hold two 32-token
  // blocks; BF16 tiles one).
  switch (p.heads) {
    case 128:
    case 64: return launch_one<FP8, DENSE, 4, 1>(p, stream);
    case 32:
      if constexpr (FP8) return launch_one<FP8, DENSE, 4, 2>(p, stream);
      else return launch_one<FP8, DENSE, 2, 1>(p, stream);
    case 16:
      if constexpr (FP8) return launch_one<FP8, DENSE, 2, 2>(p, stream);
      else return launch_one<FP8, DENSE, 1, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, bool fp8, bool dense, hipStream_t stream) {
  if (fp8) return dense ? launch_heads<true, true>(p, stream) : launch_heads<true, false>(p, stream);
  return dense ? launch_heads<false, true>(p, stream) : launch_heads<false, false>(p, stream);
}

}  // namespace dcp
