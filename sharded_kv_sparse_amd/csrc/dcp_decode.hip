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
//   * the KV rows of a tile (64 tokens FP8, 32 tokens BF16: 36 KB either
//     way, four stages) are copied straight from HBM into LDS with global->LDS DMA,
//     granule-major (each copy instruction moves one 64-byte granule of 16
//     tokens, so a lane keeps one token, and one id, for all its copies of
//     a tile), chunks swizzled against bank conflicts; the tile's slot or
//     page ids arrive two tiles ahead in an LDS ring, by the same DMA;
//   * S^T = K Q^T: FP8 KV on the fp8 MFMA 16x16x128 (block-scaled), the K
//     codes straight from LDS and Q * 2^e split into E4M3 hi + lo; BF16 KV on
//     the bf16 MFMA 16x16x32; Q stays in registers for the block;
//   * online softmax in base 2, row statistics kept per head = per lane
//     column, reductions over the four lanes of a head with shuffles;
//   * O^T += V^T P^T: V^T operands come straight out of the row-major tile
//     with the gfx950 transposing LDS reads (ds_read_b64_tr_b8 / _b16).  FP8:
//     fp16 MFMA with P' = p * per-token scale in fp16 (V codes exact in fp16).
//     BF16: bf16 MFMA twice, P split into bf16 hi + lo.
// Epilogue: O / l and LSE = ln(sum) per head; partials go to o_part and/or
// the workspace.  An arrival word per (row, head block) [and a counter per
// (row, shard, head block) when a shard is split] orders the merge with LSE
// weights: when the whole grid is resident, the row's blocks wait for each
// other and each merges a share of the row, else the last block to arrive
// merges it; either way the word is left ready for the next call.
#include "dcp_device.h"
#include "dcp_epilogue.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

// Tiles are stored granule-major: [granule G (64 bytes of the row)][token t]
// [4 x 16-byte chunks], the chunks of token t permuted by XOR with
// chunk_sw(t), which keeps the 16-byte operand reads of S^T = K Q^T free of
// bank conflicts.  FP8: 64-token tiles of 9 granules (576-byte rows) plus the
// tile's 64 fp32 token scales; BF16: 32-token tiles of 18 granules
// (1,152-byte rows).  36 KB either way, four stages: one tile computed while
// the next three are in flight.
template <bool FP8> struct Tile;
template <> struct Tile<true> {
  static constexpr int T = 64;         // tokens per tile
  static constexpr int GR = 9;         // granules per row
  static constexpr int SCALE_BYTES = 256;
};
template <> struct Tile<false> {
  static constexpr int T = 32;
  static constexpr int GR = 18;
  static constexpr int SCALE_BYTES = 0;
};
constexpr int kStages = 4;
// The ids of a tile enter the ring kIdsAhead tiles before its rows are
// copied; kRingSlots covers every tile whose ids are in flight or in use.
constexpr int kIdsAhead = kStages - 2;
constexpr int kRingSlots = kStages + kIdsAhead;

// Chunk permutation of token t inside its 64-byte granule.
__device__ __forceinline__ int chunk_sw(int t) { return ((t >> 1) ^ (t >> 3) ^ (t >> 4)) & 3; }

// The page table of a prefill chunk: one page, id 0, holding the whole chunk.
__device__ int kChunkPageId[1] = {0};

template <bool FP8, bool DENSE, int NW, int TS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const DecodeParams p) {
  using TL = Tile<FP8>;
  constexpr int T = TL::T, GR = TL::GR;
  constexpr int kPlane = T * 64;                   // bytes of one granule plane of a tile
  constexpr int kTileBytes = GR * kPlane;
  constexpr int kStageBytes = kTileBytes + TL::SCALE_BYTES;
  constexpr int kRingOff = kStages * kStageBytes;
  constexpr int kSmemBytes = kRingOff + kRingSlots * 64 * 4;
  constexpr int NT = NW * 64;
  constexpr int HG = NW / TS;          // head groups of 16 in this block
  constexpr int TSUB = T / TS;         // tokens of a tile per token group
  constexpr int CT = TSUB >= 32 ? 32 : 16;   // tokens per softmax / PV chunk
  constexpr int CST = CT / 16;         // 16-token S tiles per chunk
  constexpr int NKB = TSUB / CT;       // chunks per wave per tile
  // Row copies: TGT groups of 16 tokens per tile; a wave copies whole token
  // groups (TGW of them) or, with more waves than groups, every WPT-th
  // granule of one group.
  constexpr int TGT = T / 16;
  constexpr int TGW = TGT >= NW ? TGT / NW : 1;
  constexpr int WPT = NW >= TGT ? NW / TGT : 1;
  constexpr int IPW = TGW * GR / WPT;  // row copies per wave per tile
  constexpr int kRingWave = NW - 1;    // copies each tile's ids into the ring
  static_assert(NKB >= 1 && GR % WPT == 0 && NW * IPW == TGT * GR && (TGT % NW == 0 || NW % TGT == 0),
                "tile split");
  static_assert(!FP8 || CT == 32, "FP8 chunks are 32 tokens");
  static_assert(NW > 1, "the ring wave is not wave 0");
  static_assert((TS - 1) * HG * 64 * 130 * 4 <= kRingOff, "token-group merge space");
  static_assert(kMaxMergeInputs * kHeadsPerBlock * 8 + 256 <= kRingOff, "merge space");
  // vector-memory operations a wave queues per tile (rows; FP8 wave 0 also
  // the scales), and what may stay in flight at the top of a tile in steady
  // state: the rows of the next kStages - 2 tiles (and for the ring wave the
  // ids queued between them)
  constexpr int kOps0 = IPW + (FP8 ? 1 : 0), kOps = IPW;
  static_assert((kStages - 2) * kOps0 + kIdsAhead - 1 < 63, "vmcnt range");

  __shared__ __attribute__((aligned(16))) char smem_raw[kSmemBytes];
  __shared__ int s_flag;
  DCP_LDS char* smem = (DCP_LDS char*)smem_raw;
  DCP_LDS int* ring = (DCP_LDS int*)(smem + kRingOff);

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
    n_tok = p.chunk_mode ? p.chunk_len
                         : (int)min((long long)sh.local_len[row], (long long)p.max_pages * p.page_size);
  } else {
    n_tok = min(p.counts[(long long)shard * p.rows + row], p.k);
  }
  n_tok = max(n_tok, 0);
  // splits of whole tiles (the last one takes the remainder)
  const int chunk = ((n_tok + S - 1) / S + T - 1) / T * T;
  const int start = min(n_tok, split * chunk);
  const int end = min(n_tok, start + chunk);
  const int ntiles = (end - start + T - 1) / T;

  // ---- ids.  Local token j's id is its compacted slot id (sparse) or the id
  // of its logical page (dense).  A tile's ids are copied into a ring slot of
  // LDS by global->LDS DMA (one 4-byte copy per token) kIdsAhead tiles before
  // its rows, so that the row copies need no dependent global load.  Tokens
  // past a tile's valid count stand in for its first token: they are masked
  // out of the softmax, and a real row keeps their V values finite.
  const int page = DENSE ? p.page_size : 1;
  const int* ids = DENSE ? (p.chunk_mode ? kChunkPageId : p.block_table + row * p.max_pages)
                         : p.topk_local + ((long long)shard * p.rows + row) * p.k;
  auto tile_tok0 = [&](int it) { return start + it * T; };
  auto eff = [&](int it, int t) { return t < end - tile_tok0(it) ? t : 0; };
  auto pool_row = [&](int j, int id) -> long long {
    const long long r = DENSE ? (long long)id * page + (j - (j / page) * page) : (long long)id;
    return min(max(r, 0LL), max_prow);
  };
  // (wave kRingWave) ids of tile `it` into its ring slot; a tile past the
  // last one copies the last tile's ids (never read), so that every tile
  // queues the same operations
  auto issue_ring = [&](int it) {
    const int src_it = min(it, ntiles - 1);
    const int j = tile_tok0(src_it) + eff(src_it, lane);
    dma4(DENSE ? ids + j / page : ids + j, ring + (it % kRingSlots) * 64);
  };
  // Rows of tile `it` into its stage, its ids already in the ring: lane l of
  // a copy covers token 16 tg + l / 4 of the tile and the 16-byte chunk
  // (l & 3) ^ chunk_sw of a granule of its row.  Wave 0 also copies the
  // tile's 64 fp32 scales (FP8).
  auto issue_tile = [&](int it) {
    DCP_LDS char* sb = smem + (it % kStages) * kStageBytes;
    const DCP_LDS int* rg = ring + (it % kRingSlots) * 64;
    const int tok0 = tile_tok0(it);
#pragma unroll
    for (int jg = 0; jg < TGW; ++jg) {
      const int tg = TGT >= NW ? wave * TGW + jg : wave % TGT;
      const int t = 16 * tg + (lane >> 2);
      const int te = eff(it, t);
      const char* src = kvbase + pool_row(tok0 + te, rg[te]) * sh.row_stride +
                        16 * ((lane & 3) ^ chunk_sw(t));
#pragma unroll
      for (int k = 0; k < GR / WPT; ++k) {
        const int G = TGT >= NW ? k : wave / TGT + WPT * k;
        dma16(src + 64 * G, sb + G * kPlane + tg * 1024);
      }
    }
    if constexpr (FP8) {
      if (wave == 0) {
        const int te = eff(it, lane);
        dma4(reinterpret_cast<const float*>(reinterpret_cast<const char*>(sh.scale) +
                                            pool_row(tok0 + te, rg[te]) * sh.scale_stride),
             sb + kTileBytes);
      }
    }
  };
  // ids of the tiles whose rows are copied before the loop or in its first
  // kIdsAhead iterations
  if (wave == kRingWave && ntiles > 0) {
#pragma unroll
    for (int it = 0; it < kStages - 1 + kIdsAhead; ++it) issue_ring(it);
  }

  // ---- query fragments (B operand of S^T = K Q^T), kept for the whole block.
  // BF16 KV: bf16 Q on the bf16 MFMA; k-step s covers dims 32s..32s+31 and
  // lane group g holds dims 32s + 8g .. +8.
  // FP8 KV: Q * 2^e is split into E4M3 hi + lo for the fp8 MFMA (K = 128):
  // k-step s covers dims 128s..128s+127, lane group g holds dims 128s + 32g
  // .. +32, dims >= 576 are zero.  e is per head, the largest power of two
  // with max|q| * 2^e <= 448; hi + lo reproduces every bf16 element whose
  // scaled magnitude is >= 2^-2 exactly, smaller ones to within 2^-10
  // (scaled), i.e. to ~2^-16 of max|q|.
  const int head = hblk * kHeadsPerBlock + hg * 16 + i16;
  // In the last head block of a head count that is not a multiple of 64, a
  // head group past the last head loads no query (zeros) and stores nothing;
  // its waves still copy rows and take part in every barrier and merge.
  const bool active = hblk * kHeadsPerBlock + hg * 16 < H;
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((size_t)row * H + (active ? head : 0)) * kHeadDim;
  [[maybe_unused]] bf16x8 qf[FP8 ? 1 : 18];
  [[maybe_unused]] i32x8 qhi[FP8 ? 5 : 1], qlo[FP8 ? 5 : 1];
  float z_scale = p.sm_scale_log2;     // multiplies the raw MFMA logit
  if constexpr (FP8) {
    bf16x8 raw[5][4];
    float qmax = 0.f;
#pragma unroll
    for (int s = 0; s < 5; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dim = 128 * s + 32 * g + 8 * u;
        raw[s][u] = active && dim < kHeadDim ? *reinterpret_cast<const bf16x8*>(qrow + dim) : bf16x8{};
#pragma unroll
        for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(bf16_to_f32(raw[s][u][j])));
      }
    qmax = wave_xor_max(qmax, 16);
    qmax = wave_xor_max(qmax, 32);
    int e = 0;
    if (qmax > 0.f) {
      int ex;
      frexpf(448.0f / qmax, &ex);
      e = min(max(ex - 1, -120), 120);
      while (e > -120 && ldexpf(qmax, e) > 448.0f) --e;
    }
    const float qs = ldexpf(1.0f, e);
    z_scale = p.sm_scale_log2 * ldexpf(1.0f, -e);
#pragma unroll
    for (int s = 0; s < 5; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = bf16_to_f32(raw[s][u][4 * half + j]) * qs;
          int h = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
          h = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h, true);
          const float r[4] = {x[0] - __builtin_amdgcn_cvt_f32_fp8(h, 0),
                              x[1] - __builtin_amdgcn_cvt_f32_fp8(h, 1),
                              x[2] - __builtin_amdgcn_cvt_f32_fp8(h, 2),
                              x[3] - __builtin_amdgcn_cvt_f32_fp8(h, 3)};
          int l = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
          l = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], l, true);
          qhi[s][2 * u + half] = h;
          qlo[s][2 * u + half] = l;
        }
  } else {
#pragma unroll
    for (int s = 0; s < 18; ++s) qf[s] = active ? *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * g) : bf16x8{};
#pragma unroll
    for (int s = 0; s < 18; ++s) touch(qf[s]);
  }

  // ---- the first tiles' ids are in the ring: copy their rows
  wait_vmcnt<0>();
  lds_barrier();
#pragma unroll
  for (int it = 0; it < kStages - 1; ++it)
    if (it < ntiles) issue_tile(it);

  // ---- online-softmax state: per lane, head = hg*16 + i16; O^T tiles
  float m_run = kNegInf;    // reference max (base-2 logits), see the softmax below
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 oacc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  // FP8: P' = p * scale goes to fp16 times 2^pe_run, one power of two per
  // head that puts the head's largest P' so far in [2^14, 2^15): no overflow
  // whatever the token scales, and O^T carries the same factor until the end
  // of the tile loop.  kNoExp: no P' above zero seen yet.
  constexpr int kNoExp = 1000;
  [[maybe_unused]] int pe_run = kNoExp;

  for (int it = 0; it < ntiles; ++it) {
    // Tile `it` (and the ids of tile it + kStages - 1) have landed once at
    // most the rows of tiles it + 1 .. it + kStages - 2 (and, for the ring
    // wave after the first tile, the ids queued between them) are in flight.
    if (it + kStages - 2 < ntiles) {
      if (wave == 0) wait_vmcnt<(kStages - 2) * kOps0>();
      else if (wave == kRingWave && it > 0) wait_vmcnt<(kStages - 2) * kOps + kIdsAhead - 1>();
      else wait_vmcnt<(kStages - 2) * kOps>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (wave == kRingWave) issue_ring(it + kStages - 1 + kIdsAhead);
    if (it + kStages - 1 < ntiles) issue_tile(it + kStages - 1);

    const DCP_LDS char* sbase = smem + (it % kStages) * kStageBytes;
    const int tok0 = tile_tok0(it);

    // The wave's share of the tile in chunks of CT tokens: S^T for the
    // chunk's 16-token S tiles, the softmax update, then O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int sub0 = ts * TSUB + CT * kb;

      // S^T = K Q^T; two independent accumulators, interleaved so that
      // back-to-back MFMAs never wait on each other (the chunk's two S tiles,
      // or a 16-token chunk's even and odd k-steps).  The operands of k-step
      // s + 1 (FP8) or s + 2 (BF16) are read from LDS while step s multiplies.
      f32x4 sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
        // k-step s, lane group g: dims 128s + 32g .. +32 = chunks 2(g & 1),
        // 2(g & 1) + 1 of granule 2s + (g >> 1) (dims >= 576 are padding)
        auto load_k = [&](int s, i32x8* a) {
          const bool live = (s < 4) || (g < 2);
          const int G = live ? 2 * s + (g >> 1) : 0;
          const int c0 = 2 * (g & 1);
#pragma unroll
          for (int st = 0; st < CST; ++st) {
            const int t = sub0 + st * 16 + i16;
            const DCP_LDS char* rp = sbase + G * kPlane + t * 64;
            const int sw = chunk_sw(t);
            const i32x4 lo4 = *reinterpret_cast<const DCP_LDS i32x4*>(rp + 16 * (c0 ^ sw));
            const i32x4 hi4 = *reinterpret_cast<const DCP_LDS i32x4*>(rp + 16 * ((c0 + 1) ^ sw));
            a[st] = live ? i32x8{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w} : i32x8{};
          }
        };
        i32x8 a[2][CST];
        load_k(0, a[0]);
#pragma unroll
        for (int s = 0; s < 5; ++s) {
          if (s + 1 < 5) load_k(s + 1, a[(s + 1) & 1]);
#pragma unroll
          for (int st = 0; st < CST; ++st)
            sacc[st] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[s & 1][st], qhi[s], sacc[st],
                                                                        0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int st = 0; st < CST; ++st)
            sacc[st] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[s & 1][st], qlo[s], sacc[st],
                                                                        0, 0, 0, 127, 0, 127);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // k-step s, lane group g: dims 32s + 8g .. +8 = chunk g of granule s
        auto load_k = [&](int s, bf16x8* a) {
#pragma unroll
          for (int st = 0; st < CST; ++st) {
            const int t = sub0 + st * 16 + i16;
            a[st] = *reinterpret_cast<const DCP_LDS bf16x8*>(sbase + s * kPlane + t * 64 +
                                                            16 * (g ^ chunk_sw(t)));
          }
        };
        bf16x8 a[3][CST];
        load_k(0, a[0]);
        load_k(1, a[1]);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          if (s + 2 < 18) load_k(s + 2, a[(s + 2) % 3]);
          if constexpr (CST == 2) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
              sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s % 3][st], qf[s], sacc[st], 0, 0, 0);
          } else {
            sacc[s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s % 3][0], qf[s], sacc[s & 1], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (CST == 1) sacc[0] += sacc[1];
      }

      // First V^T operands of the chunk, read before the softmax so their
      // LDS latency hides behind it (see the PV loop below for the layout).
      const int blk0 = sub0;
      [[maybe_unused]] i32x2 vraw[2][8];
      [[maybe_unused]] i16x4 vr16[2][4][CST];
      [[maybe_unused]] const DCP_LDS char* vp = nullptr;
      [[maybe_unused]] int vsw = 0;
      [[maybe_unused]] const DCP_LDS char* va = nullptr;
      [[maybe_unused]] const DCP_LDS char* vb = nullptr;
      [[maybe_unused]] int swa = 0, swb = 0, vhalf = 0;
      if constexpr (FP8) {
        // tr8: lane i of a 16-lane group receives byte i%8 from the lanes
        // (i/8) + 2j; lane L therefore points at token slot L/2, bytes
        // [16d + 8(L%2), +8) of the row (chunk d & 3 of granule d >> 2) --
        // lane i ends up with dim 16d + i of 8 tokens.
        const int jj = i16 >> 1;
        const int tk = blk0 + (jj < 4 ? 4 * g + jj : 16 + 4 * g + (jj - 4));
        vp = sbase + tk * 64 + 8 * (i16 & 1);
        vsw = chunk_sw(tk);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          vraw[0][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (DCP_LDS i32x2*)(vp + (j >> 2) * kPlane + 16 * ((j & 3) ^ vsw)));
      } else {
        // tr16: lane i receives element i%4 from the lanes (i/4) + 4j; lane L
        // points at token slot L/4 (and 16 + L/4 for the second S tile),
        // elements [16d + 4(L%4), +4) = bytes 32d + 8(L%4) of the row (chunk
        // 2(d & 1) + (L%4)/2 of granule d >> 1) -- lane i ends up with dim
        // 16d + i of 4 tokens.
        const int tka = blk0 + 4 * g + (i16 >> 2);
        const int tkb = tka + 16;
        swa = chunk_sw(tka);
        swb = chunk_sw(tkb);
        vhalf = (i16 & 3) >> 1;
        va = sbase + tka * 64 + 8 * (i16 & 1);
        vb = sbase + tkb * 64 + 8 * (i16 & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 2 * (j & 1) + vhalf, off = (j >> 1) * kPlane;
          vr16[0][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DCP_LDS i16x4*)(va + off + 16 * (c ^ swa)));
          if constexpr (CST == 2)
            vr16[0][j][CST - 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DCP_LDS i16x4*)(vb + off + 16 * (c ^ swb)));
        }
      }

      // Online softmax (lane: head column, tokens 4g..4g+3 of each S tile).
      // The reference max m_run only moves when the chunk max exceeds it by
      // more than 8 (base 2): p = 2^(z - m_run) then stays <= 2^8, and O and
      // l are rescaled rarely instead of on every chunk.
      float z[CST][4];
      float sc[CST][4];
      float tmax = kNegInf;
#pragma unroll
      for (int st = 0; st < CST; ++st) {
        const int tk = sub0 + st * 16 + 4 * g;
        if constexpr (FP8) {
          const f32x4 s4 = *reinterpret_cast<const DCP_LDS f32x4*>(sbase + kTileBytes + 4 * tk);
          sc[st][0] = s4[0]; sc[st][1] = s4[1]; sc[st][2] = s4[2]; sc[st][3] = s4[3];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[st][i] * z_scale;
          if constexpr (FP8) v *= sc[st][i];
          v = (tok0 + tk + i < end) ? v : kNegInf;
          z[st][i] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = wave_xor_max(tmax, 16);
      tmax = wave_xor_max(tmax, 32);
      const bool bump = tmax > m_run + 8.0f;
      if (__any(bump)) {
        const float m_new = bump ? tmax : m_run;
        const float alpha = bump ? fast_exp2(m_run - m_new) : 1.0f;   // m_run = -inf -> 0
        if (__any(bump && m_run != kNegInf)) {
#pragma unroll
          for (int d = 0; d < 32; ++d) oacc[d] *= alpha;
        }
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == kNegInf) ? 0.f : m_run;
      float pr[CST][4];
#pragma unroll
      for (int st = 0; st < CST; ++st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(z[st][i] - m_use);
          l_run += e;
          pr[st][i] = FP8 ? e * sc[st][i] : e;
        }
      }

      // O^T += V^T P^T over the chunk.  32-token chunks: k-slot j of lane
      // group g is token 4g+j (j < 4) or 16+4g+(j-4) (j >= 4) of the chunk,
      // exactly the tokens this lane holds in the two S tiles, so P needs no
      // shuffle.  16-token chunks (BF16): k-slots j < 4 carry P's bf16 hi
      // part of token 4g+j and j >= 4 its lo part, against the V^T of token
      // 4g+(j-4) read once and used twice.  V^T operands are read in groups
      // of 8 (FP8) / 4 (BF16) 16-dim tiles, one group ahead of the MFMAs
      // that consume them.
      if constexpr (FP8) {
        // The head's largest P' over its four lanes sets the power of two; a
        // larger P' than before lowers it, and O^T is scaled down to match
        // (an exact power-of-two multiply).
        float pmax = 0.f;
#pragma unroll
        for (int st = 0; st < CST; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) pmax = fmaxf(pmax, pr[st][i]);
        pmax = max_xor32(max_xor16(pmax));
        if (pmax > 0.f) {
          const int pe = -half_exponent(pmax);
          if (pe < pe_run) {
            if (pe_run != kNoExp) {
              const float f = pow2i(pe - pe_run);
#pragma unroll
              for (int d = 0; d < 32; ++d) oacc[d] *= f;
            }
            pe_run = pe;
          }
        }
        const float ps = pe_run != kNoExp ? pow2i(pe_run) : 1.0f;
        const f16x8 bp = f16x8{(_Float16)(pr[0][0] * ps), (_Float16)(pr[0][1] * ps),
                               (_Float16)(pr[0][2] * ps), (_Float16)(pr[0][3] * ps),
                               (_Float16)(pr[CST - 1][0] * ps), (_Float16)(pr[CST - 1][1] * ps),
                               (_Float16)(pr[CST - 1][2] * ps), (_Float16)(pr[CST - 1][3] * ps)};
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          if (grp + 1 < 4) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              vraw[(grp + 1) & 1][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (DCP_LDS i32x2*)(vp + (2 * (grp + 1) + (j >> 2)) * kPlane + 16 * ((j & 3) ^ vsw)));
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const i32x2 raw = vraw[grp & 1][j];
            oacc[8 * grp + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(raw.x, raw.y), bp,
                                                                       oacc[8 * grp + j], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        bf16x8 bh, bl;
        if constexpr (CST == 2) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float v = pr[(j >> 2) & (CST - 1)][j & 3];
            const __bf16 hi = f32_to_bf16(v);
            bh[j] = hi;
            bl[j] = f32_to_bf16(v - bf16_to_f32(hi));
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = pr[0][j];
            const __bf16 hi = f32_to_bf16(v);
            bh[j] = hi;
            bh[4 + j] = f32_to_bf16(v - bf16_to_f32(hi));
          }
        }
#pragma unroll
        for (int grp = 0; grp < 8; ++grp) {
          if (grp + 1 < 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int d = 4 * (grp + 1) + j;
              const int c = 2 * (d & 1) + vhalf, off = (d >> 1) * kPlane;
              vr16[(grp + 1) & 1][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (DCP_LDS i16x4*)(va + off + 16 * (c ^ swa)));
              if constexpr (CST == 2)
                vr16[(grp + 1) & 1][j][CST - 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DCP_LDS i16x4*)(vb + off + 16 * (c ^ swb)));
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 4 * grp + j;
            const i32x2 ra2 = __builtin_bit_cast(i32x2, vr16[grp & 1][j][0]);
            const i32x2 rb2 = __builtin_bit_cast(i32x2, vr16[grp & 1][j][CST - 1]);
            const bf16x8 a = __builtin_bit_cast(bf16x8, i32x4{ra2.x, ra2.y, rb2.x, rb2.y});
            oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, oacc[d], 0, 0, 0);
            if constexpr (CST == 2) oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, oacc[d], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  if constexpr (FP8) {          // remove the P' power of two from O^T
    if (pe_run != kNoExp) {
      const float f = pow2i(-pe_run);
#pragma unroll
      for (int d = 0; d < 32; ++d) oacc[d] *= f;
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

  finish_block<NT>(p, row, shard, split, head, g, ts == 0 && active, oacc, m_run, l_tot, smem, &s_flag);
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
  // heads per block = min(H, 64): four 16-head groups (from 48 heads on;
  // the last block of a count that is not a multiple of 64 leaves groups
  // idle), or fewer groups with each tile's token halves shared between
  // waves (16 and 32 heads).
  if (p.heads % 16 != 0 || p.heads > 128) return hipErrorInvalidValue;
  if (p.heads >= 48) return launch_one<FP8, DENSE, 4, 1>(p, stream);
  if (p.heads == 32) return launch_one<FP8, DENSE, 4, 2>(p, stream);
  return launch_one<FP8, DENSE, 2, 2>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, bool fp8, bool dense, hipStream_t stream) {
  if (fp8 && p.heads >= 48) return launch_decode_fp8(p, dense, stream);
  if (fp8) return dense ? launch_heads<true, true>(p, stream) : launch_heads<true, false>(p, stream);
  return dense ? launch_heads<false, true>(p, stream) : launch_heads<false, false>(p, stream);
}

}  // namespace dcp
