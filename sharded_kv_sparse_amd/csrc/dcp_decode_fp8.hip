// Step 2 (+ step 3 fused) for FP8 E4M3 KV with 48 to 128 gathered heads:
// absorbed-weight MLA decode with LSE over one DCP shard's paged latent KV,
// the shards' partials merged in the epilogue of the last block of a row.
//
// Pages: [P3] "[DSA] Fix decode context parallelism for RoPE sparse attention
// on Blackwell" -- Motivation (output and LSE from the backend; every rank
// runs the heads of the whole DCP group), Modifications (Backend: return_lse,
// rows without local KV fixed up, partials merged), Follow-ups item 1 (pack
// and combine fused).  [P1] "feat: support decode context parallelism for
// PyTorch MLA", Summary (dense and sparse FlashMLA with FP8 KV).
//
// Both contractions run on the gfx950 fp8 MFMA (16x16x128, f8f6f4 with E8M0
// block scales), so no KV element is ever converted in registers:
//   * S^T = K Q^T: K codes straight from LDS; Q*2^e split into E4M3 hi + lo
//     once per block (exact for all but the tiniest elements).
//   * O^T += V^T P'^T with P' = p * scale_t: P' of each lane's 32 tokens is
//     scaled by a power of two to the top of the E4M3 range and split into
//     three E4M3 terms (12 significant bits, like fp16), and the MFMA's B
//     block scale (2^-e) undoes the power of two exactly.
//
// Data movement.  A tile is 128 tokens.  Its 576-byte rows are copied from
// HBM straight into LDS with global->LDS DMA.  Each copy instruction moves
// one 64-byte granule of 16 tokens, four lanes per granule.  LDS layout of a
// stage: [granule G: bytes 64G.. of the row, 9][token / 16][token % 16][4 x
// 16-byte chunks], the chunks of token t permuted by XOR with sw(t) =
// ((t >> 1) ^ (t >> 3) ^ (t >> 4)) & 3, which keeps the 16-byte operand
// reads of S^T = K Q^T and the 8-byte transposing reads of V^T free of bank
// conflicts on 32- and 64-bank LDS alike; then the tile's 128 fp32 token
// scales.  Two stages: tile it+1 streams in while tile it is computed, its
// copies issued among the QK MFMAs of tile it.  The slot ids (sparse) or
// page ids (dense) of tile it+2 are DMA'd into a three-deep ring at the same
// time, so the row addresses of the next tile are ready without a dependent
// global load.
//
// Per wave: 16 heads (4 waves = 64 heads; more heads use more blocks, the
// waves of the last block past the last head idle).  Per
// tile: 8 S tiles x (4 latent k-steps x 2 (hi, lo) + 1 RoPE k-step) + 32 dim
// tiles x 3 (P' terms) = 168 MFMAs of 16x16x128.
#include "dcp_device.h"
#include "dcp_epilogue.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kT = 128;                            // tokens per tile
constexpr int kGranules = 9;                       // 64-byte granules per row
constexpr int kGranPlane = kT * 64;                // LDS bytes of one granule plane
constexpr int kTileBytes = kGranules * kGranPlane; // 73728
constexpr int kStageBytes = kTileBytes + kT * 4;   // + per-token scales
constexpr int kRingOff = 2 * kStageBytes;          // slot/page-id ring, 3 tiles
constexpr int kSmem = kRingOff + 3 * kT * 4;       // 150016 bytes
constexpr int kThreads = 256;

template <bool B> struct BoolC { static constexpr bool value = B; };
template <int V> struct IntC { static constexpr int value = V; };

// The page table of a prefill chunk: one page, id 0, holding the whole chunk.
__device__ int kChunkPage[1] = {0};

// Chunk permutation of token t inside its 64-byte granule.
__device__ __forceinline__ int chunk_sw(int t) { return ((t >> 1) ^ (t >> 3) ^ (t >> 4)) & 3; }

// Four E4M3 codes (RNE) of four floats, in byte order.
__device__ __forceinline__ int pack_e4m3(float a, float b, float c, float d) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, h, true);
}
// The same of four floats divided by a power of two `div` (the gfx950 scaled
// conversion divides its inputs by its scale operand: for a power of two the
// codes are those of the exact quotients, with no separate multiply).
__device__ __forceinline__ int pack_e4m3_div(float a, float b, float c, float d, float div) {
  typedef short s2 __attribute__((ext_vector_type(2)));
  s2 v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s2{0, 0}, a, b, div, false);
  v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, c, d, div, true);
  return __builtin_bit_cast(int, v);
}

// PARTIAL: the head count is not a multiple of 64 (the last head block has
// idle waves).
template <bool DENSE, bool PARTIAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_fp8_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kSmem];
  __shared__ int s_flag;
  DCP_LDS char* smem = (DCP_LDS char*)smem_raw;
  DCP_LDS int* ring = (DCP_LDS int*)(smem + kRingOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;             // 16-lane group of the MFMA layouts
  const int i16 = lane & 15;

  // ---- block -> (row, shard, split, head block); a row's blocks are
  // consecutive within one XCD's share of the grid
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
  const char* scbase = reinterpret_cast<const char*>(sh.scale);
  const int max_prow = (int)min(sh.pool_rows - 1, (long long)0x7fffffff);

  // ---- this block's token range [start, end) of the shard's local tokens
  int n_tok;
  if constexpr (DENSE) {
    n_tok = p.chunk_mode ? p.chunk_len
                         : (int)min((long long)sh.local_len[row], (long long)p.max_pages * p.page_size);
  } else {
    n_tok = min(p.counts[(long long)shard * p.rows + row], p.k);
  }
  n_tok = max(n_tok, 0);
  const int chunk = ((n_tok + S - 1) / S + kT - 1) / kT * kT;
  // (split 0 starts at 0 without waiting for the count)
  const int start = split == 0 ? 0 : min(n_tok, split * chunk);
  const int end = min(n_tok, start + chunk);
  const int ntiles = (end - start + kT - 1) / kT;
  // When the tokens leave a remainder of 1..64 past whole tiles, that short
  // tile goes first ("lead"): its compute then overlaps the prologue's wait
  // for the first full tile's rows instead of lengthening the block's end,
  // which the row's merge waits for.  Tile it covers [tb(it), te(it)).
  const int rem = (end - start) % kT;
  const int lead = (ntiles > 1 && rem > 0 && rem <= 64) ? rem : 0;
  const int shift = lead > 0 ? kT - lead : 0;
  auto tb = [&](int it) { return start + it * kT - (it > 0 ? shift : 0); };
  auto te = [&](int it) { return (it == 0 && lead > 0) ? start + lead : min(end, tb(it) + kT); };

  // Where the id of local token j lives: the compacted slot id (sparse) or
  // the page id of its logical page (dense).
  const int page = DENSE ? p.page_size : 1;
  const int* ids = DENSE ? (p.chunk_mode ? kChunkPage : p.block_table + row * p.max_pages)
                         : p.topk_local + ((long long)shard * p.rows + row) * p.k;
  auto id_ptr = [&](int j) -> const int* { return DENSE ? ids + j / page : ids + j; };
  auto pool_row = [&](int j, int id) -> int {
    const int r = DENSE ? id * page + (j - (j / page) * page) : id;
    return min(max(r, 0), max_prow);
  };

  // ---- copies.  Rows of tile `it` into stage it & 1: wave w fills token
  // groups 2w and 2w+1 (16 tokens each) for all 9 granules; lane l covers
  // token 16(2w + h) + l/4 and the 16-byte chunk (l & 3) ^ sw of its granule.
  // Waves 0 and 1 also copy the tile's 128 scales (token 64w + lane).
  const int dma_tok = 32 * wave + (lane >> 2);     // + 16h
  const int sc_tok = 64 * (wave & 1) + lane;
  // Tokens past the tile's valid count copy the tile's first token: they are
  // masked out of the softmax, and a real row keeps their V codes finite
  // (P' = 0 times a NaN code would still be NaN).
  auto eff = [&](int it, int t) { return t < te(it) - tb(it) ? t : 0; };
  // A tile's copies are issued in pieces (copy c = 0..17: granule c / 2 of
  // token group 2w + (c & 1), granule-major) so that they can be spread over
  // the MFMA work of the previous tile and the next tile's first k-steps can
  // start on the first granules.  Only the pool rows are kept between the
  // copies (three registers); the addresses are formed at issue time.
  struct RowCopies {
    int prow[2];
    int prow_sc;
  };
  struct TileIds {
    int id[2];
    int sc;
  };
  const int chunk_off0 = 16 * ((lane & 3) ^ chunk_sw(dma_tok));
  const int chunk_off1 = 16 * ((lane & 3) ^ chunk_sw(dma_tok + 16));
  auto plan_rows = [&](int it, const TileIds& id) {
    RowCopies rc;
    const int tok0 = tb(it);
    rc.prow[0] = pool_row(tok0 + eff(it, dma_tok), id.id[0]);
    rc.prow[1] = pool_row(tok0 + eff(it, dma_tok + 16), id.id[1]);
    rc.prow_sc = pool_row(tok0 + eff(it, sc_tok), id.sc);
    return rc;
  };
  auto issue_copy = [&](const RowCopies& rc, int it, int c) {
    const int h = c & 1, G = c >> 1;
    const char* src = kvbase + (long long)rc.prow[h] * sh.row_stride + (h ? chunk_off1 : chunk_off0) + 64 * G;
    dma16(src, smem + (it & 1) * kStageBytes + (2 * wave + h) * 1024 + G * kGranPlane);
  };
  auto issue_scales = [&](const RowCopies& rc, int it) {
    if (wave < 2)
      dma4(reinterpret_cast<const float*>(scbase + (long long)rc.prow_sc * sh.scale_stride),
           smem + (it & 1) * kStageBytes + kTileBytes + 256 * wave);
  };
  // Ids of the tokens this lane copies in tile `it`, from the ring.
  auto ring_ids = [&](int it, TileIds& id) {
    const DCP_LDS int* rg = ring + (it % 3) * kT;
    id.id[0] = rg[eff(it, dma_tok)];
    id.id[1] = rg[eff(it, dma_tok + 16)];
    id.sc = rg[eff(it, sc_tok)];
  };
  // Ids of tile `it` into ring slot `slot` (waves 2 and 3, 64 tokens each).
  auto issue_ring_slot = [&](int it, int slot) {
    const int t = (wave - 2) * 64 + lane;
    dma4(id_ptr(tb(it) + eff(it, t)), ring + slot * kT + (wave - 2) * 64);
  };

  // ---- tile 0's ids go into ring slot 0 by DMA (waves 2 and 3, like every
  // ring slot), and the query right behind them, so that neither waits for
  // the other's latency.  For split 0 the ids do not wait for the count: they
  // are bounded by the id table (cap entries) instead, and the ids of tokens
  // past the count are replaced by the first token's once the count is
  // known, when the copies are planned.
  const int cap = DENSE ? p.max_pages * p.page_size : p.k;
  auto tok_cap = [&](int t) { return start + t < cap ? t : 0; };
  if (wave >= 2 && start < cap) {
    const int t = (wave - 2) * 64 + lane;
    dma4(id_ptr(start + tok_cap(t)), ring + (wave - 2) * 64);
  }

  // ---- the query of the wave's 16 heads (18 KB, contiguous) is copied into
  // stage 1, idle until tile 1's copies, by the same global->LDS DMA as the
  // keys, so that it streams in together with tile 0.  (Register loads would
  // have to land before the first copy is queued: the waits the compiler
  // places before a load's first use do not count the inline copies, so a
  // use after them would also wait for every copy of tile 0.)
  const int head = hblk * kHeadsPerBlock + wave * 16 + i16;
  // In the last head block of a head count that is not a multiple of 64,
  // the waves past the last head copy rows and take part in every barrier
  // and merge, but load no query and store nothing of their own.
  const bool active = !PARTIAL || hblk * kHeadsPerBlock + wave * 16 < H;
  constexpr int kQWaveBytes = 16 * kHeadDim * 2;
  DCP_LDS char* q_lds = smem + kStageBytes + wave * kQWaveBytes;
  if (active) {
    const char* qw = static_cast<const char*>(p.q) +
                     ((size_t)row * H + hblk * kHeadsPerBlock + wave * 16) * kHeadDim * 2;
#pragma unroll
    for (int i = 0; i < kQWaveBytes / 1024; ++i) dma16(qw + 1024 * i + 16 * lane, q_lds + 1024 * i);
  }
  if (wave >= 2) {                     // the ids (the query stays in flight)
    if (active) wait_vmcnt<18>();
    else wait_vmcnt<0>();
  }
  lds_barrier();
  TileIds ids0;
  ids0.id[0] = ring[dma_tok];
  ids0.id[1] = ring[dma_tok + 16];
  ids0.sc = ring[sc_tok];
  const int id_first = ring[0];

  // ---- tile 0: the scales (waves 0, 1) or the ids of tile 1 (waves 2, 3)
  // first, as at the top of every tile, then all its copies.
  const bool issue0 = ntiles > 0, ring1 = ntiles > 1;
  {
    auto valid0 = [&](int t) { return start + t < te(0); };
#pragma unroll
    for (int h = 0; h < 2; ++h) ids0.id[h] = valid0(dma_tok + 16 * h) ? ids0.id[h] : id_first;
    ids0.sc = valid0(sc_tok) ? ids0.sc : id_first;
  }
  const RowCopies rc0 = plan_rows(0, ids0);
  if (issue0 && wave < 2) issue_scales(rc0, 0);
  if (wave >= 2 && ring1) issue_ring_slot(1, 1);
  if (issue0) {
#pragma unroll
    for (int c = 0; c < 18; ++c) issue_copy(rc0, 0, c);
    wait_vmcnt<18>();                  // the query (tile 0's 18 copies stay in flight)
  } else {
    wait_vmcnt<0>();
  }

  // ---- query from LDS.  Latent k-step s < 4: lane group g holds dims 128s +
  // 32g .. +32; RoPE: dims 512 + 16g .. +16.
  bf16x8 raw[4][4], raw_r[2];
  {
    const DCP_LDS char* qh = q_lds + i16 * (kHeadDim * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        raw[s][u] = *reinterpret_cast<const DCP_LDS bf16x8*>(qh + 2 * (128 * s + 32 * g + 8 * u));
#pragma unroll
    for (int u = 0; u < 2; ++u)
      raw_r[u] = *reinterpret_cast<const DCP_LDS bf16x8*>(qh + 2 * (512 + 16 * g + 8 * u));
    if (!active) {                     // no query: zeros (its results are never stored)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[s][u] = bf16x8{};
#pragma unroll
      for (int u = 0; u < 2; ++u) raw_r[u] = bf16x8{};
    }
  }

  // ---- query: Q * 2^e as E4M3 hi + lo (e per head: the largest with
  // max |Q| * 2^e <= 448; a bf16 value has 8 significant bits, so hi + lo is
  // exact unless it falls below the E4M3 range), and the MFMA's B block scale
  // 2^-e undoes the power of two.  qr packs the RoPE dims: hi in bytes 0..15,
  // lo in bytes 16..31 (one MFMA against the RoPE chunk twice).  The query
  // operands live in AGPRs (read by the MFMA as its B operand).
  i32x8 qhi[4], qlo[4], qr;
  int qscale;
  {
    float qmax = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(bf16_to_f32(raw[s][u][j])));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(bf16_to_f32(raw_r[u][j])));
    qmax = max_xor32(max_xor16(qmax));
    const int e = e4m3_exponent(qmax);
    const float qs = pow2i(e);
    qscale = 127 - e;
    // four bf16 values -> (E4M3 hi, E4M3 lo) of their scaled copies
    auto split4 = [&](const bf16x8& v, int off) -> i32x2 {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = bf16_to_f32(v[off + j]) * qs;
      const int h = pack_e4m3(x[0], x[1], x[2], x[3]);
      const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
      const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
      return i32x2{h, pack_e4m3(x[0] - b01[0], x[1] - b01[1], x[2] - b23[0], x[3] - b23[1])};
    };
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const i32x2 hl = split4(raw[s][u], 4 * half);
          qhi[s][2 * u + half] = hl.x;
          qlo[s][2 * u + half] = hl.y;
        }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const i32x2 hl = split4(raw_r[u], 4 * half);
        qr[2 * u + half] = hl.x;
        qr[4 + 2 * u + half] = hl.y;
      }
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+a"(qhi[s]), "+a"(qlo[s]));
    asm volatile("" : "+a"(qr));
  }

  // ---- online-softmax state; lane: head column, O^T dims 16d + 4g + i.
  // Logits are kept as y = q.k * scale_t; the base-2 logit is c * y.
  const float c = p.sm_scale_log2;
  const float bump_gap = 8.0f / c;   // the reference moves when a tile beats it by 2^8
  float m_run = kNegInf;    // reference max of y, moves lazily
  float l_run = 0.f;        // this lane's share of sum 2^(c (y - m_run))
  float smax = 0.f;         // largest |token scale| this lane has read
  // Set by the last tile: the block's l, the fp16 exponent of its workspace
  // partial and whether that partial was stored during the last PV.
  float l_fin = 0.f;
  int ex_ws = kExFromValues;
  bool pre_stored = false;
  f32x4 oacc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets (bytes) inside a stage.
  // QK: S tile st, latent k-step s, lane (token i16, group g) reads chunks
  // 2(g & 1) + cc (cc = 0, 1) of granule 2s + (g >> 1) of token 16st + i16;
  // the RoPE k-step reads chunk g of granule 8.  The chunk permutation of
  // token 16st + i16 is sw0(i16) ^ cst(st).
  const int sw0 = ((i16 >> 1) ^ (i16 >> 3)) & 3;
  int qk_lat[2][4], qk_rope[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      qk_lat[cc][c] = (g >> 1) * kGranPlane + 64 * i16 + 16 * ((2 * (g & 1) + cc) ^ sw0 ^ c);
    qk_rope[c] = 8 * kGranPlane + 64 * i16 + 16 * (g ^ sw0 ^ c);
  }
  // PV: tr8 read r of lane L (group g) fetches token 32r + 16(jj >= 4) + 4g +
  // (jj & 3), jj = L/2, bytes 8(L & 1) of chunk d & 3 of granule d >> 2: lane i
  // of the group then holds dim 16d + i of the 8 tokens of k-slots 8r..8r+7.
  // That token's chunk permutation is swl ^ 2(r & 1).
  const int jj = i16 >> 1;
  const int pv_hi = jj >> 2, pv_p = 4 * g + (jj & 3);
  const int swl = ((pv_p >> 1) ^ (pv_p >> 3) ^ (3 * pv_hi)) & 3;
  int pv_off[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) pv_off[v] = 1024 * pv_hi + 64 * pv_p + 8 * (i16 & 1) + 16 * (v ^ swl);
  // softmax: the scales of tokens 16st + 4g .. +3
  const int sc_off = kTileBytes + 16 * g;

  // Copy schedule of tile it + 1 while tile it is computed (per wave, in
  // this order): one 4-byte copy at the top (scales of it + 1 on waves 0, 1;
  // ids of it + 2 on waves 2, 3), copies 0..8 behind the first nine k-steps
  // of QK, 9..13 spread over the softmax and 14..17 behind the first four PV
  // pairs: about one copy per 400 cycles, the rate at which a CU's share of
  // the memory system drains them when every CU is copying, so the wave
  // rarely stalls at an issue.  Tile it + 1 waits for granules 0..3 (copies
  // 0..7) at its top, for granules 4..7 (copies 8..15) before it loads
  // k-step 2 and for the RoPE granule (16, 17) before it loads k-step 4.  The
  // vmcnt values count the copies issued after the awaited ones.
  // The tile body is instantiated twice: with the next tile's copies
  // (every tile but the last) and without, so that it has no branches on it.
  // The last tile, when at most 64 of its tokens are valid ("short"),
  // skips the QK pass over S tiles 4..7 and packs the three P' terms of its
  // 64 tokens into the k slots of two MFMAs per dim tile instead of three.
  auto tile = [&](auto next_c, auto lead_c, int it) {
    constexpr bool next = decltype(next_c)::value;
    // the lead tile: 33..64 tokens ("short") or 1..32 ("tiny")
    constexpr bool first_short = decltype(lead_c)::value > 0;
    constexpr bool first_tiny = decltype(lead_c)::value == 2;
    constexpr int NS = 8, NQ = 4, NH = 2;
    wait_vmcnt<10>();
    lds_barrier();                       // granules 0..3 of tile it, its scales, ring(it + 1)
    RowCopies rc{};
    if constexpr (next) {
      TileIds id;
      ring_ids(it + 1, id);
      rc = plan_rows(it + 1, id);
      if (wave < 2) issue_scales(rc, it + 1);
      else issue_ring_slot(min(it + 2, ntiles - 1), (it + 2) % 3);
    }

    // Copy c of the next tile at this point of the instruction stream.
    auto copy_at = [&](int c) {
      if constexpr (next) {
        __builtin_amdgcn_sched_barrier(0);
        issue_copy(rc, it + 1, c);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const DCP_LDS char* sb = smem + (it & 1) * kStageBytes;
    const int tok0 = tb(it);
    const int tend = te(it);
    const bool short_tile = first_short || (!next && tend - tok0 <= 64);

    // ---- S^T = K Q^T (base-2 logits), eight 16-token S tiles in two passes of four
    f32x4 sacc[NS];
    i32x8 a[NQ];
#pragma unroll
    for (int half = 0; half < NH; ++half) {
      if (half == 1 && short_tile) {       // S tiles 4..7 are all masked
#pragma unroll
        for (int q = 0; q < NQ; ++q) sacc[4 + q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (next) {              // the copies pass 1 would have carried
#pragma unroll
          for (int j = 5; j < 9; ++j) issue_copy(rc, it + 1, j);
        }
        break;
      }
      // S tiles of this pass (a tiny lead tile's tokens all sit in S tiles 0, 1)
      const int nq = (half == 0 && first_tiny) ? 2 : NQ;
      f32x4 acc[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Operand of S tile 4 half + q for k-step s.
      auto load_kq = [&](int hf, int s, int q) -> i32x8 {
        const int st = 4 * hf + q;
        const int cst = ((2 * st) ^ st) & 3;
        if (s < 4) {
          const i32x4 lo4 = *reinterpret_cast<const DCP_LDS i32x4*>(sb + qk_lat[0][cst] + 2 * s * kGranPlane + 1024 * st);
          const i32x4 hi4 = *reinterpret_cast<const DCP_LDS i32x4*>(sb + qk_lat[1][cst] + 2 * s * kGranPlane + 1024 * st);
          return i32x8{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
        }
        const i32x4 r4 = *reinterpret_cast<const DCP_LDS i32x4*>(sb + qk_rope[cst] + 1024 * st);
        return i32x8{r4.x, r4.y, r4.z, r4.w, r4.x, r4.y, r4.z, r4.w};
      };
      // One operand set, rolled: the operand of S tile q for the next k-step
      // is loaded as soon as q's MFMAs of this k-step are issued, so it has
      // the rest of the k-step to arrive.  (Half 0's RoPE step loads half 1's
      // first operands.)
      if (half == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          if (q < nq) a[q] = load_kq(0, 0, q);
      }
      const bool more = half == 0 && !short_tile;
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        // Before k-step s + 1 is loaded: at s = 1 granules 4..7 (copies up to
        // 15; behind them copies 16, 17 of this tile and, with a next tile,
        // its top copy and copy 0), at s = 3 the RoPE granule (copy 17;
        // behind it the top copy and copies 0..2 of the next tile).
        if (half == 0 && s == 1) {
          if constexpr (next) wait_vmcnt<4>(); else wait_vmcnt<2>();
          lds_barrier();
        }
        if (half == 0 && s == 3) {
          if constexpr (next) wait_vmcnt<4>(); else wait_vmcnt<0>();
          lds_barrier();
        }
        if (s < 4) {
#pragma unroll
          for (int q = 0; q < NQ; q += 2) {
            if (q >= nq) break;
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q], qhi[s], acc[q], 0, 0, 0, 127, 0, qscale);
            acc[q + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q + 1], qhi[s], acc[q + 1], 0, 0, 0, 127, 0, qscale);
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q], qlo[s], acc[q], 0, 0, 0, 127, 0, qscale);
            a[q] = load_kq(half, s + 1, q);
            acc[q + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q + 1], qlo[s], acc[q + 1], 0, 0, 0, 127, 0, qscale);
            a[q + 1] = load_kq(half, s + 1, q + 1);
          }
          // issue order: per pair of S tiles three MFMAs, q's next operand,
          // one MFMA, q + 1's next operand
#pragma unroll
          for (int q = 0; q < NQ; q += 2) {
            if (q >= nq) break;
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else {
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            if (q >= nq) break;
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q], qr, acc[q], 0, 0, 0, 127, 0, qscale);
            if (more) a[q] = load_kq(1, 0, q);
          }
        }
        if constexpr (next) {
          const int j = 5 * half + s;
          if (j < 9) issue_copy(rc, it + 1, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) sacc[4 * half + q] = acc[q];
    }

    // First V^T operands, read before the softmax so their latency hides.
    // The short lead tile's 64 tokens need only the first two tr8 reads of a
    // dim tile, and its softmax only the first four S tiles; the tiny one's
    // 32 tokens one read and two S tiles.
    constexpr int NR = first_tiny ? 1 : first_short ? 2 : 4;        // tr8 reads per dim tile
    constexpr int NSS = first_tiny ? 2 : first_short ? 4 : NS;      // S tiles the softmax covers
    i32x2 vr[2][2][NR];
    auto load_v = [&](int d, i32x2* r4) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        r4[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (DCP_LDS i32x2*)(sb + (d >> 2) * kGranPlane + 2048 * r + pv_off[(d & 3) ^ (2 * (r & 1))]));
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) load_v(j, vr[0][j]);

    // ---- online softmax over the tile (lane: tokens 16st + 4g + i).  The
    // reference max only moves when the tile max exceeds it by more than 8
    // (base 2), so O and l are rescaled rarely; p stays <= 2^8.
    // The token scales are read from LDS once, all together, and kept in
    // registers for both passes.
    float z[NS][4];
    float tmax = kNegInf;
    // Only the short lead tile and the last tile can be partial: every other
    // tile holds kT valid tokens (the lead takes the remainder up front).
    const bool full = (next && !first_short) || tok0 + kT <= tend;
    f32x4 s4v[NSS];
#pragma unroll
    for (int st = 0; st < NSS; ++st) s4v[st] = *reinterpret_cast<const DCP_LDS f32x4*>(sb + sc_off + 64 * st);
#pragma unroll
    for (int st = 0; st < NSS; ++st) {
      const f32x4 s4 = s4v[st];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[st][i] = sacc[st][i] * s4[i];
    }
    copy_at(9);
    if (!full) {                           // the last tile of the row: mask its tail
#pragma unroll
      for (int st = 0; st < NSS; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * st + 4 * g + i >= tend) z[st][i] = kNegInf;
    }
#pragma unroll
    for (int st = 0; st < NSS; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, z[st][i]);
    tmax = max_xor32(max_xor16(tmax));
    copy_at(10);
    const bool bump = tmax > m_run + bump_gap;
    if (__any(bump)) {
      const float m_new = bump ? tmax : m_run;
      const float alpha = bump ? fast_exp2((m_run - m_new) * c) : 1.0f;   // m_run = -inf -> 0
      if (__any(bump && m_run != kNegInf)) {
#pragma unroll
        for (int d = 0; d < 32; ++d) oacc[d] *= alpha;
      }
      l_run *= alpha;
      m_run = m_new;
    }
    const float neg_mc = (m_run == kNegInf) ? 0.f : -m_run * c;
    float (&pr)[NS][4] = z;                // P' = p * scale replaces the logits
    float pmax = 0.f;
#pragma unroll
    for (int st = 0; st < NSS; ++st) {
      const f32x4 s4 = s4v[st];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(fmaf(z[st][i], c, neg_mc));
        l_run += e;
        smax = fmaxf(smax, fabsf(s4[i]));
        pr[st][i] = e * s4[i];
        pmax = fmaxf(pmax, pr[st][i]);
      }
    }
    copy_at(11);

    // ---- P' of the head's 128 tokens as three E4M3 terms at one power of two
    // per head; the MFMA's B block scale (127 - ep) multiplies it back out.
    // The power must be the same in the head's four lanes: in the 16x16x128
    // operand layout lane group g holds k = 16g..16g+15 (bytes 0..15) and
    // 64+16g..64+16g+15 (bytes 16..31), while the scale of the 32-wide k block
    // kb is taken from lane group kb, so every scale block spans two groups.
    pmax = max_xor32(max_xor16(pmax));
    const int ep = e4m3_exponent(pmax);
    const float ps = pow2i(ep), ps_div = pow2i(-ep);
    const int pscale = 127 - ep;
    i32x8 pb[3] = {};                      // pb[term] byte 4st + i
#pragma unroll
    for (int st = 0; st < NSS; ++st) {
      float x[4];                          // (only in the residuals: fused there)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = pr[st][i] * ps;
      const int h = pack_e4m3_div(pr[st][0], pr[st][1], pr[st][2], pr[st][3], ps_div);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
      const float r0 = x[0] - h01[0], r1 = x[1] - h01[1], r2 = x[2] - h23[0], r3 = x[3] - h23[1];
      const int m = pack_e4m3(r0, r1, r2, r3);
      const auto m01 = __builtin_amdgcn_cvt_pk_f32_fp8(m, false);
      const auto m23 = __builtin_amdgcn_cvt_pk_f32_fp8(m, true);
      const int l = pack_e4m3(r0 - m01[0], r1 - m01[1], r2 - m23[0], r3 - m23[1]);
      pb[0][st] = h;
      pb[1][st] = m;
      pb[2][st] = l;
      if (st == (NSS > 2 ? 2 : NSS - 1)) copy_at(12);
      if (st == (NSS > 5 ? 5 : NSS - 1)) copy_at(13);
    }

    // ---- The last tile stores the workspace partial during its PV, each
    // dim-tile pair right behind its final MFMAs.  l is complete once the
    // softmax has run, and |O / l| <= 448 * (largest token scale), since O / l
    // is a convex combination of scaled E4M3 values: that bound fixes the
    // fp16 exponent before O is known.  (Only the fp16 partial of the row
    // merge is stored early; the fp32 one of a split shard is stored after
    // the loop.)
    const bool ws_early = !next && p.o != nullptr && !(p.o_part != nullptr && p.num_splits > 1);
    if constexpr (!next) {
      l_fin = sum_xor32(sum_xor16(l_run));
      ex_ws = half_exponent(448.0f * max_xor32(max_xor16(smax)));
      pre_stored = ws_early;
    }
    const WsPartial<kThreads, true, true> wsp(p, row, shard, split, head, g,
                                         l_fin > 0.f ? 1.0f / l_fin : 0.f, ex_ws);
    // No branch per store: the own dim tiles (kept in registers for the
    // merge) and an idle wave's tiles are stored past the end of the
    // workspace resource, where the store is dropped.
    auto store_pair = [&](int pair) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int d = 2 * pair + j;
        wsp.store_half(d, oacc[d], active && !wsp.is_own(d));
      }
    };

    // ---- O^T += V^T P'^T: 32 dim tiles in 16 pairs, operands one pair ahead.
    // k slot byte 4st + i of lane group g is token 16st + 4g + i, one MFMA
    // per P' term.  A short tile's 64 tokens sit in bytes 0..15 (tr8 reads
    // 0, 1); its operands repeat them, with the terms (hi, mid) in one MFMA
    // and (lo, zero) in a second.  A tiny lead tile's 32 tokens sit in bytes
    // 0..7 (tr8 read 0): hi, mid and lo go into bytes 0..23 of one MFMA.
    auto pv = [&](auto short_c, auto store_c) {
      constexpr bool sh = decltype(short_c)::value;
      constexpr bool st = decltype(store_c)::value;   // the last tile's early stores
      constexpr bool ty = first_tiny;                 // all three terms in one MFMA
      constexpr int NT3 = ty ? 1 : sh ? 2 : 3;        // MFMAs per dim tile
      i32x8 pf[2];
      if constexpr (ty) {
        pf[0] = i32x8{pb[0][0], pb[0][1], pb[1][0], pb[1][1], pb[2][0], pb[2][1], 0, 0};
      } else if constexpr (sh) {
        pf[0] = i32x8{pb[0][0], pb[0][1], pb[0][2], pb[0][3], pb[1][0], pb[1][1], pb[1][2], pb[1][3]};
        pf[1] = i32x8{pb[2][0], pb[2][1], pb[2][2], pb[2][3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int grp = 0; grp < 16; ++grp) {
        if (grp + 1 < 16) {
#pragma unroll
          for (int j = 0; j < 2; ++j) load_v(2 * (grp + 1) + j, vr[(grp + 1) & 1][j]);
        }
        i32x8 vt[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const i32x2* r4 = vr[grp & 1][j];
          if constexpr (ty)
            vt[j] = i32x8{r4[0].x, r4[0].y, r4[0].x, r4[0].y, r4[0].x, r4[0].y, r4[0].x, r4[0].y};
          else if constexpr (sh)
            vt[j] = i32x8{r4[0].x, r4[0].y, r4[1].x, r4[1].y, r4[0].x, r4[0].y, r4[1].x, r4[1].y};
          else
            vt[j] = i32x8{r4[0].x, r4[0].y, r4[1].x, r4[1].y, r4[NR - 2].x, r4[NR - 2].y, r4[NR - 1].x, r4[NR - 1].y};
        }
        if constexpr (next) {
          if (grp < 4) issue_copy(rc, it + 1, 14 + grp);
        }
        // term-major: two independent accumulators between dependent MFMAs
#pragma unroll
        for (int term = 0; term < NT3; ++term)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            oacc[2 * grp + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                vt[j], (ty || sh) ? pf[term] : pb[term], oacc[2 * grp + j], 0, 0, 0, 127, 0, pscale);
        if constexpr (st) {
          if (grp > 0) store_pair(grp - 1);
        }
        // issue order: the next pair's V^T reads first, then this pair's MFMAs
        if (grp + 1 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NR, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NT3, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (st) store_pair(15);
    };
    auto run_pv = [&](auto store_c) {
      if constexpr (first_short) {
        pv(BoolC<true>{}, store_c);
      } else {
        if (!short_tile) pv(BoolC<false>{}, store_c);
        else pv(BoolC<true>{}, store_c);
      }
    };
    if constexpr (next) {
      run_pv(BoolC<false>{});
    } else {
      if (ws_early) run_pv(BoolC<true>{});
      else run_pv(BoolC<false>{});
    }
  };
  // Tile 0's copies are waited for at its top like any tile's.
  int it = 0;
  if (lead > 32) tile(BoolC<true>{}, IntC<1>{}, it++);       // (lead > 0 implies ntiles > 1)
  else if (lead > 0) tile(BoolC<true>{}, IntC<2>{}, it++);
  for (; it + 1 < ntiles; ++it) tile(BoolC<true>{}, IntC<0>{}, it);
  if (it < ntiles) tile(BoolC<false>{}, IntC<0>{}, it);
  wait_vmcnt<0>();   // copies queued for tiles that turned out empty

  const float l_tot = sum_xor32(sum_xor16(l_run));
  finish_block<kThreads, true, true>(p, row, shard, split, head, g, active, oacc, m_run * c, l_tot, smem, &s_flag,
                               ex_ws, pre_stored);
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeParams& p, bool dense, hipStream_t stream) {
  const long long blocks = p.rows * p.num_shards * (long long)p.num_splits * p.head_blocks;
  void* args[] = {(void*)&p};
  const bool partial = p.heads % kHeadsPerBlock != 0;
  const void* fn = dense ? (partial ? (const void*)decode_fp8_kernel<true, true>
                                    : (const void*)decode_fp8_kernel<true, false>)
                         : (partial ? (const void*)decode_fp8_kernel<false, true>
                                    : (const void*)decode_fp8_kernel<false, false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

}  // namespace dcp
