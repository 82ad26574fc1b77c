// Step 2 (+ step 3 fused) for FP8 E4M3 KV with 64 or 128 gathered heads:
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
// one 64-byte granule of 16 tokens, four lanes per granule, so the global
// side of every instruction is 16 whole 64-byte segments.  LDS layout of a
// stage: [granule G: bytes 64G.. of the row, 9][token / 16][token % 16][4 x
// 16-byte chunks], the chunks of token t permuted by XOR with sw(t) =
// ((t >> 1) ^ (t >> 3) ^ (t >> 4)) & 3, which keeps the 16-byte operand
// reads of S^T = K Q^T and the 8-byte transposing reads of V^T free of bank
// conflicts on 32- and 64-bank LDS alike.  Two stages: tile it+1 streams in
// while tile it is computed.  The slot ids (sparse) or page ids (dense) of
// tile it+2 are DMA'd into a three-deep ring at the same time, so the row
// addresses of the next tile are ready without a dependent global load.
//
// Per wave: 16 heads (4 waves = 64 heads; 128 heads use two blocks).  Per
// tile: 8 S tiles x 5 k-steps x 2 (hi, lo) + 32 dim tiles x 3 (P' terms) =
// 176 MFMAs of 16x16x128.
#include "dcp_device.h"
#include "dcp_epilogue.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kT = 128;                            // tokens per tile
constexpr int kRowBytes = 576;                     // E4M3 codes per key row
constexpr int kGranules = 9;                       // 64-byte granules per row
constexpr int kGranPlane = kT * 64;                // LDS bytes of one granule plane
constexpr int kTileBytes = kGranules * kGranPlane; // 73728
constexpr int kStageBytes = kTileBytes + kT * 4;   // + per-token scales
constexpr int kRingOff = 2 * kStageBytes;          // slot/page-id ring, 3 tiles
constexpr int kSmem = kRingOff + 3 * kT * 4;       // 150016 bytes
constexpr int kThreads = 256;

template <bool B> struct BoolC { static constexpr bool value = B; };

// Chunk permutation of token t inside its 64-byte granule.
__device__ __forceinline__ int chunk_sw(int t) { return ((t >> 1) ^ (t >> 3) ^ (t >> 4)) & 3; }

// Four E4M3 codes (RNE) of four floats, in byte order.
__device__ __forceinline__ int pack_e4m3(float a, float b, float c, float d) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, h, true);
}

template <bool DENSE>
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
  const int max_prow = (int)min(sh.pool_rows - 1, (long long)0x7fffffff);

  // ---- this block's token range [start, end) of the shard's local tokens
  int n_tok;
  if constexpr (DENSE) {
    n_tok = (int)min((long long)sh.local_len[row], (long long)p.max_pages * p.page_size);
  } else {
    n_tok = min(p.counts[(long long)shard * p.rows + row], p.k);
  }
  n_tok = max(n_tok, 0);
  const int chunk = ((n_tok + S - 1) / S + kT - 1) / kT * kT;
  const int start = min(n_tok, split * chunk);
  const int end = min(n_tok, start + chunk);
  const int ntiles = (end - start + kT - 1) / kT;

  // Where the id of local token j lives: the compacted slot id (sparse) or
  // the page id of its logical page (dense).
  const int page = DENSE ? p.page_size : 1;
  const int* ids = DENSE ? p.block_table + row * p.max_pages
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
  // Tokens past the tile's valid count re-read token 0 (never used).
  auto eff = [&](int it, int t) { return t < min(kT, end - (start + it * kT)) ? t : 0; };
  // A tile's copies are issued in pieces (copy c = 0..17: token group 2w +
  // c / 9, granule c % 9) so that they can be spread over the MFMA work of
  // the previous tile.
  // Only the pool rows are kept between the copies (three registers); the
  // addresses are formed at issue time.
  struct RowCopies {
    int prow[2];
    int prow_sc;
  };
  const int chunk_off0 = 16 * ((lane & 3) ^ chunk_sw(dma_tok));
  const int chunk_off1 = 16 * ((lane & 3) ^ chunk_sw(dma_tok + 16));
  auto plan_rows = [&](int it, int id0, int id1, int idsc) {
    RowCopies rc;
    const int tok0 = start + it * kT;
    rc.prow[0] = pool_row(tok0 + eff(it, dma_tok), id0);
    rc.prow[1] = pool_row(tok0 + eff(it, dma_tok + 16), id1);
    rc.prow_sc = pool_row(tok0 + eff(it, sc_tok), idsc);
    return rc;
  };
  // Copy c of a tile: granule c / 2 of token group 2w + (c & 1) (granule-major,
  // so that the k-steps of the next tile can start on the first granules).
  auto issue_copy = [&](const RowCopies& rc, int it, int c) {
    const int h = c & 1, G = c >> 1;
    const char* src = kvbase + (long long)rc.prow[h] * kRowBytes + (h ? chunk_off1 : chunk_off0) + 64 * G;
    dma16(src, smem + (it & 1) * kStageBytes + (2 * wave + h) * 1024 + G * kGranPlane);
  };
  auto issue_scales = [&](const RowCopies& rc, int it) {
    if (wave < 2) dma4(sh.scale + rc.prow_sc, smem + (it & 1) * kStageBytes + kTileBytes + 256 * wave);
  };
  auto issue_rows = [&](int it, int id0, int id1, int idsc) {
    const RowCopies rc = plan_rows(it, id0, id1, idsc);
#pragma unroll
    for (int c = 0; c < 2 * kGranules; ++c) issue_copy(rc, it, c);
    issue_scales(rc, it);
  };
  // Ids of the tokens this lane copies in tile `it`, from the ring.
  auto ring_ids = [&](int it, int& id0, int& id1, int& idsc) {
    const DCP_LDS int* rg = ring + (it % 3) * kT;
    id0 = rg[eff(it, dma_tok)];
    id1 = rg[eff(it, dma_tok + 16)];
    idsc = rg[eff(it, sc_tok)];
  };
  // Ids of tile `it` into ring slot `slot` (waves 2 and 3, 64 tokens each).
  auto issue_ring_slot = [&](int it, int slot) {
    const int t = (wave - 2) * 64 + lane;
    dma4(id_ptr(start + it * kT + eff(it, t)), ring + slot * kT + (wave - 2) * 64);
  };

  // ---- tile 0's ids with plain loads (padding tokens re-read token 0)
  int id0 = 0, id1 = 0, idsc = 0;
  if (ntiles > 0) {
    id0 = *id_ptr(start + eff(0, dma_tok));
    id1 = *id_ptr(start + eff(0, dma_tok + 16));
    idsc = *id_ptr(start + eff(0, sc_tok));
  }

  // ---- query loads (consumed after tile 0's copies are queued).  Latent
  // k-step s < 4: lane group g holds dims 128s + 32g .. +32; RoPE: dims
  // 512 + 16g .. +16.
  const int head = hblk * kHeadsPerBlock + wave * 16 + i16;
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + ((size_t)row * H + head) * kHeadDim;
  bf16x8 raw[4][4], raw_r[2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      raw[s][u] = *reinterpret_cast<const bf16x8*>(qrow + 128 * s + 32 * g + 8 * u);
#pragma unroll
  for (int u = 0; u < 2; ++u) raw_r[u] = *reinterpret_cast<const bf16x8*>(qrow + 512 + 16 * g + 8 * u);
  __builtin_amdgcn_sched_barrier(0);   // the query loads go out before the ids are waited for

  if (ntiles > 0) issue_rows(0, id0, id1, idsc);
  if (wave >= 2 && ntiles > 1) issue_ring_slot(1, 1);

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
  // ids of it + 2 on waves 2, 3), copies 0..9 behind the ten k-steps of QK,
  // copies 10..17 behind the first eight PV pairs.  Copies are granule-major,
  // so tile it + 1 waits for granules 0..3 (copies 0..7) at its top, for
  // granules 4..7 before it loads k-step 2 and for the RoPE granule before it
  // loads k-step 4.  The vmcnt values count the copies issued after the
  // awaited ones.
  // The tile body is instantiated twice: with the next tile's copies
  // (every tile but the last) and without, so that it has no branches on it.
  auto tile = [&](auto next_c, int it) {
    constexpr bool next = decltype(next_c)::value;
    wait_vmcnt<10>();
    lds_barrier();                       // granules 0..3 of tile it, its scales, ring(it + 1)
    RowCopies rc{};
    if constexpr (next) {
      ring_ids(it + 1, id0, id1, idsc);
      rc = plan_rows(it + 1, id0, id1, idsc);
      if (wave < 2) issue_scales(rc, it + 1);
      else issue_ring_slot(min(it + 2, ntiles - 1), (it + 2) % 3);
    }

    const DCP_LDS char* sb = smem + (it & 1) * kStageBytes;
    const int tok0 = start + it * kT;

    // ---- S^T = K Q^T (base-2 logits), eight 16-token S tiles in two passes of four
    f32x4 sacc[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto load_k = [&](int s, i32x8* a) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int st = 4 * half + q;
          const int cst = ((2 * st) ^ st) & 3;
          if (s < 4) {
            const i32x4 lo4 = *reinterpret_cast<const DCP_LDS i32x4*>(sb + qk_lat[0][cst] + 2 * s * kGranPlane + 1024 * st);
            const i32x4 hi4 = *reinterpret_cast<const DCP_LDS i32x4*>(sb + qk_lat[1][cst] + 2 * s * kGranPlane + 1024 * st);
            a[q] = i32x8{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
          } else {
            const i32x4 r4 = *reinterpret_cast<const DCP_LDS i32x4*>(sb + qk_rope[cst] + 1024 * st);
            a[q] = i32x8{r4.x, r4.y, r4.z, r4.w, r4.x, r4.y, r4.z, r4.w};
          }
        }
      };
      // One operand set: step s + 1 is loaded once step s's MFMAs are
      // issued (they have eight MFMAs of work queued to cover the latency).
      i32x8 a[4];
      load_k(0, a);
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
          for (int q = 0; q < 4; ++q)
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q], qhi[s], acc[q], 0, 0,
                                                                     0, 127, 0, qscale);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q], qlo[s], acc[q], 0, 0,
                                                                     0, 127, 0, qscale);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[q], qr, acc[q], 0, 0,
                                                                     0, 127, 0, qscale);
        }
        if constexpr (next) issue_copy(rc, it + 1, 5 * half + s);
        if (s + 1 < 5) load_k(s + 1, a);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sacc[4 * half + q] = acc[q];
    }

    // First V^T operands, read before the softmax so their latency hides.
    i32x2 vr[2][2][4];
    auto load_v = [&](int d, i32x2* r4) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        r4[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (DCP_LDS i32x2*)(sb + (d >> 2) * kGranPlane + 2048 * r + pv_off[(d & 3) ^ (2 * (r & 1))]));
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) load_v(j, vr[0][j]);

    // ---- online softmax over the tile (lane: tokens 16st + 4g + i).  The
    // reference max only moves when the tile max exceeds it by more than 8
    // (base 2), so O and l are rescaled rarely; p stays <= 2^8.
    // The token scales are read from LDS twice rather than kept in registers.
    float z[8][4];
    float tmax = kNegInf;
    const bool full = tok0 + kT <= end;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const f32x4 s4 = *reinterpret_cast<const DCP_LDS f32x4*>(sb + sc_off + 64 * st);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[st][i] = sacc[st][i] * s4[i];
    }
    if (!full) {                           // the last tile of the row: mask its tail
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * st + 4 * g + i >= end) z[st][i] = kNegInf;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, z[st][i]);
    tmax = max_xor32(max_xor16(tmax));
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
    float (&pr)[8][4] = z;                 // P' = p * scale replaces the logits
    float pmax = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const f32x4 s4 = *reinterpret_cast<const DCP_LDS f32x4*>(sb + sc_off + 64 * st);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(fmaf(z[st][i], c, neg_mc));
        l_run += e;
        pr[st][i] = e * s4[i];
        pmax = fmaxf(pmax, pr[st][i]);
      }
    }

    // ---- P' of the head's 128 tokens as three E4M3 terms at one power of two
    // per head; the MFMA's B block scale (127 - ep) multiplies it back out.
    // The power must be the same in the head's four lanes: in the 16x16x128
    // operand layout lane group g holds k = 16g..16g+15 (bytes 0..15) and
    // 64+16g..64+16g+15 (bytes 16..31), while the scale of the 32-wide k block
    // kb is taken from lane group kb, so every scale block spans two groups.
    pmax = max_xor32(max_xor16(pmax));
    const int ep = e4m3_exponent(pmax);
    const float ps = pow2i(ep);
    const int pscale = 127 - ep;
    i32x8 p3[3];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = pr[st][i] * ps;
      const int h = pack_e4m3(x[0], x[1], x[2], x[3]);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
      const float r0 = x[0] - h01[0], r1 = x[1] - h01[1], r2 = x[2] - h23[0], r3 = x[3] - h23[1];
      const int m = pack_e4m3(r0, r1, r2, r3);
      const auto m01 = __builtin_amdgcn_cvt_pk_f32_fp8(m, false);
      const auto m23 = __builtin_amdgcn_cvt_pk_f32_fp8(m, true);
      const int l = pack_e4m3(r0 - m01[0], r1 - m01[1], r2 - m23[0], r3 - m23[1]);
      p3[0][st] = h;
      p3[1][st] = m;
      p3[2][st] = l;
    }

    // ---- O^T += V^T P'^T: 32 dim tiles in 16 pairs, operands one pair ahead
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
        vt[j] = i32x8{r4[0].x, r4[0].y, r4[1].x, r4[1].y, r4[2].x, r4[2].y, r4[3].x, r4[3].y};
      }
      if constexpr (next) {
        if (grp < 8) issue_copy(rc, it + 1, 10 + grp);
      }
      // term-major: two independent accumulators between dependent MFMAs
#pragma unroll
      for (int term = 0; term < 3; ++term)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          oacc[2 * grp + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              vt[j], p3[term], oacc[2 * grp + j], 0, 0, 0, 127, 0, pscale);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  wait_vmcnt<0>();                       // everything the prologue queued
  int it = 0;
  for (; it + 1 < ntiles; ++it) tile(BoolC<true>{}, it);
  if (it < ntiles) tile(BoolC<false>{}, it);

  const float l_tot = sum_xor32(sum_xor16(l_run));
  finish_block<kThreads>(p, row, shard, split, head, g, true, oacc, m_run * c, l_tot, smem, &s_flag);
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeParams& p, bool dense, hipStream_t stream) {
  const long long blocks = p.rows * p.num_shards * (long long)p.num_splits * p.head_blocks;
  void* args[] = {(void*)&p};
  const void* fn = dense ? (const void*)decode_fp8_kernel<true> : (const void*)decode_fp8_kernel<false>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

}  // namespace dcp
