// Sharded index cache and distributed top-k: every shard scores its own
// tokens' index keys and keeps its local top-k; the shards' candidates are
// merged into the global top-k, whose slots feed the index remap.
//
// Pages: [P3] "[DSA] Fix decode context parallelism for RoPE sparse attention
// on Blackwell", Follow-ups item 2 (index keys of 128 FP8 values + one fp32
// scale per token, 132 bytes, split across the ranks like the KV; the local
// top-k candidates merged by one more collective per indexer layer); [P1]
// "feat: support decode context parallelism for PyTorch MLA", Summary (DSA
// merges local candidates into the global top-k), File summaries
// (distributed candidate packing and merging) and the review note that the
// merge needs dcp * k to be a multiple of 512.
//
// Score (the DSA indexer form; the pages give none): for a query row with
// index heads h (E4M3FN codes q_h, fp32 weight w_h) and a token with index
// key codes k_t and scale s_t > 0,
//     score(t) = s_t * sum_h w_h * max(0, q_h . k_t),
// with q_h . k_t on the fp8 MFMA (16 tokens x 16 heads x 128 dims per
// instruction; every product of two E4M3 values is exact, and the
// instruction's sum keeps about 14 bits below its largest product).
// One wave scores 256 tokens, sixteen 16-token groups loaded four at a time;
// its A operands come straight from global memory (a token's 128-byte key
// row is one line, and the 16 tokens of a group are contiguous rows of a
// page).  The sum over a group's 16 heads runs on DPP row moves.
//
// Selection: score descending, then position ascending, as one 64-bit key
// (the order-preserving image of the fp32 score above the complement of the
// position), so every key is distinct and the top k is unique.  One block
// per list finds the k-th largest key by radix select (eight 8-bit digits,
// histograms in LDS, the list re-read from L2 per pass), gathers the keys
// above it and sorts them (bitonic, in LDS).
#include "dcp_device.h"
#include "dcp_internal.h"

namespace dcp {
namespace {

constexpr int kScoreThreads = 256;                 // 4 waves
constexpr int kScoreWaveGroups = 16;               // 16-token groups per wave
constexpr int kScoreBatch = 4;                     // groups loaded together
constexpr int kScoreTokens = 4 * 16 * kScoreWaveGroups;   // 1024 tokens per block
constexpr int kSelectThreads = 1024;

// ---------------------------------------------------------------- scores

// Sum over the 16 lanes of each row of the wave (every lane gets its row's
// sum): the quads first, then the row's half mirror and full mirror, all by
// DPP moves (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_move<0xb1>(x);     // quad_perm 1,0,3,2
  x += dpp_move<0x4e>(x);     // quad_perm 2,3,0,1
  x += dpp_move<0x141>(x);    // row_half_mirror: quad 0 <-> 1, 2 <-> 3
  x += dpp_move<0x140>(x);    // row_mirror: the two halves
  return x;
}

// HG: index head groups of 16.
template <int HG>
__global__ __launch_bounds__(kScoreThreads) void index_score_kernel(IndexScoreParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  long long b = blockIdx.x;
  const int tiles = p.tiles_per_list;
  const int tile = (int)(b % tiles);
  b /= tiles;
  const int shard = (int)(b % p.num_shards);
  const long long row = b / p.num_shards;
  const IndexShardArg sh = p.shard[shard];
  const int n_local = min(max(sh.local_len[row], 0), p.max_local);
  const int t0 = tile * kScoreTokens + wave * (16 * kScoreWaveGroups);
  if (t0 >= n_local) return;

  // query operands (B of S^T = K Q^T): head group hg, lane (head i16, g) holds
  // bytes 16g .. +16 and 64 + 16g .. +16 of its head's 128 codes (the keys'
  // A operands take the same bytes, so the products pair up)
  typedef __attribute__((ext_vector_type(4))) int i32x4_t;
  const unsigned char* qrow = p.q + (size_t)row * p.hi * kIndexDim;
  const float* wrow = p.w + (size_t)row * p.hi;
  i32x8 qb[HG];
  float wv[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const unsigned char* qh = qrow + (size_t)(16 * hg + i16) * kIndexDim;
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(qh + 16 * g);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(qh + 64 + 16 * g);
    qb[hg] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    wv[hg] = wrow[16 * hg + i16];
  }
  const int* bt = p.block_table + row * p.max_pages;
  const long long max_prow = sh.pool_rows - 1;
  auto pool_row = [&](int j) -> long long {
    const int pg = min(j / p.page_size, p.max_pages - 1);
    const long long r = (long long)bt[pg] * p.page_size + (j - (j / p.page_size) * p.page_size);
    return min(max(r, 0LL), max_prow);
  };
  const char* keys = static_cast<const char*>(sh.keys);
  const char* scl = reinterpret_cast<const char*>(sh.scale);
  float* out_row = p.scores + ((long long)shard * p.rows + row) * p.max_local;

  for (int gb = 0; gb < kScoreWaveGroups; gb += kScoreBatch) {
    if (t0 + 16 * gb >= n_local) break;
    // the batch's key rows and scales first (lane: token 16 grp + i16)
    i32x8 ka[kScoreBatch];
    float scv[kScoreBatch];
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      const int j = min(t0 + 16 * (gb + u) + i16, n_local - 1);
      const long long pr = pool_row(j);
      const char* kr = keys + pr * sh.row_stride;
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kr + 16 * g);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(kr + 64 + 16 * g);
      ka[u] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      scv[u] = *reinterpret_cast<const float*>(scl + pr * sh.scale_stride);
    }
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      // lane (head i16, g): tokens 4g .. 4g + 3 of the group, summed over head groups
      f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            ka[u], qb[hg], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] += wv[hg] * fmaxf(d[i], 0.f);
      }
      // sum over the 16 heads of the group's lanes
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = row16_sum(part[i]);
      // token 4g + i's scale sits in lane 4g + i (its A row)
      f32x4 res;
#pragma unroll
      for (int i = 0; i < 4; ++i) res[i] = __shfl(scv[u], 4 * g + i, 64) * part[i];
      const int j0 = t0 + 16 * (gb + u) + 4 * g;
      if (i16 == 0) {
        if (j0 + 3 < n_local && (reinterpret_cast<uintptr_t>(out_row + j0) & 15u) == 0) {
          *reinterpret_cast<f32x4*>(out_row + j0) = res;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (j0 + i < n_local) out_row[j0 + i] = res[i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- selection

// Order-preserving image of an fp32 score (larger score, larger key).
__device__ __forceinline__ unsigned score_bits(float s) {
  const unsigned u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float bits_score(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ unsigned long long make_key(float s, int pos) {
  const float v = s == 0.f ? 0.f : s;               // -0 ranks as +0 (they are equal scores)
  return ((unsigned long long)score_bits(v) << 32) | (unsigned)(0xffffffffu - (unsigned)pos);
}

// Element e of list `list`: its key, or 0 (below every real key: position
// 0xffffffff never occurs) when it is not a candidate.
struct ListSource {
  const TopkParams& p;
  long long list;
  int n;
  __device__ unsigned long long key(int e) const {
    if (p.merge) {
      const long long row = list;
      const int r = e / p.k_in, idx = e - r * p.k_in;
      const long long at = ((long long)r * p.rows + row) * p.k_in + idx;
      const int pos = p.in_pos[at];
      return pos >= 0 ? make_key(p.in_score[at], pos) : 0ull;
    }
    const int shard = (int)(list / p.rows);
    return make_key(p.in_score[list * p.max_local + e], e * p.num_shards + shard);
  }
};

__global__ __launch_bounds__(kSelectThreads) void topk_select_kernel(TopkParams p) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ unsigned s_need, s_count;
  __shared__ unsigned long long sel[kMaxTopk];
  const int tid = threadIdx.x;
  const long long list = blockIdx.x;
  int n;
  if (p.merge) {
    n = p.num_shards * p.k_in;
  } else {
    const int shard = (int)(list / p.rows);
    const long long row = list - (long long)shard * p.rows;
    n = min(max(p.local_len[(long long)shard * p.rows + row], 0), p.max_local);
  }
  const ListSource src{p, list, n};
  const int k = p.k;

  // ---- count the candidates (merge lists may hold padding)
  if (tid == 0) s_count = 0;
  __syncthreads();
  unsigned mine = 0;
  for (int e = tid; e < n; e += kSelectThreads) mine += src.key(e) != 0ull;
  atomicAdd(&s_count, mine);
  __syncthreads();
  const unsigned valid = s_count;

  // ---- the k-th largest key (all keys are distinct), digit by digit
  unsigned long long thresh = 1ull;                 // every candidate when valid <= k
  if (valid > (unsigned)k) {
    if (tid == 0) { s_prefix = 0ull; s_need = (unsigned)k; }
    unsigned long long mask = 0ull;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelectThreads) hist[i] = 0;
      __syncthreads();
      const unsigned long long prefix = s_prefix;
      for (int e = tid; e < n; e += kSelectThreads) {
        const unsigned long long kv = src.key(e);
        if (kv != 0ull && (kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned need = s_need, above = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (above + hist[d] >= need) break;
          above += hist[d];
        }
        s_need = need - above;
        s_prefix = prefix | ((unsigned long long)d << shift);
      }
      mask |= 255ull << shift;
      __syncthreads();
    }
    thresh = s_prefix;
  }

  // ---- gather the selected keys, then sort them (descending)
  const unsigned m = valid < (unsigned)k ? valid : (unsigned)k;
  if (tid == 0) s_count = 0;
  __syncthreads();
  for (int e = tid; e < n; e += kSelectThreads) {
    const unsigned long long kv = src.key(e);
    if (kv != 0ull && kv >= thresh) {
      const unsigned at = atomicAdd(&s_count, 1u);
      if (at < m) sel[at] = kv;                     // exactly m pass (keys are distinct)
    }
  }
  __syncthreads();
  int np2 = 1;
  while (np2 < (int)m) np2 <<= 1;
  for (int i = (int)m + tid; i < np2; i += kSelectThreads) sel[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < np2 / 2; i += kSelectThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const unsigned long long a = sel[lo], c = sel[hi];
        if ((a < c) == desc) {
          sel[lo] = c;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  // ---- write the list's top k in order, padded with (-inf, -1)
  for (int i = tid; i < k; i += kSelectThreads) {
    float s = kNegInf;
    int pos = -1;
    if (i < (int)m) {
      const unsigned long long kv = sel[i];
      s = bits_score((unsigned)(kv >> 32));
      pos = (int)(0xffffffffu - (unsigned)(kv & 0xffffffffull));
    }
    if (p.out_score) p.out_score[list * k + i] = s;
    if (p.out_pos) p.out_pos[list * k + i] = pos;
    if (p.out_slot) {
      int slot = -1;
      if (pos >= 0) {
        const long long span = (long long)p.page_size * p.num_shards;
        const long long lp = min((long long)pos / span, (long long)p.max_pages - 1);
        slot = (int)((long long)p.block_table[list * p.max_pages + lp] * span + pos % span);
      }
      p.out_slot[list * k + i] = slot;
    }
  }
}

// Local top-k of lists of at most kLocalFastMax scores, held in registers
// (32 per thread): radix select on the 32-bit order image of the score (four
// 8-bit digits, stopping early when a digit's bucket is taken whole), the
// tied scores at the threshold taken by position, then the k keys sorted.
// Histogram updates are combined per wave when a wave's values share a
// bucket (the leading digits of nearby scores usually do).
constexpr int kLocalVpt = 32;
constexpr int kLocalFastMax = kSelectThreads * kLocalVpt;   // 32768

__device__ __forceinline__ void hist_add(unsigned* hist, unsigned bin, bool on) {
  const unsigned lead = __builtin_amdgcn_readfirstlane(on ? bin : 0xffffffffu);
  const unsigned long long same = __ballot(on && bin == lead);
  const int n_same = __popcll(same);
  if (n_same >= 8) {
    if (on && bin == lead) {
      const unsigned long long lower = same & ((1ull << (threadIdx.x & 63)) - 1ull);
      if (lower == 0ull) atomicAdd(&hist[bin], (unsigned)n_same);
    } else if (on) {
      atomicAdd(&hist[bin], 1u);
    }
  } else if (on) {
    atomicAdd(&hist[bin], 1u);
  }
}

__global__ __launch_bounds__(kSelectThreads) void topk_local_fast_kernel(TopkParams p) {
  __shared__ unsigned whist[kSelectThreads / 64][256];   // one digit histogram per wave
  __shared__ unsigned s_word[4];
  __shared__ unsigned wave_sum[kSelectThreads / 64];
  __shared__ unsigned long long sel[kMaxTopk];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long list = blockIdx.x;
  const int shard = (int)(list / p.rows);
  const long long row = list - (long long)shard * p.rows;
  const int n = min(max(p.local_len[(long long)shard * p.rows + row], 0), p.max_local);
  const int k = p.k;
  const float* src = p.in_score + list * p.max_local;
  unsigned key[kLocalVpt];
#pragma unroll
  for (int i = 0; i < kLocalVpt; ++i) {
    const int e = tid + i * kSelectThreads;
    const float v = e < n ? src[e] : 0.f;
    key[i] = score_bits(v == 0.f ? 0.f : v);
  }
  const unsigned m = (unsigned)min(n, k);
  unsigned thresh = 0u;         // select keys above thresh, and `need` keys equal to it
  unsigned need = 0u;
  bool ties = false;
  if (n > k) {
    unsigned prefix = 0u, mask = 0u, rem = (unsigned)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      // each wave counts its own keys (no atomics across waves); the wave's
      // LDS operations stay in order, so its zeroing needs no barrier
#pragma unroll
      for (int j = 0; j < 4; ++j) whist[wv][4 * lane + j] = 0u;
#pragma unroll
      for (int i = 0; i < kLocalVpt; ++i) {
        const int e = tid + i * kSelectThreads;
        hist_add(whist[wv], (key[i] >> shift) & 255u, e < n && (key[i] & mask) == prefix);
      }
      __syncthreads();
      // wave 0: lane l sums bins 4l .. 4l + 3 over the waves; the bucket d of
      // the rem-th largest key is the largest d whose suffix count S(d) =
      // sum of bins >= d reaches rem (S(0) >= rem, S(256) = 0 < rem, so
      // exactly one lane holds it)
      if (wv == 0) {
        unsigned c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          unsigned t = 0u;
#pragma unroll
          for (int w = 0; w < kSelectThreads / 64; ++w) t += whist[w][4 * lane + j];
          c[j] = t;
        }
        const unsigned mine = c[0] + c[1] + c[2] + c[3];
        unsigned suf = mine;                  // bins >= 4 lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned t = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += t;
        }
        unsigned above = suf - mine;          // S(4 lane + 4)
        if (suf >= rem && above < rem) {
          int j = 3;
          for (; j > 0; --j) {
            if (above + c[j] >= rem) break;
            above += c[j];
          }
          const int d = 4 * lane + j;
          s_word[0] = prefix | ((unsigned)d << shift);
          s_word[1] = rem - above;            // still to take from bucket d
          s_word[2] = c[j];                   // bucket d's size
        }
      }
      __syncthreads();
      prefix = s_word[0];
      rem = s_word[1];
      mask |= 255u << shift;
      if (s_word[2] == rem) {                 // bucket d is taken whole
        thresh = prefix;                      // every key >= prefix (its low bits are 0)
        need = 0u;
        ties = false;
        break;
      }
      if (shift == 0) {                       // prefix is the k-th key's score image
        thresh = prefix;
        need = rem;
        ties = true;
      }
      __syncthreads();
    }
  }
  // ---- gather: keys above the threshold, and (ties) the first `need` keys
  // equal to it by position (element order), with their 64-bit keys
  if (tid == 0) s_word[3] = 0u;
  __syncthreads();
  unsigned base = 0u;
#pragma unroll
  for (int i = 0; i < kLocalVpt; ++i) {
    const int e = tid + i * kSelectThreads;
    const bool valid = e < n;
    const bool above = valid && (ties ? key[i] > thresh : key[i] >= thresh);
    bool take = above;
    if (ties) {
      // rank of this tie among the ties of round i, in element order
      const bool tie = valid && key[i] == thresh;
      const unsigned long long bal = __ballot(tie);
      const unsigned before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_sum[wv] = __popcll(bal);
      __syncthreads();
      unsigned wbase = 0u, total = 0u;
      for (int w = 0; w < kSelectThreads / 64; ++w) {
        const unsigned c = wave_sum[w];
        if (w < wv) wbase += c;
        total += c;
      }
      take = above || (tie && base + wbase + before < need);
      base += total;
      __syncthreads();
    }
    if (take) {
      const unsigned at = atomicAdd(&s_word[3], 1u);
      if (at < m)
        sel[at] = ((unsigned long long)key[i] << 32) |
                  (unsigned)(0xffffffffu - (unsigned)(e * p.num_shards + shard));
    }
  }
  __syncthreads();
  int np2 = 1;
  while (np2 < (int)m) np2 <<= 1;
  for (int i = (int)m + tid; i < np2; i += kSelectThreads) sel[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < np2 / 2; i += kSelectThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const unsigned long long a = sel[lo], c = sel[hi];
        if ((a < c) == desc) {
          sel[lo] = c;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kSelectThreads) {
    float sc = kNegInf;
    int pos = -1;
    if (i < (int)m) {
      const unsigned long long kv = sel[i];
      sc = bits_score((unsigned)(kv >> 32));
      pos = (int)(0xffffffffu - (unsigned)(kv & 0xffffffffull));
    }
    p.out_score[list * k + i] = sc;
    p.out_pos[list * k + i] = pos;
  }
}

// Merge of sorted candidate lists by rank: the lists of a row (each in
// selection order, padding last) are staged in LDS as keys; an element's
// place in the merged order is its index in its own list plus, for every
// other list, the number of that list's keys above it (a binary search; keys
// are distinct).  Elements whose place is below k are written there.  Four
// blocks share a row: each stages all of the row's keys and places a fourth
// of them.
constexpr int kMergeThreads = 1024;
constexpr int kMergeMaxKeys = 8192;                 // num_shards * k staged in LDS
constexpr int kMergeParts = 4;                     // blocks per row, each placing a fourth of the elements
constexpr int kMergeRun = kMergeMaxKeys / (kMergeThreads * kMergeParts);   // consecutive elements per thread

__global__ __launch_bounds__(kMergeThreads) void topk_merge_rank_kernel(TopkParams p) {
  __shared__ unsigned long long keys[kMergeMaxKeys];
  __shared__ int s_valid;
  const int tid = threadIdx.x;
  const long long row = blockIdx.x / kMergeParts;
  const int part = (int)(blockIdx.x % kMergeParts);
  const int K = p.k_in, N = p.num_shards, k = p.k;
  if (tid == 0) s_valid = 0;
  __syncthreads();
  int valid = 0;
  for (int e = tid; e < N * K; e += kMergeThreads) {
    const int r = e / K, idx = e - r * K;
    const long long at = ((long long)r * p.rows + row) * K + idx;
    const int pos = p.in_pos[at];
    const unsigned long long kv = pos >= 0 ? make_key(p.in_score[at], pos) : 0ull;
    keys[e] = kv;
    valid += kv != 0ull;
  }
  atomicAdd(&s_valid, valid);
  __syncthreads();
  const int m = min(s_valid, k);
  // Each thread takes kMergeRun consecutive elements of one list (descending
  // keys): the first one's count in every other list by binary search, the
  // next ones by walking on from the previous count (counts only grow).
  const int e0 = (part * kMergeThreads + tid) * kMergeRun;
  int cnt[kMaxShards];
  for (int e = e0; e < min(e0 + kMergeRun, N * K); ++e) {
    const unsigned long long kv = keys[e];
    if (kv == 0ull) break;                          // padding: the rest of the run too
    const int r = e / K;
    int place = e - r * K;
    for (int o = 0; o < N; ++o) {
      if (o == r) continue;
      const unsigned long long* lst = keys + o * K;
      int c;
      if (e == e0 || (e % K) == 0) {
        int lo = 0, hi = K;
        while (lo < hi) {                           // first index whose key is below kv
          const int mid = (lo + hi) >> 1;
          if (lst[mid] > kv) lo = mid + 1;
          else hi = mid;
        }
        c = lo;
      } else {
        c = cnt[o];
        while (c < K && lst[c] > kv) ++c;
      }
      cnt[o] = c;
      place += c;
    }
    if (place < k) {
      const float sc = bits_score((unsigned)(kv >> 32));
      const int pos = (int)(0xffffffffu - (unsigned)(kv & 0xffffffffull));
      if (p.out_score) p.out_score[row * k + place] = sc;
      if (p.out_pos) p.out_pos[row * k + place] = pos;
      if (p.out_slot) {
        const long long span = (long long)p.page_size * p.num_shards;
        const long long lp = min((long long)pos / span, (long long)p.max_pages - 1);
        p.out_slot[row * k + place] = (int)((long long)p.block_table[row * p.max_pages + lp] * span + pos % span);
      }
    }
  }
  for (int i = m + part * kMergeThreads + tid; i < k; i += kMergeThreads * kMergeParts) {
    if (p.out_score) p.out_score[row * k + i] = kNegInf;
    if (p.out_pos) p.out_pos[row * k + i] = -1;
    if (p.out_slot) p.out_slot[row * k + i] = -1;
  }
}

}  // namespace

hipError_t launch_topk_merge(const TopkParams& p, long long rows, hipStream_t stream) {
  void* args[] = {(void*)&p};
  if ((long long)p.num_shards * p.k_in > kMergeMaxKeys)
    return hipLaunchKernel((const void*)topk_select_kernel, dim3((unsigned)rows), dim3(kSelectThreads),
                           args, 0, stream);
  return hipLaunchKernel((const void*)topk_merge_rank_kernel, dim3((unsigned)(rows * kMergeParts)), dim3(kMergeThreads),
                         args, 0, stream);
}

hipError_t launch_index_score(const IndexScoreParams& p, hipStream_t stream) {
  const long long blocks = p.rows * p.num_shards * (long long)p.tiles_per_list;
  void* args[] = {(void*)&p};
  const void* fn;
  switch (p.hi / 16) {
    case 1: fn = (const void*)index_score_kernel<1>; break;
    case 2: fn = (const void*)index_score_kernel<2>; break;
    case 3: fn = (const void*)index_score_kernel<3>; break;
    case 4: fn = (const void*)index_score_kernel<4>; break;
    case 5: fn = (const void*)index_score_kernel<5>; break;
    case 6: fn = (const void*)index_score_kernel<6>; break;
    case 7: fn = (const void*)index_score_kernel<7>; break;
    case 8: fn = (const void*)index_score_kernel<8>; break;
    default: return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kScoreThreads), args, 0, stream);
}

hipError_t launch_topk_select(const TopkParams& p, long long lists, hipStream_t stream) {
  void* args[] = {(void*)&p};
  const void* fn = (!p.merge && p.max_local <= kLocalFastMax) ? (const void*)topk_local_fast_kernel
                                                              : (const void*)topk_select_kernel;
  return hipLaunchKernel(fn, dim3((unsigned)lists), dim3(kSelectThreads), args, 0, stream);
}

int index_score_tokens_per_block() { return kScoreTokens; }

}  // namespace dcp
