// Host side of the C ABI: argument checks, split and workspace planning, and
// dispatch to the HIP kernels.  Every check runs before anything is queued, so
// a rejected call writes nothing.  No allocation, no synchronisation.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "dcp_internal.h"

namespace dcp {

namespace {

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool valid_heads(int heads) { return heads >= 16 && heads <= 128 && heads % 16 == 0; }

// Smallest split count that keeps every block's slot list within its LDS
// budget (sparse: slot ids; dense: pages).
long long min_splits_for_list(long long tokens_max, bool dense, int page_size) {
  long long cap = dense ? (long long)(kMaxList - 2) * page_size : (long long)(kMaxList - 64);
  if (tokens_max <= 0) return 1;
  return ceil_div(tokens_max, cap);
}

dcp_status resolve_splits(long long rows, int num_shards, int heads, long long tok_expected,
                          long long tok_max, bool dense, int page_size, int requested,
                          int* splits_out) {
  if (requested < 0) return DCP_ERR_INVALID_ARGUMENT;
  long long need = min_splits_for_list(tok_max, dense, page_size);
  long long s = requested > 0 ? requested
                              : std::max<long long>(need, default_splits(rows, num_shards, heads,
                                                                        tok_expected, tok_max));
  if (s < need) return DCP_ERR_UNSUPPORTED;
  if (s * num_shards > kMaxMergeInputs) return DCP_ERR_UNSUPPORTED;
  *splits_out = (int)s;
  return DCP_OK;
}

// Sparse: a shard holds about k / N of a row's k slots (at most k).
// Dense: a shard holds up to max_local_len tokens of a sequence.
dcp_status plan_splits(bool dense, long long rows, int num_shards, int heads,
                       long long tokens_per_shard, int page_size, int requested, int* splits_out) {
  long long expected = dense ? tokens_per_shard : ceil_div(tokens_per_shard, num_shards);
  return resolve_splits(rows, num_shards, heads, expected, tokens_per_shard, dense, page_size,
                        requested, splits_out);
}

}  // namespace

// Token splits per (row, shard): enough blocks to cover the chip once, at
// least one tile of tokens per split (128 from 48 heads on, the FP8
// kernel's tile; 64 for 16 or 32 heads, whose kernel uses 32- or 64-token
// tiles), at most 32K tokens per split.  Depends on the heads, not the KV
// dtype, so the workspace size query plans the same splits as the call.
int default_splits(long long rows, int num_shards, int heads, long long tok_expected,
                   long long tok_max) {
  (void)tok_max;
  const long long min_tok = heads <= 32 ? 64 : 128;
  long long units = std::max<long long>(1, rows * num_shards);
  long long s = ceil_div(kAssumedCUs, units);
  s = std::max(s, ceil_div(std::max<long long>(tok_expected, 1), 32768));
  s = std::min(s, std::max<long long>(1, ceil_div(std::max<long long>(tok_expected, 1), min_tok)));
  s = std::min<long long>(s, kMaxMergeInputs / num_shards);
  return (int)std::max<long long>(1, s);
}

WorkspacePlan plan_workspace(long long rows, int heads, int num_shards, int splits,
                             bool want_partials, bool want_merged) {
  WorkspacePlan w{};
  w.splits = splits;
  w.fused = want_merged;
  w.partials = want_partials;
  w.needs_block_partials = want_merged || (want_partials && splits > 1);
  size_t off = 0;
  w.cnt_row_off = off;
  const size_t hb = (size_t)(heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  if (want_merged) off += 4 * sizeof(int) * (size_t)rows * hb;      // per (row, head block)
  w.cnt_shard_off = off;
  if (want_partials && splits > 1) off += sizeof(int) * (size_t)rows * num_shards * hb;
  off = align256(off);
  w.ws_o_off = off;
  size_t blocks = (size_t)rows * num_shards * splits;
  if (w.needs_block_partials) off += sizeof(float) * blocks * heads * kVDim;
  off = align256(off);
  w.ws_lse_off = off;
  if (w.needs_block_partials) off += sizeof(float) * blocks * heads;
  off = align256(off);
  w.ws_exp_off = off;
  if (w.needs_block_partials) off += sizeof(int) * blocks * heads;
  w.total = (want_merged || (want_partials && splits > 1)) ? align256(off) : 0;
  return w;
}

namespace {

dcp_status check_shards(const dcp_kv_shard* shards, int num_shards, dcp_kv_dtype kv_dtype,
                        bool dense) {
  if (!shards) return DCP_ERR_INVALID_ARGUMENT;
  for (int r = 0; r < num_shards; ++r) {
    const dcp_kv_shard& s = shards[r];
    if (!s.kv || s.pool_rows < 1) return DCP_ERR_INVALID_ARGUMENT;
    if (kv_dtype == DCP_KV_FP8_E4M3 && !s.kv_scale) return DCP_ERR_INVALID_ARGUMENT;
    // every row is copied in 16-byte pieces, every scale in 4 bytes
    const long long row_bytes = kv_dtype == DCP_KV_FP8_E4M3 ? kHeadDim : 2 * kHeadDim;
    if (reinterpret_cast<uintptr_t>(s.kv) % 16 != 0) return DCP_ERR_INVALID_ARGUMENT;
    if (s.row_stride != 0 && (s.row_stride < row_bytes || s.row_stride % 16 != 0))
      return DCP_ERR_INVALID_ARGUMENT;
    if (kv_dtype == DCP_KV_FP8_E4M3) {
      if (reinterpret_cast<uintptr_t>(s.kv_scale) % 4 != 0) return DCP_ERR_INVALID_ARGUMENT;
      if (s.scale_stride < 0 || s.scale_stride % 4 != 0) return DCP_ERR_INVALID_ARGUMENT;
    }
    if (dense && !s.local_len) return DCP_ERR_INVALID_ARGUMENT;
  }
  return DCP_OK;
}

struct CommonArgs {
  const void* q;
  long long rows;
  int heads;
  const dcp_kv_shard* shards;
  int num_shards;
  dcp_kv_dtype kv_dtype;
  float softmax_scale;
  float* o_part;
  float* lse_part;
  void* o;
  float* lse;
  dcp_out_dtype out_dtype;
  int num_splits;
  void* workspace;
  size_t workspace_bytes;
};

dcp_status check_common(const CommonArgs& a, bool dense) {
  if (a.rows < 0 || a.num_shards < 1 || a.num_shards > kMaxShards) return DCP_ERR_INVALID_ARGUMENT;
  if (a.kv_dtype != DCP_KV_BF16 && a.kv_dtype != DCP_KV_FP8_E4M3) return DCP_ERR_INVALID_ARGUMENT;
  if (a.out_dtype != DCP_OUT_F32 && a.out_dtype != DCP_OUT_BF16) return DCP_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(a.softmax_scale) || !(a.softmax_scale > 0.f)) return DCP_ERR_INVALID_ARGUMENT;
  if (a.heads < 1 || a.num_splits < 0) return DCP_ERR_INVALID_ARGUMENT;
  if ((a.o_part == nullptr) != (a.lse_part == nullptr)) return DCP_ERR_INVALID_ARGUMENT;
  if ((a.o == nullptr) != (a.lse == nullptr)) return DCP_ERR_INVALID_ARGUMENT;
  if (!a.o_part && !a.o) return DCP_ERR_INVALID_ARGUMENT;
  if (a.rows == 0) return DCP_OK;
  if (!a.q) return DCP_ERR_INVALID_ARGUMENT;
  dcp_status st = check_shards(a.shards, a.num_shards, a.kv_dtype, dense);
  if (st != DCP_OK) return st;
  if (!valid_heads(a.heads)) return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

// Compute units of the current device (cached per device).
long long device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kAssumedCUs;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kAssumedCUs;
    cached[dev] = n;
  }
  return cached[dev];
}

// Bound of the wait for the other blocks of a row before merging, in
// microseconds (0 disables waiting, so the last block to arrive merges the
// whole row).  Starts from DCP_MERGE_WAIT_US, read from the environment once
// at the first decode call (default 30); dcp_set_merge_wait_us changes it.
constexpr int kMergeWaitUnset = -1;
std::atomic<int> g_merge_wait_us{kMergeWaitUnset};

int merge_wait_us_from_env() {
  const char* e = std::getenv("DCP_MERGE_WAIT_US");
  long v = 30;
  if (e && *e) {
    char* end = nullptr;
    const long x = std::strtol(e, &end, 10);
    if (end != e && x >= 0 && x <= kMaxMergeWaitUs) v = x;
  }
  return (int)v;
}

// The bound in 100 MHz ticks (the kernels' s_memrealtime clock).
int merge_wait_ticks() {
  int v = g_merge_wait_us.load(std::memory_order_relaxed);
  if (v == kMergeWaitUnset) {
    int expect = kMergeWaitUnset;
    g_merge_wait_us.compare_exchange_strong(expect, merge_wait_us_from_env(),
                                            std::memory_order_relaxed);
    v = g_merge_wait_us.load(std::memory_order_relaxed);
  }
  return v * 100;
}

// A shard as the kernels see it: strides resolved (0 = packed).
ShardArg shard_arg(const dcp_kv_shard& s, dcp_kv_dtype kv_dtype) {
  ShardArg a;
  a.kv = s.kv;
  a.scale = s.kv_scale;
  a.pool_rows = s.pool_rows;
  a.local_len = s.local_len;
  a.row_stride = s.row_stride != 0 ? s.row_stride
                                   : (kv_dtype == DCP_KV_FP8_E4M3 ? kHeadDim : 2 * kHeadDim);
  a.scale_stride = s.scale_stride != 0 ? s.scale_stride : 4;
  return a;
}

DecodeParams make_params(const CommonArgs& a, const WorkspacePlan& w) {
  DecodeParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a.q;
  for (int r = 0; r < a.num_shards; ++r) p.shard[r] = shard_arg(a.shards[r], a.kv_dtype);
  p.rows = a.rows;
  p.heads = a.heads;
  p.num_shards = a.num_shards;
  p.num_splits = w.splits;
  p.head_blocks = (a.heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  p.sm_scale_log2 = a.softmax_scale * 1.4426950408889634f;
  p.o_part = a.o_part;
  p.lse_part = a.lse_part;
  p.o = a.o;
  p.lse = a.lse;
  p.out_bf16 = a.out_dtype == DCP_OUT_BF16;
  char* ws = static_cast<char*>(a.workspace);
  if (w.total > 0) {
    p.cnt_row = reinterpret_cast<int*>(ws + w.cnt_row_off);
    p.cnt_shard = reinterpret_cast<int*>(ws + w.cnt_shard_off);
    p.ws_o = reinterpret_cast<float*>(ws + w.ws_o_off);
    p.ws_lse = reinterpret_cast<float*>(ws + w.ws_lse_off);
    p.ws_exp = reinterpret_cast<int*>(ws + w.ws_exp_off);
  }
  long long blocks = a.rows * a.num_shards * w.splits * p.head_blocks;
  p.xcd_swizzle = (blocks % 8 == 0) ? 1 : 0;
  // The blocks of a row may wait for each other to share its merge only
  // when the whole grid is resident at once (one block per compute unit).
  p.merge_wait_ticks = blocks <= device_cus() ? merge_wait_ticks() : 0;
  return p;
}

dcp_status launch_checked(const DecodeParams& p, bool fp8, bool dense, hipStream_t stream) {
  long long blocks = p.rows * p.num_shards * (long long)p.num_splits * p.head_blocks;
  if (blocks > 0x7fffffffLL) return DCP_ERR_UNSUPPORTED;
  return launch_decode(p, fp8, dense, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

// A prefill chunk's attention as dense decode launches: every query of
// every token attends the same chunk with no mask, so the tokens * heads
// (token, head) queries, contiguous in that order in q, o and lse, are
// regrouped into rows of 64 (64 queries per block read the chunk once); the
// last tokens * heads mod 64 of them (a multiple of 16) run as a second
// launch of one row with that many heads.
struct PrefillLaunch {
  long long rows;      // rows of this launch
  int heads;           // heads per row
  long long pair_off;  // first (token, head) query of this launch
};

int prefill_launches(long long tokens, int heads, PrefillLaunch out[2]) {
  int n = 0;
  const long long pairs = tokens * heads;
  const long long main_rows = pairs / 64;
  const int rem = (int)(pairs - main_rows * 64);
  if (main_rows > 0) out[n++] = PrefillLaunch{main_rows, 64, 0};
  if (rem > 0) out[n++] = PrefillLaunch{1, rem, main_rows * 64};
  return n;
}

size_t prefill_plan_bytes(long long tokens, int heads, long long chunk_len) {
  PrefillLaunch l[2];
  const int n = prefill_launches(tokens, heads, l);
  size_t need = 0;
  const int page = (int)std::max<long long>(chunk_len, 1);
  for (int i = 0; i < n; ++i) {
    int splits = 0;
    if (plan_splits(true, l[i].rows, 1, l[i].heads, chunk_len, page, 0, &splits) != DCP_OK)
      return std::numeric_limits<size_t>::max();
    need = std::max(need, plan_workspace(l[i].rows, l[i].heads, 1, splits, true, false).total);
  }
  return need;
}

// The sparse decode call, with the caller's workspace or (noalloc) the
// library's static scratch: counters at its start, partials after
// kNoallocCounterBytes.
dcp_status sparse_decode(const CommonArgs& a, const int32_t* topk_local, const int32_t* counts,
                         int32_t k, bool noalloc, hipStream_t stream) {
  dcp_status st = check_common(a, false);
  if (st != DCP_OK) return st;
  if (k < 0) return DCP_ERR_INVALID_ARGUMENT;
  if (a.rows == 0) return DCP_OK;
  if (!counts || (k > 0 && !topk_local)) return DCP_ERR_INVALID_ARGUMENT;
  int splits = 0;
  st = plan_splits(false, a.rows, a.num_shards, a.heads, k, 1, a.num_splits, &splits);
  if (st != DCP_OK) return st;
  WorkspacePlan w = plan_workspace(a.rows, a.heads, a.num_shards, splits, a.o_part != nullptr,
                                   a.o != nullptr);
  DecodeParams p;
  if (!noalloc) {
    if (w.total > 0 && (!a.workspace || a.workspace_bytes < w.total))
      return DCP_ERR_WORKSPACE_TOO_SMALL;
    p = make_params(a, w);
  } else {
    // counters occupy [0, ws_o_off) of the plan, partials [ws_o_off, total)
    const size_t parts = w.total > w.ws_o_off ? w.total - w.ws_o_off : 0;
    if (w.total > 0 && (w.ws_o_off > (size_t)kNoallocCounterBytes ||
                        parts > (size_t)(kNoallocScratchBytes - kNoallocCounterBytes)))
      return DCP_ERR_SCRATCH_TOO_SMALL;
    void* base = nullptr;
    if (w.total > 0 && noalloc_scratch(stream, &base) != hipSuccess) return DCP_ERR_LAUNCH;
    CommonArgs b = a;
    b.workspace = base;
    p = make_params(b, w);
    if (w.total > 0) {
      char* part_base = static_cast<char*>(base) + kNoallocCounterBytes;
      p.ws_o = reinterpret_cast<float*>(part_base);
      p.ws_lse = reinterpret_cast<float*>(part_base + (w.ws_lse_off - w.ws_o_off));
      p.ws_exp = reinterpret_cast<int*>(part_base + (w.ws_exp_off - w.ws_o_off));
    }
  }
  p.topk_local = topk_local;
  p.counts = counts;
  p.k = k;
  return launch_checked(p, a.kv_dtype == DCP_KV_FP8_E4M3, false, stream);
}

}  // namespace
}  // namespace dcp

using namespace dcp;

extern "C" {

const char* dcp_status_string(dcp_status status) {
  switch (status) {
    case DCP_OK: return "DCP_OK";
    case DCP_ERR_INVALID_ARGUMENT: return "DCP_ERR_INVALID_ARGUMENT";
    case DCP_ERR_UNSUPPORTED: return "DCP_ERR_UNSUPPORTED";
    case DCP_ERR_WORKSPACE_TOO_SMALL: return "DCP_ERR_WORKSPACE_TOO_SMALL";
    case DCP_ERR_LAUNCH: return "DCP_ERR_LAUNCH";
    case DCP_ERR_SCRATCH_TOO_SMALL: return "DCP_ERR_SCRATCH_TOO_SMALL";
  }
  return "DCP_ERR_UNKNOWN";
}

int32_t dcp_abi_version(void) { return DCP_ABI_VERSION; }

dcp_status dcp_set_merge_wait_us(int32_t us) {
  if (us < 0 || us > kMaxMergeWaitUs) return DCP_ERR_INVALID_ARGUMENT;
  g_merge_wait_us.store(us, std::memory_order_relaxed);
  return DCP_OK;
}

dcp_status dcp_remap_topk(const int32_t* topk_global, int64_t rows, int32_t k,
                          int32_t num_shards, int32_t shard, int32_t* topk_local,
                          int32_t* counts, hipStream_t stream) {
  if (rows < 0 || k < 0 || num_shards < 1 || num_shards > kMaxShards) return DCP_ERR_INVALID_ARGUMENT;
  if (shard >= num_shards) return DCP_ERR_INVALID_ARGUMENT;
  if (rows == 0) return DCP_OK;
  if (!counts || (k > 0 && (!topk_global || !topk_local))) return DCP_ERR_INVALID_ARGUMENT;
  if (rows > 0x7fffffffLL) return DCP_ERR_UNSUPPORTED;
  return launch_remap(topk_global, rows, k, num_shards, shard, topk_local, counts, stream) == hipSuccess
             ? DCP_OK : DCP_ERR_LAUNCH;
}

size_t dcp_decode_workspace_size(int32_t dense, int64_t rows, int32_t heads,
                                 int32_t num_shards, int64_t tokens_per_shard,
                                 int32_t page_size, int32_t num_splits,
                                 int32_t want_partials, int32_t want_merged) {
  const size_t bad = std::numeric_limits<size_t>::max();
  if (rows < 0 || !valid_heads(heads) || num_shards < 1 || num_shards > kMaxShards || tokens_per_shard < 0)
    return bad;
  if (dense && page_size < 1) return bad;
  if (!want_partials && !want_merged) return bad;
  if (rows == 0) return 0;
  int splits = 0;
  if (plan_splits(dense != 0, rows, num_shards, heads, tokens_per_shard, page_size, num_splits, &splits) != DCP_OK)
    return bad;
  return plan_workspace(rows, heads, num_shards, splits, want_partials != 0, want_merged != 0).total;
}

int32_t dcp_decode_splits(int32_t dense, int64_t rows, int32_t heads, int32_t num_shards,
                          int64_t tokens_per_shard, int32_t page_size, int32_t num_splits) {
  if (rows < 0 || !valid_heads(heads) || num_shards < 1 || num_shards > kMaxShards || tokens_per_shard < 0)
    return -1;
  if (dense && page_size < 1) return -1;
  int splits = 0;
  if (plan_splits(dense != 0, std::max<int64_t>(rows, 1), num_shards, heads, tokens_per_shard, page_size,
                  num_splits, &splits) != DCP_OK)
    return -1;
  return splits;
}

dcp_status mla_sparse_decode_lse(const void* q, int64_t rows, int32_t heads,
                                 const dcp_kv_shard* shards, int32_t num_shards,
                                 dcp_kv_dtype kv_dtype, const int32_t* topk_local,
                                 const int32_t* counts, int32_t k, float softmax_scale,
                                 float* o_part, float* lse_part, void* o, float* lse,
                                 dcp_out_dtype out_dtype, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  CommonArgs a{q, rows, heads, shards, num_shards, kv_dtype, softmax_scale, o_part, lse_part,
               o, lse, out_dtype, num_splits, workspace, workspace_bytes};
  return sparse_decode(a, topk_local, counts, k, false, stream);
}

dcp_status mla_sparse_decode_lse_noalloc(const void* q, int64_t rows, int32_t heads,
                                         const dcp_kv_shard* shards, int32_t num_shards,
                                         dcp_kv_dtype kv_dtype, const int32_t* topk_local,
                                         const int32_t* counts, int32_t k, float softmax_scale,
                                         float* o_part, float* lse_part, void* o, float* lse,
                                         dcp_out_dtype out_dtype, int32_t num_splits,
                                         hipStream_t stream) {
  CommonArgs a{q, rows, heads, shards, num_shards, kv_dtype, softmax_scale, o_part, lse_part,
               o, lse, out_dtype, num_splits, nullptr, 0};
  return sparse_decode(a, topk_local, counts, k, true, stream);
}

dcp_status mla_dense_decode_lse(const void* q, int64_t rows, int32_t heads,
                                const dcp_kv_shard* shards, int32_t num_shards,
                                dcp_kv_dtype kv_dtype, const int32_t* block_table,
                                int32_t max_pages, int32_t page_size,
                                int64_t max_local_len, float softmax_scale,
                                float* o_part, float* lse_part, void* o, float* lse,
                                dcp_out_dtype out_dtype, int32_t num_splits,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  CommonArgs a{q, rows, heads, shards, num_shards, kv_dtype, softmax_scale, o_part, lse_part,
               o, lse, out_dtype, num_splits, workspace, workspace_bytes};
  dcp_status st = check_common(a, true);
  if (st != DCP_OK) return st;
  if (max_pages < 1 || page_size < 1 || max_local_len < 0) return DCP_ERR_INVALID_ARGUMENT;
  if (max_local_len > (long long)max_pages * page_size) return DCP_ERR_INVALID_ARGUMENT;
  if (rows == 0) return DCP_OK;
  if (!block_table) return DCP_ERR_INVALID_ARGUMENT;
  int splits = 0;
  st = plan_splits(true, rows, num_shards, heads, max_local_len, page_size, num_splits, &splits);
  if (st != DCP_OK) return st;
  WorkspacePlan w = plan_workspace(rows, heads, num_shards, splits, o_part != nullptr, o != nullptr);
  if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return DCP_ERR_WORKSPACE_TOO_SMALL;
  DecodeParams p = make_params(a, w);
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_size = page_size;
  return launch_checked(p, kv_dtype == DCP_KV_FP8_E4M3, true, stream);
}

size_t dcp_prefill_workspace_size(int64_t tokens, int32_t heads, int64_t chunk_len) {
  if (tokens < 0 || chunk_len < 0 || chunk_len > 0x7fffffffLL || !valid_heads(heads))
    return std::numeric_limits<size_t>::max();
  if (tokens == 0) return 0;
  return prefill_plan_bytes(tokens, heads, chunk_len);
}

dcp_status mla_prefill_chunk_lse(const void* q, int64_t tokens, int32_t heads,
                                 const void* chunk_kv, const float* chunk_scale,
                                 int64_t chunk_len, dcp_kv_dtype kv_dtype, float softmax_scale,
                                 float* o, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (tokens < 0 || chunk_len < 0 || chunk_len > 0x7fffffffLL) return DCP_ERR_INVALID_ARGUMENT;
  if (kv_dtype != DCP_KV_BF16 && kv_dtype != DCP_KV_FP8_E4M3) return DCP_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DCP_ERR_INVALID_ARGUMENT;
  if (tokens == 0) return DCP_OK;
  if (!q || !o || !lse) return DCP_ERR_INVALID_ARGUMENT;
  if (chunk_len == 0) {
    // an empty chunk: the kernels read no KV row; the query stands in for the
    // pool so that no address they form is null (one query row holds 1152 bytes)
    if (!chunk_kv) chunk_kv = q;
    if (!chunk_scale) chunk_scale = static_cast<const float*>(q);
  }
  if (!chunk_kv || (kv_dtype == DCP_KV_FP8_E4M3 && !chunk_scale)) return DCP_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(chunk_kv) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(chunk_scale) % 4 != 0)
    return DCP_ERR_INVALID_ARGUMENT;
  if (!valid_heads(heads)) return DCP_ERR_UNSUPPORTED;
  const size_t need = prefill_plan_bytes(tokens, heads, chunk_len);
  if (need == std::numeric_limits<size_t>::max()) return DCP_ERR_UNSUPPORTED;
  if (need > 0 && (!workspace || workspace_bytes < need)) return DCP_ERR_WORKSPACE_TOO_SMALL;
  dcp_kv_shard chunk{chunk_kv, chunk_scale, std::max<int64_t>(chunk_len, 1), nullptr, 0, 0};
  PrefillLaunch l[2];
  const int n = prefill_launches(tokens, heads, l);
  for (int i = 0; i < n; ++i) {
    const long long off = l[i].pair_off;                   // first (token, head) query
    CommonArgs a{static_cast<const char*>(q) + off * kHeadDim * 2, l[i].rows, l[i].heads, &chunk, 1,
                 kv_dtype, softmax_scale, o + off * kVDim, lse + off, nullptr, nullptr, DCP_OUT_F32, 0,
                 workspace, workspace_bytes};
    int splits = 0;
    const int page = (int)std::max<int64_t>(chunk_len, 1);
    dcp_status st = plan_splits(true, a.rows, 1, a.heads, chunk_len, page, 0, &splits);
    if (st != DCP_OK) return st;
    WorkspacePlan w = plan_workspace(a.rows, a.heads, 1, splits, true, false);
    DecodeParams p = make_params(a, w);
    p.block_table = nullptr;
    p.max_pages = 1;
    p.page_size = page;
    p.chunk_mode = 1;
    p.chunk_len = (int)chunk_len;
    st = launch_checked(p, kv_dtype == DCP_KV_FP8_E4M3, true, stream);
    if (st != DCP_OK) return st;
  }
  return DCP_OK;
}

dcp_status lse_merge_into(void* o_acc, float* lse_acc, const float* o_new, const float* lse_new,
                          int64_t rows, int32_t heads, int32_t dv, dcp_out_dtype acc_dtype,
                          hipStream_t stream) {
  if (rows < 0 || heads < 1 || dv < 4 || dv % 4 != 0) return DCP_ERR_INVALID_ARGUMENT;
  if (acc_dtype != DCP_OUT_F32 && acc_dtype != DCP_OUT_BF16) return DCP_ERR_INVALID_ARGUMENT;
  if (rows == 0) return DCP_OK;
  if (!o_acc || !lse_acc || !o_new || !lse_new) return DCP_ERR_INVALID_ARGUMENT;
  const size_t ea = acc_dtype == DCP_OUT_BF16 ? 8 : 16;
  if (reinterpret_cast<uintptr_t>(o_acc) % ea != 0 || reinterpret_cast<uintptr_t>(o_new) % 16 != 0)
    return DCP_ERR_INVALID_ARGUMENT;
  if (rows * heads > 0x7fffffffLL * 4) return DCP_ERR_UNSUPPORTED;
  return launch_merge_into(o_acc, lse_acc, o_new, lse_new, rows, heads, dv,
                           acc_dtype == DCP_OUT_BF16, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

dcp_status dcp_gather_prefix(const int32_t* block_table, int32_t max_pages, int32_t page_size,
                             const dcp_kv_shard* shards, int32_t num_shards, dcp_kv_dtype kv_dtype,
                             const int32_t* pos_begin, const int32_t* out_offset, int32_t num_seqs,
                             int32_t max_len, void* out_kv, float* out_scale, hipStream_t stream) {
  if (num_seqs < 0 || max_len < 0 || num_shards < 1 || num_shards > kMaxShards)
    return DCP_ERR_INVALID_ARGUMENT;
  if (kv_dtype != DCP_KV_BF16 && kv_dtype != DCP_KV_FP8_E4M3) return DCP_ERR_INVALID_ARGUMENT;
  if (max_pages < 1 || page_size < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0 || max_len == 0) return DCP_OK;
  if (!block_table || !pos_begin || !out_offset || !out_kv) return DCP_ERR_INVALID_ARGUMENT;
  if (kv_dtype == DCP_KV_FP8_E4M3 && !out_scale) return DCP_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(out_kv) % 16 != 0) return DCP_ERR_INVALID_ARGUMENT;
  if (num_seqs > 65535) return DCP_ERR_UNSUPPORTED;
  dcp_status st = check_shards(shards, num_shards, kv_dtype, false);
  if (st != DCP_OK) return st;
  GatherParams p;
  std::memset(&p, 0, sizeof(p));
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_size = page_size;
  p.num_shards = num_shards;
  p.pos_begin = pos_begin;
  p.out_offset = out_offset;
  p.num_seqs = num_seqs;
  p.out_kv = out_kv;
  p.out_scale = out_scale;
  for (int r = 0; r < num_shards; ++r) p.shard[r] = shard_arg(shards[r], kv_dtype);
  return launch_gather_prefix(p, kv_dtype == DCP_KV_FP8_E4M3, max_len, stream) == hipSuccess
             ? DCP_OK : DCP_ERR_LAUNCH;
}

dcp_status dcp_index_score(const void* q, const float* w, int64_t rows, int32_t index_heads,
                           const dcp_index_shard* shards, int32_t num_shards,
                           const int32_t* block_table, int32_t max_pages, int32_t page_size,
                           int32_t max_local, float* scores, hipStream_t stream) {
  if (rows < 0 || num_shards < 1 || num_shards > kMaxShards || max_local < 0)
    return DCP_ERR_INVALID_ARGUMENT;
  if (index_heads < 16 || index_heads % 16 != 0) return DCP_ERR_INVALID_ARGUMENT;
  if (index_heads > kMaxIndexHeads) return DCP_ERR_UNSUPPORTED;
  if (max_pages < 1 || page_size < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (rows == 0 || max_local == 0) return DCP_OK;
  if (!q || !w || !block_table || !scores || !shards) return DCP_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return DCP_ERR_INVALID_ARGUMENT;
  IndexScoreParams p;
  std::memset(&p, 0, sizeof(p));
  for (int r = 0; r < num_shards; ++r) {
    const dcp_index_shard& s = shards[r];
    if (!s.keys || !s.key_scale || !s.local_len || s.pool_rows < 1) return DCP_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(s.keys) % 16 != 0 || reinterpret_cast<uintptr_t>(s.key_scale) % 4 != 0)
      return DCP_ERR_INVALID_ARGUMENT;
    if (s.row_stride != 0 && (s.row_stride < kIndexDim || s.row_stride % 16 != 0))
      return DCP_ERR_INVALID_ARGUMENT;
    if (s.scale_stride < 0 || s.scale_stride % 4 != 0) return DCP_ERR_INVALID_ARGUMENT;
    p.shard[r] = IndexShardArg{s.keys, s.key_scale, s.pool_rows, s.local_len,
                               s.row_stride != 0 ? s.row_stride : kIndexDim,
                               s.scale_stride != 0 ? s.scale_stride : 4};
  }
  p.q = static_cast<const unsigned char*>(q);
  p.w = w;
  p.rows = rows;
  p.hi = index_heads;
  p.num_shards = num_shards;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_size = page_size;
  p.max_local = max_local;
  p.tiles_per_list = (max_local + index_score_tokens_per_block() - 1) / index_score_tokens_per_block();
  p.scores = scores;
  if (rows * num_shards * (long long)p.tiles_per_list > 0x7fffffffLL) return DCP_ERR_UNSUPPORTED;
  return launch_index_score(p, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

dcp_status dcp_topk_local(const float* scores, int64_t rows, int32_t num_shards, int32_t max_local,
                          const int32_t* local_len, int32_t k, float* cand_score, int32_t* cand_pos,
                          hipStream_t stream) {
  if (rows < 0 || num_shards < 1 || num_shards > kMaxShards || max_local < 0)
    return DCP_ERR_INVALID_ARGUMENT;
  if (k < 1 || k > kMaxTopk) return DCP_ERR_INVALID_ARGUMENT;
  if (rows == 0) return DCP_OK;
  if (!local_len || !cand_score || !cand_pos || (max_local > 0 && !scores))
    return DCP_ERR_INVALID_ARGUMENT;
  if ((long long)max_local * num_shards > 0x7fffffffLL) return DCP_ERR_UNSUPPORTED;
  TopkParams p;
  std::memset(&p, 0, sizeof(p));
  p.merge = 0;
  p.rows = rows;
  p.num_shards = num_shards;
  p.k = k;
  p.in_score = scores;
  p.max_local = max_local;
  p.local_len = local_len;
  p.out_score = cand_score;
  p.out_pos = cand_pos;
  return launch_topk_select(p, rows * num_shards, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

dcp_status dcp_topk_merge(const float* cand_score, const int32_t* cand_pos, int64_t rows,
                          int32_t num_shards, int32_t k, const int32_t* block_table,
                          int32_t max_pages, int32_t page_size, float* top_score,
                          int32_t* top_pos, int32_t* topk_global, hipStream_t stream) {
  if (rows < 0 || num_shards < 1 || num_shards > kMaxShards) return DCP_ERR_INVALID_ARGUMENT;
  if (k < 1 || k > kMaxTopk || max_pages < 1 || page_size < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (((long long)num_shards * k) % 512 != 0) return DCP_ERR_UNSUPPORTED;
  if (rows == 0) return DCP_OK;
  if (!cand_score || !cand_pos || !block_table || !topk_global) return DCP_ERR_INVALID_ARGUMENT;
  TopkParams p;
  std::memset(&p, 0, sizeof(p));
  p.merge = 1;
  p.rows = rows;
  p.num_shards = num_shards;
  p.k = k;
  p.in_score = cand_score;
  p.in_pos = cand_pos;
  p.k_in = k;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_size = page_size;
  p.out_score = top_score;
  p.out_pos = top_pos;
  p.out_slot = topk_global;
  return launch_topk_merge(p, rows, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

dcp_status lse_combine(const float* o_part, const float* lse_part, int32_t num_shards,
                       int64_t rows, int32_t heads, int32_t dv, void* o, float* lse,
                       dcp_out_dtype out_dtype, hipStream_t stream) {
  if (num_shards < 1 || rows < 0 || heads < 1 || dv < 4 || dv % 4 != 0) return DCP_ERR_INVALID_ARGUMENT;
  if (out_dtype != DCP_OUT_F32 && out_dtype != DCP_OUT_BF16) return DCP_ERR_INVALID_ARGUMENT;
  if (rows == 0) return DCP_OK;
  if (!o_part || !lse_part || !o || !lse) return DCP_ERR_INVALID_ARGUMENT;
  if (rows * heads > 0x7fffffffLL * 4) return DCP_ERR_UNSUPPORTED;
  return launch_combine(o_part, lse_part, num_shards, rows, heads, dv, o, lse,
                        out_dtype == DCP_OUT_BF16, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

dcp_status dcp_kv_write(const void* kv_new, int64_t tokens, const int32_t* slots,
                        const dcp_kv_shard* shards, int32_t num_shards, dcp_kv_dtype kv_dtype,
                        hipStream_t stream) {
  if (tokens < 0 || num_shards < 1 || num_shards > kMaxShards) return DCP_ERR_INVALID_ARGUMENT;
  if (kv_dtype != DCP_KV_BF16 && kv_dtype != DCP_KV_FP8_E4M3) return DCP_ERR_INVALID_ARGUMENT;
  if (tokens == 0) return DCP_OK;
  if (!kv_new || !slots || reinterpret_cast<uintptr_t>(kv_new) % 16 != 0) return DCP_ERR_INVALID_ARGUMENT;
  dcp_status st = check_shards(shards, num_shards, kv_dtype, false);
  if (st != DCP_OK) return st;
  if (tokens > 0x7fffffffLL * 4) return DCP_ERR_UNSUPPORTED;
  KvWriteParams p;
  std::memset(&p, 0, sizeof(p));
  p.kv_new = kv_new;
  p.slots = slots;
  p.tokens = tokens;
  p.num_shards = num_shards;
  for (int r = 0; r < num_shards; ++r) p.shard[r] = shard_arg(shards[r], kv_dtype);
  return launch_kv_write(p, kv_dtype == DCP_KV_FP8_E4M3, stream) == hipSuccess ? DCP_OK : DCP_ERR_LAUNCH;
}

}  // extern "C"
