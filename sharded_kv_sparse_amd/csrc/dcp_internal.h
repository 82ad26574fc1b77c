// Internal declarations shared by the host API (dcp_api.cpp) and the kernel
// translation units.  Not part of the public ABI (include/dcp_mla.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "dcp_mla.h"

namespace dcp {

constexpr int kHeadDim = DCP_HEAD_DIM;   // 512 latent + 64 RoPE
constexpr int kVDim = DCP_V_DIM;         // values = first 512 dims of the key row
constexpr int kMaxShards = DCP_MAX_SHARDS;
constexpr int kHeadsPerBlock = 64;       // heads one decode block handles
constexpr int kMaxList = 4096;           // slot ids / pages a decode block stages in LDS
constexpr int kMaxMergeInputs = 64;      // partials one merge may combine (N * splits)
constexpr int kAssumedCUs = 256;         // MI355X compute units (split heuristic only)
constexpr int kMaxMergeWaitUs = 100000;  // upper bound of the merge wait setting
// Static scratch of mla_sparse_decode_lse_noalloc: counters first, partials after.
constexpr long long kNoallocScratchBytes = DCP_NOALLOC_SCRATCH_BYTES;
constexpr long long kNoallocCounterBytes = DCP_NOALLOC_COUNTER_BYTES;

struct ShardArg {
  const void* kv;
  const float* scale;
  long long pool_rows;
  const int* local_len;
  long long row_stride;          // bytes between pool rows (resolved, never 0)
  long long scale_stride;        // bytes between FP8 scales (resolved, never 0)
};

struct DecodeParams {
  const void* q;                 // bf16 [rows, heads, 576]
  ShardArg shard[kMaxShards];
  long long rows;
  int heads;                     // total gathered heads
  int num_shards;
  int num_splits;
  int head_blocks;               // heads / 64 rounded up (1 for heads <= 64)
  float sm_scale_log2;           // softmax_scale * log2(e)
  // sparse
  const int* topk_local;         // [N, rows, k]
  const int* counts;             // [N, rows]
  int k;
  // dense
  const int* block_table;        // [rows, max_pages]
  int max_pages;
  int page_size;
  // outputs
  float* o_part;                 // [N, rows, heads, 512] or null
  float* lse_part;               // [N, rows, heads] or null
  void* o;                       // [rows, heads, 512] fp32 / bf16, or null
  float* lse;                    // [rows, heads] or null
  int out_bf16;
  // workspace
  float* ws_o;                   // [rows, N, S, heads, 512]
  float* ws_lse;                 // [rows, N, S, heads]
  int* ws_exp;                   // [rows, N, S, heads]: power of two of an fp16 row-merge partial
  int* cnt_row;                  // [rows, head blocks, 4]: 64-bit arrival word (two words spare)
  int* cnt_shard;                // [rows, N, head blocks]
  int xcd_swizzle;               // grid is a multiple of 8: keep a row's blocks on one XCD
  int merge_wait_ticks;          // >0: blocks wait up to this many 100 MHz ticks to share a merge
  // dense, prefill chunk: every row attends tokens 0 .. chunk_len - 1 of one
  // contiguous pool (no block table, no local_len; page_size >= chunk_len)
  int chunk_mode;
  int chunk_len;
};

// Index cache of one shard (the DSA indexer's keys): 128 E4M3FN codes per
// token at a row stride, one fp32 scale per token at a scale stride.
constexpr int kIndexDim = DCP_INDEX_DIM;
constexpr int kMaxIndexHeads = 128;
constexpr int kMaxTopk = 4096;
struct IndexShardArg {
  const void* keys;
  const float* scale;
  long long pool_rows;
  const int* local_len;          // [rows]
  long long row_stride;          // bytes (resolved, never 0)
  long long scale_stride;        // bytes (resolved, never 0)
};

struct IndexScoreParams {
  const unsigned char* q;        // [rows, hi, 128] E4M3FN
  const float* w;                // [rows, hi]
  long long rows;
  int hi;                        // index heads, a multiple of 16
  int num_shards;
  const int* block_table;        // [rows, max_pages]
  int max_pages;
  int page_size;
  int max_local;                 // row length of scores
  int tiles_per_list;
  float* scores;                 // [N, rows, max_local]
  IndexShardArg shard[kMaxShards];
};

// Top-k selection over lists of (score, position): local (a shard's scores,
// position = j * N + shard) or merge (the shards' candidates of a row).
struct TopkParams {
  int merge;
  long long rows;
  int num_shards;
  int k;                         // output width
  // local
  const float* in_score;         // local: [N, rows, max_local]; merge: [N, rows, k_in]
  int max_local;
  const int* local_len;          // [N, rows]
  // merge
  const int* in_pos;             // [N, rows, k_in]
  int k_in;
  const int* block_table;        // [rows, max_pages] (merge: positions -> slots)
  int max_pages;
  int page_size;
  // outputs [lists, k]
  float* out_score;
  int* out_pos;
  int* out_slot;                 // merge only, may be null
};

// Arguments of the prefix gather kernel.
struct GatherParams {
  const int* block_table;        // [num_seqs, max_pages] DCP-wide logical pages
  int max_pages;
  int page_size;
  int num_shards;
  const int* pos_begin;          // [num_seqs] first position of each sequence's chunk
  const int* out_offset;         // [num_seqs + 1] chunk rows of sequence b: out_offset[b] ..
  int num_seqs;
  void* out_kv;                  // [total, 576] codes or bf16
  float* out_scale;              // [total] (FP8)
  ShardArg shard[kMaxShards];
};

// Arguments of the KV-cache write kernel.
struct KvWriteParams {
  const void* kv_new;            // bf16 [tokens, 576]
  const int* slots;              // [tokens] global slot ids, < 0: skipped
  long long tokens;
  int num_shards;
  ShardArg shard[kMaxShards];
};

// Workspace plan shared by the size query and the decode calls.
struct WorkspacePlan {
  int splits;
  bool fused;
  bool partials;
  bool needs_block_partials;     // blocks write split partials to the workspace
  size_t cnt_row_off, cnt_shard_off, ws_o_off, ws_lse_off, ws_exp_off, total;
};

int default_splits(long long rows, int num_shards, int heads, long long tokens_per_shard_expected,
                   long long tokens_per_shard_max);
WorkspacePlan plan_workspace(long long rows, int heads, int num_shards, int splits,
                             bool want_partials, bool want_merged);

// Kernel launchers (return the hipError_t of the launch).
hipError_t launch_remap(const int* topk_global, long long rows, int k, int num_shards,
                        int shard, int* topk_local, int* counts, hipStream_t stream);
hipError_t launch_combine(const float* o_part, const float* lse_part, int num_shards,
                          long long rows, int heads, int dv, void* o, float* lse,
                          int out_bf16, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, bool fp8, bool dense, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeParams& p, bool dense, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteParams& p, bool fp8, hipStream_t stream);

hipError_t launch_index_score(const IndexScoreParams& p, hipStream_t stream);
hipError_t launch_topk_select(const TopkParams& p, long long lists, hipStream_t stream);
hipError_t launch_topk_merge(const TopkParams& p, long long rows, hipStream_t stream);
int index_score_tokens_per_block();
hipError_t launch_gather_prefix(const GatherParams& p, bool fp8, int max_len, hipStream_t stream);
hipError_t launch_merge_into(void* o_acc, float* lse_acc, const float* o_new, const float* lse_new,
                             long long rows, int heads, int dv, int acc_bf16, hipStream_t stream);

// Device address of this device's static scratch (looked up, and its counter
// area cleared on `stream`, at the first call on each device).
hipError_t noalloc_scratch(hipStream_t stream, void** out);

}  // namespace dcp
