/*
 * dcp_mla.h -- C ABI of libdcpmla.so: the decode hot path of decode context
 * parallelism (DCP) for MLA / DSA models, as hand-written HIP for gfx950.
 *
 * Pages cited (the text of three public pull-request pages):
 *   [P1] "feat: support decode context parallelism for PyTorch MLA"
 *        (LMDeploy pull request 4952)
 *   [P2] "Feat[DCP] Support decode context parallelism for DSA models with
 *        the flashmla_kv backend" (SGLang pull request 36990)
 *   [P3] "[DSA] Fix decode context parallelism for RoPE sparse attention on
 *        Blackwell" (SGLang pull request 42536)
 *
 * The method.  The KV cache of every sequence is split token by token over N
 * shards with interleave 1: position t lives on shard t mod N ([P1] Server
 * and client commands, the vLLM run with interleave 1 and block size 64).
 * Each shard runs the query heads of the whole DCP group over its own tokens
 * only, returns the output together with its log-sum-exp, and the partials
 * are merged with LSE weights ([P1] Summary; [P3] Motivation and
 * Modifications, Backend).  Here the N shards are N cache slices on one GPU.
 *
 * Conventions for every entry point.
 *   - All sizes are element counts; all arrays are row-major and contiguous.
 *   - Pointers marked "device" are GPU memory; "host" pointers are read
 *     during the call only.  The caller owns every buffer; the library never
 *     allocates, frees or synchronises, so the calls may be captured in a
 *     HIP graph.  Work is queued on `stream` and completes asynchronously.
 *   - Outputs must not alias inputs.
 *   - Argument checks run on the host before anything is queued.  On any
 *     error nothing is launched and nothing is written; the status says why.
 *     A failed launch is reported as DCP_ERR_LAUNCH.
 *   - Not checked (undefined if violated): device pointers really point to
 *     buffers of the stated sizes; table entries are -1 or a valid slot;
 *     the valid entries of a top-k row are distinct.
 *   - Key rows have DCP_HEAD_DIM = 576 values (512 latent + 64 RoPE); the
 *     value of a token is the first DCP_V_DIM = 512 values of its key row
 *     (absorbed-weight MLA).
 */
#ifndef DCP_MLA_H
#define DCP_MLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCP_ABI_VERSION 4
#define DCP_HEAD_DIM 576
#define DCP_V_DIM 512
#define DCP_MAX_SHARDS 16
#define DCP_INDEX_DIM 128
#define DCP_MAX_TOPK 4096
/* Static device scratch of mla_sparse_decode_lse_noalloc, per GPU: the
 * first DCP_NOALLOC_COUNTER_BYTES hold merge counters, the rest partials. */
#define DCP_NOALLOC_SCRATCH_BYTES (64LL << 20)
#define DCP_NOALLOC_COUNTER_BYTES (64LL << 10)

typedef enum dcp_status {
  DCP_OK = 0,
  DCP_ERR_INVALID_ARGUMENT = 1,  /* null pointer, non-positive size, bad index   */
  DCP_ERR_UNSUPPORTED = 2,       /* valid but not implemented (e.g. heads = 40)  */
  DCP_ERR_WORKSPACE_TOO_SMALL = 3,
  DCP_ERR_LAUNCH = 4,            /* the HIP runtime rejected a kernel launch     */
  DCP_ERR_SCRATCH_TOO_SMALL = 5  /* a no-allocation call needs more than the
                                    library's static scratch                    */
} dcp_status;

typedef enum dcp_kv_dtype {
  DCP_KV_BF16 = 0,       /* bfloat16 rows, 1152 bytes per token                     */
  DCP_KV_FP8_E4M3 = 1    /* OCP E4M3FN codes, 576 bytes per token, value =
                            code * scale with one fp32 scale per token            */
} dcp_kv_dtype;

typedef enum dcp_out_dtype {
  DCP_OUT_F32 = 0,       /* merged output stored as float32                      */
  DCP_OUT_BF16 = 1       /* merged in fp32, stored as bfloat16 ([P1] review of
                            the prefix merge: fp32 arithmetic, BF16 storage)      */
} dcp_out_dtype;

/*
 * One shard's paged latent KV cache (device pointers).  Pool row r (576
 * bf16 values, or 576 E4M3FN codes) starts at (char*)kv + r * row_stride;
 * the fp32 scale of an FP8 row r sits at (char*)kv_scale + r * scale_stride.
 * The scale may live inside the row's own padding: with row_stride = 640
 * and kv_scale = (char*)kv + 576, scale_stride = 640, a 128-byte-aligned
 * row spans exactly five 128-byte lines, scale included, where separate
 * 576-byte rows and a scale array touch six (five for the row, one for the
 * scale).  Requirements (else DCP_ERR_INVALID_ARGUMENT): kv 16-byte aligned;
 * row_stride 0 (packed: 576 FP8 / 1152 BF16) or a multiple of 16 no smaller
 * than the row; kv_scale 4-byte aligned; scale_stride 0 (packed fp32 array)
 * or a positive multiple of 4.
 */
typedef struct dcp_kv_shard {
  const void* kv;           /* pool rows, bf16 or uint8 E4M3FN codes               */
  const float* kv_scale;    /* per-token fp32 scales (FP8); NULL for BF16          */
  int64_t pool_rows;        /* rows in this shard's pool = physical pages * page  */
  const int32_t* local_len; /* dense only: [num_seqs] tokens of each sequence held
                               by this shard (0 = none); NULL for sparse          */
  int64_t row_stride;       /* bytes from one pool row to the next (0 = packed)   */
  int64_t scale_stride;     /* bytes from one scale to the next (0 = 4)           */
} dcp_kv_shard;

/* Human-readable name of a status code (static storage). */
const char* dcp_status_string(dcp_status status);

/* DCP_ABI_VERSION of the built library. */
int32_t dcp_abi_version(void);

/*
 * Process-wide bound, in microseconds (0..100000), of how long the blocks of
 * a row wait for each other to share the fused merge of the decode calls (see
 * dcp_decode_workspace_size).  Takes effect for calls queued after it; the
 * results are bit-identical for every value.  DCP_ERR_INVALID_ARGUMENT out of
 * range.
 */
dcp_status dcp_set_merge_wait_us(int32_t us);

/*
 * Step 1 -- index remap ([P3] Modifications, Index remap; remapped tables are
 * reused by the layers that share a top-k, [P3] Modifications, Decode latency).
 *
 * For every row i and shard r: keep the entries g >= 0 of topk_global[i] with
 * g mod N == r, in their original order, write g div N to the front of
 * topk_local[r][i], fill the rest of that row with -1 and write the number
 * kept to counts[r][i].  A slot id g names row g div N of shard g mod N's pool
 * (the DCP-wide logical page holds page * N tokens; [P1] review note that the
 * scheduling unit becomes block_size * dcp).  Negative entries are padding.
 *
 *   topk_global  device int32 [rows, k]
 *   num_shards   N, 1 <= N <= DCP_MAX_SHARDS
 *   shard        < 0: all shards, outputs [N, rows, k] and [N, rows];
 *                0 <= shard < N: that shard only, outputs [1, rows, k], [1, rows]
 *   topk_local   device int32 output
 *   counts       device int32 output
 * Bit-exact and deterministic.
 */
dcp_status dcp_remap_topk(const int32_t* topk_global, int64_t rows, int32_t k,
                          int32_t num_shards, int32_t shard, int32_t* topk_local,
                          int32_t* counts, hipStream_t stream);

/*
 * Workspace for the decode entry points.  Pass the same arguments as the
 * decode call: dense = 0 for mla_sparse_decode_lse (tokens_per_shard = k,
 * page_size ignored) and dense = 1 for mla_dense_decode_lse
 * (tokens_per_shard = max_local_len); num_splits as passed to that call
 * (0 = library default); want_partials / want_merged = whether
 * (o_part, lse_part) / (o, lse) will be given.  Returns 0 when the call needs
 * no workspace, and SIZE_MAX for arguments the decode call would reject.
 * The first bytes hold the merge's arrival counters: zero the workspace once
 * after allocating it; every call leaves them ready for the next call (counts
 * and flags cleared, a generation byte advanced).
 * Calls that share one workspace must be ordered on one stream.
 *
 * Merge scheduling.  When the whole grid of a call fits on the device at
 * once, the blocks of a row wait for each other (for at most the merge wait
 * set by dcp_set_merge_wait_us, else DCP_MERGE_WAIT_US microseconds read from
 * the environment once, at the first decode call; default 30, 0 = never
 * wait) so that each merges a share of the row; a block that stops waiting
 * hands its share to the block that arrives last.  The result is
 * bit-identical either way.
 */
size_t dcp_decode_workspace_size(int32_t dense, int64_t rows, int32_t heads,
                                 int32_t num_shards, int64_t tokens_per_shard,
                                 int32_t page_size, int32_t num_splits,
                                 int32_t want_partials, int32_t want_merged);

/*
 * The token splits per (row, shard) that a decode call with these arguments
 * uses (same arguments as dcp_decode_workspace_size, without the outputs):
 * num_splits itself when it is > 0 and allowed, else the library's default
 * for the shape.  Returns -1 for arguments the decode call would reject.
 * Split s of a row's n local tokens covers [s * c, min(n, (s + 1) * c)) with
 * c = ceil(ceil(n / splits) / T) * T, T the kernel's tile: 128 tokens for FP8
 * KV with 48 heads or more, 64 otherwise.  Informational: a caller never
 * needs it to run a decode.
 */
int32_t dcp_decode_splits(int32_t dense, int64_t rows, int32_t heads, int32_t num_shards,
                          int64_t tokens_per_shard, int32_t page_size, int32_t num_splits);

/*
 * Step 2 (+ step 3 fused) -- sparse absorbed-MLA decode with LSE over the
 * shards' compacted local slots ([P3] Modifications, Backend: attention with
 * return_lse, rows without local KV fixed up, partials merged; [P3] Follow-ups,
 * item 1: pack and combine fused into the attention).
 *
 * For every row i, head h and shard r with J = topk_local[r][i][0:counts[r][i]]:
 *   z_j   = softmax_scale * sum_d q[i][h][d] * K_r[j][d]    (d < 576)
 *   O_r   = sum_j e^{z_j} V_r[j] / sum_j e^{z_j}             (V = K[:, :512])
 *   LSE_r = ln sum_j e^{z_j};   J empty -> O_r = 0, LSE_r = -inf.
 * K_r[j] is pool row j of shard r (FP8: code * kv_scale[j]).
 * Merge over shards ([P1] Summary; [P3] Fixes in shared code; [P2] review of
 * the LSE combine): M = max_r LSE_r over shards with LSE_r > -inf,
 *   O = sum_r e^{LSE_r - M} O_r / sum_r e^{LSE_r - M},  LSE = M + ln sum(...),
 *   and O = 0, LSE = -inf when every shard is empty.
 *
 *   q            device bf16 [rows, heads, 576]; heads a multiple of 16 from
 *                16 to 128, else DCP_ERR_UNSUPPORTED (the gathered heads of a
 *                DCP group, [P3] Motivation)
 *   shards       host array [num_shards] of device pool descriptors
 *   topk_local   device int32 [num_shards, rows, k]   (dcp_remap_topk output)
 *   counts       device int32 [num_shards, rows]
 *   o_part, lse_part  optional device fp32 [num_shards, rows, heads, 512] and
 *                [num_shards, rows, heads]: the per-shard partials
 *   o, lse       optional device [rows, heads, 512] (fp32 or bf16 per out_dtype)
 *                and fp32 [rows, heads]: the merged result
 *   At least one of the pairs (o_part, lse_part) / (o, lse) must be given,
 *   each pair complete.
 *   softmax_scale  finite and > 0 (else DCP_ERR_INVALID_ARGUMENT)
 *   num_splits   token splits per (row, shard); 0 = library default
 *   workspace    device, >= dcp_decode_workspace_size(...) bytes (may be NULL
 *                when that size is 0)
 */
dcp_status mla_sparse_decode_lse(const void* q, int64_t rows, int32_t heads,
                                 const dcp_kv_shard* shards, int32_t num_shards,
                                 dcp_kv_dtype kv_dtype, const int32_t* topk_local,
                                 const int32_t* counts, int32_t k, float softmax_scale,
                                 float* o_part, float* lse_part, void* o, float* lse,
                                 dcp_out_dtype out_dtype, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * mla_sparse_decode_lse without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and results
 * as mla_sparse_decode_lse (the same kernels run); the partials and counters
 * of the fused merge live in a static device array of the library,
 * DCP_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the first call until
 * the process ends.  This call allocates and frees nothing.
 *   - A call whose merge needs more than the scratch (more than
 *     DCP_NOALLOC_COUNTER_BYTES of counters, or more than the rest for
 *     partials; e.g. 64 rows x 64 heads x 4 shards needs about 34 MB, 128 such
 *     rows too much) returns DCP_ERR_SCRATCH_TOO_SMALL before queuing anything.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's partials.  The counters start at zero and every call leaves them
 *     ready for the next (counts and flags cleared); calls that overlap on one GPU (other streams, other threads, an
 *     unordered graph) race and give wrong results: order them.
 *   - The first call on a device looks up the scratch's device address and
 *     queues a small kernel on `stream` that clears the counters.
 */
dcp_status mla_sparse_decode_lse_noalloc(const void* q, int64_t rows, int32_t heads,
                                         const dcp_kv_shard* shards, int32_t num_shards,
                                         dcp_kv_dtype kv_dtype, const int32_t* topk_local,
                                         const int32_t* counts, int32_t k, float softmax_scale,
                                         float* o_part, float* lse_part, void* o, float* lse,
                                         dcp_out_dtype out_dtype, int32_t num_splits,
                                         hipStream_t stream);

/*
 * Step 2 (+ step 3 fused) -- dense absorbed-MLA decode with LSE over every
 * local token of each sequence ([P1] Summary, dense FlashMLA decode with DCP).
 * One query row per sequence.  Local token j < local_len[b] of shard r is
 * pool row block_table[b][j / page_size] * page_size + j % page_size: the
 * block table holds DCP-wide logical pages and each shard stores page_size
 * tokens of every page ([P1] review note on block_size * dcp).  Otherwise as
 * mla_sparse_decode_lse; a shard with local_len[b] == 0 contributes nothing.
 *
 *   block_table  device int32 [rows, max_pages]
 *   max_local_len  upper bound of every shards[r].local_len[b]; sizes splits
 */
dcp_status mla_dense_decode_lse(const void* q, int64_t rows, int32_t heads,
                                const dcp_kv_shard* shards, int32_t num_shards,
                                dcp_kv_dtype kv_dtype, const int32_t* block_table,
                                int32_t max_pages, int32_t page_size,
                                int64_t max_local_len, float softmax_scale,
                                float* o_part, float* lse_part, void* o, float* lse,
                                dcp_out_dtype out_dtype, int32_t num_splits,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Step 3 standalone -- LSE-weighted merge of partials ([P1] Summary; [P3]
 * Fixes in shared code: zero when every shard is empty; [P2] review of the
 * LSE combine: safe denominator, -inf global LSE).  Shards whose LSE is -inf
 * are skipped, never multiplied by zero, so NaN garbage in their O is ignored.
 *
 *   o_part   device fp32 [num_shards, rows, heads, dv]
 *   lse_part device fp32 [num_shards, rows, heads]
 *   o        device [rows, heads, dv], fp32 or bf16 per out_dtype
 *   lse      device fp32 [rows, heads]
 *   dv       value width, a positive multiple of 4 (512 for MLA)
 */
dcp_status lse_combine(const float* o_part, const float* lse_part, int32_t num_shards,
                       int64_t rows, int32_t heads, int32_t dv, void* o, float* lse,
                       dcp_out_dtype out_dtype, hipStream_t stream);

/*
 * Sharded index cache and distributed top-k ([P3] "[DSA] Fix decode context
 * parallelism for RoPE sparse attention on Blackwell", Follow-ups, item 2:
 * the index keys -- 128 FP8 values and one fp32 scale per token -- split
 * across the ranks like the KV, every rank scoring its own tokens, the local
 * top-k candidates merged into the global top-k; [P1] "feat: support decode
 * context parallelism for PyTorch MLA", Summary, decode bullet, and File
 * summaries: distributed candidate packing and merging).
 *
 * One shard's index cache: token row r holds DCP_INDEX_DIM E4M3FN codes at
 * (char*)keys + r * row_stride (0 = packed 128 bytes), its fp32 scale (> 0)
 * at (char*)key_scale + r * scale_stride (0 = packed).  The rows follow the
 * KV cache's paging: local token j of a sequence is row block_table[b][j /
 * page_size] * page_size + j % page_size.  keys 16-byte aligned, row_stride
 * a multiple of 16 >= 128, key_scale 4-byte aligned, scale_stride a multiple
 * of 4.  local_len: device int32 [rows], the sequence's tokens on this shard.
 */
typedef struct dcp_index_shard {
  const void* keys;
  const float* key_scale;
  int64_t pool_rows;
  const int32_t* local_len;
  int64_t row_stride;
  int64_t scale_stride;
} dcp_index_shard;

/*
 * Index scores of every local token of every (row, shard).  The pages give
 * no score; the one computed (the DSA indexer form), for query row i with
 * index heads h (E4M3FN codes q[i][h][0:128], fp32 weight w[i][h]):
 *   score(j) = key_scale[j] * sum_h w[i][h] * max(0, q[i][h] . keys[j])
 * in fp32 (the dot products on the fp8 MFMA: every product exact, the sums
 * fp32; then the weighted sum over heads and the scale).
 *   q        device uint8 [rows, index_heads, 128]; index_heads a multiple of
 *            16, at most 128
 *   w        device fp32 [rows, index_heads]
 *   shards   host array of num_shards index caches (local_len required)
 *   block_table  device int32 [rows, max_pages] (one query row per sequence)
 *   scores   device fp32 [num_shards, rows, max_local]; entries j <
 *            min(local_len, max_local) are written, the rest are left alone
 */
dcp_status dcp_index_score(const void* q, const float* w, int64_t rows, int32_t index_heads,
                           const dcp_index_shard* shards, int32_t num_shards,
                           const int32_t* block_table, int32_t max_pages, int32_t page_size,
                           int32_t max_local, float* scores, hipStream_t stream);

/*
 * Local top-k of every (row, shard): the first k of the shard's local tokens
 * j < min(local_len[r][i], max_local) in the order score descending, then
 * position ascending, where local token j of shard r is position j * N + r
 * of its sequence (interleave 1).  Output in that order, padded with
 * (-inf, -1) when a shard holds fewer than k tokens.
 *   scores     device fp32 [num_shards, rows, max_local] (dcp_index_score)
 *   local_len  device int32 [num_shards, rows]
 *   cand_score, cand_pos  device fp32 / int32 [num_shards, rows, k]
 *   1 <= k <= DCP_MAX_TOPK.
 */
dcp_status dcp_topk_local(const float* scores, int64_t rows, int32_t num_shards, int32_t max_local,
                          const int32_t* local_len, int32_t k, float* cand_score, int32_t* cand_pos,
                          hipStream_t stream);

/*
 * Merge of the shards' candidates into the global top-k of every row: the
 * first k of the num_shards * k candidates (positions < 0 are padding) in the
 * same order, with their slots (slot of position t: block_table[i][t div
 * (page*N)] * page*N + t mod (page*N), the slot naming of dcp_remap_topk),
 * padded with (-inf, -1, -1).  The pages' merge kernel needs num_shards * k
 * to be a multiple of 512 ([P1] review note); the same is required here
 * (else DCP_ERR_UNSUPPORTED).
 *   cand_score, cand_pos  device [num_shards, rows, k], each shard's list in
 *                selection order with its padding last (as dcp_topk_local
 *                writes them; the merge relies on that order)
 *   top_score, top_pos  device fp32 / int32 [rows, k] (each may be NULL)
 *   topk_global  device int32 [rows, k]: slots, the input of dcp_remap_topk
 */
dcp_status dcp_topk_merge(const float* cand_score, const int32_t* cand_pos, int64_t rows,
                          int32_t num_shards, int32_t k, const int32_t* block_table,
                          int32_t max_pages, int32_t page_size, float* top_score,
                          int32_t* top_pos, int32_t* topk_global, hipStream_t stream);

/*
 * Prefill over a cached prefix, step 1 -- gather ([P1] "feat: support decode
 * context parallelism for PyTorch MLA", Summary, prefill bullet: the
 * cached-prefix KV is gathered in bounded chunks; [P2] "Feat[DCP] Support
 * decode context parallelism for DSA models with the flashmla_kv backend",
 * summary: with an FP8 cache the gathered buffer keeps the packed FP8 rows,
 * nothing is dequantised).
 *
 * For every sequence b < num_seqs and j < out_offset[b+1] - out_offset[b]:
 * position t = pos_begin[b] + j, slot g = block_table[b][t div (page*N)] *
 * page*N + t mod (page*N) (the DCP-wide logical page holds page*N positions),
 * and row g div N of shard g mod N is copied unchanged to chunk row
 * out_offset[b] + j (its fp32 scale to out_scale[out_offset[b] + j] for FP8).
 *   block_table  device int32 [num_seqs, max_pages]
 *   shards       host array of num_shards pools (local_len ignored)
 *   pos_begin    device int32 [num_seqs]; out_offset device int32 [num_seqs + 1],
 *                non-decreasing, out_offset[0] = 0
 *   max_len      host bound of every out_offset[b+1] - out_offset[b] (sizes the grid)
 *   out_kv       device [out_offset[num_seqs], 576] E4M3FN codes or bf16, 16-byte aligned
 *   out_scale    device fp32 [out_offset[num_seqs]] (FP8; may be NULL for BF16)
 * Positions past the block table or rows past a pool are clamped into range
 * (unspecified data, nothing read out of bounds).  num_seqs <= 65535.
 */
dcp_status dcp_gather_prefix(const int32_t* block_table, int32_t max_pages, int32_t page_size,
                             const dcp_kv_shard* shards, int32_t num_shards, dcp_kv_dtype kv_dtype,
                             const int32_t* pos_begin, const int32_t* out_offset, int32_t num_seqs,
                             int32_t max_len, void* out_kv, float* out_scale, hipStream_t stream);

/* Workspace bytes of mla_prefill_chunk_lse (0 = none; SIZE_MAX for arguments
 * it would reject).  Zero it once after allocating; calls leave it ready for
 * the next call. */
size_t dcp_prefill_workspace_size(int64_t tokens, int32_t heads, int64_t chunk_len);

/*
 * Prefill, step 2 -- attention of the new tokens to one gathered chunk, with
 * LSE ([P1] Summary, prefill bullet).  The cached prefix precedes every new
 * token, so each query row attends every chunk token:
 *   z_j = softmax_scale * q[t][h] . K[j],  O[t][h] = sum_j e^{z_j} V[j] / sum_j e^{z_j},
 *   lse[t][h] = ln sum_j e^{z_j};  chunk_len == 0 gives O = 0, lse = -inf.
 *   q          device bf16 [tokens, heads, 576]; heads a multiple of 16 from 16
 *              to 128, else DCP_ERR_UNSUPPORTED
 *   chunk_kv   device [chunk_len, 576] E4M3FN codes (value = code * chunk_scale)
 *              or bf16, packed rows, 16-byte aligned (dcp_gather_prefix output);
 *              chunk_kv and chunk_scale may be NULL when chunk_len == 0
 *   o, lse     device fp32 [tokens, heads, 512] and [tokens, heads]
 * Runs the dense decode kernels with the (token, head) queries regrouped 64
 * to a row, so that a block reads the chunk once for 64 queries.
 */
dcp_status mla_prefill_chunk_lse(const void* q, int64_t tokens, int32_t heads,
                                 const void* chunk_kv, const float* chunk_scale,
                                 int64_t chunk_len, dcp_kv_dtype kv_dtype, float softmax_scale,
                                 float* o, float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Prefill, step 3 -- running LSE merge of chunk partials ([P1] review
 * exchange on prefix_output: fp32 merge arithmetic, the running output stored
 * in BF16 or kept in fp32).  In place, for every (row, head):
 *   (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_new, lse_new))
 * with the merge of lse_combine (a side with LSE = -inf is skipped; both
 * empty gives O = 0, LSE = -inf).  Start the accumulator at lse = -inf (its O
 * is then never read) or at the first chunk's result.
 *   o_acc    device [rows, heads, dv], fp32 or bf16 per acc_dtype
 *   lse_acc  device fp32 [rows, heads]
 *   o_new, lse_new  device fp32 [rows, heads, dv], [rows, heads]
 */
dcp_status lse_merge_into(void* o_acc, float* lse_acc, const float* o_new, const float* lse_new,
                          int64_t rows, int32_t heads, int32_t dv, dcp_out_dtype acc_dtype,
                          hipStream_t stream);

/*
 * Interleaved KV-cache write with FP8 quantisation ([P1] "feat: support
 * decode context parallelism for PyTorch MLA", File summaries: the KV-cache
 * fill writes new tokens interleaved over the DCP ranks; [P2] "Feat[DCP]
 * Support decode context parallelism for DSA models with the flashmla_kv
 * backend", summary: FP8 caches hold packed FP8, and the review of the
 * gathered buffer: rows are quantised when written to the persistent cache).
 *
 * Token i with slot g = slots[i] >= 0 is written to row g div num_shards of
 * shard g mod num_shards (interleave 1, the slot naming of dcp_remap_topk).
 * BF16 pools receive the 576 values unchanged.  FP8 pools receive
 *   scale = amax / 448 and inv = 448 / amax, amax = max_d |x[d]| (fp32
 *   divisions; both 1 for an all-zero token),
 *   code[d] = E4M3FN(clamp(x[d] * inv, -448, 448)) (fp32 product), round to
 *   nearest even,
 * at the shard's row and scale strides.
 *   kv_new   device bf16 [tokens, 576], 16-byte aligned
 *   slots    device int32 [tokens]; negative = skip.  Slots must be distinct
 *            (unchecked: two writes to one row race); a slot whose row is
 *            beyond its shard's pool_rows is skipped.
 *   shards   host array of num_shards pools (as for the decode calls;
 *            local_len is ignored).  This call writes the rows and scales
 *            that dcp_kv_shard's kv and kv_scale point to: the struct
 *            declares them const for the decode calls, which only read
 *            them, so the caller must pass writable device memory here.
 * Errors (nothing written): DCP_ERR_INVALID_ARGUMENT for tokens < 0, null or
 * misaligned pointers, num_shards outside 1..16, an unknown dtype or a
 * shard failing the dcp_kv_shard rules.  tokens == 0 is a no-op.  Ordered
 * after earlier work on `stream`; a decode reading the same pools must be
 * ordered after it.
 */
dcp_status dcp_kv_write(const void* kv_new, int64_t tokens, const int32_t* slots,
                        const dcp_kv_shard* shards, int32_t num_shards, dcp_kv_dtype kv_dtype,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DCP_MLA_H */
