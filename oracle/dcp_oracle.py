"""Plain fp64 CPU oracle for decode context parallelism (DCP) on MLA/DSA decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never does, and this module imports nothing from it: the two share no
code, headers, tables or helpers.  Slow and obviously correct on purpose: every
function is the plain definition, written out with numpy in float64.

Pages this follows (the text of three public pull-request pages):

  [P1] "feat: support decode context parallelism for PyTorch MLA"
       (LMDeploy pull request 4952)
  [P2] "Feat[DCP] Support decode context parallelism for DSA models with the
       flashmla_kv backend" (SGLang pull request 36990)
  [P3] "[DSA] Fix decode context parallelism for RoPE sparse attention on
       Blackwell" (SGLang pull request 42536)

What the path computes, in the pages' terms:

* The KV cache of a sequence is split token by token over N shards with
  interleave 1: position t lives on shard t mod N ([P1] "Server and client
  commands", the vLLM run that selected interleave 1 and block size 64).
* Each shard attends the query heads of the whole DCP group to its own KV only
  and returns the output together with its log-sum-exp ([P1] Summary, decode
  bullet; [P3] Motivation, first cause, and Modifications, Backend).
* For sparse (DSA) attention the global top-k slot table is first turned into
  this shard's local slot ids, moved to the front of the row, with a count per
  row ([P3] Modifications, Index remap).
* The partial results are merged with LSE weights ([P1] Summary); a row with no
  local KV contributes nothing and the merge returns zero when every shard is
  empty ([P3] Modifications, Fixes in shared code; [P2] review of the LSE
  combine, which asks for a zero output and a -inf global LSE in that case).

Readings taken where the pages are silent (all listed in the design notes):

* Key rows have 576 dims (512 latent + 64 RoPE); the value is the first 512
  dims of the same row (absorbed-weight MLA).
* A global slot id g names row g div N of shard g mod N's pool (the DCP-wide
  logical block holds page_size*N tokens; [P1] review note that the scheduler
  unit becomes block_size*dcp, and [P2] review note that locations span
  (size + page_size)*dcp).
* Compaction keeps the original relative order; entries past the count are -1;
  any negative entry is padding.
* LSE is the natural log of the sum of exp of the scaled logits; an empty row
  gives output 0 and LSE -inf.
* FP8 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN) and the stored
  value is code * per-token scale, one fp32 scale for all 576 dims of a token.
* Dense attention of a row reads local tokens j < n_r(b) of its sequence b,
  found through the block table: row BT[b][j div page] * page + j mod page of
  the shard's pool.  One query row per sequence (no causal mask is defined).
"""

import numpy as np

D_K = 576   # key width: 512 latent + 64 RoPE
D_V = 512   # value width: the latent part of the same row

# E4M3FN: exponent and mantissa all ones is NaN, for either sign.
E4M3_NAN_CODES = (0x7F, 0xFF)


# ---------------------------------------------------------------------------
# Element decoders (exact in float64)
# ---------------------------------------------------------------------------

def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 is the upper half of an IEEE binary32, so the bits shifted left
    by 16 and read as float32 give the value; widening to float64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes):
    """OCP FP8 E4M3FN codes (uint8) -> float64, from the bit definition.

    sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e == 0: (-1)^s * m * 2^-9 (subnormal); otherwise (-1)^s * (1 + m/8) * 2^(e-7).
    Codes 0x7F and 0xFF are NaN; the format has no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    subnormal = m.astype(np.float64) * 2.0 ** -9
    normal = (1.0 + m.astype(np.float64) / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


_E4M3_TABLE = decode_e4m3fn(np.arange(256, dtype=np.uint8))


def dequant_rows(pool, rows, kv_dtype, scale=None):
    """Gather pool rows and return their exact float64 values, shape [n, 576].

    kv_dtype "bf16": pool holds bfloat16 bit patterns (uint16) [pool_rows, 576].
    kv_dtype "fp8":  pool holds E4M3FN codes (uint8) [pool_rows, 576] and
                     ``scale`` holds one float32 per row; value = code * scale.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if kv_dtype == "bf16":
        return decode_bf16(np.asarray(pool)[rows])
    if kv_dtype == "fp8":
        codes = np.asarray(pool)[rows]
        s = np.asarray(scale, dtype=np.float32)[rows].astype(np.float64)
        return _E4M3_TABLE[codes] * s[:, None]
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


# ---------------------------------------------------------------------------
# Step 1: index remap ([P3] Modifications, Index remap)
# ---------------------------------------------------------------------------

def remap_topk(table, num_shards, pool_rows=None):
    """Global top-k slot table -> per-shard compacted local slot ids and counts.

    For shard r and row i: keep the entries g >= 0 of row i with g mod N == r,
    in their original order, replace each by g div N, put them at the front of
    the row and record how many there are.  The rest of the row is -1.

    Returns (local [N, R, k] int32, counts [N, R] int32).
    Preconditions (asserted): the valid entries of a row are distinct and, when
    ``pool_rows`` is given, below N * pool_rows.
    """
    t = np.asarray(table, dtype=np.int64)
    rows, k = t.shape
    n = int(num_shards)
    assert n >= 1
    local = np.full((n, rows, k), -1, dtype=np.int32)
    counts = np.zeros((n, rows), dtype=np.int32)
    for i in range(rows):
        valid = t[i][t[i] >= 0]
        assert np.unique(valid).size == valid.size, "duplicate slot in a top-k row"
        if pool_rows is not None:
            assert (valid < n * int(pool_rows)).all(), "slot beyond the pool"
        for r in range(n):
            own = valid[valid % n == r] // n
            local[r, i, : own.size] = own
            counts[r, i] = own.size
    return local, counts


# ---------------------------------------------------------------------------
# Step 2: attention with LSE over one shard ([P3] Modifications, Backend;
# [P1] Summary, decode bullet)
# ---------------------------------------------------------------------------

def attend(q, keys, sigma):
    """Softmax attention of H query rows over n key rows, with its LSE.

    q [H, 576], keys [n, 576] (float64).  Logits z = sigma * q . k over all 576
    dims; values are keys[:, :512].  Returns (O [H, 512], lse [H]) with
    O = sum_j e^{z_j} v_j / sum_j e^{z_j} and lse = ln sum_j e^{z_j}, computed
    with the row maximum subtracted.  n == 0 gives O = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    h = q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((h, D_V)), np.full(h, -np.inf)
    z = sigma * (q @ keys.T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ keys[:, :D_V]) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def sparse_attn_shard(q, pool, kv_dtype, scale, local_table, counts, sigma):
    """Per-shard sparse attention: row i attends local_table[i, :counts[i]].

    q [R, H, 576] float64; pool/scale as in ``dequant_rows``.
    Returns (O_r [R, H, 512], lse_r [R, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    rows, heads, _ = q.shape
    o = np.zeros((rows, heads, D_V))
    lse = np.full((rows, heads), -np.inf)
    for i in range(rows):
        sel = np.asarray(local_table[i][: int(counts[i])], dtype=np.int64)
        keys = dequant_rows(pool, sel, kv_dtype, scale)
        o[i], lse[i] = attend(q[i], keys, sigma)
    return o, lse


def dense_local_rows(block_table_row, n_local, page_size):
    """Pool rows of local tokens j < n_local: BT[j div page]*page + j mod page."""
    j = np.arange(int(n_local), dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[j // page_size]
    return pages * page_size + j % page_size


def dense_attn_shard(q, pool, kv_dtype, scale, block_table, local_len, page_size,
                     sigma):
    """Per-shard dense attention: row b attends all its local tokens.

    One query row per sequence; local_len[b] = n_r(b) tokens of sequence b live
    on this shard, addressed through block_table[b].
    Returns (O_r [B, H, 512], lse_r [B, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    rows, heads, _ = q.shape
    o = np.zeros((rows, heads, D_V))
    lse = np.full((rows, heads), -np.inf)
    for b in range(rows):
        sel = dense_local_rows(block_table[b], local_len[b], page_size)
        keys = dequant_rows(pool, sel, kv_dtype, scale)
        o[b], lse[b] = attend(q[b], keys, sigma)
    return o, lse


# ---------------------------------------------------------------------------
# Step 3: LSE-weighted merge ([P1] Summary; [P3] Fixes in shared code;
# [P2] review of the LSE combine; [P1] review: merge arithmetic in fp32 there,
# float64 here)
# ---------------------------------------------------------------------------

def lse_merge(o_parts, lse_parts):
    """Merge N partial (O_r, lse_r) into (O, lse).

    M = max over shards with lse_r > -inf.  w_r = e^{lse_r - M} for those shards;
    shards with lse_r = -inf are skipped (their O_r is never read, so garbage
    or NaN there cannot leak).  O = sum w_r O_r / sum w_r, lse = M + ln sum w_r.
    If no shard is valid: O = 0 and lse = -inf.

    o_parts [N, R, H, Dv], lse_parts [N, R, H] -> (O [R, H, Dv], lse [R, H]).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    assert not np.isnan(lse_parts).any(), "NaN LSE in a partial"
    valid = lse_parts > -np.inf
    any_valid = valid.any(axis=0)
    m = np.where(valid, lse_parts, -np.inf).max(axis=0)
    m_safe = np.where(any_valid, m, 0.0)
    w = np.where(valid, np.exp(np.where(valid, lse_parts - m_safe, 0.0)), 0.0)
    w_sum = w.sum(axis=0)
    contrib = np.where(valid[..., None], o_parts, 0.0) * w[..., None]
    denom = np.where(any_valid, w_sum, 1.0)
    o = np.where(any_valid[..., None], contrib.sum(axis=0) / denom[..., None], 0.0)
    lse = np.where(any_valid, m_safe + np.log(denom), -np.inf)
    return o, lse


# ---------------------------------------------------------------------------
# Unsharded references: one softmax over the union of the selected tokens.
# DCP reaches exactly this result (up to rounding order).
# ---------------------------------------------------------------------------

def unsharded_sparse(q, pools, kv_dtype, scales, table, sigma):
    """Attention of each row over all valid slots of its global top-k row.

    Slot g is row g div N of shard g mod N's pool.  pools/scales are lists of N
    per-shard arrays (scales entries None for bf16).
    """
    q = np.asarray(q, dtype=np.float64)
    n = len(pools)
    t = np.asarray(table, dtype=np.int64)
    rows, heads, _ = q.shape
    o = np.zeros((rows, heads, D_V))
    lse = np.full((rows, heads), -np.inf)
    for i in range(rows):
        g = t[i][t[i] >= 0]
        keys = np.zeros((g.size, D_K))
        for r in range(n):
            on_r = g % n == r
            keys[on_r] = dequant_rows(pools[r], g[on_r] // n, kv_dtype, scales[r])
        o[i], lse[i] = attend(q[i], keys, sigma)
    return o, lse


def unsharded_dense(q, pools, kv_dtype, scales, block_table, local_lens, page_size,
                    sigma):
    """Attention of each sequence row over the union of every shard's tokens.

    local_lens [N, B]: tokens of sequence b held by shard r (0 = shard empty).
    """
    q = np.asarray(q, dtype=np.float64)
    n = len(pools)
    rows, heads, _ = q.shape
    o = np.zeros((rows, heads, D_V))
    lse = np.full((rows, heads), -np.inf)
    for b in range(rows):
        parts = [
            dequant_rows(pools[r], dense_local_rows(block_table[b], local_lens[r][b],
                                                    page_size), kv_dtype, scales[r])
            for r in range(n)
        ]
        o[b], lse[b] = attend(q[b], np.concatenate(parts, axis=0), sigma)
    return o, lse


# ---------------------------------------------------------------------------
# Interleaved KV-cache write with FP8 quantisation
# ---------------------------------------------------------------------------
#
# [P1] "feat: support decode context parallelism for PyTorch MLA", File
# summaries: the KV-cache fill kernel writes the new tokens interleaved over
# the DCP ranks.  [P2] "Feat[DCP] Support decode context parallelism for DSA
# models with the flashmla_kv backend", summary (FP8 KV caches are packed FP8)
# and the review of the gathered buffer (rows are quantised when they are
# written to the persistent cache).  The pages do not give the scale rule;
# the reading taken here: one fp32 scale per token, the largest magnitude of
# its 576 values divided by 448 (the largest E4M3FN value), and 1 for an
# all-zero token; code = E4M3FN of x times the inverse scale 448 / amax,
# rounded to nearest even.  Every step is one fp32 operation, as in the
# kernel (a quantised code is an integer decided by floating point, so both
# sides decide it in the same precision): the scale and the inverse scale are
# fp32 divisions, x times the inverse scale an fp32 product.

E4M3_MAX = 448.0


def encode_e4m3fn(values):
    """float32 values with |v| <= 448 -> OCP E4M3FN codes (uint8), rounding to
    nearest, ties to even, from the bit definition (the inverse of
    decode_e4m3fn on its grid).  -0.0 keeps its sign bit."""
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("encode_e4m3fn takes finite values with |v| <= 448")
    sign = np.signbit(v)
    a = np.abs(v)
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6                               # below the smallest normal
    # subnormal grid: m * 2^-9, m = 0..7 (m = 8 is the smallest normal, code 8)
    codes[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)      # rint: ties to even
    nrm = ~sub
    if np.any(nrm):
        mant, ex = np.frexp(a[nrm])                   # a = mant * 2^ex, mant in [0.5, 1)
        e = ex - 1                                    # a = (2 mant) * 2^e, 2 mant in [1, 2)
        m8 = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)   # exact operand, ties to even
        carry = m8 == 8
        e = np.where(carry, e + 1, e)
        m8 = np.where(carry, 0, m8)
        codes[nrm] = ((e + 7) << 3) | m8
    codes = codes | np.where(sign, 0x80, 0)
    return codes.astype(np.uint8)


def quantize_row_e4m3(x_bits):
    """One token's 576 bfloat16 values (bit patterns) -> (codes uint8 [576],
    scale float32): scale = amax / 448 and inv = 448 / amax, each one fp32
    division (both 1 when amax is 0); code = E4M3FN(x * inv), the fp32
    product clamped to +-448."""
    x = decode_bf16(x_bits).astype(np.float32)        # exact: a bf16 fits in fp32
    amax = np.float32(np.max(np.abs(x)))
    e4m3_max = np.float32(E4M3_MAX)
    scale = np.float32(amax / e4m3_max) if amax > 0 else np.float32(1.0)
    inv = np.float32(e4m3_max / amax) if amax > 0 else np.float32(1.0)
    q = (x * inv).astype(np.float32)                  # one fp32 product per element
    q = np.clip(q, -e4m3_max, e4m3_max)
    return encode_e4m3fn(q), scale


def kv_write(kv_new_bits, slots, num_shards, pools, scales, kv_dtype):
    """Write new tokens into the shards' pools: token i with global slot
    g = slots[i] >= 0 goes to row g div N of shard g mod N (interleave 1, the
    same slot naming as remap_topk); a negative slot is skipped.  BF16 pools
    get the bit patterns as they are; FP8 pools get quantize_row_e4m3's codes
    and scale.  Returns new lists (the inputs are not modified)."""
    kv_new_bits = np.asarray(kv_new_bits, dtype=np.uint16)
    slots = np.asarray(slots, dtype=np.int64)
    assert kv_new_bits.ndim == 2 and kv_new_bits.shape[1] == D_K
    assert slots.shape == (kv_new_bits.shape[0],)
    pools = [np.array(p, copy=True) for p in pools]
    scales = [None if s is None else np.array(s, copy=True) for s in scales]
    valid = slots[slots >= 0]
    assert len(np.unique(valid)) == len(valid), "slots must be distinct"
    for i, g in enumerate(slots):
        if g < 0:
            continue
        r, row = int(g % num_shards), int(g // num_shards)
        assert row < pools[r].shape[0], "slot beyond the shard's pool"
        if kv_dtype == "bf16":
            pools[r][row] = kv_new_bits[i]
        else:
            codes, sc = quantize_row_e4m3(kv_new_bits[i])
            pools[r][row] = codes
            scales[r][row] = sc
    return pools, scales


# ---------------------------------------------------------------------------
# Prefill over a cached prefix: bounded chunks gathered from the shards, one
# attention per chunk with its LSE, and a running LSE merge of the chunks
# ([P1] "feat: support decode context parallelism for PyTorch MLA", Summary,
# prefill bullet: the cached-prefix KV is gathered in bounded chunks; review
# exchange on prefix_output: merge arithmetic in fp32, the running result
# stored in BF16.  [P2] "Feat[DCP] Support decode context parallelism for DSA
# models with the flashmla_kv backend", summary: with an FP8 cache the
# gathered temporary buffer keeps the cache's packed FP8, no dequantisation.)
# ---------------------------------------------------------------------------

def prefix_slot(block_table_row, num_shards, page_size, position):
    """Global slot of a sequence position: the DCP-wide logical page holds
    page_size * N positions, so position t sits in logical page
    t div (page_size * N) at offset t mod (page_size * N)."""
    span = int(page_size) * int(num_shards)
    t = int(position)
    return int(block_table_row[t // span]) * span + t % span


def gather_prefix(block_table_row, num_shards, page_size, pools, scales, kv_dtype, begin,
                  length):
    """Positions begin .. begin + length - 1 of one sequence, gathered from the
    shards into one contiguous chunk in the cache's own format: the stored
    rows (bf16 bit patterns or E4M3FN codes) and, for FP8, their scales.
    Slot g is row g div N of shard g mod N (as for remap_topk)."""
    n = int(num_shards)
    rows = np.zeros((int(length), D_K), dtype=np.asarray(pools[0]).dtype)
    sc = np.zeros(int(length), dtype=np.float32) if kv_dtype == "fp8" else None
    for j in range(int(length)):
        g = prefix_slot(block_table_row, n, page_size, int(begin) + j)
        r, row = g % n, g // n
        rows[j] = pools[r][row]
        if sc is not None:
            sc[j] = scales[r][row]
    return rows, sc


def prefix_chunk_attention(q, chunk_rows, chunk_scales, kv_dtype, sigma):
    """Every query row of every new token attends every token of the chunk
    (the cached prefix precedes all new tokens, so nothing is masked).
    q [T, H, 576] float64 -> (O [T, H, 512], lse [T, H])."""
    q = np.asarray(q, dtype=np.float64)
    t, h, _ = q.shape
    keys = dequant_rows(chunk_rows, np.arange(len(chunk_rows)), kv_dtype, chunk_scales)
    o, lse = attend(q.reshape(t * h, D_K), keys, sigma)
    return o.reshape(t, h, D_V), lse.reshape(t, h)


def round_bf16(x):
    """float64 -> the nearest bfloat16 value, ties to even, as float64: a
    bfloat16 keeps 8 significant bits, so with x = m * 2^e (m in [0.5, 1))
    the result is rint(m * 2^8) * 2^(e - 8) (exact in float64; values here
    stay far inside bfloat16's exponent range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def merge_running(o_acc, lse_acc, o_new, lse_new, store_bf16=False):
    """One step of the running merge of chunk partials: the LSE merge of the
    accumulated (O, LSE) and a new chunk's (O, LSE).  store_bf16: the merged O
    is stored rounded to bfloat16 (the LSE stays fp32)."""
    o, lse = lse_merge(np.stack([o_acc, o_new]), np.stack([lse_acc, lse_new]))
    if store_bf16:
        o = round_bf16(o)
    return o, lse


# ---------------------------------------------------------------------------
# Sharded index cache and distributed top-k ([P3] "[DSA] Fix decode context
# parallelism for RoPE sparse attention on Blackwell", Follow-ups, item 2:
# the index keys -- 128 FP8 values and one fp32 scale per token, 132 bytes --
# split across the ranks like the KV, each rank scoring its own tokens and
# the local top-k candidates merged into the global top-k; [P1] "feat:
# support decode context parallelism for PyTorch MLA", Summary, decode
# bullet: local candidates merged into the global top-k, and File summaries:
# distributed candidate packing and merging; review note: dcp * k a multiple
# of 512 for the merge kernel.)
#
# The pages do not define the score.  Reading taken (the DSA indexer): for a
# query row with index heads h (128-dim E4M3FN query codes q_h, fp32 weight
# w_h) and a token with index key codes k_t and scale s_t > 0,
#     score(t) = sum_h w_h * max(0, q_h . (s_t k_t)) = s_t * sum_h w_h * max(0, q_h . k_t).
# Selection order: score descending, then position ascending (earlier
# tokens first on equal scores); the global top-k is the first k positions
# in that order, and its slots follow the cache's slot naming.
# ---------------------------------------------------------------------------

D_INDEX = 128


def index_scores(q_codes, w, key_codes, key_scales):
    """Scores of n tokens for one query row: q_codes uint8 [Hi, 128] (E4M3FN),
    w [Hi], key_codes uint8 [n, 128], key_scales [n] (> 0).  Returns float64
    [n]; the dot products of E4M3 values are exact in float64."""
    q = _E4M3_TABLE[np.asarray(q_codes, dtype=np.uint8)]                   # [Hi, 128]
    k = _E4M3_TABLE[np.asarray(key_codes, dtype=np.uint8)]                 # [n, 128]
    # every product of two E4M3 values is a multiple of 2^-18 below 2^18, so
    # the 128-term sums are exact in float64 whatever the summation order
    dots = k @ q.T                                                          # [n, Hi]
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    s = np.asarray(key_scales, dtype=np.float32).astype(np.float64)
    # the weighted sum over heads, per token in one fixed order (so a token's
    # score does not depend on how many tokens are scored together)
    return s * (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)


def topk_order(scores, positions, k):
    """Indices of the k best entries: score descending, then position
    ascending; fewer when there are fewer entries."""
    scores = np.asarray(scores, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    order = np.lexsort((positions, -scores))
    return order[: int(k)]


def index_local_topk(q_codes, w, index_pool, index_scale, block_table_row, n_local, page_size,
                     num_shards, shard, k, score_fn=None):
    """One shard's candidates for one query row: the scores of its local
    tokens j < n_local (pool row BT[j div page] * page + j mod page, position
    j * N + shard) and their top k.  score_fn(j_rows) may supply the scores
    (e.g. float32 scores computed elsewhere).  Returns (scores [m], positions
    [m]) in selection order, m = min(k, n_local)."""
    rows = dense_local_rows(block_table_row, n_local, page_size)
    if score_fn is None:
        sc = index_scores(q_codes, w, np.asarray(index_pool)[rows], np.asarray(index_scale)[rows])
    else:
        sc = np.asarray(score_fn(rows), dtype=np.float64)
    pos = np.arange(int(n_local), dtype=np.int64) * int(num_shards) + int(shard)
    sel = topk_order(sc, pos, k)
    return sc[sel], pos[sel]


def merge_topk(cand_scores, cand_positions, k):
    """The global top k of the shards' candidates (lists of (scores,
    positions), one per shard), in selection order."""
    sc = np.concatenate([np.asarray(c, dtype=np.float64) for c in cand_scores])
    pos = np.concatenate([np.asarray(c, dtype=np.int64) for c in cand_positions])
    sel = topk_order(sc, pos, k)
    return sc[sel], pos[sel]


def positions_to_slots(block_table_row, num_shards, page_size, positions):
    """Slots of sequence positions (the slot naming of remap_topk)."""
    return np.array([prefix_slot(block_table_row, num_shards, page_size, t) for t in positions],
                    dtype=np.int64)


def sharded_topk(q_codes, w, index_pools, index_scales, block_table_row, local_lens, page_size, k):
    """Distributed top-k of one query row: every shard's local top-k, then
    their merge.  local_lens[r]: tokens of the sequence held by shard r.
    Returns (scores [m], positions [m], slots [m]) of the global top k."""
    n = len(index_pools)
    cs, cp = [], []
    for r in range(n):
        s, p = index_local_topk(q_codes, w, index_pools[r], index_scales[r], block_table_row,
                                local_lens[r], page_size, n, r, k)
        cs.append(s)
        cp.append(p)
    s, p = merge_topk(cs, cp, k)
    return s, p, positions_to_slots(block_table_row, n, page_size, p)


def unsharded_topk(q_codes, w, index_pools, index_scales, block_table_row, context, page_size, k):
    """The same top k from one pass over every position of the sequence
    (position t: shard t mod N, local token t div N)."""
    n = len(index_pools)
    sc = np.zeros(int(context))
    for t in range(int(context)):
        r, j = t % n, t // n
        row = dense_local_rows(block_table_row, j + 1, page_size)[j]
        sc[t] = index_scores(q_codes, w, np.asarray(index_pools[r])[row:row + 1],
                             np.asarray(index_scales[r])[row:row + 1])[0]
    sel = topk_order(sc, np.arange(int(context)), k)
    return sc[sel], sel.astype(np.int64), positions_to_slots(block_table_row, n, page_size, sel)
