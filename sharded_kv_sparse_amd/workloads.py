"""Seeded synthetic inputs for the DCP decode path (no method arithmetic here).

This module only draws inputs: query rows, per-shard KV pools, per-token FP8
scales, block tables, global top-k slot tables and per-shard dense lengths.  It
computes no remap, no attention and no merge.  Tests feed the same arrays to
the HIP library and to the CPU oracle; the benchmark uses the same recipes.

Recipe (the shapes follow the workloads the pages describe: 64-token pages,
interleave-1 token sharding over N shards, the gathered heads of a DCP group,
top-k 2048 sparse decode, MTP rows, million-token dense contexts):

* Physical pages are a seeded permutation of all pages of all sequences; each
  sequence has ceil(context / (page * N)) DCP-wide logical pages of page * N
  tokens.  Every shard's pool holds ``page`` rows for every physical page.
* Position t of sequence b has global slot
  g = BT[b][t div (page*N)] * page * N + t mod (page*N); the pool that holds it
  and the row inside it are a property of the layout, decided by the remap.
* Sparse rows draw top-k distinct positions uniformly from the context (or
  causally up to the row's own position), unsorted, and map them to slots.
* Q ~ N(0,1) rounded to bfloat16.  BF16 KV ~ N(0,1) rounded to bfloat16.  FP8
  KV codes are N(0,1) rounded to E4M3FN by torch's conversion; the per-token
  fp32 scale is 2^U(-6, 2).
* FP8 pools come in two layouts with the same values: 576-byte rows plus a
  separate fp32 scale array, or (row_bytes = 640) each row padded to 640
  bytes with its scale in bytes 576..579 (the pool and scale tensors are then
  strided views of one buffer).
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

D_K = 576
D_V = 512


@dataclass(frozen=True)
class Preset:
    name: str
    kind: str                 # "sparse" | "dense"
    kv_dtype: str             # "bf16" | "fp8"
    batch: int                # sequences
    q_per_seq: int            # query rows per sequence (MTP: draft + 1)
    heads: int                # gathered heads of the DCP group
    context: int              # tokens per sequence
    num_shards: int
    page_size: int = 64
    topk: int = 0             # sparse only
    pad_tail: int = 0         # sparse: trailing -1 entries per row
    causal: bool = False      # sparse MTP rows: slots <= own position
    mtp_empty_rows: bool = False   # sparse MTP: constructed zero-slot rows
    forced_empty: bool = False     # dense: one shard empty for b mod 4 == 0
    short_rows: int = 0       # sparse: if > 0, rows keep 1..short_rows valid slots
    row_bytes: int = 0        # FP8: 0 = 576-byte rows + scale array; 640 = scale in the row
    sigma: float = 1.0 / math.sqrt(192.0)
    seed: int = 0
    note: str = ""

    @property
    def rows(self):
        return self.batch * self.q_per_seq

    @property
    def lpages(self):
        return -(-self.context // (self.page_size * self.num_shards))

    @property
    def pool_rows(self):
        return self.batch * self.lpages * self.page_size


# The five workloads: a tiny dense case, the three sparse decode shapes and the
# million-token dense shard.  Seeds 101..105.
PRESETS = {
    "tiny_dense_bf16_ctx256": Preset(
        "tiny_dense_bf16_ctx256", "dense", "bf16", batch=1, q_per_seq=1, heads=16,
        context=256, num_shards=2, seed=101,
        note="dense MLA decode, 1 row, 16 heads, 256 tokens over 2 shards, BF16"),
    "sparse_bf16_b8_k2048": Preset(
        "sparse_bf16_b8_k2048", "sparse", "bf16", batch=8, q_per_seq=1, heads=64,
        context=32768, num_shards=4, topk=2048, pad_tail=102, seed=102,
        note="sparse DSA decode, 8 rows, 64 heads, 32K context, 4 shards, BF16, "
             "top-k 2048 with the last 5% padded"),
    "sparse_fp8_b64_k2048": Preset(
        "sparse_fp8_b64_k2048", "sparse", "fp8", batch=64, q_per_seq=1, heads=64,
        context=131072, num_shards=4, topk=2048, seed=103,
        note="sparse DSA decode, 64 rows, 64 heads, 128K context, 4 shards, "
             "FP8 E4M3 KV + fp32 per-token scale, top-k 2048"),
    "mtp_sparse_bf16_b16x6_k2048": Preset(
        "mtp_sparse_bf16_b16x6_k2048", "sparse", "bf16", batch=16, q_per_seq=6,
        heads=32, context=65536, num_shards=2, topk=2048, causal=True,
        mtp_empty_rows=True, seed=104,
        note="MTP sparse decode, 16 sequences x 6 query tokens, 32 heads, 64K "
             "context, 2 shards, BF16, causal top-k 2048 with empty-shard rows"),
    "dense_fp8_b32_ctx1m": Preset(
        "dense_fp8_b32_ctx1m", "dense", "fp8", batch=32, q_per_seq=1, heads=128,
        context=1048576, num_shards=8, forced_empty=True, seed=105,
        note="dense MLA decode, 32 rows, 128 heads, 1M context over 8 shards, "
             "FP8 E4M3 KV + fp32 per-token scale, one shard empty on some rows"),
}


def preset(name, **overrides):
    p = PRESETS[name]
    return replace(p, **overrides) if overrides else p


# ---------------------------------------------------------------------------
# Host-side structure (numpy, exact and platform independent)
# ---------------------------------------------------------------------------

def make_block_table(p, rng):
    """[batch, lpages] int32: a seeded permutation of all physical pages."""
    return rng.permutation(p.batch * p.lpages).astype(np.int32).reshape(p.batch, p.lpages)


def positions_to_slots(p, block_table, b, positions):
    """Global slot ids of positions of sequence b under the DCP-wide pages."""
    span = p.page_size * p.num_shards
    pos = np.asarray(positions, dtype=np.int64)
    return (block_table[b][pos // span].astype(np.int64) * span + pos % span)


def _draw(rng, candidates, k):
    if candidates.size <= k:
        return rng.permutation(candidates)
    return rng.choice(candidates, size=k, replace=False)


def make_topk_table(p, block_table, rng):
    """[rows, topk] int32 global slot table, -1 padded (sparse presets)."""
    k = p.topk
    table = np.full((p.rows, k), -1, dtype=np.int64)
    n_valid_default = k - p.pad_tail
    for b in range(p.batch):
        for j in range(p.q_per_seq):
            i = b * p.q_per_seq + j
            if p.causal:
                last = p.context - p.q_per_seq + j        # own position, inclusive
            else:
                last = p.context - 1
            cand = np.arange(last + 1, dtype=np.int64)
            n_valid = n_valid_default
            if p.mtp_empty_rows:
                if b % 4 == 1 and j == 0:
                    cand = cand[cand % p.num_shards == 0]   # only shard 0 owns slots
                elif b % 4 == 2 and j == p.q_per_seq - 1:
                    cand = cand[cand % p.num_shards == 1]   # shard 0 owns none
                if b == p.batch - 1 and j == 3:
                    n_valid = 0                              # all-empty row
            if p.short_rows:
                n_valid = int(rng.integers(1, p.short_rows + 1))
            pos = _draw(rng, cand, min(n_valid, k))
            table[i, : pos.size] = positions_to_slots(p, block_table, b, pos)
    return table.astype(np.int32)


def make_local_lens(p):
    """[N, batch] int32 tokens of each sequence held by each shard (dense)."""
    n = p.num_shards
    lens = np.zeros((n, p.batch), dtype=np.int64)
    for r in range(n):
        lens[r] = max(0, -(-(p.context - r) // n))
    if p.forced_empty:
        for b in range(p.batch):
            if b % 4 == 0:
                lens[(b // 4) % n, b] = 0
    return lens.astype(np.int32)


def make_scales(p, rng):
    """Per-token fp32 scales 2^U(-6, 2) for one shard's pool."""
    return np.exp2(rng.uniform(-6.0, 2.0, size=p.pool_rows)).astype(np.float32)


# ---------------------------------------------------------------------------
# Large arrays (torch, on the requested device)
# ---------------------------------------------------------------------------

def _generator(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _fill_kv(rows, kv_dtype, device, gen, chunk_rows=1 << 17, out=None):
    if out is not None:
        pass
    elif kv_dtype == "bf16":
        out = torch.empty((rows, D_K), dtype=torch.bfloat16, device=device)
    else:
        out = torch.empty((rows, D_K), dtype=torch.uint8, device=device)
    for s in range(0, rows, chunk_rows):
        e = min(rows, s + chunk_rows)
        x = torch.randn((e - s, D_K), generator=gen, device=device)
        if kv_dtype == "bf16":
            out[s:e] = x.to(torch.bfloat16)
        else:
            out[s:e] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


@dataclass
class Workload:
    p: Preset
    device: str
    block_table: np.ndarray
    table: np.ndarray = None          # sparse
    local_lens: np.ndarray = None     # dense
    q: torch.Tensor = None
    pools: list = field(default_factory=list)    # [layer][shard] tensor
    scales: list = field(default_factory=list)   # [layer][shard] tensor or None
    scales_host: list = field(default_factory=list)

    # device copies of the small integer arrays
    def dev(self, arr, dtype=torch.int32):
        return torch.from_numpy(np.ascontiguousarray(arr)).to(self.device, dtype)

    def q_host_bits(self):
        return self.q.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    def pool_host(self, layer, r):
        t = self.pools[layer][r].detach().cpu().contiguous()
        if self.p.kv_dtype == "bf16":
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def scale_host(self, layer, r):
        return None if self.p.kv_dtype == "bf16" else self.scales_host[layer][r]


def make_workload(p, device="cpu", layers=1, seed=None):
    """Draw every input of preset ``p`` (a Preset or a preset name)."""
    if isinstance(p, str):
        p = PRESETS[p]
    seed = p.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    w = Workload(p=p, device=device, block_table=make_block_table(p, rng))
    if p.kind == "sparse":
        w.table = make_topk_table(p, w.block_table, rng)
    else:
        w.local_lens = make_local_lens(p)
    gen = _generator(device, seed)
    w.q = torch.randn((p.rows, p.heads, D_K), generator=gen, device=device).to(torch.bfloat16)
    for layer in range(layers):
        lgen = _generator(device, seed * 1000 + layer + 1)
        pools, scales, scales_h = [], [], []
        for _ in range(p.num_shards):
            inline = p.kv_dtype == "fp8" and p.row_bytes > 0
            if inline:
                assert p.row_bytes % 16 == 0 and p.row_bytes >= D_K + 4
                buf = torch.zeros((p.pool_rows, p.row_bytes), dtype=torch.uint8, device=device)
                pools.append(_fill_kv(p.pool_rows, p.kv_dtype, device, lgen, out=buf[:, :D_K]))
            else:
                pools.append(_fill_kv(p.pool_rows, p.kv_dtype, device, lgen))
            if p.kv_dtype == "fp8":
                s = make_scales(p, rng)
                scales_h.append(s)
                if inline:
                    sc = buf.view(torch.float32)[:, D_K // 4]
                    sc.copy_(torch.from_numpy(s).to(device))
                    scales.append(sc)
                else:
                    scales.append(torch.from_numpy(s).to(device))
            else:
                scales_h.append(None)
                scales.append(None)
        w.pools.append(pools)
        w.scales.append(scales)
        w.scales_host.append(scales_h)
    return w


# ---------------------------------------------------------------------------
# Prefill over a cached prefix (the new tokens of a sequence attend its cached
# prefix, gathered from the shards in bounded chunks)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefillPreset:
    name: str
    kv_dtype: str             # "bf16" | "fp8"
    batch: int                # sequences
    heads: int                # query heads of one rank
    prefix: int               # cached tokens per sequence
    new_tokens: int           # new (prefill) tokens per sequence
    num_shards: int
    chunk: int                # gathered chunk bound (tokens)
    page_size: int = 64
    sigma: float = 1.0 / math.sqrt(192.0)
    seed: int = 0
    note: str = ""

    @property
    def lpages(self):
        return -(-self.prefix // (self.page_size * self.num_shards))

    @property
    def pool_rows(self):
        return self.batch * self.lpages * self.page_size

    # the decode generator's view of the same cache (dense rows, one per sequence)
    def as_dense(self):
        return Preset(self.name, "dense", self.kv_dtype, batch=self.batch, q_per_seq=1,
                      heads=self.heads, context=self.prefix, num_shards=self.num_shards,
                      page_size=self.page_size, sigma=self.sigma, seed=self.seed)


PREFILL_PRESETS = {
    "prefill_fp8_prefix16k_new2k": PrefillPreset(
        "prefill_fp8_prefix16k_new2k", "fp8", batch=1, heads=16, prefix=16384, new_tokens=2048,
        num_shards=4, chunk=4096, seed=111,
        note="prefill of 2,048 new tokens over a 16K cached prefix held by 4 shards, FP8 KV, "
             "16 query heads, the prefix gathered in chunks of 4,096 tokens"),
}


@dataclass
class PrefillWorkload:
    p: PrefillPreset
    cache: Workload           # block table, pools and scales of the cached prefix
    q: torch.Tensor           # bf16 [batch, new_tokens, heads, 576]


def make_prefill_workload(p, device="cpu"):
    """The cached prefix (pools, scales, block table as for dense decode) and
    the new tokens' queries, Q ~ N(0,1) rounded to bfloat16."""
    if isinstance(p, str):
        p = PREFILL_PRESETS[p]
    cache = make_workload(p.as_dense(), device=device)
    gen = _generator(device, p.seed + 7)
    q = torch.randn((p.batch, p.new_tokens, p.heads, D_K), generator=gen, device=device).to(torch.bfloat16)
    return PrefillWorkload(p=p, cache=cache, q=q)


def prefix_chunks(p):
    """[(begin, length)] of the bounded chunks covering a sequence's prefix."""
    return [(b, min(p.chunk, p.prefix - b)) for b in range(0, p.prefix, p.chunk)]


# ---------------------------------------------------------------------------
# Sharded index cache (the DSA indexer's keys, split over the shards like the
# KV) and its query rows
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class IndexPreset:
    name: str
    batch: int                # sequences, one query row each
    context: int              # tokens per sequence
    num_shards: int
    index_heads: int = 64
    topk: int = 2048
    page_size: int = 64
    seed: int = 0
    note: str = ""

    @property
    def rows(self):
        return self.batch

    def as_dense(self):
        return Preset(self.name, "dense", "fp8", batch=self.batch, q_per_seq=1, heads=16,
                      context=self.context, num_shards=self.num_shards, page_size=self.page_size,
                      seed=self.seed)

    @property
    def pool_rows(self):
        return self.as_dense().pool_rows

    @property
    def max_local(self):
        return -(-self.context // self.num_shards)


INDEX_PRESETS = {
    "index_topk_b64_ctx128k_k2048": IndexPreset(
        "index_topk_b64_ctx128k_k2048", batch=64, context=131072, num_shards=4, index_heads=64,
        topk=2048, seed=106,
        note="sharded index cache + distributed top-k: 64 rows, 128K context over 4 shards, "
             "64 index heads x 128 FP8 dims + fp32 scale per token (132 bytes), top-k 2048"),
}


@dataclass
class IndexWorkload:
    p: IndexPreset
    block_table: np.ndarray   # [batch, lpages]
    local_lens: np.ndarray    # [N, batch]
    q: torch.Tensor           # uint8 [rows, hi, 128] E4M3FN codes
    w: torch.Tensor           # fp32 [rows, hi]
    keys: list                # [N] uint8 [pool_rows, 128]
    scales: list              # [N] fp32 [pool_rows]
    scales_host: list
    device: str = "cpu"

    def dev(self, arr, dtype=torch.int32):
        return torch.from_numpy(np.ascontiguousarray(arr)).to(self.device, dtype)


def make_index_workload(p, device="cpu", empty_shard_rows=False):
    """Index keys: E4M3FN codes of N(0,1) draws (torch's conversion), one fp32
    scale 2^U(-6, 2) per token; queries: E4M3FN codes of N(0,1); weights
    N(0,1) / sqrt(heads).  Paging and local lengths as for dense decode.
    empty_shard_rows: rows with b mod 4 == 0 give shard (b / 4) mod N no tokens."""
    if isinstance(p, str):
        p = INDEX_PRESETS[p]
    d = p.as_dense()
    rng = np.random.default_rng(p.seed)
    bt = make_block_table(d, rng)
    lens = make_local_lens(replace(d, forced_empty=empty_shard_rows))
    gen = _generator(device, p.seed)
    q = torch.randn((p.rows, p.index_heads, 128), generator=gen, device=device) \
        .to(torch.float8_e4m3fn).view(torch.uint8)
    w = (torch.randn((p.rows, p.index_heads), generator=gen, device=device)
         / math.sqrt(p.index_heads)).float()
    keys, scales, scales_h = [], [], []
    for _ in range(p.num_shards):
        k = torch.empty((d.pool_rows, 128), dtype=torch.uint8, device=device)
        for s in range(0, d.pool_rows, 1 << 18):
            e = min(d.pool_rows, s + (1 << 18))
            k[s:e] = torch.randn((e - s, 128), generator=gen, device=device) \
                .to(torch.float8_e4m3fn).view(torch.uint8)
        keys.append(k)
        sh = make_scales(d, rng)
        scales_h.append(sh)
        scales.append(torch.from_numpy(sh).to(device))
    return IndexWorkload(p=p, block_table=bt, local_lens=lens, q=q, w=w, keys=keys, scales=scales,
                         scales_host=scales_h, device=device)
