"""ctypes binding of libdcpmla.so (declared in include/dcp_mla.h).

Argument marshalling only: every step of the path runs in the HIP library.
Tensors supply device memory and the current HIP stream; nothing here
computes a remap, an attention or a merge.  If the library is missing this
module raises -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcpmla.so")

ABI_VERSION = 4           # DCP_ABI_VERSION this binding's structures follow
HEAD_DIM = 576
V_DIM = 512
MAX_SHARDS = 16

DCP_OK = 0
STATUS_NAMES = {0: "DCP_OK", 1: "DCP_ERR_INVALID_ARGUMENT", 2: "DCP_ERR_UNSUPPORTED",
                3: "DCP_ERR_WORKSPACE_TOO_SMALL", 4: "DCP_ERR_LAUNCH",
                5: "DCP_ERR_SCRATCH_TOO_SMALL"}
KV_BF16, KV_FP8_E4M3 = 0, 1
OUT_F32, OUT_BF16 = 0, 1

EXPORTS = ("dcp_status_string", "dcp_abi_version", "dcp_set_merge_wait_us", "dcp_remap_topk",
           "dcp_decode_workspace_size", "dcp_decode_splits", "mla_sparse_decode_lse", "mla_sparse_decode_lse_noalloc",
           "mla_dense_decode_lse",
           "lse_combine", "dcp_kv_write", "dcp_gather_prefix", "dcp_prefill_workspace_size",
           "mla_prefill_chunk_lse", "lse_merge_into", "dcp_index_score", "dcp_topk_local",
           "dcp_topk_merge")


class DcpError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")


class IndexShard(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("key_scale", ctypes.c_void_p),
                ("pool_rows", ctypes.c_int64), ("local_len", ctypes.c_void_p),
                ("row_stride", ctypes.c_int64), ("scale_stride", ctypes.c_int64)]


class KvShard(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p),
                ("pool_rows", ctypes.c_int64), ("local_len", ctypes.c_void_p),
                ("row_stride", ctypes.c_int64), ("scale_stride", ctypes.c_int64)]


_lib = None


def lib():
    """Open libdcpmla.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sharded_kv_sparse_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    L.dcp_status_string.argtypes = [ctypes.c_int]
    L.dcp_status_string.restype = ctypes.c_char_p
    L.dcp_abi_version.argtypes = []
    L.dcp_abi_version.restype = i32
    L.dcp_set_merge_wait_us.argtypes = [i32]
    L.dcp_set_merge_wait_us.restype = ctypes.c_int
    L.dcp_remap_topk.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    L.dcp_remap_topk.restype = ctypes.c_int
    L.dcp_decode_workspace_size.argtypes = [i32, i64, i32, i32, i64, i32, i32, i32, i32]
    L.dcp_decode_workspace_size.restype = sz
    L.dcp_decode_splits.argtypes = [i32, i64, i32, i32, i64, i32, i32]
    L.dcp_decode_splits.restype = i32
    L.mla_sparse_decode_lse.argtypes = [vp, i64, i32, ctypes.POINTER(KvShard), i32, ctypes.c_int,
                                        vp, vp, i32, f32, vp, vp, vp, vp, ctypes.c_int, i32,
                                        vp, sz, vp]
    L.mla_sparse_decode_lse.restype = ctypes.c_int
    L.mla_sparse_decode_lse_noalloc.argtypes = [vp, i64, i32, ctypes.POINTER(KvShard), i32,
                                                ctypes.c_int, vp, vp, i32, f32, vp, vp, vp, vp,
                                                ctypes.c_int, i32, vp]
    L.mla_sparse_decode_lse_noalloc.restype = ctypes.c_int
    L.mla_dense_decode_lse.argtypes = [vp, i64, i32, ctypes.POINTER(KvShard), i32, ctypes.c_int,
                                       vp, i32, i32, i64, f32, vp, vp, vp, vp, ctypes.c_int, i32,
                                       vp, sz, vp]
    L.mla_dense_decode_lse.restype = ctypes.c_int
    L.lse_combine.argtypes = [vp, vp, i32, i64, i32, i32, vp, vp, ctypes.c_int, vp]
    L.lse_combine.restype = ctypes.c_int
    L.dcp_kv_write.argtypes = [vp, i64, vp, ctypes.POINTER(KvShard), i32, ctypes.c_int, vp]
    L.dcp_kv_write.restype = ctypes.c_int
    L.dcp_gather_prefix.argtypes = [vp, i32, i32, ctypes.POINTER(KvShard), i32, ctypes.c_int, vp, vp,
                                    i32, i32, vp, vp, vp]
    L.dcp_gather_prefix.restype = ctypes.c_int
    L.dcp_prefill_workspace_size.argtypes = [i64, i32, i64]
    L.dcp_prefill_workspace_size.restype = sz
    L.mla_prefill_chunk_lse.argtypes = [vp, i64, i32, vp, vp, i64, ctypes.c_int, f32, vp, vp, vp, sz,
                                        vp]
    L.mla_prefill_chunk_lse.restype = ctypes.c_int
    L.lse_merge_into.argtypes = [vp, vp, vp, vp, i64, i32, i32, ctypes.c_int, vp]
    L.lse_merge_into.restype = ctypes.c_int
    L.dcp_index_score.argtypes = [vp, vp, i64, i32, ctypes.POINTER(IndexShard), i32, vp, i32, i32,
                                  i32, vp, vp]
    L.dcp_index_score.restype = ctypes.c_int
    L.dcp_topk_local.argtypes = [vp, i64, i32, i32, vp, i32, vp, vp, vp]
    L.dcp_topk_local.restype = ctypes.c_int
    L.dcp_topk_merge.argtypes = [vp, vp, i64, i32, i32, vp, i32, i32, vp, vp, vp, vp]
    L.dcp_topk_merge.restype = ctypes.c_int
    if L.dcp_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.dcp_abi_version()}, the binding "
                           f"expects {ABI_VERSION}: rebuild it")
    _lib = L
    return L


def _check(status, what):
    if status != DCP_OK:
        raise DcpError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _kv_dtype(pool):
    if pool.dtype == torch.bfloat16:
        return KV_BF16
    if pool.dtype == torch.uint8:
        return KV_FP8_E4M3
    raise TypeError("KV pools are bfloat16 rows or uint8 E4M3FN codes")


def set_merge_wait_us(us):
    """Bound (microseconds) of the wait of a row's blocks for each other in
    the fused merge; process-wide, results bit-identical for every value."""
    _check(lib().dcp_set_merge_wait_us(int(us)), "dcp_set_merge_wait_us")


# ---------------------------------------------------------------- step 1

def remap_topk(topk_global, num_shards, shard=-1, out=None, counts=None, stream=None):
    """Global top-k slot table [rows, k] -> (local [S', rows, k], counts [S', rows])."""
    return prepare_remap_topk(topk_global, num_shards, shard, out, counts, stream)()


def prepare_remap_topk(topk_global, num_shards, shard=-1, out=None, counts=None, stream=None):
    """As remap_topk, but returns a PreparedCall instead of calling."""
    _need(topk_global, torch.int32, "topk_global")
    rows, k = topk_global.shape
    n_out = num_shards if shard < 0 else 1
    if out is None:
        out = torch.empty((n_out, rows, k), dtype=torch.int32, device=topk_global.device)
    if counts is None:
        counts = torch.empty((n_out, rows), dtype=torch.int32, device=topk_global.device)
    _need(out, torch.int32, "out", (n_out, rows, k))
    _need(counts, torch.int32, "counts", (n_out, rows))
    args = (_ptr(topk_global), rows, k, num_shards, shard, _ptr(out), _ptr(counts),
            _stream(topk_global.device, stream))
    return PreparedCall(lib().dcp_remap_topk, args, "dcp_remap_topk", (out, counts),
                        topk_global.device, (topk_global,))


# ---------------------------------------------------------------- workspace

def workspace_size(dense, rows, heads, num_shards, tokens_per_shard, page_size=64, num_splits=0,
                   want_partials=False, want_merged=True):
    n = lib().dcp_decode_workspace_size(int(bool(dense)), rows, heads, num_shards,
                                        tokens_per_shard, page_size, num_splits,
                                        int(bool(want_partials)), int(bool(want_merged)))
    if n == ctypes.c_size_t(-1).value:
        raise DcpError(1, "dcp_decode_workspace_size")
    return n


def decode_splits(dense, rows, heads, num_shards, tokens_per_shard, page_size=64, num_splits=0):
    """Token splits per (row, shard) a decode call with these arguments uses."""
    s = lib().dcp_decode_splits(int(bool(dense)), rows, heads, num_shards, tokens_per_shard,
                                page_size, num_splits)
    if s < 0:
        raise DcpError(1, "dcp_decode_splits")
    return s


def alloc_workspace(nbytes, device):
    """Zeroed once; every call leaves the library's counters ready for the next."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- step 2 (+3)

def _shards(pools, scales, local_lens=None):
    n = len(pools)
    if not 1 <= n <= MAX_SHARDS:
        raise ValueError("1..16 shards")
    arr = (KvShard * n)()
    kv_dtype = _kv_dtype(pools[0])
    for r, pool in enumerate(pools):
        if pool.dtype != pools[0].dtype:
            raise TypeError("all shards share one KV dtype")
        # pools may be row-strided views (rows padded, e.g. with the scale
        # inside), scales strided views; the library checks the alignment
        _need(pool, pool.dtype, f"pool[{r}]", contiguous=False)
        if pool.dim() != 2 or pool.shape[1] != HEAD_DIM or pool.stride(1) != 1:
            raise ValueError(f"pool[{r}] must be [rows, {HEAD_DIM}] with unit inner stride")
        sc = None
        if kv_dtype == KV_FP8_E4M3:
            sc = scales[r]
            _need(sc, torch.float32, f"scale[{r}]", (pool.shape[0],), contiguous=False)
        ll = None
        if local_lens is not None:
            ll = local_lens[r]
            _need(ll, torch.int32, f"local_len[{r}]")
        arr[r] = KvShard(pool.data_ptr(), None if sc is None else sc.data_ptr(), pool.shape[0],
                         None if ll is None else ll.data_ptr(),
                         pool.stride(0) * pool.element_size(),
                         0 if sc is None else sc.stride(0) * 4)
    return arr, kv_dtype


def _outputs(q, num_shards, want_partials, want_merged, out_dtype, out=None):
    rows, heads, _ = q.shape
    dev = q.device
    res = {}
    if want_partials:
        res["o_part"] = torch.empty((num_shards, rows, heads, V_DIM), dtype=torch.float32, device=dev)
        res["lse_part"] = torch.empty((num_shards, rows, heads), dtype=torch.float32, device=dev)
    if want_merged:
        odt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
        res["o"] = torch.empty((rows, heads, V_DIM), dtype=odt, device=dev)
        res["lse"] = torch.empty((rows, heads), dtype=torch.float32, device=dev)
    if out:
        res.update(out)
    return res


class PreparedCall:
    """A library call with every argument marshalled once (for launch loops).

    Holds references to the tensors it points at.  Calling it queues the work
    on the stream captured at preparation time (or the one given)."""

    def __init__(self, fn, args, name, result, device, keep):
        self._fn, self._args, self._name = fn, args, name
        self.result, self._device, self._keep = result, device, keep

    def __call__(self, stream=None):
        args = self._args if stream is None else self._args[:-1] + (_stream(self._device, stream),)
        _check(self._fn(*args), self._name)
        return self.result


def sparse_decode(q, pools, scales, topk_local, counts, softmax_scale, want_partials=False,
                  want_merged=True, out_dtype=OUT_F32, num_splits=0, workspace=None, out=None,
                  stream=None):
    """Per-shard sparse MLA decode with LSE, merged in the epilogue when asked.

    q bf16 [rows, heads, 576]; pools[r] bf16 or uint8 [pool_rows, 576];
    scales[r] fp32 [pool_rows] for FP8; topk_local int32 [N, rows, k];
    counts int32 [N, rows].  Returns a dict with o/lse and/or o_part/lse_part.
    """
    return prepare_sparse_decode(q, pools, scales, topk_local, counts, softmax_scale,
                                 want_partials, want_merged, out_dtype, num_splits, workspace,
                                 out, stream)()


def prepare_sparse_decode(q, pools, scales, topk_local, counts, softmax_scale,
                          want_partials=False, want_merged=True, out_dtype=OUT_F32, num_splits=0,
                          workspace=None, out=None, stream=None):
    """As sparse_decode, but returns a PreparedCall instead of calling."""
    _need(q, torch.bfloat16, "q")
    rows, heads, _ = q.shape
    n = len(pools)
    _need(topk_local, torch.int32, "topk_local")
    k = topk_local.shape[-1]
    _need(topk_local, torch.int32, "topk_local", (n, rows, k))
    _need(counts, torch.int32, "counts", (n, rows))
    shards, kv_dtype = _shards(pools, scales)
    res = _outputs(q, n, want_partials, want_merged, out_dtype, out)
    if workspace is None:
        nb = workspace_size(False, rows, heads, n, k, 1, num_splits, want_partials, want_merged)
        workspace = alloc_workspace(nb, q.device) if nb else None
    args = (_ptr(q), rows, heads, shards, n, kv_dtype, _ptr(topk_local), _ptr(counts), k,
            float(softmax_scale), _ptr(res.get("o_part")), _ptr(res.get("lse_part")),
            _ptr(res.get("o")), _ptr(res.get("lse")), out_dtype, num_splits, _ptr(workspace),
            0 if workspace is None else workspace.numel(), _stream(q.device, stream))
    keep = (q, pools, scales, topk_local, counts, workspace)
    return PreparedCall(lib().mla_sparse_decode_lse, args, "mla_sparse_decode_lse", res, q.device,
                        keep)


def sparse_decode_noalloc(q, pools, scales, topk_local, counts, softmax_scale,
                          want_partials=False, want_merged=True, out_dtype=OUT_F32, num_splits=0,
                          out=None, stream=None):
    """As sparse_decode, through mla_sparse_decode_lse_noalloc: the fused
    merge uses the library's static scratch instead of a workspace."""
    return prepare_sparse_decode_noalloc(q, pools, scales, topk_local, counts, softmax_scale,
                                         want_partials, want_merged, out_dtype, num_splits, out,
                                         stream)()


def prepare_sparse_decode_noalloc(q, pools, scales, topk_local, counts, softmax_scale,
                                  want_partials=False, want_merged=True, out_dtype=OUT_F32,
                                  num_splits=0, out=None, stream=None):
    """As sparse_decode_noalloc, but returns a PreparedCall instead of calling."""
    _need(q, torch.bfloat16, "q")
    rows, heads, _ = q.shape
    n = len(pools)
    _need(topk_local, torch.int32, "topk_local")
    k = topk_local.shape[-1]
    _need(topk_local, torch.int32, "topk_local", (n, rows, k))
    _need(counts, torch.int32, "counts", (n, rows))
    shards, kv_dtype = _shards(pools, scales)
    res = _outputs(q, n, want_partials, want_merged, out_dtype, out)
    args = (_ptr(q), rows, heads, shards, n, kv_dtype, _ptr(topk_local), _ptr(counts), k,
            float(softmax_scale), _ptr(res.get("o_part")), _ptr(res.get("lse_part")),
            _ptr(res.get("o")), _ptr(res.get("lse")), out_dtype, num_splits,
            _stream(q.device, stream))
    return PreparedCall(lib().mla_sparse_decode_lse_noalloc, args, "mla_sparse_decode_lse_noalloc",
                        res, q.device, (q, pools, scales, topk_local, counts))


def dense_decode(q, pools, scales, block_table, local_lens, page_size, max_local_len,
                 softmax_scale, want_partials=False, want_merged=True, out_dtype=OUT_F32,
                 num_splits=0, workspace=None, out=None, stream=None):
    """Per-shard dense MLA decode with LSE over each sequence's local tokens.

    block_table int32 [rows, max_pages]; local_lens[r] int32 [rows].
    """
    return prepare_dense_decode(q, pools, scales, block_table, local_lens, page_size,
                                max_local_len, softmax_scale, want_partials, want_merged,
                                out_dtype, num_splits, workspace, out, stream)()


def prepare_dense_decode(q, pools, scales, block_table, local_lens, page_size, max_local_len,
                         softmax_scale, want_partials=False, want_merged=True, out_dtype=OUT_F32,
                         num_splits=0, workspace=None, out=None, stream=None):
    """As dense_decode, but returns a PreparedCall instead of calling."""
    _need(q, torch.bfloat16, "q")
    rows, heads, _ = q.shape
    n = len(pools)
    _need(block_table, torch.int32, "block_table")
    if block_table.dim() != 2 or block_table.shape[0] != rows:
        raise ValueError("block_table must be [rows, max_pages]")
    shards, kv_dtype = _shards(pools, scales, local_lens)
    res = _outputs(q, n, want_partials, want_merged, out_dtype, out)
    if workspace is None:
        nb = workspace_size(True, rows, heads, n, max_local_len, page_size, num_splits,
                            want_partials, want_merged)
        workspace = alloc_workspace(nb, q.device) if nb else None
    args = (_ptr(q), rows, heads, shards, n, kv_dtype, _ptr(block_table), block_table.shape[1],
            page_size, max_local_len, float(softmax_scale), _ptr(res.get("o_part")),
            _ptr(res.get("lse_part")), _ptr(res.get("o")), _ptr(res.get("lse")), out_dtype,
            num_splits, _ptr(workspace), 0 if workspace is None else workspace.numel(),
            _stream(q.device, stream))
    keep = (q, pools, scales, block_table, local_lens, workspace)
    return PreparedCall(lib().mla_dense_decode_lse, args, "mla_dense_decode_lse", res, q.device,
                        keep)


# ---------------------------------------------------------------- step 3

def lse_combine(o_part, lse_part, out_dtype=OUT_F32, o=None, lse=None, stream=None):
    """Merge partials [N, rows, heads, dv] + [N, rows, heads] -> (o, lse)."""
    _need(o_part, torch.float32, "o_part")
    n, rows, heads, dv = o_part.shape
    _need(lse_part, torch.float32, "lse_part", (n, rows, heads))
    if o is None:
        odt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
        o = torch.empty((rows, heads, dv), dtype=odt, device=o_part.device)
    if lse is None:
        lse = torch.empty((rows, heads), dtype=torch.float32, device=o_part.device)
    _check(lib().lse_combine(_ptr(o_part), _ptr(lse_part), n, rows, heads, dv, _ptr(o), _ptr(lse),
                             out_dtype, _stream(o_part.device, stream)), "lse_combine")
    return o, lse


# ---------------------------------------------------------------- KV write

def kv_write(kv_new, slots, pools, scales, stream=None):
    """Write new tokens into the shards' pools in place: kv_new bf16
    [tokens, 576], slots int32 [tokens] (global slot ids, negative = skip);
    pools / scales as for the decode calls (FP8 pools are quantised with one
    fp32 scale per token)."""
    prepare_kv_write(kv_new, slots, pools, scales, stream)()


def prepare_kv_write(kv_new, slots, pools, scales, stream=None):
    """As kv_write, but returns a PreparedCall instead of calling."""
    _need(kv_new, torch.bfloat16, "kv_new")
    if kv_new.dim() != 2 or kv_new.shape[1] != HEAD_DIM:
        raise ValueError(f"kv_new must be [tokens, {HEAD_DIM}]")
    _need(slots, torch.int32, "slots", (kv_new.shape[0],))
    shards, kv_dtype = _shards(pools, scales)
    args = (_ptr(kv_new), kv_new.shape[0], _ptr(slots), shards, len(pools), kv_dtype,
            _stream(kv_new.device, stream))
    return PreparedCall(lib().dcp_kv_write, args, "dcp_kv_write", None, kv_new.device,
                        (kv_new, slots, pools, scales))


# ---------------------------------------------------------------- prefill over a cached prefix

def gather_prefix(block_table, pools, scales, page_size, pos_begin, lengths, out_kv=None,
                  out_scale=None, stream=None):
    """Gather positions pos_begin[b] .. + lengths[b] of every sequence b from
    the shards into one chunk buffer (rows of sequence b after those of
    b - 1), in the cache's own format.  block_table int32 [num_seqs,
    max_pages] (device); pos_begin, lengths: host sequences of ints.
    Returns (chunk rows [total, 576], chunk scales [total] or None)."""
    return prepare_gather_prefix(block_table, pools, scales, page_size, pos_begin, lengths,
                                 out_kv, out_scale, stream)()


def prepare_gather_prefix(block_table, pools, scales, page_size, pos_begin, lengths, out_kv=None,
                          out_scale=None, stream=None):
    """As gather_prefix, but returns a PreparedCall instead of calling."""
    _need(block_table, torch.int32, "block_table")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, max_pages]")
    num_seqs, max_pages = block_table.shape
    if len(pos_begin) != num_seqs or len(lengths) != num_seqs:
        raise ValueError("one pos_begin and one length per sequence")
    shards, kv_dtype = _shards(pools, scales)
    dev = block_table.device
    offs = [0]
    for n in lengths:
        offs.append(offs[-1] + int(n))
    total = offs[-1]
    pb = torch.tensor([int(x) for x in pos_begin], dtype=torch.int32).to(dev)
    oo = torch.tensor(offs, dtype=torch.int32).to(dev)
    if out_kv is None:
        out_kv = torch.empty((total, HEAD_DIM), dtype=pools[0].dtype, device=dev)
    _need(out_kv, pools[0].dtype, "out_kv", (total, HEAD_DIM))
    if kv_dtype == KV_FP8_E4M3 and out_scale is None:
        out_scale = torch.empty((total,), dtype=torch.float32, device=dev)
    if out_scale is not None:
        _need(out_scale, torch.float32, "out_scale", (total,))
    max_len = max([int(n) for n in lengths] + [0])
    args = (_ptr(block_table), max_pages, int(page_size), shards, len(pools), kv_dtype, _ptr(pb),
            _ptr(oo), num_seqs, max_len, _ptr(out_kv), _ptr(out_scale), _stream(dev, stream))
    return PreparedCall(lib().dcp_gather_prefix, args, "dcp_gather_prefix", (out_kv, out_scale), dev,
                        (block_table, pools, scales, pb, oo))


def prefill_workspace_size(tokens, heads, chunk_len):
    n = lib().dcp_prefill_workspace_size(tokens, heads, chunk_len)
    if n == ctypes.c_size_t(-1).value:
        raise DcpError(1, "dcp_prefill_workspace_size")
    return n


def prefill_chunk_attention(q, chunk_kv, chunk_scale, softmax_scale, o=None, lse=None,
                            workspace=None, stream=None):
    """Attention of every (token, head) query row of q bf16 [tokens, heads,
    576] over every row of a gathered chunk; returns fp32 (o, lse)."""
    return prepare_prefill_chunk_attention(q, chunk_kv, chunk_scale, softmax_scale, o, lse,
                                           workspace, stream)()


def prepare_prefill_chunk_attention(q, chunk_kv, chunk_scale, softmax_scale, o=None, lse=None,
                                    workspace=None, stream=None):
    """As prefill_chunk_attention, but returns a PreparedCall instead of calling."""
    _need(q, torch.bfloat16, "q")
    tokens, heads, _ = q.shape
    kv_dtype = _kv_dtype(chunk_kv)
    _need(chunk_kv, chunk_kv.dtype, "chunk_kv")
    if chunk_kv.dim() != 2 or chunk_kv.shape[1] != HEAD_DIM:
        raise ValueError(f"chunk_kv must be [chunk_len, {HEAD_DIM}]")
    c = chunk_kv.shape[0]
    if kv_dtype == KV_FP8_E4M3:
        _need(chunk_scale, torch.float32, "chunk_scale", (c,))
    if o is None:
        o = torch.empty((tokens, heads, V_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((tokens, heads), dtype=torch.float32, device=q.device)
    _need(o, torch.float32, "o", (tokens, heads, V_DIM))
    _need(lse, torch.float32, "lse", (tokens, heads))
    if workspace is None:
        nb = prefill_workspace_size(tokens, heads, c)
        workspace = alloc_workspace(nb, q.device) if nb else None
    args = (_ptr(q), tokens, heads, _ptr(chunk_kv), _ptr(chunk_scale), c, kv_dtype,
            float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace),
            0 if workspace is None else workspace.numel(), _stream(q.device, stream))
    return PreparedCall(lib().mla_prefill_chunk_lse, args, "mla_prefill_chunk_lse", (o, lse),
                        q.device, (q, chunk_kv, chunk_scale, workspace))


def merge_into(o_acc, lse_acc, o_new, lse_new, stream=None):
    """Running merge in place: (o_acc, lse_acc) <- merge with (o_new, lse_new).
    o_acc fp32 or bf16 [rows, heads, dv]; the others fp32."""
    prepare_merge_into(o_acc, lse_acc, o_new, lse_new, stream)()


def prepare_merge_into(o_acc, lse_acc, o_new, lse_new, stream=None):
    """As merge_into, but returns a PreparedCall instead of calling."""
    if o_acc.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("o_acc must be float32 or bfloat16")
    _need(o_acc, o_acc.dtype, "o_acc")
    rows, heads, dv = o_acc.shape
    _need(lse_acc, torch.float32, "lse_acc", (rows, heads))
    _need(o_new, torch.float32, "o_new", (rows, heads, dv))
    _need(lse_new, torch.float32, "lse_new", (rows, heads))
    acc_dtype = OUT_BF16 if o_acc.dtype == torch.bfloat16 else OUT_F32
    args = (_ptr(o_acc), _ptr(lse_acc), _ptr(o_new), _ptr(lse_new), rows, heads, dv, acc_dtype,
            _stream(o_acc.device, stream))
    return PreparedCall(lib().lse_merge_into, args, "lse_merge_into", None, o_acc.device,
                        (o_acc, lse_acc, o_new, lse_new))



def prefix_attention(q, block_table_row, pools, scales, page_size, prefix_len, chunk, softmax_scale,
                     acc_dtype=torch.float32, stream=None):
    """The new tokens' attention to one sequence's cached prefix, the prefix
    gathered from the shards in chunks of at most `chunk` tokens: for each
    chunk, dcp_gather_prefix, mla_prefill_chunk_lse and lse_merge_into (the
    running output kept in acc_dtype, float32 or bfloat16).  q bf16 [tokens,
    heads, 576]; block_table_row int32 [max_pages] (device).  Only calls the
    library; returns (o, lse)."""
    tokens, heads, _ = q.shape
    dev = q.device
    o = torch.zeros((tokens, heads, V_DIM), dtype=acc_dtype, device=dev)
    lse = torch.full((tokens, heads), float("-inf"), dtype=torch.float32, device=dev)
    c_max = max(min(int(chunk), int(prefix_len)), 1)
    kv = torch.empty((c_max, HEAD_DIM), dtype=pools[0].dtype, device=dev)
    sc = torch.empty((c_max,), dtype=torch.float32, device=dev) \
        if _kv_dtype(pools[0]) == KV_FP8_E4M3 else None
    o_c = torch.empty((tokens, heads, V_DIM), dtype=torch.float32, device=dev)
    lse_c = torch.empty((tokens, heads), dtype=torch.float32, device=dev)
    ws_n = prefill_workspace_size(tokens, heads, c_max)
    ws = alloc_workspace(ws_n, dev) if ws_n else None
    bt = block_table_row.reshape(1, -1)
    for b in range(0, int(prefix_len), int(chunk)):
        n = min(int(chunk), int(prefix_len) - b)
        gather_prefix(bt, pools, scales, page_size, [b], [n], out_kv=kv[:n],
                      out_scale=None if sc is None else sc[:n], stream=stream)
        prefill_chunk_attention(q, kv[:n], None if sc is None else sc[:n], softmax_scale, o_c, lse_c,
                                workspace=ws, stream=stream)
        merge_into(o, lse, o_c, lse_c, stream=stream)
    return o, lse


# ---------------------------------------------------------------- sharded index cache + top-k

def _index_shards(keys, scales, local_lens):
    n = len(keys)
    if not 1 <= n <= MAX_SHARDS:
        raise ValueError("1..16 shards")
    arr = (IndexShard * n)()
    for r in range(n):
        _need(keys[r], torch.uint8, f"keys[{r}]", contiguous=False)
        if keys[r].dim() != 2 or keys[r].shape[1] != 128 or keys[r].stride(1) != 1:
            raise ValueError(f"keys[{r}] must be [rows, 128] with unit inner stride")
        _need(scales[r], torch.float32, f"key_scale[{r}]", (keys[r].shape[0],), contiguous=False)
        _need(local_lens[r], torch.int32, f"local_len[{r}]")
        arr[r] = IndexShard(keys[r].data_ptr(), scales[r].data_ptr(), keys[r].shape[0],
                            local_lens[r].data_ptr(), keys[r].stride(0), scales[r].stride(0) * 4)
    return arr


def index_score(q, w, keys, scales, local_lens, block_table, page_size, max_local, out=None,
                stream=None):
    """Index scores [N, rows, max_local] fp32 of every local token: q uint8
    [rows, hi, 128] E4M3FN codes, w fp32 [rows, hi], keys[r] uint8 [pool_rows,
    128], scales[r] fp32 [pool_rows], local_lens[r] int32 [rows]."""
    return prepare_index_score(q, w, keys, scales, local_lens, block_table, page_size, max_local,
                               out, stream)()


def prepare_index_score(q, w, keys, scales, local_lens, block_table, page_size, max_local, out=None,
                        stream=None):
    _need(q, torch.uint8, "q")
    rows, hi, d = q.shape
    if d != 128:
        raise ValueError("index queries are [rows, heads, 128]")
    _need(w, torch.float32, "w", (rows, hi))
    _need(block_table, torch.int32, "block_table")
    n = len(keys)
    shards = _index_shards(keys, scales, local_lens)
    if out is None:
        out = torch.empty((n, rows, max_local), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "scores", (n, rows, max_local))
    args = (_ptr(q), _ptr(w), rows, hi, shards, n, _ptr(block_table), block_table.shape[1],
            int(page_size), int(max_local), _ptr(out), _stream(q.device, stream))
    return PreparedCall(lib().dcp_index_score, args, "dcp_index_score", out, q.device,
                        (q, w, keys, scales, local_lens, block_table))


def topk_local(scores, local_len, k, cand_score=None, cand_pos=None, stream=None):
    """Local top-k of every (shard, row): scores [N, rows, max_local],
    local_len int32 [N, rows] -> (cand_score, cand_pos) [N, rows, k]."""
    return prepare_topk_local(scores, local_len, k, cand_score, cand_pos, stream)()


def prepare_topk_local(scores, local_len, k, cand_score=None, cand_pos=None, stream=None):
    _need(scores, torch.float32, "scores")
    n, rows, max_local = scores.shape
    _need(local_len, torch.int32, "local_len", (n, rows))
    if cand_score is None:
        cand_score = torch.empty((n, rows, k), dtype=torch.float32, device=scores.device)
    if cand_pos is None:
        cand_pos = torch.empty((n, rows, k), dtype=torch.int32, device=scores.device)
    _need(cand_score, torch.float32, "cand_score", (n, rows, k))
    _need(cand_pos, torch.int32, "cand_pos", (n, rows, k))
    args = (_ptr(scores), rows, n, max_local, _ptr(local_len), int(k), _ptr(cand_score), _ptr(cand_pos),
            _stream(scores.device, stream))
    return PreparedCall(lib().dcp_topk_local, args, "dcp_topk_local", (cand_score, cand_pos),
                        scores.device, (scores, local_len))


def topk_merge(cand_score, cand_pos, block_table, page_size, out=None, stream=None):
    """Global top-k of every row from the shards' candidates [N, rows, k]:
    returns (scores [rows, k], positions [rows, k], slots [rows, k])."""
    return prepare_topk_merge(cand_score, cand_pos, block_table, page_size, out, stream)()


def prepare_topk_merge(cand_score, cand_pos, block_table, page_size, out=None, stream=None):
    _need(cand_score, torch.float32, "cand_score")
    n, rows, k = cand_score.shape
    _need(cand_pos, torch.int32, "cand_pos", (n, rows, k))
    _need(block_table, torch.int32, "block_table")
    dev = cand_score.device
    if out is None:
        out = (torch.empty((rows, k), dtype=torch.float32, device=dev),
               torch.empty((rows, k), dtype=torch.int32, device=dev),
               torch.empty((rows, k), dtype=torch.int32, device=dev))
    ts, tp, tg = out
    args = (_ptr(cand_score), _ptr(cand_pos), rows, n, k, _ptr(block_table), block_table.shape[1],
            int(page_size), _ptr(ts), _ptr(tp), _ptr(tg), _stream(dev, stream))
    return PreparedCall(lib().dcp_topk_merge, args, "dcp_topk_merge", out, dev,
                        (cand_score, cand_pos, block_table))
