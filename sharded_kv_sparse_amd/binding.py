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

ABI_VERSION = 3           # DCP_ABI_VERSION this binding's structures follow
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
           "dcp_decode_workspace_size", "mla_sparse_decode_lse", "mla_sparse_decode_lse_noalloc",
           "mla_dense_decode_lse",
           "lse_combine", "dcp_kv_write")


class DcpError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")


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


def alloc_workspace(nbytes, device):
    """Zeroed once; the library leaves its counters zeroed after every call."""
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
