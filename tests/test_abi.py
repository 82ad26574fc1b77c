"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before queuing work.
No call here reaches a kernel launch (every case fails validation first or is
a documented no-op)."""

import ctypes
import os
import re

import pytest

from sharded_kv_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcp_mla.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, SCRATCH_SMALL = 0, 1, 2, 3, 5
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from sharded_kv_sparse_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "defined")))


def test_header_declares_the_binding_exports():
    assert sorted(B.EXPORTS) == declared_functions()


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.dcp_abi_version() == B.ABI_VERSION == 4
    for code, name in B.STATUS_NAMES.items():
        assert L.dcp_status_string(code).decode() == name
    assert L.dcp_status_string(99).decode() == "DCP_ERR_UNKNOWN"


def test_remap_argument_checks(L):
    f = L.dcp_remap_topk
    assert f(None, 4, 16, 2, -1, FAKE, FAKE, None) == INVALID          # null input
    assert f(FAKE, 4, 16, 2, -1, None, FAKE, None) == INVALID          # null output
    assert f(FAKE, 4, 16, 2, -1, FAKE, None, None) == INVALID          # null counts
    assert f(FAKE, 4, 16, 0, -1, FAKE, FAKE, None) == INVALID          # N < 1
    assert f(FAKE, 4, 16, 17, -1, FAKE, FAKE, None) == INVALID         # N > 16
    assert f(FAKE, 4, 16, 4, 4, FAKE, FAKE, None) == INVALID           # shard >= N
    assert f(FAKE, -1, 16, 4, -1, FAKE, FAKE, None) == INVALID         # rows < 0
    assert f(FAKE, 4, -3, 4, -1, FAKE, FAKE, None) == INVALID          # k < 0
    assert f(None, 0, 16, 4, -1, None, None, None) == OK               # empty: no-op


def _shards(n, fp8=False, dense=False, pool_rows=1024):
    arr = (B.KvShard * n)()
    for r in range(n):
        arr[r] = B.KvShard(0x20000, 0x30000 if fp8 else None, pool_rows, 0x40000 if dense else None)
    return arr


def _sparse(L, **kw):
    a = dict(q=FAKE, rows=4, heads=64, shards=_shards(2), n=2, kv=B.KV_BF16, local=FAKE,
             counts=FAKE, k=64, scale=0.07, o_part=None, lse_part=None, o=FAKE, lse=FAKE,
             out=B.OUT_F32, splits=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return L.mla_sparse_decode_lse(a["q"], a["rows"], a["heads"], a["shards"], a["n"], a["kv"],
                                   a["local"], a["counts"], a["k"], a["scale"], a["o_part"],
                                   a["lse_part"], a["o"], a["lse"], a["out"], a["splits"], a["ws"],
                                   a["ws_bytes"], None)


def test_sparse_decode_argument_checks(L):
    assert _sparse(L, q=None) == INVALID
    assert _sparse(L, heads=40) == UNSUPPORTED                    # heads: a multiple of 16 ...
    assert _sparse(L, heads=8) == UNSUPPORTED
    assert _sparse(L, heads=144) == UNSUPPORTED                   # ... up to 128
    assert _sparse(L, heads=256) == UNSUPPORTED
    assert _sparse(L, n=0) == INVALID
    assert _sparse(L, n=17) == INVALID
    assert _sparse(L, kv=7) == INVALID
    assert _sparse(L, out=5) == INVALID
    assert _sparse(L, k=-1) == INVALID
    assert _sparse(L, counts=None) == INVALID
    assert _sparse(L, o=None, lse=None) == INVALID                 # no output at all
    assert _sparse(L, o=None) == INVALID                           # half a pair
    assert _sparse(L, o_part=FAKE) == INVALID
    assert _sparse(L, scale=float("nan")) == INVALID
    assert _sparse(L, scale=float("inf")) == INVALID
    assert _sparse(L, scale=0.0) == INVALID                        # the softmax scale is positive
    assert _sparse(L, scale=-0.07) == INVALID
    assert _sparse(L, splits=-2) == INVALID
    assert _sparse(L, splits=40) == UNSUPPORTED                    # 2 shards x 40 > 64 partials
    assert _sparse(L, kv=B.KV_FP8_E4M3) == INVALID                 # FP8 needs scales
    assert _sparse(L, shards=_shards(2, pool_rows=0)) == INVALID
    assert _sparse(L, ws=None, ws_bytes=0) == WS_SMALL             # merged output needs counters
    assert _sparse(L, ws_bytes=16) == WS_SMALL
    assert _sparse(L, rows=0, q=None, shards=None, local=None, counts=None) == OK


def _noalloc(L, **kw):
    a = dict(q=FAKE, rows=4, heads=64, shards=_shards(2), n=2, kv=B.KV_BF16, local=FAKE,
             counts=FAKE, k=64, scale=0.07, o_part=None, lse_part=None, o=FAKE, lse=FAKE,
             out=B.OUT_F32, splits=0)
    a.update(kw)
    return L.mla_sparse_decode_lse_noalloc(a["q"], a["rows"], a["heads"], a["shards"], a["n"],
                                           a["kv"], a["local"], a["counts"], a["k"], a["scale"],
                                           a["o_part"], a["lse_part"], a["o"], a["lse"], a["out"],
                                           a["splits"], None)


def test_noalloc_decode_argument_checks(L):
    # the same host checks as the workspace entry point, then the scratch limit
    # (checked before the scratch is touched, so no GPU is needed here)
    assert _noalloc(L, q=None) == INVALID
    assert _noalloc(L, heads=40) == UNSUPPORTED
    assert _noalloc(L, scale=0.0) == INVALID
    assert _noalloc(L, o=None, lse=None) == INVALID
    assert _noalloc(L, splits=40) == UNSUPPORTED
    assert _noalloc(L, rows=0, q=None, shards=None, local=None, counts=None) == OK
    # 1024 rows x 64 heads x 4 shards: about 537 MB of partials > the 63 MiB of scratch
    assert _noalloc(L, rows=1024, shards=_shards(4), n=4, k=2048) == SCRATCH_SMALL
    # 4096 rows x 16 heads, one shard: about 135 MB of partials
    assert _noalloc(L, rows=4096, heads=16, splits=1, shards=_shards(1), n=1) == SCRATCH_SMALL
    # per-shard partials of one split use no scratch: nothing to reject
    assert _noalloc(L, rows=0, o=None, lse=None, o_part=FAKE, lse_part=FAKE) == OK


def test_kv_layout_checks(L):
    # row and scale strides: alignment and size rules of the dcp_kv_shard layout
    def sh(kv=0x20000, scale=0x30000, row_stride=0, scale_stride=0):
        arr = (B.KvShard * 2)()
        for r in range(2):
            arr[r] = B.KvShard(kv, scale, 1024, None, row_stride, scale_stride)
        return arr
    fp8 = B.KV_FP8_E4M3
    assert _sparse(L, kv=fp8, shards=sh(row_stride=600)) == INVALID     # not a multiple of 16
    assert _sparse(L, kv=fp8, shards=sh(row_stride=560)) == INVALID     # shorter than a row
    assert _sparse(L, kv=fp8, shards=sh(row_stride=-640)) == INVALID
    assert _sparse(L, kv=fp8, shards=sh(kv=0x20008)) == INVALID         # kv not 16-byte aligned
    assert _sparse(L, kv=fp8, shards=sh(scale=0x30002)) == INVALID      # scale not 4-byte aligned
    assert _sparse(L, kv=fp8, shards=sh(scale_stride=6)) == INVALID
    assert _sparse(L, kv=fp8, shards=sh(scale_stride=-4)) == INVALID
    assert _sparse(L, shards=sh(scale=None, row_stride=1136)) == INVALID   # BF16 rows are 1152 bytes
    assert _sparse(L, shards=sh(scale=None, row_stride=640)) == INVALID


def test_kv_write_argument_checks(L):
    def kw(kv_new=0x50000, tokens=4, slots=FAKE, shards=None, n=2, kv=B.KV_FP8_E4M3):
        return L.dcp_kv_write(kv_new, tokens, slots, _shards(2, fp8=True) if shards is None else shards,
                              n, kv, None)
    assert kw(tokens=0, kv_new=None, slots=None) == OK                # no-op
    assert kw(tokens=-1) == INVALID
    assert kw(kv_new=None) == INVALID
    assert kw(kv_new=0x50008) == INVALID                              # not 16-byte aligned
    assert kw(slots=None) == INVALID
    assert kw(n=0) == INVALID
    assert kw(n=17) == INVALID
    assert kw(kv=7) == INVALID
    assert kw(shards=_shards(2, fp8=False)) == INVALID                # FP8 needs scales
    assert kw(shards=_shards(2, fp8=True, pool_rows=0)) == INVALID


def test_dense_decode_argument_checks(L):
    def dense(**kw):
        a = dict(q=FAKE, rows=2, heads=64, shards=_shards(2, dense=True), n=2, kv=B.KV_BF16,
                 bt=FAKE, max_pages=8, page=64, max_len=400, scale=0.07, o=FAKE, lse=FAKE,
                 ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return L.mla_dense_decode_lse(a["q"], a["rows"], a["heads"], a["shards"], a["n"], a["kv"],
                                      a["bt"], a["max_pages"], a["page"], a["max_len"], a["scale"],
                                      None, None, a["o"], a["lse"], B.OUT_F32, 0, a["ws"],
                                      a["ws_bytes"], None)
    assert dense(shards=_shards(2, dense=False)) == INVALID        # local_len required
    assert dense(bt=None) == INVALID
    assert dense(page=0) == INVALID
    assert dense(max_pages=0) == INVALID
    assert dense(max_len=-1) == INVALID
    assert dense(max_len=8 * 64 + 1) == INVALID                    # beyond the block table
    assert dense(heads=24) == UNSUPPORTED
    assert dense(scale=0.0) == INVALID
    assert dense(scale=-1.0) == INVALID


def test_merge_wait_setting_range(L):
    assert L.dcp_set_merge_wait_us(-1) == INVALID
    assert L.dcp_set_merge_wait_us(100001) == INVALID
    assert L.dcp_set_merge_wait_us(0) == OK
    assert L.dcp_set_merge_wait_us(30) == OK


def test_prefill_argument_checks(L):
    def gather(bt=FAKE, max_pages=4, page=64, shards=None, n=2, kv=B.KV_FP8_E4M3, pb=FAKE, oo=FAKE,
               seqs=2, max_len=100, out=FAKE, sc=FAKE):
        return L.dcp_gather_prefix(bt, max_pages, page, _shards(2, fp8=True) if shards is None else shards,
                                   n, kv, pb, oo, seqs, max_len, out, sc, None)
    assert gather(seqs=0, bt=None) == OK                                 # nothing to gather
    assert gather(max_len=0) == OK
    assert gather(bt=None) == INVALID
    assert gather(pb=None) == INVALID
    assert gather(oo=None) == INVALID
    assert gather(out=None) == INVALID
    assert gather(sc=None) == INVALID                                    # FP8 needs the scales
    assert gather(out=0x50008) == INVALID                                # not 16-byte aligned
    assert gather(n=0) == INVALID
    assert gather(page=0) == INVALID
    assert gather(max_pages=0) == INVALID
    assert gather(kv=9) == INVALID
    assert gather(shards=_shards(2, fp8=False)) == INVALID
    assert gather(seqs=70000) == UNSUPPORTED

    def chunk(q=FAKE, tokens=37, heads=16, kv_ptr=FAKE, sc=FAKE, c=1000, kv=B.KV_FP8_E4M3, scale=0.07,
              o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return L.mla_prefill_chunk_lse(q, tokens, heads, kv_ptr, sc, c, kv, scale, o, lse, ws, ws_bytes,
                                       None)
    assert chunk(tokens=0, q=None) == OK
    assert chunk(q=None) == INVALID
    assert chunk(kv_ptr=None) == INVALID
    assert chunk(sc=None) == INVALID
    assert chunk(o=None) == INVALID
    assert chunk(lse=None) == INVALID
    assert chunk(scale=0.0) == INVALID
    assert chunk(c=-1) == INVALID
    assert chunk(kv=4) == INVALID
    assert chunk(heads=24) == UNSUPPORTED
    assert chunk(kv_ptr=0x50008) == INVALID
    bad = ctypes.c_size_t(-1).value
    assert L.dcp_prefill_workspace_size(37, 24, 1000) == bad
    assert L.dcp_prefill_workspace_size(-1, 16, 1000) == bad
    assert L.dcp_prefill_workspace_size(0, 16, 1000) == 0
    for h in (48, 80, 112):                                              # leftover queries: one row of 16-48
        assert 0 < L.dcp_prefill_workspace_size(37, h, 1000) < bad
    need = L.dcp_prefill_workspace_size(4, 16, 100000)                  # one row: split, workspace
    assert need > 0 and chunk(tokens=4, c=100000, ws_bytes=need - 1) == WS_SMALL

    def merge(o=FAKE, lse=FAKE, on=FAKE, ln=FAKE, rows=4, heads=16, dv=512, acc=B.OUT_F32):
        return L.lse_merge_into(o, lse, on, ln, rows, heads, dv, acc, None)
    assert merge(rows=0, o=None) == OK
    assert merge(o=None) == INVALID
    assert merge(ln=None) == INVALID
    assert merge(dv=6) == INVALID
    assert merge(acc=3) == INVALID
    assert merge(heads=0) == INVALID
    assert merge(o=0x50008) == INVALID                                   # fp32 accumulator: 16 bytes
    assert merge(o=0x50004, acc=B.OUT_BF16) == INVALID                   # bf16 accumulator: 8 bytes


def test_combine_argument_checks(L):
    f = L.lse_combine
    assert f(None, FAKE, 2, 4, 16, 512, FAKE, FAKE, 0, None) == INVALID
    assert f(FAKE, FAKE, 0, 4, 16, 512, FAKE, FAKE, 0, None) == INVALID
    assert f(FAKE, FAKE, 2, 4, 16, 6, FAKE, FAKE, 0, None) == INVALID   # dv % 4
    assert f(FAKE, FAKE, 2, 4, 0, 512, FAKE, FAKE, 0, None) == INVALID
    assert f(FAKE, FAKE, 2, 4, 16, 512, FAKE, FAKE, 3, None) == INVALID
    assert f(None, None, 2, 0, 16, 512, None, None, 0, None) == OK      # empty: no-op


def test_workspace_size_rules(L):
    bad = ctypes.c_size_t(-1).value
    ws = lambda *a: L.dcp_decode_workspace_size(*a)                    # noqa: E731
    # (dense, rows, heads, shards, tokens, page, splits, partials, merged)
    assert ws(0, 4, 64, 2, 64, 1, 0, 0, 0) == bad                      # no output requested
    assert ws(0, 4, 64, 0, 64, 1, 0, 0, 1) == bad
    assert ws(0, -1, 64, 2, 64, 1, 0, 0, 1) == bad
    assert ws(1, 4, 64, 2, 64, 0, 0, 0, 1) == bad                      # dense needs a page size
    assert ws(0, 0, 64, 2, 64, 1, 0, 0, 1) == 0
    assert ws(0, 4, 40, 2, 64, 1, 0, 0, 1) == bad                      # a head count the decode rejects
    assert ws(0, 4, 48, 2, 64, 1, 0, 0, 1) not in (0, bad)
    assert ws(0, 64, 64, 4, 2048, 1, 1, 1, 0) == 0                     # partials, one split: none
    fused = ws(0, 64, 64, 4, 2048, 1, 1, 0, 1)
    # counters + one fp32 partial (O and LSE) per (row, shard, split, head)
    assert fused >= 64 * 4 * 64 * (512 + 1) * 4
    assert ws(0, 64, 64, 4, 2048, 1, 2, 0, 1) > fused                  # more splits, more partials
    assert ws(0, 128, 64, 4, 2048, 1, 1, 0, 1) > fused
    assert ws(0, 64, 64, 4, 2048, 1, 2, 1, 1) >= ws(0, 64, 64, 4, 2048, 1, 2, 0, 1)


def test_decode_splits_rules(L):
    sp = lambda *a: L.dcp_decode_splits(*a)                            # noqa: E731
    # (dense, rows, heads, shards, tokens, page, splits)
    assert sp(0, 64, 64, 0, 2048, 1, 0) == -1
    assert sp(0, -1, 64, 4, 2048, 1, 0) == -1
    assert sp(1, 4, 64, 2, 64, 0, 0) == -1                           # dense needs a page size
    assert sp(0, 64, 64, 4, 2048, 1, 0) == 1                          # 256 (row, shard) units fill the chip
    assert sp(0, 8, 64, 4, 2048, 1, 0) == 4                           # 32 units: 4 splits of 128 tokens
    assert sp(0, 8, 64, 4, 2048, 1, 8) == 8                           # asked for
    assert sp(0, 8, 64, 4, 2048, 1, 17) == -1                         # 17 x 4 partials: too many to merge
    # every multiple of 16 up to 128 is a supported head count
    for h in range(16, 129, 16):
        assert sp(0, 8, h, 4, 2048, 1, 0) >= 1
        assert sp(1, 8, h, 4, 2048, 64, 0) >= 1
    assert sp(0, 8, 40, 4, 2048, 1, 0) == -1
    assert sp(0, 8, 144, 4, 2048, 1, 0) == -1
    # the workspace query plans the same splits
    for args in [(0, 8, 64, 4, 2048, 1), (1, 32, 128, 8, 131072, 64), (0, 96, 32, 2, 2048, 1),
                 (0, 8, 48, 4, 2048, 1), (1, 4, 112, 2, 4096, 64)]:
        s = sp(*args, 0)
        assert s >= 1
        assert L.dcp_decode_workspace_size(*args, s, 0, 1) == L.dcp_decode_workspace_size(*args, 0, 0, 1)


def test_binding_refuses_without_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        B.remap_topk(torch.zeros((2, 4), dtype=torch.int32), 2)
