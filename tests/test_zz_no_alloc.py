"""The decode entry point that allocates nothing (mla_sparse_decode_lse_noalloc)
against the workspace entry point (mla_sparse_decode_lse), through the C ABI.

Two calls in a row on the library's static scratch, the second with a smaller
input (fewer rows, other heads and shard count, so a different split of the
scratch): each result bit-identical to the workspace call's on the same
inputs (the same kernels run) and within tolerance of the CPU oracle.
"""

import numpy as np
import pytest
import torch

from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

from ._support import check_against_oracle, make, oracle_sparse

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


CASES = [
    # first call: 32 rows x 64 heads x 4 shards, FP8, top-k 2048 (about 17 MB of scratch)
    wl.Preset("noalloc-a", "sparse", "fp8", batch=32, q_per_seq=1, heads=64, context=32768,
              num_shards=4, topk=2048, pad_tail=40, seed=301),
    # second call, smaller: 6 rows x 128 heads x 2 shards, BF16, short rows included
    wl.Preset("noalloc-b", "sparse", "bf16", batch=6, q_per_seq=1, heads=128, context=5000,
              num_shards=2, topk=300, short_rows=40, seed=302),
]


def test_noalloc_matches_workspace_call_twice(gpu):
    for p in CASES:
        w = make(p)
        local, counts = B.remap_topk(w.dev(w.table), p.num_shards)
        say(f"noalloc {p.name}: {p.rows} rows x {p.heads} heads x {p.num_shards} shards {p.kv_dtype}")
        ref = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma,
                              want_partials=False, want_merged=True)
        got = B.sparse_decode_noalloc(w.q, w.pools[0], w.scales[0], local, counts, p.sigma,
                                      want_partials=False, want_merged=True)
        torch.cuda.synchronize()
        assert torch.equal(got["o"], ref["o"]), p.name
        assert torch.equal(got["lse"], ref["lse"]), p.name
        check_against_oracle(got, oracle_sparse(w), f"noalloc {p.name}")
        # the same call again on the scratch the first left behind
        again = B.sparse_decode_noalloc(w.q, w.pools[0], w.scales[0], local, counts, p.sigma,
                                        want_partials=False, want_merged=True)
        torch.cuda.synchronize()
        assert torch.equal(again["o"], ref["o"]) and torch.equal(again["lse"], ref["lse"]), p.name


def test_noalloc_rejects_calls_beyond_the_scratch(gpu):
    # 256 rows x 64 heads x 4 shards would need about 135 MB of partials
    p = wl.Preset("noalloc-big", "sparse", "fp8", batch=256, q_per_seq=1, heads=64, context=4096,
                  num_shards=4, topk=64, seed=303)
    w = make(p)
    local, counts = B.remap_topk(w.dev(w.table), p.num_shards)
    with pytest.raises(B.DcpError) as e:
        B.sparse_decode_noalloc(w.q, w.pools[0], w.scales[0], local, counts, p.sigma)
    assert e.value.status == 5
    # per-shard partials with one split need no scratch at all
    res = B.sparse_decode_noalloc(w.q, w.pools[0], w.scales[0], local, counts, p.sigma,
                                  want_partials=True, want_merged=False, num_splits=1)
    ref = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma,
                          want_partials=True, want_merged=False, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(res["o_part"], ref["o_part"]) and torch.equal(res["lse_part"], ref["lse_part"])
    assert np.isfinite(res["o_part"].cpu().numpy()).all()
