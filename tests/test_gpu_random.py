"""GPU parity on seeded random configurations: head count, shard count,
splits, KV dtype and layout, page size, row lengths and output options drawn
together (and, for the prefill chunk attention, token count, head count and
chunk length), so that combinations the fixed cases do not name are checked.
Same bar as the fixed cases: remap bit-exact, max |dO| <= 1e-2 and max |dLSE|
<= 1e-3 against the fp64 oracle, -inf matched exactly, no NaN.
"""

import numpy as np
import pytest
import torch

import oracle
from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

from ._support import (assert_attn_close, check_against_oracle, gpu_dense, gpu_sparse, make, oracle_dense,
                       oracle_sparse, to_np)
from .test_gpu_prefix import _chunk, _chunk_host


def draw_case(seed):
    """One configuration: (preset, num_splits, want_partials, want_merged, out_dtype)."""
    rng = np.random.default_rng(seed)
    kind = "sparse" if rng.random() < 0.6 else "dense"
    kv = "fp8" if rng.random() < 0.55 else "bf16"
    heads = int(rng.integers(1, 9)) * 16
    n = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    batch = int(rng.integers(1, 5))
    row_bytes = 640 if kv == "fp8" and rng.random() < 0.25 else 0
    if kind == "sparse":
        q_per_seq = 3 if rng.random() < 0.3 else 1
        context = int(rng.integers(300, 6000))
        topk = int(rng.integers(1, min(context - q_per_seq, 1500) + 1))
        pad = int(rng.integers(0, topk // 4 + 1))
        short = int(rng.integers(1, 17)) if rng.random() < 0.15 else 0
        p = wl.Preset(f"rand{seed}", "sparse", kv, batch=batch, q_per_seq=q_per_seq, heads=heads,
                      context=context, num_shards=n, topk=topk, pad_tail=pad,
                      causal=q_per_seq > 1, short_rows=short, row_bytes=row_bytes, seed=seed)
    else:
        page = int(rng.choice([16, 32, 64, 128]))
        context = int(rng.integers(1, 4000))
        p = wl.Preset(f"rand{seed}", "dense", kv, batch=batch, q_per_seq=1, heads=heads,
                      context=context, num_shards=n, page_size=page,
                      forced_empty=bool(rng.random() < 0.4), row_bytes=row_bytes, seed=seed)
    splits = 0 if rng.random() < 0.5 else int(rng.integers(1, max(1, min(8, 64 // n)) + 1))
    want_partials = bool(rng.random() < 0.6)
    want_merged = (not want_partials) or bool(rng.random() < 0.7)
    out_dtype = B.OUT_BF16 if want_merged and rng.random() < 0.3 else B.OUT_F32
    return p, splits, want_partials, want_merged, out_dtype


SEEDS = list(range(9001, 9201))


def test_random_cases_are_varied():
    # the draw covers both kinds, both KV dtypes and several head / shard counts
    cases = [draw_case(s) for s in SEEDS]
    assert {c[0].kind for c in cases} == {"sparse", "dense"}
    assert {c[0].kv_dtype for c in cases} == {"bf16", "fp8"}
    assert len({c[0].heads for c in cases}) >= 5
    assert len({c[0].num_shards for c in cases}) >= 4


@pytest.mark.gpu
@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(gpu, seed):
    p, splits, want_partials, want_merged, out_dtype = draw_case(seed)
    print(f"[gpu-case] random seed={seed} {p.kind} {p.kv_dtype} H={p.heads} N={p.num_shards} "
          f"rows={p.rows} ctx={p.context} k={p.topk} page={p.page_size} splits={splits} "
          f"row_bytes={p.row_bytes} partials={want_partials} merged={want_merged} "
          f"out={'bf16' if out_dtype == B.OUT_BF16 else 'f32'}", flush=True)
    w = make(p)
    if p.kind == "sparse":
        res = gpu_sparse(w, want_partials=want_partials, want_merged=want_merged, num_splits=splits,
                         out_dtype=out_dtype)
        torch.cuda.synchronize()
        ref = oracle_sparse(w)
        np.testing.assert_array_equal(res["local"].cpu().numpy(), ref["local"])
        np.testing.assert_array_equal(res["counts"].cpu().numpy(), ref["counts"])
    else:
        res = gpu_dense(w, want_partials=want_partials, want_merged=want_merged, num_splits=splits,
                        out_dtype=out_dtype)
        torch.cuda.synchronize()
        ref = oracle_dense(w)
    assert ("o_part" in res) == want_partials and ("o" in res) == want_merged
    check_against_oracle(res, ref, f"random seed={seed}")


PREFILL_SEEDS = list(range(9101, 9151))


@pytest.mark.gpu
@pytest.mark.parametrize("seed", PREFILL_SEEDS)
def test_random_prefill_chunk(gpu, seed):
    rng = np.random.default_rng(seed)
    kv = "fp8" if rng.random() < 0.5 else "bf16"
    heads = int(rng.integers(1, 9)) * 16
    tokens = int(rng.integers(1, 81))
    c = int(rng.integers(0, 3001))
    print(f"[gpu-case] random prefill seed={seed} {kv} H={heads} T={tokens} C={c}", flush=True)
    rows, sc = _chunk(kv, c, seed=seed)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 500000)        # independent of the chunk's draw
    q = torch.randn((tokens, heads, 576), generator=gen, device="cuda").to(torch.bfloat16)
    o, lse = B.prefill_chunk_attention(q, rows, sc, 1.0 / np.sqrt(192.0))
    torch.cuda.synchronize()
    hr, hs = _chunk_host(kv, rows, sc)
    qh = oracle.decode_bf16(q.cpu().view(torch.int16).numpy().view(np.uint16))
    o_ref, lse_ref = oracle.prefix_chunk_attention(qh, hr, hs, kv, 1.0 / np.sqrt(192.0))
    assert_attn_close(to_np(o), to_np(lse), o_ref, lse_ref, f"random prefill seed={seed}")
