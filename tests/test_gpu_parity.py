"""GPU parity of the HIP path against the CPU fp64 oracle, through the C ABI.

Remap: bit-exact.  Attention partials and the merged result: max |dO| <= 1e-2,
max |dLSE| <= 1e-3 (fp32 outputs), -inf matched exactly, no NaN.  Sizes span
several tiles with ragged tails; full-size workloads are checked whole (sparse)
or on sampled rows and heads (the million-token dense shard).
"""

import numpy as np
import pytest
import torch

import oracle
from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

from ._support import (assert_attn_close, check_against_oracle, gpu_dense, gpu_sparse, host_inputs,
                       make, oracle_dense, oracle_sparse, to_np)

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


# ---------------------------------------------------------------- remap

def test_remap_bit_exact_small_exhaustive(gpu):
    rng = np.random.default_rng(0)
    for n in (1, 2, 3, 4, 7, 16):
        for k in (1, 2, 5, 63, 64, 65, 300, 2048):
            rows = 5
            table = rng.integers(-1, 4 * n * 64, size=(rows, k)).astype(np.int32)
            for i in range(rows):          # make valid entries distinct
                seen = set()
                for j in range(k):
                    if table[i, j] >= 0 and table[i, j] in seen:
                        table[i, j] = -1
                    seen.add(int(table[i, j]))
            table[rows - 1] = -1           # an all-padding row
            say(f"remap n={n} k={k}")
            ref_local, ref_counts = oracle.remap_topk(table, n)
            local, counts = B.remap_topk(torch.from_numpy(table).to(gpu), n)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(local.cpu().numpy(), ref_local)
            np.testing.assert_array_equal(counts.cpu().numpy(), ref_counts)
            for s in (0, n - 1):
                l1, c1 = B.remap_topk(torch.from_numpy(table).to(gpu), n, shard=s)
                np.testing.assert_array_equal(l1.cpu().numpy()[0], ref_local[s])
                np.testing.assert_array_equal(c1.cpu().numpy()[0], ref_counts[s])


@pytest.mark.parametrize("n", [1, 3, 4])
def test_remap_bit_exact_multi_segment(gpu, n):
    # rows wider than one 2048-entry segment: the kept-entry counts of one
    # segment carry into the next, in order; rows with many, few or no kept
    # entries, and padding spread through the row
    rng = np.random.default_rng(40 + n)
    for k in (2049, 4096, 8000):
        rows = 6
        table = np.full((rows, k), -1, dtype=np.int32)
        for i in range(rows - 1):
            nv = [k, k - 1, k // 2, 3, 2048][i]
            vals = rng.choice(50 * k, size=nv, replace=False).astype(np.int32)
            pos = np.sort(rng.choice(k, size=nv, replace=False))
            table[i, pos] = vals
        if n > 1:                      # a row owned entirely by shard n - 1
            table[1] = (rng.choice(30 * k, size=k, replace=False) * n + (n - 1)).astype(np.int32)
        say(f"remap multi-segment n={n} k={k}")
        ref_local, ref_counts = oracle.remap_topk(table, n)
        local, counts = B.remap_topk(torch.from_numpy(table).to(gpu), n)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(local.cpu().numpy(), ref_local)
        np.testing.assert_array_equal(counts.cpu().numpy(), ref_counts)
        s = n - 1
        l1, c1 = B.remap_topk(torch.from_numpy(table).to(gpu), n, shard=s)
        np.testing.assert_array_equal(l1.cpu().numpy()[0], ref_local[s])
        np.testing.assert_array_equal(c1.cpu().numpy()[0], ref_counts[s])


@pytest.mark.parametrize("name", ["sparse_bf16_b8_k2048", "sparse_fp8_b64_k2048",
                                  "mtp_sparse_bf16_b16x6_k2048"])
def test_remap_bit_exact_workload_tables(gpu, name):
    p = wl.preset(name)
    rng = np.random.default_rng(p.seed)
    table = wl.make_topk_table(p, wl.make_block_table(p, rng), rng)
    say(f"remap {name}")
    ref_local, ref_counts = oracle.remap_topk(table, p.num_shards, p.pool_rows)
    t = torch.from_numpy(table).to(gpu)
    first = None
    for rep in range(3):               # repeat launches are bit-identical
        local, counts = B.remap_topk(t, p.num_shards)
        torch.cuda.synchronize()
        got = (local.cpu().numpy(), counts.cpu().numpy())
        np.testing.assert_array_equal(got[0], ref_local)
        np.testing.assert_array_equal(got[1], ref_counts)
        if first is not None:
            assert all((a == b).all() for a, b in zip(first, got))
        first = got


def test_remap_empty_rows_and_k_zero(gpu):
    say("remap rows=0 / k=0")
    t0 = torch.empty((0, 16), dtype=torch.int32, device=gpu)
    local, counts = B.remap_topk(t0, 4)
    assert local.shape == (4, 0, 16)
    t1 = torch.empty((3, 0), dtype=torch.int32, device=gpu)
    local, counts = B.remap_topk(t1, 2)
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == 0).all()


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("n,dv", [(1, 512), (2, 512), (4, 512), (8, 64), (5, 4)])
def test_lse_combine_matches_oracle(gpu, n, dv):
    rng = np.random.default_rng(n * 100 + dv)
    rows, heads = 7, 16
    o_parts = rng.standard_normal((n, rows, heads, dv)).astype(np.float32)
    lse_parts = (3 * rng.standard_normal((n, rows, heads))).astype(np.float32)
    lse_parts[:, 0, 0] = -np.inf                         # every shard empty
    if n > 1:
        lse_parts[1:, 1, :] = -np.inf                    # only shard 0 present
        lse_parts[0, 2, 3] = -np.inf                     # shard 0 empty
    o_parts[lse_parts == -np.inf] = np.nan               # garbage must never leak
    say(f"combine n={n} dv={dv}")
    o_ref, lse_ref = oracle.lse_merge(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    for out_dtype in (B.OUT_F32, B.OUT_BF16):
        o, lse = B.lse_combine(torch.from_numpy(o_parts).to(gpu), torch.from_numpy(lse_parts).to(gpu),
                               out_dtype=out_dtype)
        torch.cuda.synchronize()
        rel = 2.0 ** -8 if out_dtype == B.OUT_BF16 else 0.0
        assert_attn_close(to_np(o), to_np(lse), o_ref, lse_ref, f"combine n={n}", o_tol=1e-5,
                          lse_tol=1e-5, o_rel=rel)


# ---------------------------------------------------------------- sparse decode

SPARSE_SMALL = [
    # (kv, heads, shards, topk, context, pad, rows)
    ("bf16", 64, 4, 300, 5000, 7, 3),
    ("fp8", 64, 4, 300, 5000, 7, 3),
    ("fp8", 32, 2, 257, 3000, 0, 4),
    ("bf16", 32, 2, 257, 3000, 0, 4),
    ("fp8", 16, 3, 130, 2000, 3, 2),
    ("bf16", 16, 1, 200, 2000, 0, 2),
    ("fp8", 128, 2, 190, 4000, 11, 2),
    ("bf16", 128, 4, 190, 4000, 0, 2),
    # head counts that are not a multiple of 64: the last head block's waves
    # past the last head load no query and store nothing
    ("fp8", 48, 2, 300, 4000, 5, 3),
    ("bf16", 48, 3, 250, 3000, 0, 2),
    ("fp8", 80, 4, 260, 5000, 9, 2),
    ("bf16", 96, 2, 190, 3000, 4, 2),
    ("fp8", 112, 3, 333, 4000, 0, 2),
    ("bf16", 112, 1, 200, 2000, 2, 1),
]


@pytest.mark.parametrize("kv,heads,n,k,ctx,pad,rows", SPARSE_SMALL)
def test_sparse_decode_small(gpu, kv, heads, n, k, ctx, pad, rows):
    p = wl.Preset("t", "sparse", kv, batch=rows, q_per_seq=1, heads=heads, context=ctx,
                  num_shards=n, topk=k, pad_tail=pad, seed=heads * 7 + n * 3 + k)
    w = make(p)
    say(f"sparse small {kv} H={heads} N={n} k={k}")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    ref = oracle_sparse(w)
    np.testing.assert_array_equal(res["counts"].cpu().numpy(), ref["counts"])
    check_against_oracle(res, ref, f"sparse {kv} H={heads} N={n}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 2, 3, 5])
def test_sparse_decode_splits(gpu, kv, splits):
    p = wl.Preset("t", "sparse", kv, batch=3, q_per_seq=1, heads=64, context=6000, num_shards=2,
                  topk=700, pad_tail=5, seed=splits)
    w = make(p)
    say(f"sparse splits={splits} {kv}")
    res = gpu_sparse(w, num_splits=splits)
    torch.cuda.synchronize()
    check_against_oracle(res, oracle_sparse(w), f"splits={splits}")


@pytest.mark.parametrize("kv,splits", [("fp8", 8), ("fp8", 12), ("fp8", 20), ("fp8", 24), ("fp8", 25),
                                       ("fp8", 32), ("bf16", 32)])
def test_sparse_decode_many_partials(gpu, kv, splits):
    # 16, 24, 40, 48, 50 or 64 partials per row (2 shards x splits): the
    # merge's wide load groups (16 or 32 members per pass, several groups),
    # two rounds of LSE loads, abandon bits above bit 31 of the arrival word
    # (40 and 48 members merging in parallel, 48 the most that have abandon
    # bits), rows merged by their last block alone (50 and 64 partials), and
    # empty splits; merged and per-shard outputs within tolerance
    p = wl.Preset("t", "sparse", kv, batch=2, q_per_seq=1, heads=64, context=40000, num_shards=2,
                  topk=8000, pad_tail=300, seed=60 + splits)
    w = make(p)
    say(f"sparse {kv} splits={splits} ({2 * splits} partials per row)")
    res = gpu_sparse(w, num_splits=splits)
    torch.cuda.synchronize()
    ref = oracle_sparse(w)
    np.testing.assert_array_equal(res["local"].cpu().numpy(), ref["local"])    # k = 8000: 4 segments
    np.testing.assert_array_equal(res["counts"].cpu().numpy(), ref["counts"])
    check_against_oracle(res, ref, f"{kv} splits={splits}")


@pytest.mark.parametrize("kv,heads", [("fp8", 64), ("fp8", 128), ("bf16", 64), ("bf16", 32)])
def test_sparse_decode_short_rows(gpu, kv, heads):
    """Rows with 1..16 selected slots and many heads (a case another stack's
    sparse kernel got wrong for short FP8 rows with more than 32 heads)."""
    p = wl.Preset("t", "sparse", kv, batch=6, q_per_seq=1, heads=heads, context=4000,
                  num_shards=4, topk=64, short_rows=16, seed=heads + 1)
    w = make(p)
    say(f"sparse short rows {kv} H={heads}")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    ref = oracle_sparse(w)
    assert (ref["counts"] == 0).any()          # some shard owns nothing on some row
    check_against_oracle(res, ref, f"short rows {kv} H={heads}")


def test_sparse_all_empty_rows(gpu):
    p = wl.Preset("t", "sparse", "fp8", batch=3, q_per_seq=1, heads=64, context=1000,
                  num_shards=2, topk=32, pad_tail=32, seed=3)
    w = make(p)
    say("sparse all-empty")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    assert (to_np(res["o"]) == 0).all() and (to_np(res["lse"]) == -np.inf).all()
    assert (to_np(res["o_part"]) == 0).all()


@pytest.mark.parametrize("heads", [16, 32])
def test_fp8_large_token_scales(gpu, heads):
    # Tokens with scales 2^9 .. 2^11 and codes of magnitude 0 or 2^-9 (their
    # values, at most 4, and the logits stay moderate): P' = p * scale reaches
    # 2^19, beyond fp16, so the 16/32-head kernel must scale P' per head before
    # converting it to fp16.  Partials and the merge within tolerance of the
    # oracle.  (The kernel for 48 heads or more has no fp16 P': it splits P' into E4M3
    # terms at a power of two per head, whose 17 binades cover the P' that
    # carry the output as long as a token's scale is not thousands of times
    # what its codes need, which this construction is on purpose.)
    p = wl.Preset("t", "sparse", "fp8", batch=3, q_per_seq=1, heads=heads, context=3000,
                  num_shards=2, topk=300, seed=70 + heads)
    w = make(p)
    rng = np.random.default_rng(80 + heads)
    local, counts = oracle.remap_topk(w.table, p.num_shards, p.pool_rows)
    for r in range(p.num_shards):
        used = np.unique(np.concatenate([local[r, i, :counts[r, i]] for i in range(p.rows)]))
        big = rng.choice(used, size=min(40, used.size), replace=False)
        idx = torch.from_numpy(big.astype(np.int64)).to(gpu)
        w.pools[0][r][idx] = w.pools[0][r][idx] & 0x81      # codes 0 and +-2^-9
        s = w.scales_host[0][r].copy()
        s[big] = np.exp2(rng.integers(9, 12, size=big.size)).astype(np.float32)
        w.scales_host[0][r] = s
        w.scales[0][r].copy_(torch.from_numpy(s).to(gpu))
    say(f"sparse fp8 large token scales H={heads}")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    check_against_oracle(res, oracle_sparse(w), f"large scales H={heads}")


@pytest.mark.parametrize("name", ["sparse_bf16_b8_k2048", "sparse_fp8_b64_k2048",
                                  "mtp_sparse_bf16_b16x6_k2048"])
def test_sparse_decode_full_workload(gpu, name):
    p = wl.preset(name)
    say(f"sparse full {name}: generating")
    w = make(p)
    say(f"sparse full {name}: gpu")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    say(f"sparse full {name}: oracle")
    ref = oracle_sparse(w)
    np.testing.assert_array_equal(res["local"].cpu().numpy(), ref["local"])
    np.testing.assert_array_equal(res["counts"].cpu().numpy(), ref["counts"])
    err = check_against_oracle(res, ref, name)
    say(f"{name}: {err}")


def test_fused_equals_unfused_and_counters_reset(gpu):
    p = wl.preset("sparse_fp8_b64_k2048", batch=8, context=16384)
    w = make(p)
    say("fused vs unfused")
    table = w.dev(w.table)
    local, counts = B.remap_topk(table, p.num_shards)
    nb = B.workspace_size(False, p.rows, p.heads, p.num_shards, p.topk, want_merged=True,
                          want_partials=False, num_splits=2)
    ws = B.alloc_workspace(nb, gpu)
    a = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma, num_splits=2,
                        workspace=ws)
    b = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma, num_splits=2,
                        workspace=ws)                       # counters must have reset
    parts = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma, num_splits=2,
                            want_partials=True, want_merged=False)
    o_c, lse_c = B.lse_combine(parts["o_part"], parts["lse_part"])
    torch.cuda.synchronize()
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])
    hb = (p.heads + 63) // 64
    # arrival words (64 bits, the first of two per (row, head block)): count
    # and abandon bits clear after every call, the generation byte moved on
    words = ws[: 16 * p.rows * hb].view(torch.int64).view(p.rows * hb, 2)[:, 0].cpu().numpy()
    assert ((words.astype(np.uint64) & np.uint64((1 << 56) - 1)) == 0).all()
    assert (words.astype(np.uint64) >> np.uint64(56) == 2).all()      # two fused calls
    # The fused merge exchanges the partials as fp16 with a power of two per
    # (partial, head) that puts the head's largest magnitude in [2^14, 2^15):
    # every value is off by at most 2^-11 of its head's largest partial value
    # (the merge weights sum to 1); the LSEs are exchanged in fp32.
    bound = 2.0 ** -11 * float(parts["o_part"].abs().max()) + 1e-5
    np.testing.assert_allclose(to_np(a["o"]), to_np(o_c), rtol=0, atol=bound)
    np.testing.assert_allclose(to_np(a["lse"]), to_np(lse_c), rtol=0, atol=1e-5)
    check_against_oracle(a, oracle_sparse(w), "fused")


@pytest.mark.parametrize("name", ["sparse_fp8_b64_k2048", "sparse_bf16_b8_k2048"])
def test_fused_merge_modes_agree(gpu, name):
    # The row's blocks share the merge (bounded wait), give up at once (1 us),
    # or never wait (the last block merges everything): bit-identical results,
    # arrival counts and flags clear after every call (the generation byte
    # advancing by one per call), and within tolerance of the oracle.
    p = wl.preset(name)
    w = make(p)
    table = w.dev(w.table)
    local, counts = B.remap_topk(table, p.num_shards)
    nb = B.workspace_size(False, p.rows, p.heads, p.num_shards, p.topk, want_merged=True,
                          want_partials=False)
    ws = B.alloc_workspace(nb, gpu)
    hb = (p.heads + 63) // 64
    res = {}
    for call, us in enumerate(["30", "1", "0", "30"]):
        say(f"merge wait {us} us")
        B.set_merge_wait_us(int(us))
        try:
            r = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma, workspace=ws)
            torch.cuda.synchronize()
        finally:
            B.set_merge_wait_us(30)
        words = ws[: 16 * p.rows * hb].view(torch.int64).view(p.rows * hb, 2)[:, 0].cpu().numpy()
        assert ((words.astype(np.uint64) & np.uint64((1 << 56) - 1)) == 0).all()
        assert (words.astype(np.uint64) >> np.uint64(56) == call + 1).all()
        if us in res:
            assert torch.equal(r["o"], res[us]["o"]) and torch.equal(r["lse"], res[us]["lse"])
        res[us] = r
    for us in ["1", "0"]:
        assert torch.equal(res[us]["o"], res["30"]["o"]) and torch.equal(res[us]["lse"], res["30"]["lse"])
    check_against_oracle(res["30"], oracle_sparse(w), f"{name} fused")


def test_bf16_output(gpu):
    p = wl.Preset("t", "sparse", "fp8", batch=4, q_per_seq=1, heads=64, context=8000,
                  num_shards=4, topk=512, seed=11)
    w = make(p)
    say("bf16 output")
    res = gpu_sparse(w, want_partials=False, out_dtype=B.OUT_BF16)
    torch.cuda.synchronize()
    assert res["o"].dtype == torch.bfloat16
    check_against_oracle(res, oracle_sparse(w), "bf16 out")


# ---------------------------------------------------------------- dense decode

DENSE_SMALL = [
    # (kv, heads, shards, context, page, rows, forced_empty)
    ("bf16", 16, 2, 256, 64, 1, False),
    ("fp8", 64, 4, 3001, 64, 3, False),
    ("bf16", 64, 3, 2500, 16, 2, True),
    ("fp8", 128, 8, 5000, 64, 4, True),
    ("fp8", 32, 2, 777, 128, 3, False),
    ("bf16", 32, 1, 1000, 64, 2, False),
    ("fp8", 48, 2, 1500, 64, 2, True),
    ("bf16", 80, 3, 1200, 64, 2, False),
    ("fp8", 96, 4, 2100, 16, 2, False),
    ("fp8", 112, 2, 900, 64, 3, False),
]


@pytest.mark.parametrize("kv,heads,n,ctx,page,rows,empty", DENSE_SMALL)
def test_dense_decode_small(gpu, kv, heads, n, ctx, page, rows, empty):
    p = wl.Preset("t", "dense", kv, batch=rows, q_per_seq=1, heads=heads, context=ctx,
                  num_shards=n, page_size=page, forced_empty=empty, seed=ctx + heads)
    w = make(p)
    say(f"dense small {kv} H={heads} N={n} ctx={ctx} page={page}")
    res = gpu_dense(w)
    torch.cuda.synchronize()
    check_against_oracle(res, oracle_dense(w), f"dense {kv} H={heads} N={n}")


def test_dense_tiny_workload(gpu):
    w = make(wl.preset("tiny_dense_bf16_ctx256"))
    say("dense tiny preset")
    res = gpu_dense(w)
    torch.cuda.synchronize()
    ref = oracle_dense(w)
    check_against_oracle(res, ref, "tiny dense")
    q, pools, scales = host_inputs(w)
    o_u, lse_u = oracle.unsharded_dense(q, pools, "bf16", scales, w.block_table, w.local_lens,
                                        w.p.page_size, w.p.sigma)
    assert_attn_close(to_np(res["o"]), to_np(res["lse"]), o_u, lse_u, "tiny dense vs unsharded")


def test_dense_equals_sparse_on_gpu(gpu):
    """Dense over every local token == sparse with a table listing them all."""
    p = wl.Preset("t", "dense", "fp8", batch=2, q_per_seq=1, heads=64, context=1500,
                  num_shards=2, seed=5)
    w = make(p)
    say("dense == sparse")
    dres = gpu_dense(w, want_partials=True)
    table = np.stack([wl.positions_to_slots(p, w.block_table, b, np.arange(p.context))
                      for b in range(p.batch)]).astype(np.int32)
    local, counts = B.remap_topk(torch.from_numpy(table).to(gpu), p.num_shards)
    sres = B.sparse_decode(w.q, w.pools[0], w.scales[0], local, counts, p.sigma,
                           want_partials=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(dres["lse"]), to_np(sres["lse"]), rtol=0, atol=1e-4)
    np.testing.assert_allclose(to_np(dres["o"]), to_np(sres["o"]), rtol=0, atol=2e-3)


def test_dense_million_token_sampled(gpu):
    p = wl.preset("dense_fp8_b32_ctx1m")
    say("dense 1M: generating")
    w = make(p)
    say("dense 1M: gpu")
    res = gpu_dense(w, want_partials=False)
    torch.cuda.synchronize()
    rows = [0, 1, 4, 31]                    # rows 0 and 4 have a forced-empty shard
    heads = list(range(0, 8)) + list(range(120, 128))
    say("dense 1M: host copies")
    host = host_inputs(w)
    say("dense 1M: oracle on sampled rows/heads")
    ref = oracle_dense(w, rows=rows, heads=heads, host=host)
    err = check_against_oracle(res, ref, "dense 1M", rows=rows, heads=heads)
    say(f"dense 1M: {err}")


@pytest.mark.parametrize("kv,heads", [("fp8", 64), ("fp8", 128), ("fp8", 32), ("bf16", 64)])
def test_strided_pool_layout_is_bit_identical(gpu, kv, heads):
    # The same codes and scales in packed rows (+ a scale array) and in padded
    # rows with the scale inside (FP8: 640-byte rows, scale at byte 576; BF16:
    # 1280-byte rows): identical outputs, partials and LSEs, and both within
    # tolerance of the oracle.
    p = wl.Preset("layout", "sparse", kv, batch=6, q_per_seq=1, heads=heads, context=9000,
                  num_shards=4, topk=700, pad_tail=13, seed=31)
    w = make(p)
    packed = gpu_sparse(w)
    pools, scales = [], []
    for r in range(p.num_shards):
        src = w.pools[0][r]
        rb = 640 if kv == "fp8" else 1280
        buf = torch.zeros((src.shape[0], rb), dtype=torch.uint8, device=gpu)
        if kv == "fp8":
            buf[:, :576] = src
            sc = buf.view(torch.float32)[:, 144]
            sc.copy_(w.scales[0][r])
            pools.append(buf[:, :576])
            scales.append(sc)
        else:
            bv = buf.view(torch.bfloat16)
            bv[:, :576] = src
            pools.append(bv[:, :576])
            scales.append(None)
    assert pools[0].stride(0) * pools[0].element_size() == (640 if kv == "fp8" else 1280)
    local, counts = B.remap_topk(w.dev(w.table), p.num_shards)
    say(f"strided layout {kv} heads={heads}")
    strided = B.sparse_decode(w.q, pools, scales, local, counts, p.sigma, want_partials=True,
                              want_merged=True)
    torch.cuda.synchronize()
    for key in ("o", "lse", "o_part", "lse_part"):
        assert torch.equal(packed[key], strided[key]), key
    check_against_oracle(strided, oracle_sparse(w), f"strided {kv} {heads}")


def test_inline_scale_workload_layout(gpu):
    # The workload generator's 640-byte-row layout (scale inside the row) at a
    # few-tile size: pool and scale are strided views of one buffer, and the
    # result matches the oracle on the same values.
    p = wl.Preset("inline", "sparse", "fp8", batch=5, q_per_seq=1, heads=64, context=12000,
                  num_shards=4, topk=900, pad_tail=40, seed=37, row_bytes=640)
    w = make(p)
    assert w.pools[0][0].stride(0) == 640 and w.scales[0][0].stride(0) == 160
    assert w.pools[0][0].data_ptr() + 576 == w.scales[0][0].data_ptr()
    say("inline-scale workload")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    check_against_oracle(res, oracle_sparse(w), "inline scale")


# ---------------------------------------------------------------- KV write

def _kv_write_case(gpu, n, kv, rows, tokens, seed, row_bytes=0):
    rng = np.random.default_rng(seed)
    pools, scales = [], []
    for r in range(n):
        if kv == "bf16":
            pools.append(torch.randn((rows, 576), device=gpu).to(torch.bfloat16))
            scales.append(None)
        elif row_bytes:
            buf = torch.randint(0, 0x7F, (rows, row_bytes), dtype=torch.uint8, device=gpu)
            sc = buf.view(torch.float32)[:, 144]
            sc.copy_(torch.rand(rows, device=gpu) + 0.5)
            pools.append(buf[:, :576])
            scales.append(sc)
        else:
            pools.append(torch.randint(0, 0x7F, (rows, 576), dtype=torch.uint8, device=gpu))
            scales.append(torch.rand(rows, device=gpu) + 0.5)
    slots = rng.choice(n * rows, size=tokens, replace=False).astype(np.int32)
    slots[rng.random(tokens) < 0.1] = -1                   # skipped tokens
    slots[0] = n * rows + 3                               # beyond every pool: skipped
    mag = np.exp2(rng.uniform(-8, 8, size=(tokens, 1)))
    x = rng.normal(0, 1, size=(tokens, 576)) * mag
    x[1] = 0.0                                            # an all-zero token
    x[2, :] = 0.0
    x[2, 7] = -3.0e-3                                     # one value: codes 0 except +-448
    kv_new = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(gpu)
    host_p = [p.cpu().contiguous() for p in pools]
    host_p = [p.view(torch.int16).numpy().view(np.uint16) if kv == "bf16" else p.numpy() for p in host_p]
    host_s = [None if s is None else s.cpu().contiguous().numpy() for s in scales]
    bits = kv_new.cpu().view(torch.int16).numpy().view(np.uint16)
    ref_p, ref_s = oracle.kv_write(bits, np.where(slots >= n * rows, -1, slots), n, host_p, host_s, kv)
    say(f"kv write n={n} {kv} rows={rows} tokens={tokens} row_bytes={row_bytes}")
    B.kv_write(kv_new, torch.from_numpy(slots).to(gpu), pools, scales)
    torch.cuda.synchronize()
    for r in range(n):
        got = pools[r].cpu().contiguous()
        got = got.view(torch.int16).numpy().view(np.uint16) if kv == "bf16" else got.numpy()
        np.testing.assert_array_equal(got, ref_p[r])
        if kv == "fp8":
            np.testing.assert_array_equal(scales[r].cpu().numpy().view(np.uint32),
                                          ref_s[r].view(np.uint32))


@pytest.mark.parametrize("n", [1, 2, 4, 8])
@pytest.mark.parametrize("kv,row_bytes", [("fp8", 0), ("fp8", 640), ("bf16", 0)])
def test_kv_write_bit_exact(gpu, n, kv, row_bytes):
    # every pool byte and every scale bit equal to the oracle's, skipped and
    # out-of-pool slots leave the pools untouched
    _kv_write_case(gpu, n, kv, rows=700, tokens=900 if n > 1 else 500, seed=40 + n,
                   row_bytes=row_bytes)


def test_kv_write_headline_shape(gpu):
    # one new token per row of the 64-row FP8 workload, into its 4 pools of
    # 2M rows: the written rows equal the oracle's quantisation, sampled other
    # rows are untouched, and the sparse decode of a table that selects the new
    # tokens matches the oracle on the written values
    p = wl.preset("sparse_fp8_b64_k2048")
    w = make(p)
    n, rows = p.num_shards, p.pool_rows
    rng = np.random.default_rng(7)
    pos = p.context - 1
    slots = np.array([wl.positions_to_slots(p, w.block_table, b, np.array([pos]))[0]
                      for b in range(p.batch)], dtype=np.int32)
    kv_new = (torch.randn((p.batch, 576), device=gpu) * 2.0).to(torch.bfloat16)
    sample = rng.integers(0, rows, 256)
    before = [(w.pools[0][r][sample].cpu(), w.scales[0][r][sample].cpu()) for r in range(n)]
    say("kv write headline shape")
    B.kv_write(kv_new, torch.from_numpy(slots).to(gpu), w.pools[0], w.scales[0])
    torch.cuda.synchronize()
    bits = kv_new.cpu().view(torch.int16).numpy().view(np.uint16)
    touched = set()
    for i, g in enumerate(slots):
        r, row = int(g) % n, int(g) // n
        touched.add((r, row))
        codes, sc = oracle.quantize_row_e4m3(bits[i])
        np.testing.assert_array_equal(w.pools[0][r][row].cpu().numpy(), codes)
        assert w.scales[0][r][row].item() == float(sc)
    for r in range(n):
        keep = np.array([(r, int(s)) not in touched for s in sample])
        np.testing.assert_array_equal(w.pools[0][r][sample].cpu().numpy()[keep], before[r][0].numpy()[keep])
        np.testing.assert_array_equal(w.scales[0][r][sample].cpu().numpy()[keep], before[r][1].numpy()[keep])
    # the decode reads what was written: each row's new slot joins its table
    # (in column 0 unless the row already selects it), and the oracle sees
    # the new scales
    table = w.table.copy()
    for b in range(p.batch):
        if slots[b] not in table[b]:
            table[b, 0] = slots[b]
    w.table = table
    for r in range(n):
        w.scales_host[0][r] = w.scales[0][r].cpu().numpy()
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    check_against_oracle(res, oracle_sparse(w), "decode after kv write")


@pytest.mark.parametrize("golden", ["kv_write_worked_example.json", "kv_write_product_vs_division.json"])
def test_kv_write_hand_worked_example(gpu, golden):
    # the kernel's codes and scale equal the ones derived by hand in
    # tests/golden (exact products, ties to even, subnormals; a token whose
    # scale is not a power of two, where the product by the inverse scale is
    # a tie that dividing by the scale would not give), written to slot 5 of
    # a 2-shard FP8 pool (shard 1, row 2)
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", golden)) as f:
        ex = json.load(f)
    x = torch.zeros((1, 576), dtype=torch.float32)
    x[0, :len(ex["values"])] = torch.tensor(ex["values"])
    pools = [torch.full((4, 576), 0x55, dtype=torch.uint8, device=gpu) for _ in range(2)]
    scales = [torch.ones(4, dtype=torch.float32, device=gpu) for _ in range(2)]
    say("kv write hand-worked example")
    B.kv_write(x.to(torch.bfloat16).to(gpu), torch.tensor([5], dtype=torch.int32, device=gpu), pools, scales)
    torch.cuda.synchronize()
    row = pools[1][2].cpu().numpy()
    np.testing.assert_array_equal(row[:len(ex["codes"])], np.array(ex["codes"], dtype=np.uint8))
    assert (row[len(ex["codes"]):] == ex["rest_code"]).all()
    assert format(int(scales[1][2].cpu().numpy().view(np.uint32)), "08x") == ex["scale_bits_hex"]
    assert (pools[0].cpu().numpy() == 0x55).all() and (pools[1][[0, 1, 3]].cpu().numpy() == 0x55).all()


@pytest.mark.parametrize("kind,heads,splits", [("sparse", 64, 0), ("sparse", 128, 0), ("sparse", 64, 2),
                                               ("dense", 64, 0), ("dense", 128, 0)])
def test_fp8_lead_short_tile(gpu, kind, heads, splits):
    # rows whose token counts leave 1..64 tokens past whole 128-token tiles
    # (the short tile then runs first: 1..32 tokens on the one-MFMA PV path,
    # 33..64 on the two-MFMA one), with 32 / 33 / 64 / 65 / whole-tile
    # boundaries
    lens = [129, 150, 160, 161, 192, 193, 256, 257, 288, 289, 320, 321, 449, 512]
    if kind == "sparse":
        p = wl.Preset("t", "sparse", "fp8", batch=len(lens), q_per_seq=1, heads=heads, context=4000,
                      num_shards=1, topk=max(lens), seed=71 + heads)
        w = make(p)
        table = w.table.copy()
        for i, n in enumerate(lens):
            table[i, n:] = -1
        w.table = table
        say(f"fp8 lead tile sparse H={heads} splits={splits}")
        res = gpu_sparse(w, num_splits=splits)
        torch.cuda.synchronize()
        ref = oracle_sparse(w)
        np.testing.assert_array_equal(res["counts"].cpu().numpy()[0], np.array(lens))
    else:
        p = wl.Preset("t", "dense", "fp8", batch=len(lens), q_per_seq=1, heads=heads, context=1024,
                      num_shards=1, seed=73 + heads)
        w = make(p)
        w.local_lens = np.array([lens], dtype=np.int32)
        say(f"fp8 lead tile dense H={heads}")
        res = gpu_dense(w, num_splits=splits)
        torch.cuda.synchronize()
        ref = oracle_dense(w)
    check_against_oracle(res, ref, f"lead tile {kind} H={heads}")


@pytest.mark.parametrize("kv,heads,n", [("fp8", 64, 16), ("fp8", 128, 16), ("bf16", 64, 16),
                                        ("fp8", 32, 16), ("fp8", 64, 1), ("bf16", 16, 1)])
def test_sparse_decode_shard_count_extremes(gpu, kv, heads, n):
    # the largest shard count the library takes (16: 16 partials per row, the
    # own-part merge off) and a single shard (the merge is the identity)
    p = wl.Preset("t", "sparse", kv, batch=3, q_per_seq=1, heads=heads, context=20000,
                  num_shards=n, topk=1500, pad_tail=30, seed=80 + n + heads)
    w = make(p)
    say(f"sparse {kv} H={heads} N={n}")
    res = gpu_sparse(w)
    torch.cuda.synchronize()
    ref = oracle_sparse(w)
    np.testing.assert_array_equal(res["counts"].cpu().numpy(), ref["counts"])
    check_against_oracle(res, ref, f"{kv} H={heads} N={n}")
