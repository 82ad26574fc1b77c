"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a swapped index, the wrong slice for the values, a weight applied
to an empty shard) fails at least one of them:

* decoders against torch's own bfloat16 / float8_e4m3fn conversions;
* remap: hand-worked fixture, exhaustive small tables checked by invariants;
* attention: scipy's softmax/logsumexp, single-token and equal-logit closed
  forms, a hand-worked two-token fixture;
* merge: sharded == unsharded, permutation and shift invariance, N = 1
  identity, the all-empty case with NaN garbage in the partials;
* dense == sparse when the table lists every local token.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from sharded_kv_sparse_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoders

def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isin(codes, oracle.E4M3_NAN_CODES)
    assert np.isnan(mine[nan]).all() and np.isnan(ref[nan]).all()
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    # a few values by the format's definition
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9
    assert mine[0x80] == 0.0 and mine[0xB8] == -1.0


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # drop inf/NaN patterns
    mine = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_fp8_dequant_matches_torch_times_scale():
    rng = np.random.default_rng(1)
    pool = rng.integers(0, 256, size=(40, 576), dtype=np.uint8)
    pool[np.isin(pool, oracle.E4M3_NAN_CODES)] = 0
    scale = np.exp2(rng.uniform(-6, 2, size=40)).astype(np.float32)
    rows = np.array([3, 0, 39, 17])
    mine = oracle.dequant_rows(pool, rows, "fp8", scale)
    ref = (torch.from_numpy(pool[rows]).view(torch.float8_e4m3fn).to(torch.float64)
           * torch.from_numpy(scale[rows]).to(torch.float64)[:, None]).numpy()
    np.testing.assert_array_equal(mine, ref)


# ---------------------------------------------------------------- remap

def test_remap_hand_worked_fixture():
    d = json.load(open(os.path.join(GOLDEN, "remap_worked_example.json")))
    local, counts = oracle.remap_topk(np.array(d["table"]), d["num_shards"])
    np.testing.assert_array_equal(local, np.array(d["local"]))
    np.testing.assert_array_equal(counts, np.array(d["counts"]))


def _check_remap_invariants(table, n, local, counts):
    rows, k = table.shape
    assert local.shape == (n, rows, k) and counts.shape == (n, rows)
    for i in range(rows):
        valid = [int(g) for g in table[i] if g >= 0]
        assert int(counts[:, i].sum()) == len(valid)
        rebuilt = []
        for r in range(n):
            c = int(counts[r, i])
            assert (local[r, i, c:] == -1).all()
            ids = [int(x) * n + r for x in local[r, i, :c]]
            assert all(g % n == r for g in ids)
            # order preserved: positions in the input row strictly increase
            where = [list(table[i]).index(g) for g in ids]
            assert where == sorted(where) and len(set(where)) == len(where)
            rebuilt += ids
        assert sorted(rebuilt) == sorted(valid)


def test_remap_exhaustive_small_tables():
    values = list(range(-1, 8))
    for n in (1, 2, 3):
        for k in (1, 2, 3):
            for row in itertools.product(values, repeat=k):
                valid = [v for v in row if v >= 0]
                if len(set(valid)) != len(valid):
                    continue
                table = np.array([row], dtype=np.int32)
                local, counts = oracle.remap_topk(table, n)
                _check_remap_invariants(table, n, local, counts)
                if n == 1:
                    assert list(local[0, 0, : counts[0, 0]]) == valid


def test_remap_random_large():
    p = wl.preset("sparse_bf16_b8_k2048")
    rng = np.random.default_rng(5)
    bt = wl.make_block_table(p, rng)
    table = wl.make_topk_table(p, bt, rng)
    local, counts = oracle.remap_topk(table, p.num_shards, p.pool_rows)
    _check_remap_invariants(table[:2], p.num_shards, local[:, :2], counts[:, :2])
    assert (counts.sum(axis=0) == 2048 - 102).all()


# ---------------------------------------------------------------- attention

def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_attend_matches_scipy_softmax_logsumexp():
    rng = np.random.default_rng(2)
    q, keys, sigma = _rand(rng, 5, 576), _rand(rng, 37, 576), 0.07
    o, lse = oracle.attend(q, keys, sigma)
    z = sigma * np.einsum("hd,nd->hn", q, keys)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=0, atol=1e-12)
    w = scipy.special.softmax(z, axis=1)
    np.testing.assert_allclose(o, w @ keys[:, :512], rtol=0, atol=1e-12)


def test_attend_single_token_returns_its_value():
    rng = np.random.default_rng(3)
    q, k, sigma = _rand(rng, 3, 576), _rand(rng, 1, 576), 0.11
    o, lse = oracle.attend(q, k, sigma)
    np.testing.assert_array_equal(o, np.repeat(k[:, :512], 3, axis=0))
    for h in range(3):
        exact = sigma * math.fsum(float(a) * float(b) for a, b in zip(q[h], k[0]))
        assert abs(lse[h] - exact) < 1e-12


def test_attend_equal_logits_give_mean_of_values():
    rng = np.random.default_rng(4)
    n = 9
    q = np.zeros((2, 576)); q[:, 512:] = _rand(rng, 2, 64)      # only RoPE dims
    keys = _rand(rng, n, 576); keys[:, 512:] = _rand(rng, 1, 64)  # shared RoPE part
    o, lse = oracle.attend(q, keys, 0.3)
    np.testing.assert_allclose(o, np.repeat(keys[:, :512].mean(axis=0, keepdims=True), 2, 0),
                               rtol=0, atol=1e-12)
    z = 0.3 * q @ keys[0]
    np.testing.assert_allclose(lse, z + math.log(n), rtol=0, atol=1e-12)


def test_attend_empty_gives_zero_and_minus_inf():
    o, lse = oracle.attend(np.ones((4, 576)), np.zeros((0, 576)), 0.1)
    assert (o == 0).all() and (lse == -np.inf).all()


def _merge_fixture():
    d = json.load(open(os.path.join(GOLDEN, "merge_worked_example.json")))
    q = np.zeros((1, 576)); q[0, d["q_nonzero"]["dim"]] = d["q_nonzero"]["value"]
    k1 = np.zeros(576); k1[:4] = d["k1"]["v_first4"]; k1[512] = d["k1"]["dim512"]
    k2 = np.zeros(576); k2[:4] = d["k2"]["v_first4"]; k2[512] = d["k2"]["dim512"]
    return d, q, k1, k2


def test_two_token_hand_worked_fixture():
    d, q, k1, k2 = _merge_fixture()
    o, lse = oracle.attend(q, np.stack([k1, k2]), math.log(3.0))
    np.testing.assert_allclose(o[0, :4], d["expected_o_first4"], rtol=0, atol=1e-14)
    assert (o[0, 4:] == 0).all()
    assert abs(lse[0] - math.log(4.0)) < 1e-14
    # the same two tokens on two shards, merged
    o1, l1 = oracle.attend(q, k1[None], math.log(3.0))
    o2, l2 = oracle.attend(q, k2[None], math.log(3.0))
    om, lm = oracle.lse_merge(np.stack([o1, o2])[:, None], np.stack([l1, l2])[:, None])
    np.testing.assert_allclose(om[0, 0, :4], d["expected_o_first4"], rtol=0, atol=1e-14)
    assert abs(lm[0, 0] - math.log(4.0)) < 1e-14


# ---------------------------------------------------------------- merge

def test_all_empty_merge_is_zero_even_with_nan_garbage():
    o_parts = np.full((3, 2, 4, 512), np.nan)
    lse_parts = np.full((3, 2, 4), -np.inf)
    o, lse = oracle.lse_merge(o_parts, lse_parts)
    assert (o == 0).all() and (lse == -np.inf).all()


def test_empty_shard_is_skipped_not_weighted():
    rng = np.random.default_rng(6)
    o_parts = _rand(rng, 3, 1, 2, 512)
    lse_parts = _rand(rng, 3, 1, 2)
    o_parts[1] = np.nan
    lse_parts[1] = -np.inf
    o, lse = oracle.lse_merge(o_parts, lse_parts)
    o_ref, lse_ref = oracle.lse_merge(o_parts[[0, 2]], lse_parts[[0, 2]])
    assert not np.isnan(o).any()
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)


def test_merge_identity_permutation_and_shift():
    rng = np.random.default_rng(7)
    o_parts, lse_parts = _rand(rng, 5, 3, 4, 512), 3 * _rand(rng, 5, 3, 4)
    o1, l1 = oracle.lse_merge(o_parts[:1], lse_parts[:1])
    np.testing.assert_array_equal(o1, o_parts[0])
    np.testing.assert_array_equal(l1, lse_parts[0])
    o, lse = oracle.lse_merge(o_parts, lse_parts)
    perm = rng.permutation(5)
    op, lp = oracle.lse_merge(o_parts[perm], lse_parts[perm])
    np.testing.assert_allclose(op, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lp, lse, rtol=0, atol=1e-13)
    os_, ls = oracle.lse_merge(o_parts, lse_parts + 2.5)
    np.testing.assert_allclose(os_, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ls, lse + 2.5, rtol=0, atol=1e-13)
    # weights follow exp(lse): a shard 40 nats above the rest dominates
    lse_dom = lse_parts.copy(); lse_dom[2] += 40.0
    od, _ = oracle.lse_merge(o_parts, lse_dom)
    np.testing.assert_allclose(od, o_parts[2], rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sharded_sparse_equals_unsharded(n, kv_dtype):
    p = wl.Preset("t", "sparse", kv_dtype, batch=5, q_per_seq=1, heads=16, context=3000,
                  num_shards=n, topk=200, pad_tail=13, seed=40 + n)
    w = wl.make_workload(p)
    q = oracle.decode_bf16(w.q_host_bits())
    pools = [w.pool_host(0, r) for r in range(n)]
    scales = [w.scale_host(0, r) for r in range(n)]
    local, counts = oracle.remap_topk(w.table, n, p.pool_rows)
    parts = [oracle.sparse_attn_shard(q, pools[r], kv_dtype, scales[r], local[r], counts[r],
                                      p.sigma) for r in range(n)]
    o, lse = oracle.lse_merge(np.stack([a for a, _ in parts]), np.stack([b for _, b in parts]))
    o_ref, lse_ref = oracle.unsharded_sparse(q, pools, kv_dtype, scales, w.table, p.sigma)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sharded_dense_equals_unsharded_with_forced_empty(kv_dtype):
    p = wl.Preset("t", "dense", kv_dtype, batch=8, q_per_seq=1, heads=16, context=700,
                  num_shards=3, forced_empty=True, seed=77)
    w = wl.make_workload(p)
    q = oracle.decode_bf16(w.q_host_bits())
    pools = [w.pool_host(0, r) for r in range(3)]
    scales = [w.scale_host(0, r) for r in range(3)]
    assert (w.local_lens == 0).any()
    parts = [oracle.dense_attn_shard(q, pools[r], kv_dtype, scales[r], w.block_table,
                                     w.local_lens[r], p.page_size, p.sigma) for r in range(3)]
    o, lse = oracle.lse_merge(np.stack([a for a, _ in parts]), np.stack([b for _, b in parts]))
    o_ref, lse_ref = oracle.unsharded_dense(q, pools, kv_dtype, scales, w.block_table,
                                            w.local_lens, p.page_size, p.sigma)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_dense_equals_sparse_over_every_local_token():
    """The block-table walk and the slot layout + remap must name the same tokens."""
    p = wl.Preset("t", "dense", "bf16", batch=3, q_per_seq=1, heads=16, context=1000,
                  num_shards=4, seed=9)
    w = wl.make_workload(p)
    q = oracle.decode_bf16(w.q_host_bits())
    k = p.context
    table = np.stack([wl.positions_to_slots(p, w.block_table, b, np.arange(p.context))
                      for b in range(p.batch)]).astype(np.int32)
    local, counts = oracle.remap_topk(table, p.num_shards, p.pool_rows)
    for r in range(p.num_shards):
        pool = w.pool_host(0, r)
        od, ld = oracle.dense_attn_shard(q, pool, "bf16", None, w.block_table,
                                         w.local_lens[r], p.page_size, p.sigma)
        os_, ls = oracle.sparse_attn_shard(q, pool, "bf16", None, local[r], counts[r], p.sigma)
        np.testing.assert_array_equal(counts[r], w.local_lens[r])
        np.testing.assert_allclose(od, os_, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ld, ls, rtol=0, atol=1e-12)
    assert k == table.shape[1]


# ---------------------------------------------------------------- input recipe

def test_preset_structure():
    p2 = wl.preset("sparse_bf16_b8_k2048")
    assert p2.pool_rows == 65536 and p2.rows == 8
    p3 = wl.preset("sparse_fp8_b64_k2048")
    assert p3.pool_rows == 2097152 and p3.lpages == 512
    p4 = wl.preset("mtp_sparse_bf16_b16x6_k2048", context=4096)
    rng = np.random.default_rng(0)
    bt = wl.make_block_table(p4, rng)
    t4 = wl.make_topk_table(p4, bt, rng)
    _, counts = oracle.remap_topk(t4, 2, p4.pool_rows)
    assert (counts[1, [6 * 1 + 0, 6 * 5 + 0]] == 0).all()      # b%4==1, j=0: shard 1 empty
    assert (counts[0, [6 * 2 + 5, 6 * 6 + 5]] == 0).all()      # b%4==2, j=5: shard 0 empty
    assert (counts[:, 6 * 15 + 3] == 0).all()                  # all-empty row
    p5 = wl.preset("dense_fp8_b32_ctx1m")
    lens = wl.make_local_lens(p5)
    assert lens[0, 0] == 0 and lens[1, 4] == 0 and lens[0, 1] == 131072
