"""Pins of the oracle's prefill over a cached prefix (CPU only): the gather's
addressing stated by hand and checked against the decode oracle's per-shard
paging (two independently written formulas), chunked attention with a
running merge equal to one attention over the whole prefix (and to the
unsharded dense oracle), the merge's identities, and the bfloat16 rounding
of the running output against torch's conversion and hand-worked ties."""

import numpy as np
import torch

import oracle

SIGMA = 1.0 / np.sqrt(192.0)


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


# (N, page, block table row, position) -> (shard, row), worked by hand: the
# logical page of position t is t div (page * N); g = BT[page] * page * N +
# t mod (page * N); the shard is g mod N and the row g div N.
HAND_SLOTS = {
    (2, 4, (3, 1), 5): (1, 14),      # g = 3 * 8 + 5 = 29
    (2, 4, (3, 1), 9): (1, 4),       # page 1 -> BT 1: g = 8 + 1 = 9
    (2, 4, (3, 1), 8): (0, 4),       # g = 8
    (4, 2, (2, 0), 3): (3, 4),       # g = 2 * 8 + 3 = 19
    (4, 2, (2, 0), 12): (0, 1),      # page 1 -> BT 0: g = 12 - 8 = 4
    (1, 64, (5, 7), 70): (0, 454),   # g = 7 * 64 + 6
}


def test_prefix_slot_hand_stated():
    for (n, page, bt, t), (r, row) in HAND_SLOTS.items():
        g = oracle.prefix_slot(np.array(bt), n, page, t)
        assert (g % n, g // n) == (r, row), (n, page, bt, t)


def _cache(rng, n, page, lpages, kv):
    pool_rows = lpages * page * 3
    bt = rng.permutation(pool_rows // page)[:lpages].astype(np.int32)
    if kv == "bf16":
        pools = [bf16_bits(rng.normal(0, 1, (pool_rows, 576))) for _ in range(n)]
        scales = [None] * n
    else:
        pools = [rng.integers(0, 0x7F, (pool_rows, 576)).astype(np.uint8) for _ in range(n)]
        scales = [np.exp2(rng.uniform(-6, 2, pool_rows)).astype(np.float32) for _ in range(n)]
    return bt, pools, scales


def test_gather_matches_decode_paging():
    # position t is local token t div N of shard t mod N, and the decode
    # oracle finds local token j at row BT[j div page] * page + j mod page
    rng = np.random.default_rng(3)
    for n, page in ((1, 4), (2, 4), (3, 2), (4, 8)):
        bt, pools, scales = _cache(rng, n, page, 5, "fp8")
        length = 5 * page * n
        rows, sc = oracle.gather_prefix(bt, n, page, pools, scales, "fp8", 0, length)
        for t in range(length):
            r, j = t % n, t // n
            prow = oracle.dense_local_rows(bt, j + 1, page)[j]
            np.testing.assert_array_equal(rows[t], pools[r][prow])
            assert sc[t] == scales[r][prow]
        # a window in the middle is the same rows
        w_rows, w_sc = oracle.gather_prefix(bt, n, page, pools, scales, "fp8", 3, length - 5)
        np.testing.assert_array_equal(w_rows, rows[3:length - 2])
        np.testing.assert_array_equal(w_sc, sc[3:length - 2])


def test_chunked_prefix_equals_whole_prefix():
    # attention over the prefix in chunks, merged as it goes, equals one
    # attention over the whole prefix, and the unsharded dense oracle
    rng = np.random.default_rng(4)
    for kv in ("bf16", "fp8"):
        n, page, lpages = 3, 4, 6
        bt, pools, scales = _cache(rng, n, page, lpages, kv)
        prefix = page * n * lpages - 5
        q = oracle.decode_bf16(bf16_bits(rng.normal(0, 1, (3, 4, 576))))     # 3 new tokens x 4 heads
        o_acc = np.zeros((3, 4, 512))
        lse_acc = np.full((3, 4), -np.inf)
        for b in range(0, prefix, 17):
            ln = min(17, prefix - b)
            rows, sc = oracle.gather_prefix(bt, n, page, pools, scales, kv, b, ln)
            o_c, lse_c = oracle.prefix_chunk_attention(q, rows, sc, kv, SIGMA)
            o_acc, lse_acc = oracle.merge_running(o_acc, lse_acc, o_c, lse_c)
        rows, sc = oracle.gather_prefix(bt, n, page, pools, scales, kv, 0, prefix)
        o_w, lse_w = oracle.prefix_chunk_attention(q, rows, sc, kv, SIGMA)
        np.testing.assert_allclose(o_acc, o_w, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse_acc, lse_w, rtol=0, atol=1e-12)
        lens = np.array([[max(0, -(-(prefix - r) // n))] for r in range(n)], dtype=np.int32)
        for t in range(3):
            o_d, lse_d = oracle.unsharded_dense(q[t:t + 1], pools, kv, scales, bt[None, :], lens,
                                                page, SIGMA)
            np.testing.assert_allclose(o_acc[t], o_d[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse_acc[t], lse_d[0], rtol=0, atol=1e-12)


def test_chunk_attention_single_token_and_empty():
    rng = np.random.default_rng(5)
    q = oracle.decode_bf16(bf16_bits(rng.normal(0, 1, (2, 3, 576))))
    rows = bf16_bits(rng.normal(0, 1, (1, 576)))
    o, lse = oracle.prefix_chunk_attention(q, rows, None, "bf16", SIGMA)
    v = oracle.decode_bf16(rows[0])
    np.testing.assert_array_equal(o, np.broadcast_to(v[:512], (2, 3, 512)))
    np.testing.assert_allclose(lse, SIGMA * (q @ v), rtol=0, atol=1e-12)
    o, lse = oracle.prefix_chunk_attention(q, rows[:0], None, "bf16", SIGMA)
    assert (o == 0).all() and (lse == -np.inf).all()


def test_merge_running_identities():
    rng = np.random.default_rng(6)
    o1, l1 = rng.normal(0, 1, (2, 3, 8)), rng.normal(0, 2, (2, 3))
    o2, l2 = rng.normal(0, 1, (2, 3, 8)), rng.normal(0, 2, (2, 3))
    empty_o, empty_l = np.full((2, 3, 8), np.nan), np.full((2, 3), -np.inf)
    o, lse = oracle.merge_running(empty_o, empty_l, o2, l2)          # first chunk: taken as is
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-15)
    o, lse = oracle.merge_running(o1, l1, empty_o, empty_l)          # empty chunk: no change
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)
    o, lse = oracle.merge_running(empty_o, empty_l, empty_o, empty_l)
    assert (o == 0).all() and (lse == -np.inf).all()
    # two chunks: weights e^l1, e^l2 (closed form)
    o, lse = oracle.merge_running(o1, l1, o2, l2)
    w1, w2 = np.exp(l1), np.exp(l2)
    np.testing.assert_allclose(o, (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None],
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(w1 + w2), rtol=0, atol=1e-12)
    # BF16 storage rounds the merged output, not the LSE
    ob, lseb = oracle.merge_running(o1, l1, o2, l2, store_bf16=True)
    np.testing.assert_array_equal(ob, oracle.round_bf16(o))
    np.testing.assert_array_equal(lseb, lse)


def test_round_bf16():
    # torch's float32 -> bfloat16 conversion (a library routine, used only as
    # a check) on values exact in float32, where it rounds once
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e3, 2000),
                        rng.normal(0, 1e-3, 2000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), ref)
    # ties to even, worked by hand: bfloat16 keeps 7 fraction bits
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0                      # tie, 1.0 is even
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6      # tie, up to even
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(-2.5 - 2.0 ** -7) == -2.5                    # tie at 2^1: step 2^-6
