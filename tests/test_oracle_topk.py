"""Pins of the oracle's sharded index scoring and distributed top-k (CPU
only): a score worked by hand from the E4M3FN codes, a selection worked by
hand with ties (score descending, then position ascending), the sharded
selection (local top-k per shard, then the merge) equal to one selection over
every position of the sequence by brute force, with forced ties, and the
selection order against Python's own sort."""

import numpy as np
import pytest

import oracle

ONE, TWO, HALF, M_ONE, M_TWO = 0x38, 0x40, 0x30, 0xB8, 0xC0    # E4M3FN: 1.0, 2.0, 0.5, -1.0, -2.0


def test_index_score_hand_worked():
    # two index heads; head 0: q = (1, 2, 0, ...), head 1: q = (-1, 0, ...)
    q = np.zeros((2, 128), dtype=np.uint8)
    q[0, 0], q[0, 1], q[1, 0] = ONE, TWO, M_ONE
    w = np.array([0.5, 3.0], dtype=np.float32)
    keys = np.zeros((2, 128), dtype=np.uint8)
    keys[0, 0], keys[0, 1] = TWO, HALF      # dots: 1*2 + 2*0.5 = 3 and -2 -> ReLU 0
    keys[1, 0] = M_TWO                      # dots: -2 -> 0 and (-1)(-2) = 2
    s = np.array([0.25, 0.125], dtype=np.float32)
    got = oracle.index_scores(q, w, keys, s)
    # token 0: 0.25 * (0.5 * 3 + 3.0 * 0) = 0.375; token 1: 0.125 * (0.5 * 0 + 3.0 * 2) = 0.75
    np.testing.assert_array_equal(got, [0.375, 0.75])


def test_selection_hand_worked_with_ties():
    # positions 0..7 over 2 shards (even positions on shard 0), scores with a
    # three-way tie at 2.0: the order is 3.0 (4), then 2.0 at positions 1, 2, 6
    scores = np.array([0.5, 2.0, 2.0, -1.0, 3.0, 0.5, 2.0, 0.0])
    pos = np.arange(8)
    assert oracle.topk_order(scores, pos, 4).tolist() == [4, 1, 2, 6]
    assert oracle.topk_order(scores, pos, 3).tolist() == [4, 1, 2]
    cs, cp = [], []
    for r in range(2):
        mine = pos[pos % 2 == r]
        sel = oracle.topk_order(scores[mine], mine, 4)
        cs.append(scores[mine][sel])
        cp.append(mine[sel])
    assert cp[0].tolist() == [4, 2, 6, 0] and cp[1].tolist() == [1, 5, 7, 3]
    s, p = oracle.merge_topk(cs, cp, 4)
    assert p.tolist() == [4, 1, 2, 6] and s.tolist() == [3.0, 2.0, 2.0, 2.0]
    s, p = oracle.merge_topk(cs, cp, 20)                    # fewer than k: everything, in order
    assert p.tolist() == [4, 1, 2, 6, 0, 5, 7, 3]


def test_selection_order_against_python_sort():
    rng = np.random.default_rng(3)
    scores = rng.integers(-3, 4, 300).astype(np.float64) / 2         # many ties
    pos = rng.permutation(1000)[:300]
    for k in (1, 7, 100, 300, 400):
        want = sorted(range(300), key=lambda i: (-scores[i], pos[i]))[:k]
        assert oracle.topk_order(scores, pos, k).tolist() == want


def _index_cache(rng, n, page, lpages, dup=0):
    pool_rows = lpages * page * 2
    bt = rng.permutation(pool_rows // page)[:lpages].astype(np.int32)
    pools = [np.where(rng.random((pool_rows, 128)) < 0.1, 0,
                      rng.integers(0, 0x7F, (pool_rows, 128))).astype(np.uint8) for _ in range(n)]
    scales = [np.exp2(rng.uniform(-6, 2, pool_rows)).astype(np.float32) for _ in range(n)]
    for _ in range(dup):                      # equal keys and scales on other shards: equal scores
        src, dst = rng.integers(0, n), rng.integers(0, n)
        a, b = rng.integers(0, pool_rows, 2)
        pools[dst][b] = pools[src][a]
        scales[dst][b] = scales[src][a]
    return bt, pools, scales


@pytest.mark.parametrize("n", [3, 1, 2, 4])
def test_sharded_topk_equals_unsharded(n):
    rng = np.random.default_rng(10 + n)
    page, lpages = 4, 7
    bt, pools, scales = _index_cache(rng, n, page, lpages, dup=40)
    context = page * n * lpages - 3
    lens = [max(0, -(-(context - r) // n)) for r in range(n)]
    q = rng.integers(0, 0xFF, (6, 128)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0                                 # no NaN codes
    w = rng.normal(0, 1, 6).astype(np.float32)
    for k in (1, 5, 40, context + 10):
        s1, p1, g1 = oracle.sharded_topk(q, w, pools, scales, bt, lens, page, k)
        s2, p2, g2 = oracle.unsharded_topk(q, w, pools, scales, bt, context, page, k)
        np.testing.assert_array_equal(p1, p2)
        np.testing.assert_array_equal(s1, s2)
        np.testing.assert_array_equal(g1, g2)
        assert len(p1) == min(k, context)
    # the copied keys made equal scores, which the order resolves by position
    s_all, _, _ = oracle.unsharded_topk(q, w, pools, scales, bt, context, page, context)
    assert len(np.unique(s_all)) < len(s_all)
