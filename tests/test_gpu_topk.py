"""GPU parity of the sharded index cache and distributed top-k against the CPU
oracle, through the C ABI.

* Scores: within a bound derived from fp32 arithmetic of the exact (fp64)
  oracle scores.
* Selection (local top-k, merge): bit-exact -- scores, positions and slots --
  on score lists drawn by the input generator (many ties), where the order
  (score descending, then position ascending) is unique.
* The whole path (scores -> local top-k -> merge -> remap): the chosen set is
  valid for the exact scores (nothing left out beats anything taken, beyond
  the scores' error bound), the output is in order of the kernel's own
  scores, the slots follow the positions, and the remap of the result is
  bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _host_scores_and_bound(w):
    """Exact scores of every local token of every (shard, row) and the bound
    on an fp32 computation of them: the 128-term dot products (relative
    error of their absolute sums), the weighted sum over heads and the final
    product, each at most (terms + 2) * 2^-24 of the absolute terms."""
    p = w.p
    q = w.q.cpu().numpy()
    wv = w.w.cpu().numpy().astype(np.float64)
    keys = [k.cpu().numpy() for k in w.keys]
    ex, bound = [], []
    qv = oracle.decode_e4m3fn(q)                        # [rows, hi, 128]
    u = 2.0 ** -24
    for r in range(p.num_shards):
        ex_r, b_r = [], []
        for b in range(p.rows):
            n = int(w.local_lens[r][b])
            rows = oracle.dense_local_rows(w.block_table[b], n, p.page_size)
            s = oracle.index_scores(q[b], w.w.cpu().numpy()[b], keys[r][rows], w.scales_host[r][rows])
            kv = oracle.decode_e4m3fn(keys[r][rows])   # [n, 128]
            absdot = np.abs(kv) @ np.abs(qv[b]).T       # [n, hi]
            sc = w.scales_host[r][rows].astype(np.float64)
            dot_err = (128 + 2) * u * absdot
            bnd = sc * ((np.abs(wv[b]) * (dot_err + (p.index_heads + 2) * u * absdot)).sum(axis=1)) \
                + 4 * u * np.abs(s)
            ex_r.append(s)
            b_r.append(bnd)
        ex.append(ex_r)
        bound.append(b_r)
    return ex, bound


INDEX_SMALL = [
    wl.IndexPreset("t1", batch=3, context=3000, num_shards=3, index_heads=16, topk=512, seed=31),
    wl.IndexPreset("t2", batch=4, context=5000, num_shards=4, index_heads=64, topk=256, seed=32),
    wl.IndexPreset("t3", batch=2, context=2500, num_shards=2, index_heads=128, topk=256, seed=33),
    wl.IndexPreset("t4", batch=5, context=700, num_shards=1, index_heads=32, topk=512, seed=34),
]


def _run_scores(w):
    p = w.p
    lens = [w.dev(w.local_lens[r]) for r in range(p.num_shards)]
    bt = w.dev(w.block_table)
    scores = B.index_score(w.q, w.w, w.keys, w.scales, lens, bt, p.page_size, p.max_local)
    torch.cuda.synchronize()
    return scores, bt


@pytest.mark.parametrize("p", INDEX_SMALL, ids=[p.name for p in INDEX_SMALL])
def test_index_scores_within_bound(gpu, p):
    w = wl.make_index_workload(p, device="cuda", empty_shard_rows=True)
    say(f"index scores {p.name}: {p.rows} rows, {p.num_shards} shards, {p.index_heads} heads")
    scores, _ = _run_scores(w)
    ex, bound = _host_scores_and_bound(w)
    got = scores.cpu().numpy().astype(np.float64)
    worst = 0.0
    for r in range(p.num_shards):
        for b in range(p.rows):
            n = int(w.local_lens[r][b])
            d = np.abs(got[r, b, :n] - ex[r][b])
            assert (d <= bound[r][b]).all(), (r, b, float((d - bound[r][b]).max()))
            if n:
                worst = max(worst, float((d / np.maximum(bound[r][b], 1e-30)).max()))
    say(f"{p.name}: largest error / bound = {worst:.3f}")


def _tied_scores(rng, n_lists, max_local):
    """Scores with many exact ties (multiples of 1/4 in [-8, 8]) and a few
    large values, fp32."""
    s = rng.integers(-32, 33, (n_lists, max_local)).astype(np.float32) / 4
    s[rng.random(s.shape) < 0.01] = np.float32(1e30)
    s[rng.random(s.shape) < 0.01] = np.float32(-0.0)
    return s


@pytest.mark.parametrize("n,rows,max_local,k", [(3, 4, 900, 512), (4, 2, 5000, 128), (1, 3, 100, 512),
                                                (2, 3, 4096, 2048), (8, 1, 300, 64)])
def test_topk_local_bit_exact(gpu, n, rows, max_local, k):
    rng = np.random.default_rng(n * 100 + k)
    s = _tied_scores(rng, n * rows, max_local).reshape(n, rows, max_local)
    lens = rng.integers(0, max_local + 1, (n, rows)).astype(np.int32)
    lens[0, 0] = 0                              # an empty shard
    lens[-1, -1] = max_local                    # a full one
    say(f"topk local n={n} rows={rows} L={max_local} k={k}")
    cs, cp = B.topk_local(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), k)
    torch.cuda.synchronize()
    cs, cp = cs.cpu().numpy(), cp.cpu().numpy()
    for r in range(n):
        for b in range(rows):
            m = int(lens[r, b])
            pos = np.arange(m) * n + r
            sel = oracle.topk_order(s[r, b, :m].astype(np.float64), pos, k)
            np.testing.assert_array_equal(cp[r, b, :len(sel)], pos[sel])
            np.testing.assert_array_equal(cs[r, b, :len(sel)], s[r, b, :m][sel])
            assert (cp[r, b, len(sel):] == -1).all() and (cs[r, b, len(sel):] == -np.inf).all()


@pytest.mark.parametrize("n,rows,k", [(2, 3, 256), (4, 2, 128), (1, 2, 512), (4, 3, 2048), (8, 2, 64)])
def test_topk_merge_bit_exact(gpu, n, rows, k):
    rng = np.random.default_rng(n * 10 + k)
    page = 4
    lpages = 40
    bt = np.stack([rng.permutation(rows * lpages)[:lpages] for _ in range(rows)]).astype(np.int32)
    cs = np.full((n, rows, k), -np.inf, dtype=np.float32)
    cp = np.full((n, rows, k), -1, dtype=np.int32)
    ref = []
    for b in range(rows):
        c_s, c_p = [], []
        for r in range(n):
            m = int(rng.integers(0, min(k, page * lpages) + 1)) if (r + b) % 3 else k
            m = min(m, page * lpages)
            loc = rng.choice(page * lpages, size=m, replace=False)
            pos = loc * n + r
            sc = rng.integers(-16, 17, m).astype(np.float32) / 2
            order = oracle.topk_order(sc.astype(np.float64), pos, k)
            cs[r, b, :m], cp[r, b, :m] = sc[order], pos[order]
            c_s.append(sc[order])
            c_p.append(pos[order])
        ms, mp = oracle.merge_topk(c_s, c_p, k)
        ref.append((ms, mp, oracle.positions_to_slots(bt[b], n, page, mp)))
    say(f"topk merge n={n} rows={rows} k={k}")
    ts, tp, tg = B.topk_merge(torch.from_numpy(cs).cuda(), torch.from_numpy(cp).cuda(),
                              torch.from_numpy(bt).cuda(), page)
    torch.cuda.synchronize()
    ts, tp, tg = ts.cpu().numpy(), tp.cpu().numpy(), tg.cpu().numpy()
    for b, (ms, mp, mg) in enumerate(ref):
        m = len(mp)
        np.testing.assert_array_equal(tp[b, :m], mp)
        np.testing.assert_array_equal(ts[b, :m], ms)
        np.testing.assert_array_equal(tg[b, :m], mg)
        assert (tp[b, m:] == -1).all() and (tg[b, m:] == -1).all()


def test_topk_merge_rejects_width_not_multiple_of_512(gpu):
    cs = torch.zeros((3, 2, 100), dtype=torch.float32, device="cuda")
    cp = torch.zeros((3, 2, 100), dtype=torch.int32, device="cuda")
    bt = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(B.DcpError) as e:
        B.topk_merge(cs, cp, bt, 64)
    assert e.value.status == 2


def _check_selection(w, scores_gpu, ts, tp, tg, k, what):
    """The whole path's result against the exact scores (see module doc)."""
    p = w.p
    n = p.num_shards
    ex, bound = _host_scores_and_bound(w)
    for b in range(p.rows):
        # every position's exact score and bound, by position t = j * N + r
        total = int(sum(w.local_lens[r][b] for r in range(n)))
        s_ex = np.full(p.context, np.nan)
        s_bd = np.zeros(p.context)
        for r in range(n):
            m = int(w.local_lens[r][b])
            s_ex[np.arange(m) * n + r] = ex[r][b]
            s_bd[np.arange(m) * n + r] = bound[r][b]
        m = min(k, total)
        chosen = tp[b, :m]
        assert (chosen >= 0).all() and len(np.unique(chosen)) == m, what
        assert (tp[b, m:] == -1).all() and (tg[b, m:] == -1).all(), what
        have = np.isfinite(s_ex)
        assert have[chosen].all(), f"{what}: a chosen position is not a local token"
        rest = np.setdiff1d(np.nonzero(have)[0], chosen)
        if rest.size:
            worst_in = (s_ex[chosen] + s_bd[chosen]).min()
            best_out = (s_ex[rest] - s_bd[rest]).max()
            assert worst_in >= best_out, f"{what} row {b}: {worst_in} < {best_out}"
        # the output is in order of the kernel's own scores, which are its
        # score buffer's values at those positions
        g = np.array([scores_gpu[t % n, b, t // n] for t in chosen], dtype=np.float32)
        np.testing.assert_array_equal(ts[b, :m], g)
        want = sorted(range(m), key=lambda i: (-float(g[i]), int(chosen[i])))
        assert want == list(range(m)), f"{what} row {b}: output not in selection order"
        np.testing.assert_array_equal(tg[b, :m], oracle.positions_to_slots(w.block_table[b], n,
                                                                           p.page_size, chosen))


@pytest.mark.parametrize("p", INDEX_SMALL, ids=[p.name for p in INDEX_SMALL])
def test_distributed_topk_end_to_end(gpu, p):
    w = wl.make_index_workload(p, device="cuda", empty_shard_rows=True)
    say(f"distributed top-k {p.name}")
    scores, bt = _run_scores(w)
    lens = w.dev(w.local_lens)
    cs, cp = B.topk_local(scores, lens, p.topk)
    ts, tp, tg = B.topk_merge(cs, cp, bt, p.page_size)
    local, counts = B.remap_topk(tg, p.num_shards)
    torch.cuda.synchronize()
    tg_h = tg.cpu().numpy()
    _check_selection(w, scores.cpu().numpy(), ts.cpu().numpy(), tp.cpu().numpy(), tg_h, p.topk, p.name)
    ref_local, ref_counts = oracle.remap_topk(tg_h, p.num_shards)
    np.testing.assert_array_equal(local.cpu().numpy(), ref_local)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_counts)


def test_distributed_topk_workload_sampled(gpu):
    # the benchmark's shape (64 rows, 128K context over 4 shards, 64 index
    # heads, top-k 2048): every row computed, 3 rows checked as above
    p = wl.INDEX_PRESETS["index_topk_b64_ctx128k_k2048"]
    w = wl.make_index_workload(p, device="cuda")
    say("distributed top-k workload: gpu")
    scores, bt = _run_scores(w)
    cs, cp = B.topk_local(scores, w.dev(w.local_lens), p.topk)
    ts, tp, tg = B.topk_merge(cs, cp, bt, p.page_size)
    torch.cuda.synchronize()
    rows = [0, 31, 63]
    sub = wl.IndexWorkload(p=wl.IndexPreset("s", batch=len(rows), context=p.context,
                                            num_shards=p.num_shards, index_heads=p.index_heads,
                                            topk=p.topk, page_size=p.page_size),
                           block_table=w.block_table[rows], local_lens=w.local_lens[:, rows],
                           q=w.q[rows], w=w.w[rows], keys=w.keys, scales=w.scales,
                           scales_host=w.scales_host, device="cuda")
    say("distributed top-k workload: oracle on 3 rows")
    _check_selection(sub, scores.cpu().numpy()[:, rows], ts.cpu().numpy()[rows], tp.cpu().numpy()[rows],
                     tg.cpu().numpy()[rows], p.topk, "workload")
