"""GPU parity of the prefill path over a cached prefix against the CPU oracle,
through the C ABI: the gather bit-exact, the per-chunk attention and the
running merge within tolerance, and the whole chunked prefill against one
attention over the prefix."""

import numpy as np
import pytest
import torch

import oracle
from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

from ._support import assert_attn_close, record_margins, to_np

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _cache(kv, n, batch, context, seed, row_bytes=0):
    p = wl.Preset("t", "dense", kv, batch=batch, q_per_seq=1, heads=16, context=context,
                  num_shards=n, seed=seed, row_bytes=row_bytes)
    return wl.make_workload(p, device="cuda")


@pytest.mark.parametrize("kv,n,row_bytes", [("fp8", 1, 0), ("fp8", 2, 0), ("fp8", 4, 0),
                                            ("fp8", 4, 640), ("bf16", 3, 0), ("bf16", 4, 0)])
def test_gather_bit_exact(gpu, kv, n, row_bytes):
    w = _cache(kv, n, batch=4, context=3000, seed=200 + n, row_bytes=row_bytes)
    p = w.p
    begins = [0, 17, 5, 2500]
    lengths = [300, 1, 0, 500]
    say(f"gather {kv} N={n} row_bytes={row_bytes}")
    bt = w.dev(w.block_table)
    rows, sc = B.gather_prefix(bt, w.pools[0], w.scales[0], p.page_size, begins, lengths)
    torch.cuda.synchronize()
    pools = [w.pool_host(0, r) for r in range(n)]
    scales = [w.scale_host(0, r) for r in range(n)]
    got = rows.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if kv == "bf16" else got.numpy()
    off = 0
    for b, (beg, ln) in enumerate(zip(begins, lengths)):
        ref_rows, ref_sc = oracle.gather_prefix(w.block_table[b], n, p.page_size, pools, scales, kv,
                                                beg, ln)
        np.testing.assert_array_equal(got[off:off + ln], ref_rows)
        if kv == "fp8":
            np.testing.assert_array_equal(sc.cpu().numpy()[off:off + ln], ref_sc)
        off += ln


def _chunk(kv, c, seed):
    """A chunk buffer as the gather leaves it (drawn directly)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn((max(c, 1), 576), generator=gen, device="cuda")
    if kv == "bf16":
        return x.to(torch.bfloat16)[:c], None
    rng = np.random.default_rng(seed)
    sc = torch.from_numpy(np.exp2(rng.uniform(-6, 2, max(c, 1))).astype(np.float32)).cuda()
    return x.to(torch.float8_e4m3fn).view(torch.uint8)[:c], sc[:c]


def _chunk_host(kv, rows, sc):
    if kv == "bf16":
        return rows.cpu().view(torch.int16).numpy().view(np.uint16), None
    return rows.cpu().numpy(), sc.cpu().numpy()


CHUNK_CASES = [
    # (kv, heads, tokens, chunk_len)
    ("fp8", 16, 37, 1000), ("fp8", 32, 33, 700), ("fp8", 64, 9, 1300), ("fp8", 128, 5, 900),
    ("bf16", 16, 37, 1000), ("bf16", 32, 20, 333), ("bf16", 64, 8, 700), ("bf16", 128, 3, 260),
    ("fp8", 16, 64, 1), ("fp8", 16, 8, 0), ("bf16", 32, 6, 0), ("fp8", 16, 3, 5000),
    # (token, head) queries left over after the rows of 64: 16, 32, 48 and 48
    ("fp8", 48, 7, 900), ("bf16", 96, 5, 500), ("fp8", 80, 3, 1100), ("bf16", 112, 1, 300),
]


@pytest.mark.parametrize("kv,heads,tokens,c", CHUNK_CASES)
def test_prefill_chunk_attention(gpu, kv, heads, tokens, c):
    rows, sc = _chunk(kv, c, seed=heads * 31 + tokens + c)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(tokens * 7 + heads)
    q = torch.randn((tokens, heads, 576), generator=gen, device="cuda").to(torch.bfloat16)
    say(f"prefill chunk {kv} H={heads} T={tokens} C={c}")
    o, lse = B.prefill_chunk_attention(q, rows, sc, 1.0 / np.sqrt(192.0))
    torch.cuda.synchronize()
    hr, hs = _chunk_host(kv, rows, sc)
    qh = oracle.decode_bf16(q.cpu().view(torch.int16).numpy().view(np.uint16))
    o_ref, lse_ref = oracle.prefix_chunk_attention(qh, hr, hs, kv, 1.0 / np.sqrt(192.0))
    m = assert_attn_close(to_np(o), to_np(lse), o_ref, lse_ref, f"prefill chunk {kv} H={heads} C={c}")
    record_margins(f"prefill chunk {kv} H={heads} T={tokens} C={c}", {"chunk": m})


@pytest.mark.parametrize("acc", ["f32", "bf16"])
def test_merge_into(gpu, acc):
    rng = np.random.default_rng(9 if acc == "f32" else 10)
    rows, heads, dv = 5, 16, 512
    o_a = rng.normal(0, 2, (rows, heads, dv)).astype(np.float32)
    l_a = rng.normal(0, 3, (rows, heads)).astype(np.float32)
    o_n = rng.normal(0, 2, (rows, heads, dv)).astype(np.float32)
    l_n = rng.normal(0, 3, (rows, heads)).astype(np.float32)
    l_a[0, :4] = -np.inf                      # accumulator empty (first chunk)
    l_n[1, :4] = -np.inf                      # empty chunk
    l_a[2, 0] = l_n[2, 0] = -np.inf           # both empty
    o_a[l_a == -np.inf] = np.nan              # never read
    o_n[l_n == -np.inf] = np.nan
    dt = torch.float32 if acc == "f32" else torch.bfloat16
    oa = torch.from_numpy(o_a).to(dt).cuda()
    oa_host = oa.float().cpu().numpy().astype(np.float64)        # the accumulator as stored
    la = torch.from_numpy(l_a).cuda()
    say(f"merge into {acc}")
    B.merge_into(oa, la, torch.from_numpy(o_n).cuda(), torch.from_numpy(l_n).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge_running(oa_host, l_a.astype(np.float64), o_n.astype(np.float64),
                                        l_n.astype(np.float64), store_bf16=acc == "bf16")
    # bfloat16 storage: the kernel rounds its fp32 merge, the oracle its fp64
    # one, so near a rounding boundary the two may land one bfloat16 step
    # (2^-7 of the value) apart
    rel = 2.0 ** -7 if acc == "bf16" else 0.0
    assert_attn_close(to_np(oa), to_np(la), o_ref, l_ref, f"merge into {acc}", o_tol=1e-5,
                      lse_tol=1e-5, o_rel=rel)


def _prefill_case(p):
    pw = wl.make_prefill_workload(p, device="cuda")
    w = pw.cache
    return pw, w


SMALL_PREFILL = [
    wl.PrefillPreset("t1", "fp8", batch=2, heads=16, prefix=3000, new_tokens=37, num_shards=3,
                     chunk=1000, seed=121),
    wl.PrefillPreset("t2", "bf16", batch=1, heads=32, prefix=2100, new_tokens=16, num_shards=4,
                     chunk=512, seed=122),
    wl.PrefillPreset("t3", "fp8", batch=1, heads=64, prefix=700, new_tokens=5, num_shards=2,
                     chunk=4096, seed=123),
]


@pytest.mark.parametrize("p", SMALL_PREFILL, ids=[p.name for p in SMALL_PREFILL])
@pytest.mark.parametrize("acc", ["f32", "bf16"])
def test_chunked_prefill_matches_whole_prefix(gpu, p, acc):
    pw, w = _prefill_case(p)
    pools = [w.pool_host(0, r) for r in range(p.num_shards)]
    scales = [w.scale_host(0, r) for r in range(p.num_shards)]
    dt = torch.float32 if acc == "f32" else torch.bfloat16
    for b in range(p.batch):
        say(f"chunked prefill {p.name} acc={acc} seq {b}")
        o, lse = B.prefix_attention(pw.q[b], w.dev(w.block_table[b]), w.pools[0], w.scales[0],
                                    p.page_size, p.prefix, p.chunk, p.sigma, acc_dtype=dt)
        torch.cuda.synchronize()
        qh = oracle.decode_bf16(pw.q[b].cpu().view(torch.int16).numpy().view(np.uint16))
        if acc == "f32":
            rows, sc = oracle.gather_prefix(w.block_table[b], p.num_shards, p.page_size, pools, scales,
                                            p.kv_dtype, 0, p.prefix)
            o_ref, lse_ref = oracle.prefix_chunk_attention(qh, rows, sc, p.kv_dtype, p.sigma)
            rel = 0.0
        else:
            # the oracle's own chunk chain, its running output rounded to bfloat16 after every merge
            o_ref = np.zeros(qh.shape[:2] + (512,))
            lse_ref = np.full(qh.shape[:2], -np.inf)
            vmax = np.zeros_like(o_ref)
            for beg, ln in wl.prefix_chunks(p):
                rows, sc = oracle.gather_prefix(w.block_table[b], p.num_shards, p.page_size, pools,
                                                scales, p.kv_dtype, beg, ln)
                o_c, l_c = oracle.prefix_chunk_attention(qh, rows, sc, p.kv_dtype, p.sigma)
                o_ref, lse_ref = oracle.merge_running(o_ref, lse_ref, o_c, l_c, store_bf16=True)
                vmax = np.maximum(vmax, np.abs(o_ref))
            # every stored merge rounds the running value on each side (at most
            # 2^-8 of it), and later merges carry those roundings on with
            # weights <= 1: the two chains may differ by up to 2^-7 of the
            # largest running value per merge, on top of the kernels' own error
            bound = 1e-2 + len(wl.prefix_chunks(p)) * 2.0 ** -7 * vmax
            d = np.abs(to_np(o) - o_ref)
            assert (d <= bound).all(), f"{p.name} bf16 seq {b}: max excess {float((d - bound).max()):.3e}"
            rel = 0.0
            o_ref = to_np(o)                 # the O check is done; the LSE check follows
        m = assert_attn_close(to_np(o), to_np(lse), o_ref, lse_ref, f"{p.name} {acc} seq {b}",
                              o_rel=rel)
        record_margins(f"chunked prefill {p.name} acc={acc} seq {b}", {"merged": m})


def test_prefill_workload_sampled(gpu):
    # the benchmark's prefill (2,048 new tokens over a 16K prefix, 4 shards,
    # FP8, chunks of 4,096): every chunk run on the GPU, checked on 24 sampled
    # tokens against one attention over the whole prefix
    p = wl.PREFILL_PRESETS["prefill_fp8_prefix16k_new2k"]
    pw, w = _prefill_case(p)
    say("prefill workload: gpu")
    o, lse = B.prefix_attention(pw.q[0], w.dev(w.block_table[0]), w.pools[0], w.scales[0],
                                p.page_size, p.prefix, p.chunk, p.sigma)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.sort(np.concatenate([[0, p.new_tokens - 1], rng.choice(p.new_tokens, 22, replace=False)]))
    say("prefill workload: oracle")
    pools = [w.pool_host(0, r) for r in range(p.num_shards)]
    scales = [w.scale_host(0, r) for r in range(p.num_shards)]
    rows, sc = oracle.gather_prefix(w.block_table[0], p.num_shards, p.page_size, pools, scales,
                                    p.kv_dtype, 0, p.prefix)
    qh = oracle.decode_bf16(pw.q[0].cpu().view(torch.int16).numpy().view(np.uint16))[toks]
    o_ref, lse_ref = oracle.prefix_chunk_attention(qh, rows, sc, p.kv_dtype, p.sigma)
    m = assert_attn_close(to_np(o)[toks], to_np(lse)[toks], o_ref, lse_ref, "prefill workload")
    record_margins("prefill_fp8_prefix16k_new2k (24 sampled tokens)", {"merged": m})
