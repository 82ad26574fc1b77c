#!/usr/bin/env python3
"""Benchmark of the DCP decode hot path on one MI355X.

A step is one pass of the whole path over one batch: the index remap of a
top-k table shared by four consecutive layers, then the fused sparse MLA
decode (all shards + LSE merge) for each of those four layers, each layer with
its own KV cache.  The reported value is microseconds per layer-step
(= step time / 4).  Layers rotate over 16 distinct KV caches (4 table groups x
4 layers, 1.2 GB touched per cycle) so the 256 MB last-level cache cannot hold
a layer between its uses: the KV is read from HBM.

Output: one JSON line (rank 0), plus a roofline figure for the decode kernel
(algorithmic bytes per launch / average launch time from HIP events recorded
on the launch stream), the interleaved FP8 KV-cache write timed after the
decode loop (one decode step of new tokens, and a chunk of up to 2048 tokens
per sequence), and the CPU fp64 oracle timed on the host as a baseline.
"""

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8
ROOT = os.path.dirname(os.path.abspath(__file__))


def source_digest():
    """sha256 over the kernel sources (sorted by path): a traffic figure
    measured on other sources is stale."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "sharded_kv_sparse_amd", "csrc", "*")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by what
    the counter reads for a copy of known size), or None when there is no
    summary or it was taken on different sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_digest():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def decode_kernel_name(p):
    if p.kv_dtype == "fp8" and p.heads >= 48:
        return "decode_fp8_kernel"
    return "decode_kernel"
METRIC = "µs/layer-step and KV HBM GB/s (% of peak), sparse MLA decode B=64 top-k 2048"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="sparse_fp8_b64_k2048", choices=sorted(wl.PRESETS))
    ap.add_argument("--groups", type=int, default=4, help="table groups (4 layers each) rotated")
    ap.add_argument("--layers-per-table", type=int, default=4)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--launch", choices=["graph", "stream"], default="stream",
                    help="stream: every launch issued from the host, back to back; graph: each "
                         "step's launches captured once in a HIP graph and replayed (decode steps "
                         "run under graphs on the pages' systems; here a replayed step measured "
                         "about 6 us slower than the same launches issued from the host)")
    ap.add_argument("--min-warmup-s", type=float, default=2.0,
                    help="keep warming up (whole steps) until this much wall time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the timings of the prefill and of the distributed top-k")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the CPU-baseline sample (0 = all rows of one layer-step)")
    ap.add_argument("--out", default="", help="also write the JSON line to this file")
    ap.add_argument("--print-digest", action="store_true",
                    help="print the digest of the kernel sources that traffic figures are keyed on")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size: each launch reads and writes exactly 1 GiB."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}))


def algorithmic_bytes(w, layer_counts):
    """Bytes a decode launch must move: KV rows read once, query, slot ids,
    counts, merged output and LSE."""
    p = w.p
    per_token = 580 if p.kv_dtype == "fp8" else 1152
    kv = int(layer_counts) * per_token
    q = p.rows * p.heads * 576 * 2
    out = p.rows * p.heads * (512 * 4 + 4)
    ids = int(layer_counts) * 4 + p.num_shards * p.rows * 4 if p.kind == "sparse" else 0
    return kv, kv + q + out + ids


def flops(p, tokens):
    return 2.0 * p.heads * tokens * (576 + 512)


def fp8_kernel_mfma(p, w, splits):
    """MFMAs the FP8 decode kernel (48 to 128 heads) executes for one launch.

    Per wave (16 heads) and 128-token tile: 8 S tiles x (4 latent k-steps x 2
    query terms + 1 RoPE k-step) + 32 dim tiles x 3 P' terms = 168; a tile of
    at most 64 valid tokens (the remainder past whole tiles) skips half the
    S tiles and packs its P' terms into two MFMAs per dim tile: 100; when
    that remainder of at most 32 tokens leads a longer split, two S tiles
    and one MFMA per dim tile: 50.  Every MFMA is 16x16x128, 65,536 flops.
    None for the other kernels."""
    if p.kv_dtype != "fp8" or p.heads < 48:
        return None
    n_sh = p.num_shards
    if p.kind == "sparse":
        counts = np.zeros((n_sh, p.rows), dtype=np.int64)
        for r in range(n_sh):
            counts[r] = ((w.table >= 0) & (w.table % n_sh == r)).sum(axis=1)
    else:
        cap = p.lpages * p.page_size
        counts = np.minimum(np.repeat(w.local_lens, p.q_per_seq, axis=1), cap).astype(np.int64)
    per_wave = 0
    for n in counts.ravel():
        chunk = -(-(-(-int(n) // splits)) // 128) * 128
        for sp in range(splits):
            ln = max(0, min(int(n), (sp + 1) * chunk) - min(int(n), sp * chunk))
            tiles, rem = -(-ln // 128), ln % 128
            short = 1 if 0 < rem <= 64 else 0
            tiny = 1 if short and tiles > 1 and rem <= 32 else 0
            per_wave += 168 * (tiles - short) + 100 * (short - tiny) + 50 * tiny
    return per_wave * 4 * -(-p.heads // 64)      # idle waves of a partial head block included


def measure_kv_write(w, stream, dev, reps=50):
    """Time dcp_kv_write on layer 0 of group w: the new tokens of one decode
    step (q_per_seq per sequence) and a chunk of up to 2048 tokens per sequence, both
    at the sequences' last positions; K launches back to back between two
    events on the launch stream.  Algorithmic bytes per token: the bf16 row
    read (1152), its slot (4) and the row written (580 FP8 with its scale,
    1152 BF16)."""
    p = w.p
    per_tok = 1152 + 4 + (580 if p.kv_dtype == "fp8" else 1152)
    out = {"kernel": "kv_write_kernel (interleaved KV-cache write"
                     + (", E4M3FN quantisation)" if p.kv_dtype == "fp8" else ")")}
    gen = torch.Generator(device=dev)
    gen.manual_seed(p.seed + 77)
    for label, per_seq in (("decode_step", min(p.q_per_seq, p.context)),
                           ("chunk", min(2048, p.context))):
        slots = np.concatenate([wl.positions_to_slots(p, w.block_table, b,
                                                      np.arange(p.context - per_seq, p.context))
                                for b in range(p.batch)]).astype(np.int32)
        kv_new = torch.randn((len(slots), 576), generator=gen, device=dev).to(torch.bfloat16)
        call = B.prepare_kv_write(kv_new, torch.from_numpy(slots).to(dev), w.pools[0], w.scales[0],
                                  stream=stream)
        for _ in range(5):
            call()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            call()
        t1.record(stream)
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / reps
        nbytes = len(slots) * per_tok
        out[label] = {"tokens": int(len(slots)), "us_per_launch": round(us, 2),
                      "algorithmic_bytes": int(nbytes),
                      "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    return out


def measure_combine(p, stream, dev, reps=50):
    """The standalone LSE merge (lse_combine) of per-shard partials of the
    decode workload's shape: fp32 [N, rows, heads, 512] + LSE in, bf16 out,
    one shard's LSE -inf on every fourth row.  Events around `reps` launches
    on the launch stream."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    n, rows, heads = p.num_shards, p.rows, p.heads
    o_part = torch.randn((n, rows, heads, 512), generator=gen, device=dev)
    lse_part = torch.randn((n, rows, heads), generator=gen, device=dev) * 3
    lse_part[0, ::4] = float("-inf")
    o = torch.empty((rows, heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, heads), dtype=torch.float32, device=dev)
    call = lambda: B.lse_combine(o_part, lse_part, B.OUT_BF16, o, lse, stream=stream)  # noqa: E731
    for _ in range(5):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    alg = n * rows * heads * (512 + 1) * 4 + rows * heads * (512 * 2 + 4)
    return {"workload": f"{p.name} partials ({n} shards)", "us_per_launch": round(us, 2),
            "algorithmic_bytes": alg, "gbps": round(alg / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def measure_prefill(stream, dev, reps=20, name="prefill_fp8_prefix16k_new2k"):
    """Time the prefill over a cached prefix on its workload: for every
    bounded chunk, the gather from the shards (dcp_gather_prefix), the new
    tokens' attention to the chunk (mla_prefill_chunk_lse) and the running
    merge (lse_merge_into, fp32 accumulator); each kind of launch timed over
    `reps` passes by events on the launch stream, and the whole pass.
    Algorithmic bytes: gather 2 x 580 (FP8) or 2 x 1152 (BF16) per token,
    merge 3 x (512 x 4 + 4) per (token, head); attention flops 2 x (576 +
    512) per (token, head, chunk token)."""
    p = wl.PREFILL_PRESETS[name]
    pw = wl.make_prefill_workload(p, device=dev)
    w = pw.cache
    q = pw.q[0]
    tokens, heads = p.new_tokens, p.heads
    chunks = wl.prefix_chunks(p)
    c_max = max(ln for _, ln in chunks)
    fp8 = p.kv_dtype == "fp8"
    kv = torch.empty((c_max, 576), dtype=w.pools[0][0].dtype, device=dev)
    sc = torch.empty((c_max,), dtype=torch.float32, device=dev) if fp8 else None
    o_c = torch.empty((tokens, heads, 512), dtype=torch.float32, device=dev)
    lse_c = torch.empty((tokens, heads), dtype=torch.float32, device=dev)
    o = torch.zeros((tokens, heads, 512), dtype=torch.float32, device=dev)
    lse = torch.full((tokens, heads), float("-inf"), dtype=torch.float32, device=dev)
    ws_n = B.prefill_workspace_size(tokens, heads, c_max)
    ws = B.alloc_workspace(ws_n, dev) if ws_n else None
    bt = w.dev(w.block_table[0]).reshape(1, -1)
    calls = []
    for beg, ln in chunks:
        calls.append((
            B.prepare_gather_prefix(bt, w.pools[0], w.scales[0], p.page_size, [beg], [ln], out_kv=kv[:ln],
                                    out_scale=sc[:ln] if fp8 else None, stream=stream),
            B.prepare_prefill_chunk_attention(q, kv[:ln], sc[:ln] if fp8 else None, p.sigma, o_c, lse_c,
                                              workspace=ws, stream=stream),
            B.prepare_merge_into(o, lse, o_c, lse_c, stream=stream)))

    def mk():
        return torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        for c in calls:
            for f in c:
                f()
    torch.cuda.synchronize()
    ev = [[(mk(), mk()) for _ in range(3)] for _ in range(reps * len(calls))]
    t0, t1 = mk(), mk()
    t0.record(stream)
    for r in range(reps):
        for c in calls:
            for f in c:
                f()
    t1.record(stream)
    torch.cuda.synchronize()
    whole_us = t0.elapsed_time(t1) * 1000.0 / reps
    i = 0
    for r in range(reps):
        for c in calls:
            for k, f in enumerate(c):
                ev[i][k][0].record(stream)
                f()
                ev[i][k][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    per = [statistics.mean(e[k][0].elapsed_time(e[k][1]) * 1000.0 for e in ev) for k in range(3)]
    mean_chunk = statistics.mean(ln for _, ln in chunks)
    g_bytes = mean_chunk * (2 * 580 if fp8 else 2 * 1152)
    a_flops = 2.0 * (576 + 512) * tokens * heads * mean_chunk
    m_bytes = 3 * tokens * heads * (512 * 4 + 4)
    peak = FP8_MFMA_PEAK_TFLOPS if fp8 else BF16_MFMA_PEAK_TFLOPS
    return {
        "workload": p.name, "note": p.note,
        "us_per_prefix_pass": round(whole_us, 1),
        "chunks": len(chunks),
        "gather": {"kernel": "gather_prefix_kernel", "us_per_chunk": round(per[0], 2),
                   "gbps": round(g_bytes / (per[0] * 1e-6) / 1e9, 1),
                   "frac_hbm_peak": round(g_bytes / (per[0] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
        "attention": {"kernel": ("decode_fp8_kernel<true, false>" if fp8 and heads * tokens % 64 == 0
                                 else "decode_kernel") + " (dense, one contiguous chunk)",
                      "us_per_chunk": round(per[1], 2),
                      "tflops": round(a_flops / (per[1] * 1e-6) / 1e12, 1),
                      "frac_mfma_peak": round(a_flops / (per[1] * 1e-6) / 1e12 / peak, 4),
                      "peak_tflops": peak},
        "merge": {"kernel": "merge_into_kernel", "us_per_chunk": round(per[2], 2),
                  "gbps": round(m_bytes / (per[2] * 1e-6) / 1e9, 1),
                  "frac_hbm_peak": round(m_bytes / (per[2] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
    }


def measure_topk(stream, dev, reps=20, name="index_topk_b64_ctx128k_k2048"):
    """Time the sharded index cache and distributed top-k on its workload:
    dcp_index_score (every local token of every (row, shard)), dcp_topk_local
    and dcp_topk_merge, each over `reps` launches between events on the launch
    stream, and the three back to back.  Algorithmic bytes of the scoring: 132
    per token (128 codes + scale) + 4 (its score written) + the queries;
    flops 2 x 128 x heads per token."""
    p = wl.INDEX_PRESETS[name]
    w = wl.make_index_workload(p, device=dev)
    lens_dev = [w.dev(w.local_lens[r]) for r in range(p.num_shards)]
    lens_all = w.dev(w.local_lens)
    bt = w.dev(w.block_table)
    scores = torch.empty((p.num_shards, p.rows, p.max_local), dtype=torch.float32, device=dev)
    cs = torch.empty((p.num_shards, p.rows, p.topk), dtype=torch.float32, device=dev)
    cp = torch.empty((p.num_shards, p.rows, p.topk), dtype=torch.int32, device=dev)
    out = (torch.empty((p.rows, p.topk), dtype=torch.float32, device=dev),
           torch.empty((p.rows, p.topk), dtype=torch.int32, device=dev),
           torch.empty((p.rows, p.topk), dtype=torch.int32, device=dev))
    calls = [B.prepare_index_score(w.q, w.w, w.keys, w.scales, lens_dev, bt, p.page_size, p.max_local,
                                   out=scores, stream=stream),
             B.prepare_topk_local(scores, lens_all, p.topk, cs, cp, stream=stream),
             B.prepare_topk_merge(cs, cp, bt, p.page_size, out=out, stream=stream)]

    def mk():
        return torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        for f in calls:
            f()
    torch.cuda.synchronize()
    per = []
    for f in calls:
        t0, t1 = mk(), mk()
        t0.record(stream)
        for _ in range(reps):
            f()
        t1.record(stream)
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) * 1000.0 / reps)
    t0, t1 = mk(), mk()
    t0.record(stream)
    for _ in range(reps):
        for f in calls:
            f()
    t1.record(stream)
    torch.cuda.synchronize()
    whole = t0.elapsed_time(t1) * 1000.0 / reps
    tokens = int(w.local_lens.sum())
    s_bytes = tokens * (132 + 4) + p.rows * p.index_heads * (128 + 4)
    s_flops = 2.0 * 128 * p.index_heads * tokens
    return {
        "workload": p.name, "note": p.note, "us_per_layer": round(whole, 2),
        "score": {"kernel": "index_score_kernel", "us": round(per[0], 2),
                  "gbps": round(s_bytes / (per[0] * 1e-6) / 1e9, 1),
                  "frac_hbm_peak": round(s_bytes / (per[0] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                  "tflops": round(s_flops / (per[0] * 1e-6) / 1e12, 1),
                  "algorithmic_bytes": int(s_bytes)},
        "local_topk": {"kernel": "topk_local_fast_kernel (lists of at most 32,768 tokens)",
                       "us": round(per[1], 2),
                       "lists": p.rows * p.num_shards, "list_len": p.max_local},
        "merge": {"kernel": "topk_merge_rank_kernel", "us": round(per[2], 2),
                  "candidates_per_row": p.num_shards * p.topk},
    }


def cpu_baseline(w, host, rows, min_seconds=10.0, max_reps=30):
    """Time the CPU oracle on one layer-step (or a row sample of it),
    repeated until about min_seconds of CPU work have run."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    p = w.p
    q, pools, scales = host
    sel = np.arange(p.rows) if rows <= 0 else np.arange(min(rows, p.rows))
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_all < min_seconds and len(times) < max_reps):
        t0 = time.perf_counter()
        if p.kind == "sparse":
            local, counts = oracle.remap_topk(w.table[sel], p.num_shards, p.pool_rows)
            parts = [oracle.sparse_attn_shard(q[sel], pools[r], p.kv_dtype, scales[r], local[r],
                                              counts[r], p.sigma) for r in range(p.num_shards)]
        else:
            parts = [oracle.dense_attn_shard(q[sel], pools[r], p.kv_dtype, scales[r],
                                             w.block_table[sel], w.local_lens[r][sel],
                                             p.page_size, p.sigma) for r in range(p.num_shards)]
        oracle.lse_merge(np.stack([a for a, _ in parts]), np.stack([b for _, b in parts]))
        times.append(time.perf_counter() - t0)
    t = statistics.median(times) * (p.rows / len(sel))
    return {"value": round(t * 1e6, 1), "unit": "us/layer-step", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"{'all' if len(sel) == p.rows else len(sel)} of {p.rows} rows of one "
                       f"layer-step (remap + {p.num_shards} shard attentions + merge, fp64 numpy), "
                       f"median of {len(times)} runs ({time.perf_counter() - t_all:.1f} s of CPU work), "
                       f"scaled to {p.rows} rows; host CPU {cpu_model()}, "
                       f"{len(os.sched_getaffinity(0))} cores available")}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the DCP shards are cache slices on one device and "
              "this build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.print_digest:
        print(source_digest())
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda:0")
    p = wl.preset(args.workload)
    sparse = p.kind == "sparse"
    lpt = args.layers_per_table if sparse else 1
    n_layers = args.groups * lpt
    print(f"[bench] workload {p.name}: generating {n_layers} layer caches", file=sys.stderr, flush=True)
    groups = []
    for gi in range(args.groups):
        w = wl.make_workload(p, device=dev, layers=lpt, seed=p.seed + 1000 * gi)
        groups.append(w)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    # Per-group device inputs and preallocated outputs / workspace.
    ws_bytes = B.workspace_size(not sparse, p.rows, p.heads, p.num_shards,
                                p.topk if sparse else int(groups[0].local_lens.max()),
                                p.page_size, args.num_splits, want_partials=False, want_merged=True)
    ws = B.alloc_workspace(ws_bytes, dev)
    o = torch.empty((p.rows, p.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((p.rows, p.heads), dtype=torch.float32, device=dev)
    outs = {"o": o, "lse": lse}
    # Every call is marshalled once up front, so the timed loop is one ctypes
    # call per launch and the host stays ahead of the GPU.
    prep = []
    for w in groups:
        d = {}
        if sparse:
            table = w.dev(w.table)
            local = torch.empty((p.num_shards, p.rows, p.topk), dtype=torch.int32, device=dev)
            counts = torch.empty((p.num_shards, p.rows), dtype=torch.int32, device=dev)
            d["remap"] = B.prepare_remap_topk(table, p.num_shards, out=local, counts=counts,
                                              stream=stream)
            d["dec"] = [B.prepare_sparse_decode(w.q, w.pools[li], w.scales[li], local, counts,
                                                p.sigma, num_splits=args.num_splits, workspace=ws,
                                                out=outs, stream=stream) for li in range(lpt)]
        else:
            bt = w.dev(w.block_table)
            lens = [w.dev(w.local_lens[r]) for r in range(p.num_shards)]
            d["dec"] = [B.prepare_dense_decode(w.q, w.pools[li], w.scales[li], bt, lens,
                                               p.page_size, int(w.local_lens.max()), p.sigma,
                                               num_splits=args.num_splits, workspace=ws, out=outs,
                                               stream=stream) for li in range(lpt)]
        prep.append(d)

    def step(gi, ev=None, cap_stream=None):
        d = prep[gi]
        if sparse:
            if ev is not None:
                ev["remap"][0].record(stream)
            d["remap"](cap_stream)
            if ev is not None:
                ev["remap"][1].record(stream)
        for li in range(lpt):
            if ev is not None:
                ev["dec"][li][0].record(stream)
            d["dec"][li](cap_stream)
            if ev is not None:
                ev["dec"][li][1].record(stream)

    # HIP graphs: one per table group, each holding one step's launches (the
    # remap and the decodes of the layers sharing the table).  The library
    # queues only kernels (no memsets, no allocation), so a replay is the
    # same work as the eager step; the first replays are checked against the
    # eager result below.
    graphs = None
    if args.launch == "graph":
        eager = []
        for gi in range(args.groups):
            step(gi)
            torch.cuda.synchronize()
            eager.append((o.clone(), lse.clone()))
        graphs = []
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for gi in range(args.groups):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    step(gi, cap_stream=cap)
                graphs.append(g)
        torch.cuda.synchronize()
        for rep in range(2):
            for gi in range(args.groups):
                o.zero_()
                lse.zero_()
                torch.cuda.synchronize()
                graphs[gi].replay()
                torch.cuda.synchronize()
                if not (torch.equal(o, eager[gi][0]) and torch.equal(lse, eager[gi][1])):
                    print(f"[bench] graph replay {rep} of group {gi} differs from the eager step",
                          file=sys.stderr)
                    sys.exit(3)

    def run_step(s):
        if graphs is not None:
            graphs[s % args.groups].replay()
        else:
            step(s % args.groups)

    t_w = time.perf_counter()
    s = 0
    while s < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        run_step(s)
        s += 1
        if s % args.groups == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_steps = s

    def mk():
        return torch.cuda.Event(enable_timing=True)
    # The timed region: K steps launched back to back.  Events recorded
    # between launches would stop consecutive kernels from overlapping their
    # dispatch (measured: about 7 us per layer-step), so the per-launch
    # durations for the roofline come from a second pass over the same K
    # steps with an event pair around every launch.
    t_start, t_end = mk(), mk()
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        run_step(s)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    evs = [{"remap": (mk(), mk()), "dec": [(mk(), mk()) for _ in range(lpt)]}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(s % args.groups, evs[s])
    torch.cuda.synchronize()
    ms_per_step = total_ms / args.steps
    us_per_layer_step = ms_per_step * 1000.0 / lpt
    dec_us = [e["dec"][li][0].elapsed_time(e["dec"][li][1]) * 1000.0 for e in evs for li in range(lpt)]
    remap_us = [e["remap"][0].elapsed_time(e["remap"][1]) * 1000.0 for e in evs] if sparse else [0.0]

    # algorithmic bytes / flops of one decode launch (average over the groups)
    if sparse:
        valid = [int((w.table >= 0).sum()) for w in groups]
    else:
        valid = [int(w.local_lens.sum()) for w in groups]
    kv_b, tot_b = zip(*[algorithmic_bytes(w, v) for w, v in zip(groups, valid)])
    kv_b, tot_b, tok = statistics.mean(kv_b), statistics.mean(tot_b), statistics.mean(valid)
    dec_mean = statistics.mean(dec_us)
    fl = flops(p, tok)
    kv_gbps = kv_b / (us_per_layer_step * 1e-6) / 1e9
    # The FP8 path contracts on the fp8 MFMA, the BF16 path on the bf16 one.
    mfma_peak = FP8_MFMA_PEAK_TFLOPS if p.kv_dtype == "fp8" else BF16_MFMA_PEAK_TFLOPS
    mfma_bound = (fl / (mfma_peak * 1e12)) > (tot_b / (HBM_PEAK_GBPS * 1e9))
    kname = decode_kernel_name(p)
    traffic = measured_traffic(kname, p.name)
    if mfma_bound:
        achieved = fl / (dec_mean * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4), "traffic": traffic}
    else:
        achieved = tot_b / (dec_mean * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
    # The FP8 kernel's executed MFMA work (query hi + lo terms, three P'
    # terms, padded short tiles) against the fp8 MFMA peak, beside the roof
    # above: which of the two binds depends on the shape.
    splits = B.decode_splits(not sparse, p.rows, p.heads, p.num_shards,
                             p.topk if sparse else int(groups[0].local_lens.max()), p.page_size,
                             args.num_splits)
    mfma_n = [fp8_kernel_mfma(p, w, splits) for w in groups]
    if mfma_n[0] is not None:
        ex_flops = statistics.mean(mfma_n) * 65536.0
        ex_tf = ex_flops / (dec_mean * 1e-6) / 1e12
        roof["mfma_executed"] = {"mfma_per_launch": int(statistics.mean(mfma_n)),
                                 "flops_per_launch": ex_flops, "achieved": round(ex_tf, 1),
                                 "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(ex_tf / FP8_MFMA_PEAK_TFLOPS, 4),
                                 "floor_us": round(ex_flops / (FP8_MFMA_PEAK_TFLOPS * 1e12) * 1e6, 2)}
    roof["splits"] = splits
    roof.update({"kernel": kname + (" (fused sparse MLA decode + LSE merge)" if sparse
                                    else " (fused dense MLA decode + LSE merge)"),
                 "avg_launch_us": round(dec_mean, 2), "algorithmic_bytes_per_launch": int(tot_b),
                 "kv_bytes_per_launch": int(kv_b), "flops_per_launch": fl,
                 "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                 "copy-calibrated)"})

    result = {
        "metric": METRIC,
        "value": round(us_per_layer_step, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "launch": ("one HIP graph per step (remap + the layers' decodes), replayed"
                   if graphs is not None else "kernels launched from the host"),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if p.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "rows": p.rows, "heads": p.heads, "shards": p.num_shards,
                   "topk": p.topk if sparse else None, "context": p.context,
                   "kv": "fp8_e4m3 + fp32 per-token scale" if p.kv_dtype == "fp8" else "bf16",
                   "page_size": p.page_size, "layers_per_step": lpt, "layers_rotated": n_layers,
                   "step": ("remap once + fused decode for each layer sharing the table"
                            if sparse else "fused dense decode")},
        "kv_gbps": round(kv_gbps, 1),
        "kv_pct_hbm_peak": round(100.0 * kv_gbps / HBM_PEAK_GBPS, 2),
        "decode_us_mean": round(dec_mean, 2),
        "decode_us_p10_p90": [round(float(np.percentile(dec_us, 10)), 2),
                              round(float(np.percentile(dec_us, 90)), 2)],
        "remap_us_mean": round(statistics.mean(remap_us), 2),
        "roofline": roof,
    }
    # Warm figure, reported beside the cold one: the same layer's decode
    # relaunched back to back, so its KV (4.9 GB at the headline size, more
    # than the 256 MB last-level cache) is only partly cache-resident.
    warm = prep[0]["dec"][0]
    for _ in range(10):
        warm()
    w0, w1 = mk(), mk()
    torch.cuda.synchronize()
    w0.record(stream)
    for _ in range(args.steps):
        warm()
    w1.record(stream)
    torch.cuda.synchronize()
    result["decode_us_warm_same_layer"] = round(w0.elapsed_time(w1) * 1000.0 / args.steps, 2)
    # The KV-cache write runs after the timed decode loop (it overwrites the
    # last positions of layer 0 of the first table group).
    result["kv_write"] = measure_kv_write(groups[0], stream, dev)
    # The oracle's baseline runs on a host copy of layer 0 of the first table
    # group, before the layer caches are released for the other measurements.
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: copying one layer to the host", file=sys.stderr, flush=True)
        w = groups[0]
        host = (__import__("oracle").decode_bf16(w.q_host_bits()),
                [w.pool_host(0, r) for r in range(p.num_shards)],
                [w.scale_host(0, r) for r in range(p.num_shards)])
        print("[bench] cpu baseline: running the oracle", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, host, args.cpu_rows)
        result["cpu_baseline"] = cb
        del w, host
    if not args.no_prefill:
        del groups, prep
        torch.cuda.empty_cache()
        result["combine"] = measure_combine(p, stream, dev)
        result["prefill_prefix"] = measure_prefill(stream, dev)
        torch.cuda.empty_cache()
        result["index_topk"] = measure_topk(stream, dev)
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
