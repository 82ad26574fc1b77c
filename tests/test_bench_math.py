"""CPU checks of bench.py's roofline arithmetic on the 64-row FP8 workload:
the algorithmic bytes and flops of one decode launch, against the figures
derived independently from the workload's shape (576 FP8 codes + one fp32
scale per selected token, 2 x (576 + 512) flops per token and head)."""

import types

import bench
from sharded_kv_sparse_amd import workloads as wl


def test_headline_algorithmic_bytes_and_flops():
    p = wl.preset("sparse_fp8_b64_k2048")
    w = types.SimpleNamespace(p=p)
    tokens = p.rows * p.topk                              # every entry valid
    kv, total = bench.algorithmic_bytes(w, tokens)
    assert kv == 64 * 2048 * 580 == 76_021_760
    q = 64 * 64 * 576 * 2                                 # bf16 query, read once
    out = 64 * 64 * (512 * 4 + 4)                         # fp32 output + LSE
    ids = tokens * 4 + 4 * 64 * 4                         # local ids + counts
    assert total == kv + q + out + ids == 89_670_656
    assert bench.flops(p, tokens) == 2.0 * 64 * tokens * (576 + 512) == 18_253_611_008
    # 60 % of the 8 TB/s peak on these bytes: the 15.84 us per layer-step target
    assert abs(kv / (0.6 * bench.HBM_PEAK_GBPS * 1e9) * 1e6 - 15.84) < 0.01


def test_bf16_workload_bytes_per_token():
    p = wl.preset("sparse_bf16_b8_k2048")
    kv, _ = bench.algorithmic_bytes(types.SimpleNamespace(p=p), 1000)
    assert kv == 1000 * 1152
