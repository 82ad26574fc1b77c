"""CPU checks of bench.py's roofline arithmetic on the 64-row FP8 workload:
the algorithmic bytes and flops of one decode launch, against the figures
derived independently from the workload's shape (576 FP8 codes + one fp32
scale per selected token, 2 x (576 + 512) flops per token and head)."""

import types

import bench
import numpy as np
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


def test_fp8_kernel_mfma_hand_worked():
    # one shard, 64 heads: row 0 holds 200 tokens (a full tile and one of 72
    # tokens: 2 x 168 MFMAs per wave), row 1 holds 64 (one short tile: 100);
    # four waves per block.  Two splits cut row 0 into 128 + 72 and row 1
    # into 64 + 0: the same tiles.
    from types import SimpleNamespace
    p = SimpleNamespace(kv_dtype="fp8", heads=64, kind="sparse", num_shards=1, rows=2)
    table = np.full((2, 256), -1, dtype=np.int64)
    table[0, :200] = np.arange(200)
    table[1, :64] = np.arange(64)
    w = SimpleNamespace(table=table)
    assert bench.fp8_kernel_mfma(p, w, 1) == 4 * (2 * 168 + 100) == 1744
    assert bench.fp8_kernel_mfma(p, w, 2) == 1744
    p128 = SimpleNamespace(**{**vars(p), "heads": 128})
    assert bench.fp8_kernel_mfma(p128, w, 1) == 2 * 1744            # two 64-head blocks
    assert bench.fp8_kernel_mfma(SimpleNamespace(**{**vars(p), "kv_dtype": "bf16"}), w, 1) is None


def test_fp8_kernel_mfma_lead_tiles():
    # a remainder of at most 32 tokens ahead of a full tile is a "tiny" lead
    # (two S tiles, one MFMA per dim tile: 18 + 32 = 50 per wave); 33..64
    # ahead of one is a short lead (100); alone, any remainder up to 64 is a
    # short tile (100)
    from types import SimpleNamespace
    p = SimpleNamespace(kv_dtype="fp8", heads=64, kind="sparse", num_shards=1, rows=3)
    table = np.full((3, 256), -1, dtype=np.int64)
    table[0, :150] = np.arange(150)       # 128 + 22: 168 + 50
    table[1, :180] = np.arange(180)       # 128 + 52: 168 + 100
    table[2, :20] = np.arange(20)         # 20 alone: 100
    w = SimpleNamespace(table=table)
    assert bench.fp8_kernel_mfma(p, w, 1) == 4 * (218 + 268 + 100)
