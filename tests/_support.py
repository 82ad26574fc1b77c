"""Shared helpers for the parity tests: run the HIP path through the binding,
run the oracle on host copies of the same inputs, compare.

Tolerances (fp32 outputs, relative to the fp64 oracle on the same dequantised
KV values): max |dO| <= 1e-2, max |dLSE| <= 1e-3; -inf must match exactly and
any NaN fails.  Integer outputs (remap) must be bit-exact.
"""

import json
import os

import numpy as np
import torch

import oracle
from sharded_kv_sparse_amd import binding as B
from sharded_kv_sparse_amd import workloads as wl

O_TOL = 1e-2
LSE_TOL = 1e-3


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_attn_close(o_gpu, lse_gpu, o_ref, lse_ref, what, o_tol=O_TOL, lse_tol=LSE_TOL,
                      o_rel=0.0):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    ninf_ref = lse_ref == -np.inf
    np.testing.assert_array_equal(lse_gpu == -np.inf, ninf_ref, err_msg=f"{what}: -inf pattern")
    d_lse = np.abs(lse_gpu[~ninf_ref] - lse_ref[~ninf_ref])
    # o_rel > 0 only for bfloat16 storage: its rounding adds up to 2^-9 |O|
    d_o = np.abs(o_gpu - o_ref) - o_rel * np.abs(o_ref)
    assert (o_gpu[ninf_ref] == 0).all(), f"{what}: empty rows must give O = 0"
    max_lse = float(d_lse.max()) if d_lse.size else 0.0
    max_o = float(d_o.max()) if d_o.size else 0.0
    assert max_lse <= lse_tol, f"{what}: max |dLSE| = {max_lse:.3e} > {lse_tol}"
    assert max_o <= o_tol, f"{what}: max |dO| = {max_o:.3e} > {o_tol}"
    return max_o, max_lse


def host_inputs(w, layer=0):
    q = oracle.decode_bf16(w.q_host_bits())
    pools = [w.pool_host(layer, r) for r in range(w.p.num_shards)]
    scales = [w.scale_host(layer, r) for r in range(w.p.num_shards)]
    return q, pools, scales


def oracle_sparse(w, layer=0, rows=None, heads=None, host=None):
    p = w.p
    q, pools, scales = host if host is not None else host_inputs(w, layer)
    table = w.table
    if rows is not None:
        q, table = q[rows], table[rows]
    if heads is not None:
        q = q[:, heads]
    local, counts = oracle.remap_topk(table, p.num_shards, p.pool_rows)
    parts = [oracle.sparse_attn_shard(q, pools[r], p.kv_dtype, scales[r], local[r], counts[r],
                                      p.sigma) for r in range(p.num_shards)]
    o, lse = oracle.lse_merge(np.stack([a for a, _ in parts]), np.stack([b for _, b in parts]))
    return dict(local=local, counts=counts, parts=parts, o=o, lse=lse)


def oracle_dense(w, layer=0, rows=None, heads=None, host=None):
    p = w.p
    q, pools, scales = host if host is not None else host_inputs(w, layer)
    bt, lens = w.block_table, w.local_lens
    if rows is not None:
        q, bt, lens = q[rows], bt[rows], lens[:, rows]
    if heads is not None:
        q = q[:, heads]
    parts = [oracle.dense_attn_shard(q, pools[r], p.kv_dtype, scales[r], bt, lens[r],
                                     p.page_size, p.sigma) for r in range(p.num_shards)]
    o, lse = oracle.lse_merge(np.stack([a for a, _ in parts]), np.stack([b for _, b in parts]))
    return dict(parts=parts, o=o, lse=lse)


def gpu_sparse(w, layer=0, want_partials=True, want_merged=True, num_splits=0,
               out_dtype=B.OUT_F32, workspace=None):
    p = w.p
    table = w.dev(w.table)
    local, counts = B.remap_topk(table, p.num_shards)
    res = B.sparse_decode(w.q, w.pools[layer], w.scales[layer], local, counts, p.sigma,
                          want_partials=want_partials, want_merged=want_merged,
                          out_dtype=out_dtype, num_splits=num_splits, workspace=workspace)
    res["local"], res["counts"] = local, counts
    return res


def gpu_dense(w, layer=0, want_partials=True, want_merged=True, num_splits=0,
              out_dtype=B.OUT_F32, workspace=None):
    p = w.p
    bt = w.dev(w.block_table)
    lens = [w.dev(w.local_lens[r]) for r in range(p.num_shards)]
    max_len = int(w.local_lens.max()) if w.local_lens.size else 0
    return B.dense_decode(w.q, w.pools[layer], w.scales[layer], bt, lens, p.page_size, max_len,
                          p.sigma, want_partials=want_partials, want_merged=want_merged,
                          out_dtype=out_dtype, num_splits=num_splits, workspace=workspace)


def check_against_oracle(res, ref, what, rows=None, heads=None):
    """Compare partials (if present) and the merged result."""
    def sel(a, lead=0):
        a = to_np(a)
        if rows is not None:
            a = np.take(a, rows, axis=lead)
        if heads is not None:
            a = np.take(a, heads, axis=lead + 1)
        return a

    out = {}
    if "o_part" in res:
        for r, (o_r, l_r) in enumerate(ref["parts"]):
            out[f"part{r}"] = assert_attn_close(sel(res["o_part"][r]), sel(res["lse_part"][r]),
                                                o_r, l_r, f"{what} shard {r}")
    if "o" in res:
        bf16 = res["o"].dtype == torch.bfloat16
        out["merged"] = assert_attn_close(sel(res["o"]), sel(res["lse"]), ref["o"], ref["lse"],
                                          f"{what} merged", o_rel=2.0 ** -8 if bf16 else 0.0)
    record_margins(what, out)
    return out


def record_margins(what, margins):
    """Append the measured max |dO| / |dLSE| of a parity case as one JSON line
    to the file named by DCP_PARITY_MARGINS (nothing when it is unset)."""
    path = os.environ.get("DCP_PARITY_MARGINS")
    if not path:
        return
    with open(path, "a") as f:
        for part, (d_o, d_lse) in margins.items():
            f.write(json.dumps({"case": what, "output": part, "max_abs_dO": d_o,
                                "max_abs_dLSE": d_lse, "tol_O": O_TOL, "tol_LSE": LSE_TOL}) + "\n")


def make(p, device="cuda", layers=1):
    return wl.make_workload(p, device=device, layers=layers)
