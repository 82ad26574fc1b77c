"""CPU fp64 oracle for the decode-context-parallel MLA decode path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library and imports nothing but numpy.
"""

from .dcp_oracle import (  # noqa: F401
    E4M3_NAN_CODES,
    decode_bf16,
    decode_e4m3fn,
    dequant_rows,
    remap_topk,
    sparse_attn_shard,
    dense_local_rows,
    dense_attn_shard,
    lse_merge,
    unsharded_sparse,
    unsharded_dense,
    attend,
    E4M3_MAX,
    encode_e4m3fn,
    quantize_row_e4m3,
    kv_write,
    prefix_slot,
    gather_prefix,
    prefix_chunk_attention,
    round_bf16,
    merge_running,
    D_INDEX,
    index_scores,
    topk_order,
    index_local_topk,
    merge_topk,
    positions_to_slots,
    sharded_topk,
    unsharded_topk,
)
