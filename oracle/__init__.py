"""CPU oracle for the Block KV decode path: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. It shares no code with the HIP library.
"""

from .kvslot_oracle import (  # noqa: F401
    NULL_BLOCK_ID,
    P_MAX,
    PAD_SLOT_ID,
    OracleError,
    compute_slot_mapping,
    compute_slot_mapping_dcp,
    dcp_local_position,
    dcp_owner,
    kv_cache_tensor_bytes,
    map_to_kernel_blocks,
    merge_lse,
    paged_decode_attention,
    paged_decode_attention_dcp,
    remap_null_block_to_sentinel,
    reshape_and_cache,
    select_batch_bucket,
    select_ctx_bucket,
    smallest_bucket_at_least,
    swa_tail_trim,
    validate_buckets,
    widen,
)
