"""Block KV decode hot path for AMD Instinct MI355X (gfx950).

Slot mapping, the paged KV-cache write, GQA paged decode attention and
per-step context-length bucket selection, as hand-written HIP kernels behind
a C ABI (include/kvslot.h, libkvslot.so). This package is the thin Python
binding: it marshals torch tensors into that ABI and nothing else. There is
no CPU or PyTorch fallback; a missing library is an error.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    KVS_BF16,
    KVS_F32,
    KVS_WALK_TABLE,
    LIB_PATH,
    STATUS,
    KvslotError,
    kv_cache_write,
    kv_map_to_kernel_blocks,
    kv_slot_mapping,
    kv_slot_mapping_cache_write,
    kv_slot_mapping_dcp,
    paged_decode_attention_dcp,
    decode_lse_merge,
    load,
    make_workspace,
    paged_decode_attention,
    paged_decode_attention_noalloc,
    paged_decode_attention_append,
    paged_decode_attention_swa,
    kv_swa_tail_trim,
    paged_decode_attention_workspace_bytes,
    select_batch_bucket,
    select_ctx_bucket,
)
