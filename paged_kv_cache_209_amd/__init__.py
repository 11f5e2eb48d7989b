"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

Python binding of libpagedattn.so (C ABI in include/paged_attn.h): the
slot-mapped KV store (also fused with the rotary embedding of q and k), paged
decode attention with split-context merging, and causal paged prefill /
speculative-verify attention, and the host block manager that emits
the block tables and slot mappings (`block_manager.BlockManager`). PyTorch supplies device
memory and the current HIP stream; all computation runs in the HIP kernels.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PA_BF16,
    PA_ERR_HIP,
    PA_ERR_INVALID_ARG,
    PA_ERR_NO_BLOCKS,
    PA_ERR_UNSUPPORTED,
    PA_ERR_WORKSPACE,
    PA_F32,
    PA_OK,
    PagedAttnError,
    check_workspace,
    decode_fp8_workspace_bytes,
    decode_num_workgroups,
    decode_workspace_bytes,
    kv_store,
    kv_store_fp8,
    library,
    paged_attn_decode,
    paged_attn_decode_fp8,
    paged_attn_decode_noalloc,
    paged_attn_decode_store,
    paged_attn_prefill,
    prefill_workspace_bytes,
    qknorm_rope_kv_store,
    rope_kv_store,
    version,
)
