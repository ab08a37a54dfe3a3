"""PagedAttention decode and its slot-mapped KV writer for AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in
include/pagedkv.h (libpagedkv.so); this package only marshals torch tensors
into that ABI.  Importing it loads the library and fails loudly if it was
not built.
"""
from ._lib import (BF16, BLOCK_SIZE, DEFAULT_PARTITION_SIZE, EXPORTED, F16, F32, FP8_E4M3,
                   NOALLOC_SCRATCH_BYTES, BlockManager, LIB_PATH, PagedKVError,
                   alloc_shared_prefix_workspace, alloc_workspace, copy_blocks,
                   paged_attention_decode, paged_attention_decode_append,
                   paged_attention_decode_noalloc, paged_attention_decode_shared_prefix,
                   paged_attention_decode_shared_prefix_append, paged_kv_gather, raw, reshape_and_cache, shared_prefix_workspace_bytes,
                   workspace_bytes)

__all__ = [
    "BF16", "BLOCK_SIZE", "BlockManager", "DEFAULT_PARTITION_SIZE", "EXPORTED", "F16", "F32",
    "FP8_E4M3", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "PagedKVError",
    "alloc_shared_prefix_workspace", "alloc_workspace", "copy_blocks",
    "paged_attention_decode", "paged_attention_decode_append",
    "paged_attention_decode_noalloc", "paged_attention_decode_shared_prefix",
    "paged_attention_decode_shared_prefix_append", "paged_kv_gather", "shared_prefix_workspace_bytes", "raw", "reshape_and_cache",
    "workspace_bytes",
]
