"""MI355X-native paged KV write and paged attention.

The step (page "Add paged / block-table KV cache export (--features
paged-cache)", onnxruntime/mobius #395): scatter new K/V rows into per-layer
page pools through slot_mapping, then run causal GQA attention over each
sequence's pages (block_table row) cut to seq_lens, for a batch of sequences
described by query_start_loc.  All work runs in the HIP kernels of
libpagedkv.so (C ABI in include/pagedkv.h); this package only marshals torch
tensors into that ABI.  Build the library with
``python -m paged_kv_cache_243_amd.build``.
"""
from ._binding import (  # noqa: F401
    CHECK_NEW_ROWS_ARE_QUERY_ROWS,
    EXPORTS,
    LIB_PATH,
    PagedKVError,
    check_metadata_host,
    load,
    paged_attention,
    paged_attention_noalloc,
    paged_kv_write_attention,
    paged_block_table_from_csr,
    paged_attention_workspace_size,
    paged_kv_write,
    paged_kv_write_fp8,
    paged_validate_metadata,
)
