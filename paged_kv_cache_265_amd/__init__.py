"""Paged-attention decode for AMD MI355X (gfx950): a C-ABI HIP library
(include/pkv.h, built into libpkv.so) and its thin Python binding."""

from .pkv import (  # noqa: F401
    BF16,
    F16,
    F32,
    PkvError,
    SYMBOLS,
    copy_blocks,
    decode_partition_size,
    decode_workspace_size,
    load_library,
    mixed_workspace_size,
    paged_attention_chunked,
    paged_attention_decode,
    paged_attention_decode_static,
    paged_attention_mixed,
    read_probe,
    reshape_and_cache,
    version,
)
