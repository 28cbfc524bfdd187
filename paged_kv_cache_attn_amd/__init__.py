"""Paged KV-cache attention for AMD MI355X (gfx950).

The compute lives in ``libpagedattn.so`` (hand-written HIP kernels, C ABI in
``include/pagedattn.h``); this package only builds it and binds it.
"""

from .binding import (  # noqa: F401
    BlockManager,
    PrefixLevel,
    PA_BF16,
    PA_F32,
    bench_fill,
    block_mask,
    bench_stream_read,
    decode_cascade_plan,
    decode_cascade_workspace,
    decode_cascade_workspace_size,
    decode_split_tokens,
    decode_workspace,
    decode_workspace_size,
    kv_append,
    kv_copy_blocks,
    lib,
    lib_path,
    paged_attn_decode,
    paged_attn_decode_noalloc,
    paged_attn_decode_cascade,
    paged_attn_prefill,
    prefill_workspace,
    prefill_workspace_size,
    prefix_level,
    status_string,
)
