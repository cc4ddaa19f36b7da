"""MI355X (gfx950) paged KV-cache decode: paged attention decode and the
slot-mapped cache write, as hand-written HIP kernels behind a C ABI
(``include/pkv.h``).

``paged_attn_decode`` and ``kv_cache_write`` take torch tensors on the GPU and
call the HIP library; ``paged_attn_chunk`` scores several new tokens per
sequence (causal), ``paged_attn_decode_shared_prefix`` reads a prompt prefix
shared by a group of sequences once per group (``shared_prefix_groups``
derives the groups from host tables), and the ``_fp8`` variants work on e4m3
pools. ``BlockManager`` (host) hands out pool blocks with reference-counted
sharing and copy-on-write, whose copies ``copy_blocks`` runs on the GPU; the
library is loaded on first use and a missing build raises. ``workloads`` builds seeded synthetic inputs; ``accounting`` holds the
byte counts used to turn kernel time into bandwidth.
"""
from ._lib import (  # noqa: F401
    BlockManager,
    PkvError,
    copy_blocks,
    decode_plan,
    kv_cache_write,
    kv_cache_write_fp8,
    last_error,
    paged_attn_chunk,
    paged_attn_chunk_fp8,
    paged_attn_decode,
    paged_attn_decode_append,
    paged_attn_decode_fp8,
    paged_attn_decode_shared_prefix,
    paged_attn_decode_shared_prefix_fp8,
    release_workspace,
    set_partition_tokens,
    shared_prefix_groups,
    version,
)

__all__ = [
    "paged_attn_decode",
    "paged_attn_decode_append",
    "BlockManager",
    "copy_blocks",
    "paged_attn_decode_fp8",
    "paged_attn_chunk",
    "paged_attn_decode_shared_prefix",
    "shared_prefix_groups",
    "paged_attn_chunk_fp8",
    "paged_attn_decode_shared_prefix_fp8",
    "kv_cache_write_fp8",
    "kv_cache_write",
    "decode_plan",
    "set_partition_tokens",
    "release_workspace",
    "last_error",
    "version",
    "PkvError",
]
