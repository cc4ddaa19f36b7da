"""MI355X (gfx950) paged KV-cache decode: paged attention decode and the
slot-mapped cache write, as hand-written HIP kernels behind a C ABI
(``include/pkv.h``).

``paged_attn_decode`` and ``kv_cache_write`` take torch tensors on the GPU and
call the HIP library; the library is loaded on first use and a missing build
raises. ``workloads`` builds seeded synthetic inputs; ``accounting`` holds the
byte counts used to turn kernel time into bandwidth.
"""
from ._lib import (  # noqa: F401
    PkvError,
    decode_plan,
    kv_cache_write,
    last_error,
    paged_attn_decode,
    release_workspace,
    set_partition_tokens,
    version,
)

__all__ = [
    "paged_attn_decode",
    "kv_cache_write",
    "decode_plan",
    "set_partition_tokens",
    "release_workspace",
    "last_error",
    "version",
    "PkvError",
]
