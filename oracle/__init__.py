"""fp64 CPU oracle for paged decode, multi-token (chunk) paged attention,
shared-prefix decode, the slot-mapped cache write, the block manager and block
copy, and the FP8 (e4m3) KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The HIP library never calls it, and it imports nothing from the HIP
path (no binding, no kernel, no shared helper); it takes plain numpy arrays.

Every function here is pinned (``tests/test_oracle.py``, ``test_chunk_oracle.py``,
``test_shared_prefix_oracle.py``, ``test_block_manager.py``,
``test_fp8_oracle.py``) to facts that the
pages or plain mathematics fix (worked block-table example, permutation and
sharing invariance, softmax identities, brute force on tiny inputs, a library
attention routine on contiguous K/V). No function is "parity unpinned".
"""
from .paged_attention import (  # noqa: F401
    attention_weights,
    gather_tokens,
    paged_attn_decode,
    paged_attn_decode_partitioned,
    paged_attn_chunk,
)
from .cache_write import kv_cache_write  # noqa: F401
from .block_manager import BlockManagerModel, copy_blocks  # noqa: F401
from . import fp8  # noqa: F401
from . import shared_prefix  # noqa: F401
