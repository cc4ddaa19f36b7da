"""Oracle for the slot-mapped KV cache write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The vLLM notes page ("V1 engine" scheduler steps) allocates slots for each
step's new tokens before the forward pass, and the vLLM paper page
("PagedAttention" section) grows a sequence block by block on demand. A slot
names one token position in the pool: ``slot = physical_block * BS + offset``
(the encoding is not on the pages; this is the reading taken). A negative slot
marks a padding token that is not written.

For every token ``t`` with ``slot[t] >= 0``::

    k_pool[slot // BS, :, slot % BS, :] = k_new[t]      (all KV heads)
    v_pool[slot // BS, :, slot % BS, :] = v_new[t]

and every other pool byte is unchanged. The copy is bitwise, so the oracle
works on any dtype, including integer views of bf16 storage.
"""
from __future__ import annotations

import numpy as np


def kv_cache_write(k_pool, v_pool, k_new, v_new, slot_mapping, block_size: int):
    """Return new ``(k_pool, v_pool)`` arrays with the new tokens scattered into their slots."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    num_slots = k_out.shape[0] * block_size
    for t, slot in enumerate(np.asarray(slot_mapping).reshape(-1)):
        slot = int(slot)
        if slot < 0:
            continue
        if slot >= num_slots:
            raise ValueError(f"slot {slot} outside a pool of {num_slots} slots")
        block, offset = divmod(slot, block_size)
        k_out[block, :, offset, :] = k_new[t]
        v_out[block, :, offset, :] = v_new[t]
    return k_out, v_out
