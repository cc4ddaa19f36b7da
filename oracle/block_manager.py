"""Oracle for the KV block manager and the copy-on-write block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  - vLLM paper page, "PagedAttention" core idea and its block-pool diagram.
    A pool of equal blocks is allocated once. A sequence takes a block when
    it needs one and gives it back when it ends; a block table maps its
    logical blocks to physical ones.
  - The same page's OS-paging table pairs fork and copy-on-write with block
    sharing for parallel sampling and beam search.
  - The same page's "system implementation points": reference counts make
    sharing possible.
  - vLLM notes page, "KV Cache and PagedAttention": a block may be
    referenced by several requests (ref_count) and is copied on write. A KV
    cache manager keeps a free-block queue.
  - vLLM notes page, "Prefix Caching", eviction paragraph: a finished
    request's blocks join the free queue in reverse order, so its last
    blocks are reused first.

Readings taken where the pages leave a step open:
  - The free queue starts in block-index order. Allocation takes the front;
    a released block joins the back.
  - A sequence with n cached tokens holds ceil(n / BS) blocks. Token j lives
    in slot ``blocks[j // BS] * BS + j % BS``.
  - Appending token n:
      * n % BS == 0: a new block is taken;
      * the last block is shared (count > 1): copy-on-write. A new block
        replaces it in this sequence, the shared block's count drops by one,
        and (src, dst) is reported so its contents are copied before the
        write;
      * otherwise the slot is in the last block.
  - Sequences of one append call are served in the order given.
  - An operation that cannot get all the blocks it needs changes nothing
    and raises ``OutOfBlocks``.

``copy_blocks`` is the plain definition of the copy: ``pool[dst] = pool[src]``
for each pair.
"""
from __future__ import annotations

from collections import deque

import numpy as np


class OutOfBlocks(Exception):
    pass


class BlockManagerModel:
    """Reference model of the manager: free queue, counts, per-sequence block lists."""

    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.free = deque(range(num_blocks))
        self.ref = [0] * num_blocks
        self.blocks = {}   # seq id -> list of block ids
        self.tokens = {}   # seq id -> cached tokens

    def _take(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def add_sequence(self, sid: int, num_tokens: int) -> None:
        if sid in self.blocks:
            raise KeyError(sid)
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks(need)
        self.blocks[sid] = [self._take() for _ in range(need)]
        self.tokens[sid] = num_tokens

    def fork(self, parent: int, child: int) -> None:
        if child in self.blocks:
            raise KeyError(child)
        self.blocks[child] = list(self.blocks[parent])
        self.tokens[child] = self.tokens[parent]
        for b in self.blocks[child]:
            self.ref[b] += 1

    def _blocks_needed(self, sids) -> int:
        """Blocks an append over ``sids`` takes, following the counts as they change."""
        ref = {}
        need = 0
        for sid in sids:
            n = self.tokens[sid]
            if n % self.block_size == 0:
                need += 1
                continue
            last = self.blocks[sid][-1]
            r = ref.get(last, self.ref[last])
            if r > 1:
                need += 1
                ref[last] = r - 1
        return need

    def append_slots(self, sids):
        """Slots for the next token of each sequence, and the (src, dst) copies first needed."""
        sids = list(sids)
        if len(set(sids)) != len(sids):
            raise KeyError("duplicate sequence")
        for sid in sids:
            if sid not in self.blocks:
                raise KeyError(sid)
        if self._blocks_needed(sids) > len(self.free):
            raise OutOfBlocks()
        slots, copies = [], []
        for sid in sids:
            n = self.tokens[sid]
            blocks = self.blocks[sid]
            if n % self.block_size == 0:
                blocks.append(self._take())
            elif self.ref[blocks[-1]] > 1:
                src = blocks[-1]
                dst = self._take()
                self._release(src)
                blocks[-1] = dst
                copies.append((src, dst))
            slots.append(blocks[n // self.block_size] * self.block_size + n % self.block_size)
            self.tokens[sid] = n + 1
        return slots, copies

    def free_sequence(self, sid: int) -> None:
        for b in reversed(self.blocks.pop(sid)):
            self._release(b)
        del self.tokens[sid]

    def table(self, sid: int):
        return self.tokens[sid], list(self.blocks[sid])


def copy_blocks(k_pool, v_pool, pairs):
    """New ``(k_pool, v_pool)`` with block ``dst`` replaced by block ``src`` for each pair."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
    return k_out, v_out
