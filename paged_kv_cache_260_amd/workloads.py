"""Seeded synthetic inputs for paged decode and the slot-mapped cache write.

This module only builds inputs: block pools, block tables, sequence lengths,
slot mappings and random values. It holds none of the attention arithmetic, so
both the fp64 oracle (under ``oracle/``) and the HIP path can consume what it
makes without sharing any of the method's code.

Layouts (the pages fix none; these are the library's ABI layouts):

* ``q``                      ``[B, H, D]``
* ``k_pool`` / ``v_pool``    ``[NB, Hkv, BS, D]`` -- one (block, kv head) tile
  is one contiguous ``BS*D`` run.
* ``block_tables``           int32 ``[B, MB]``; entries past a sequence's
  allocated blocks are ``-1``.
* ``seq_lens``               int32 ``[B]``: tokens already in the cache.
* ``k_new`` / ``v_new``      ``[T, Hkv, D]`` with ``T = B``: one new token per
  sequence, appended at position ``seq_lens[s]``.
* ``slot_mapping``           int32 ``[T]``: ``slot = phys_block*BS + offset``.

Allocation follows the paged scheme of the vLLM paper page ("PagedAttention"
section and its block-pool diagram): a pool of fixed-size blocks, physical
blocks handed out in a shuffled order, one extra block allocated on demand only
when the appended token starts a new block, so internal waste stays below one
block per sequence. Parallel samples share their prompt's blocks with a
reference count (the block-manager and prefix-sharing points of the same page).

Draw order for a config with seed ``2600 + cfg_id`` (PCG64): lengths ->
physical permutation -> q -> k_pool -> v_pool -> k_new -> v_new. Values are
N(0, 1) drawn in float32 and rounded to the storage dtype by torch on the CPU
(round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    name: str
    dtype: torch.dtype
    num_seqs: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    scale: float                 # exactly representable float32 value
    seq_lens: np.ndarray         # int32 [B], tokens cached before the write
    block_tables: np.ndarray     # int32 [B, MB], -1 past allocated blocks
    num_blocks: int
    q: torch.Tensor              # [B, H, D]
    k_pool: torch.Tensor         # [NB, Hkv, BS, D]
    v_pool: torch.Tensor
    k_new: torch.Tensor          # [T, Hkv, D]
    v_new: torch.Tensor
    slot_mapping: np.ndarray     # int32 [T]
    refcount: np.ndarray         # int32 [NB], number of tables referencing each block
    seed: int = 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def seq_lens_after_write(self) -> np.ndarray:
        """Lengths once ``k_new``/``v_new`` are appended (one token each)."""
        out = self.seq_lens.copy()
        written = self.slot_mapping >= 0
        out[written[: len(out)]] += 1
        return out


def _f32_scale(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def build(
    *,
    name: str,
    rng: np.random.Generator,
    seq_lens: Sequence[int],
    n_heads: int,
    n_kv_heads: int,
    head_dim: int,
    block_size: int,
    dtype: torch.dtype,
    num_blocks: Optional[int] = None,
    pool_factor: float = 1.2,
    max_len: Optional[int] = None,
    shared_prefix_tokens: int = 0,
    samples_per_prompt: int = 1,
    scale: Optional[float] = None,
    poison: bool = False,
    values: bool = True,
    seed: int = 0,
) -> Workload:
    """Build pool, tables, values and the append slots for one batch.

    ``shared_prefix_tokens`` > 0 (a multiple of ``block_size``) gives every group
    of ``samples_per_prompt`` consecutive sequences the same prefix blocks; the
    remaining tokens of each sequence live in private blocks. ``seq_lens`` are
    the full lengths (prefix included).

    ``poison=True`` fills every pool slot that no sequence may read (blocks no
    table references, and slots at or past ``seq_len`` in each last block) with
    NaN, so a kernel that reads or mixes them in shows it.

    ``values=False`` stops after the tables (no value draws): tensors are empty,
    which keeps layout-only checks of the large configs cheap.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    BS = block_size
    if n_heads % n_kv_heads:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    if shared_prefix_tokens % BS:
        raise ValueError("shared prefix must be whole blocks")
    if shared_prefix_tokens and B % samples_per_prompt:
        raise ValueError("batch must be whole prompt groups")
    if max_len is None:
        max_len = int(seq_lens.max()) if B else 0
    # Room for the appended token: one more block only when the new token
    # starts a block (on-demand growth).
    mb = max(1, -(-(max_len + 1) // BS))

    n_prefix_blocks = shared_prefix_tokens // BS
    n_prompts = B // samples_per_prompt if shared_prefix_tokens else 0
    private_blocks = [-(-(int(L) + 1 - shared_prefix_tokens) // BS) for L in seq_lens]
    need = n_prompts * n_prefix_blocks + sum(private_blocks)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need))
    if num_blocks < need:
        raise ValueError(f"pool of {num_blocks} blocks < {need} needed")
    perm = rng.permutation(num_blocks).astype(np.int64)

    tables = np.full((B, mb), -1, dtype=np.int32)
    refcount = np.zeros(num_blocks, dtype=np.int32)
    cursor = 0
    prefix_ids = []
    for _ in range(n_prompts):
        prefix_ids.append(perm[cursor: cursor + n_prefix_blocks])
        cursor += n_prefix_blocks
    for s in range(B):
        ids = []
        if shared_prefix_tokens:
            ids.extend(prefix_ids[s // samples_per_prompt].tolist())
        ids.extend(perm[cursor: cursor + private_blocks[s]].tolist())
        cursor += private_blocks[s]
        tables[s, : len(ids)] = ids
        refcount[ids] += 1

    H, Hkv, D = n_heads, n_kv_heads, head_dim
    if values:
        q = _normal(rng, (B, H, D), dtype)
        k_pool = _normal(rng, (num_blocks, Hkv, BS, D), dtype)
        v_pool = _normal(rng, (num_blocks, Hkv, BS, D), dtype)
        k_new = _normal(rng, (B, Hkv, D), dtype)
        v_new = _normal(rng, (B, Hkv, D), dtype)
    else:
        q = k_pool = v_pool = k_new = v_new = torch.empty(0, dtype=dtype)

    slots = np.empty(B, dtype=np.int32)
    for s in range(B):
        L = int(seq_lens[s])
        slots[s] = int(tables[s, L // BS]) * BS + L % BS

    if poison and values:
        nan = float("nan")
        unused = refcount == 0
        k_pool[torch.from_numpy(unused)] = nan
        v_pool[torch.from_numpy(unused)] = nan
        for s in range(B):
            L = int(seq_lens[s])
            blk = int(tables[s, L // BS])
            k_pool[blk, :, L % BS:, :] = nan
            v_pool[blk, :, L % BS:, :] = nan

    return Workload(
        name=name, dtype=dtype, num_seqs=B, n_heads=H, n_kv_heads=Hkv, head_dim=D,
        block_size=BS, scale=_f32_scale(D) if scale is None else float(np.float32(scale)),
        seq_lens=seq_lens.astype(np.int32), block_tables=tables, num_blocks=int(num_blocks),
        q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
        slot_mapping=slots, refcount=refcount, seed=seed,
    )


def build_groups(*, name: str, rng: np.random.Generator, group_sizes: Sequence[int],
                 prefix_blocks: Sequence[int], private_lens: Sequence[int], n_heads: int, n_kv_heads: int,
                 head_dim: int, block_size: int, dtype: torch.dtype, pool_factor: float = 1.3,
                 poison: bool = False, seed: int = 0) -> Workload:
    """A batch of consecutive sequence groups: group ``i`` has ``group_sizes[i]``
    members whose tables start with the same ``prefix_blocks[i]`` physical
    blocks (full of prefix tokens); member ``s`` then holds
    ``private_lens[s]`` tokens of its own in private blocks, so
    ``seq_lens[s] = prefix_blocks[group] * block_size + private_lens[s]``.
    Physical ids are a random permutation of the pool; ``poison`` fills every
    slot no sequence may read with NaN."""
    BS = block_size
    sizes = [int(x) for x in group_sizes]
    pblk = [int(x) for x in prefix_blocks]
    priv = [int(x) for x in private_lens]
    B = sum(sizes)
    if len(pblk) != len(sizes) or len(priv) != B:
        raise ValueError("one prefix per group, one private length per sequence")
    group_of = np.repeat(np.arange(len(sizes)), sizes)
    seq_lens = np.array([pblk[group_of[s]] * BS + priv[s] for s in range(B)], dtype=np.int64)
    mb = max(1, -(-(int(seq_lens.max()) + 1) // BS)) if B else 1
    private_blocks = [-(-(priv[s] + 1) // BS) for s in range(B)]
    need = sum(pblk) + sum(private_blocks)
    num_blocks = int(math.ceil(pool_factor * need))
    perm = rng.permutation(num_blocks).astype(np.int64)
    tables = np.full((B, mb), -1, dtype=np.int32)
    refcount = np.zeros(num_blocks, dtype=np.int32)
    cursor = 0
    prefix_ids = []
    for n in pblk:
        prefix_ids.append(perm[cursor: cursor + n].tolist())
        cursor += n
    for s in range(B):
        ids = prefix_ids[group_of[s]] + perm[cursor: cursor + private_blocks[s]].tolist()
        cursor += private_blocks[s]
        tables[s, : len(ids)] = ids
        refcount[ids] += 1
    H, Hkv, D = n_heads, n_kv_heads, head_dim
    q = _normal(rng, (B, H, D), dtype)
    k_pool = _normal(rng, (num_blocks, Hkv, BS, D), dtype)
    v_pool = _normal(rng, (num_blocks, Hkv, BS, D), dtype)
    k_new = _normal(rng, (B, Hkv, D), dtype)
    v_new = _normal(rng, (B, Hkv, D), dtype)
    slots = np.array([int(tables[s, int(seq_lens[s]) // BS]) * BS + int(seq_lens[s]) % BS for s in range(B)],
                     dtype=np.int32)
    if poison:
        nan = float("nan")
        unused = torch.from_numpy(refcount == 0)
        k_pool[unused] = nan
        v_pool[unused] = nan
        for s in range(B):
            L = int(seq_lens[s])
            blk = int(tables[s, L // BS])
            k_pool[blk, :, L % BS:, :] = nan
            v_pool[blk, :, L % BS:, :] = nan
    return Workload(
        name=name, dtype=dtype, num_seqs=B, n_heads=H, n_kv_heads=Hkv, head_dim=D, block_size=BS,
        scale=_f32_scale(D), seq_lens=seq_lens.astype(np.int32), block_tables=tables, num_blocks=num_blocks,
        q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, slot_mapping=slots,
        refcount=refcount, seed=seed,
    )


CONFIG_NAMES = {
    1: "tiny fp32 paged decode, B=4, H=Hkv=4, D=64, BS=16, L~U[1,100], pool 32",
    2: "MHA bf16 paged decode, B=64, H=Hkv=32, D=128, BS=16, L~U[128,2048]",
    3: "GQA bf16 paged decode, B=128, H=32, Hkv=8, D=128, BS=16, L=lognormal(ln512,0.8) in [16,4096]",
    4: "long-context split-K bf16 paged decode, B=4, H=32, Hkv=8, D=128, BS=16, L={32K,64K,96K,128K}",
    5: "shared-prefix fp16 paged decode, 16 prompts x 4 samples, H=32, Hkv=8, D=128, BS=32, prefix 1024 + U[64,512]",
}


def make(cfg_id: int, seed: Optional[int] = None, poison: bool = False,
         values: bool = True) -> Workload:
    """The five benchmark/parity configurations (seed defaults to 2600 + cfg_id)."""
    seed = 2600 + cfg_id if seed is None else seed
    kw = dict(poison=poison, values=values, seed=seed)
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[cfg_id]
    if cfg_id == 1:
        lens = rng.integers(1, 101, size=4)
        return build(name=name, rng=rng, seq_lens=lens, n_heads=4, n_kv_heads=4, head_dim=64,
                     block_size=16, dtype=torch.float32, num_blocks=32, max_len=100,
                     **kw)
    if cfg_id == 2:
        lens = rng.integers(128, 2049, size=64)
        return build(name=name, rng=rng, seq_lens=lens, n_heads=32, n_kv_heads=32, head_dim=128,
                     block_size=16, dtype=torch.bfloat16, max_len=2048, **kw)
    if cfg_id == 3:
        lens = lognormal_lengths(rng, 128, 512.0, 0.8, 16, 4096)
        return build(name=name, rng=rng, seq_lens=lens, n_heads=32, n_kv_heads=8, head_dim=128,
                     block_size=16, dtype=torch.bfloat16, max_len=4096, **kw)
    if cfg_id == 4:
        lens = [32768, 65536, 98304, 131072]
        return build(name=name, rng=rng, seq_lens=lens, n_heads=32, n_kv_heads=8, head_dim=128,
                     block_size=16, dtype=torch.bfloat16, max_len=131072, **kw)
    if cfg_id == 5:
        private = rng.integers(64, 513, size=64)
        lens = 1024 + private
        return build(name=name, rng=rng, seq_lens=lens, n_heads=32, n_kv_heads=8, head_dim=128,
                     block_size=32, dtype=torch.float16, max_len=1024 + 512,
                     shared_prefix_tokens=1024, samples_per_prompt=4, **kw)
    raise ValueError(f"unknown config {cfg_id}")


def lognormal_lengths(rng, n, median, sigma, lo, hi) -> np.ndarray:
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def random_case(seed: int, *, num_seqs: int, n_heads: int, n_kv_heads: int, head_dim: int,
                block_size: int, dtype: torch.dtype, max_len: int, min_len: int = 1,
                poison: bool = False, pool_factor: float = 1.5) -> Workload:
    """A small random case with uniform lengths in ``[min_len, max_len]``."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=num_seqs)
    return build(name=f"random seed={seed}", rng=rng, seq_lens=lens, n_heads=n_heads,
                 n_kv_heads=n_kv_heads, head_dim=head_dim, block_size=block_size, dtype=dtype,
                 max_len=max_len, pool_factor=pool_factor, poison=poison, seed=seed)


def contiguous_case(rng: np.random.Generator, *, seq_lens, n_heads, n_kv_heads, head_dim,
                    block_size, dtype, num_blocks):
    """Contiguous per-sequence K/V plus a shuffled pool holding the same rows.

    Returns ``(q, k_seq, v_seq, k_pool, v_pool, block_tables)`` where ``k_seq[s]``
    is ``[Hkv, L_s, D]``. The pool is filled by scattering the contiguous rows
    to randomly permuted physical blocks, the inverse of the gather a paged
    kernel performs, so a test can compare paged against contiguous attention.
    """
    B = len(seq_lens)
    BS = block_size
    mb = max(1, max(-(-int(L) // BS) for L in seq_lens))
    need = sum(-(-int(L) // BS) for L in seq_lens)
    assert num_blocks >= need
    perm = rng.permutation(num_blocks)
    q = _normal(rng, (B, n_heads, head_dim), dtype)
    k_pool = _normal(rng, (num_blocks, n_kv_heads, BS, head_dim), dtype)
    v_pool = _normal(rng, (num_blocks, n_kv_heads, BS, head_dim), dtype)
    tables = np.full((B, mb), -1, dtype=np.int32)
    k_seq, v_seq = [], []
    cur = 0
    for s, L in enumerate(seq_lens):
        L = int(L)
        nb = -(-L // BS)
        ids = perm[cur: cur + nb]
        cur += nb
        tables[s, :nb] = ids
        ks = _normal(rng, (n_kv_heads, L, head_dim), dtype)
        vs = _normal(rng, (n_kv_heads, L, head_dim), dtype)
        for j in range(L):
            k_pool[ids[j // BS], :, j % BS, :] = ks[:, j, :]
            v_pool[ids[j // BS], :, j % BS, :] = vs[:, j, :]
        k_seq.append(ks)
        v_seq.append(vs)
    return q, k_seq, v_seq, k_pool, v_pool, tables
