"""Byte accounting for paged decode and the cache write.

Closed forms used by the benchmark to turn a kernel time into an effective
bandwidth, plus the KV-sizing formulas the course page states ("MLSys II"
page, section 6 example 1 for the per-request KV size; the "formal mechanism"
section for peak KV = bytes per token times the peak number of active tokens).
"""
from __future__ import annotations

import numpy as np


def kv_cache_bytes(layers: int, hidden: int, tokens: int, elem_bytes: int) -> int:
    """K and V of every layer for ``tokens`` tokens: ``2 * layers * hidden * tokens * e``."""
    return 2 * layers * hidden * tokens * elem_bytes


def peak_kv_bytes(bytes_per_token: float, max_active_tokens: int) -> float:
    """Peak KV reserve: bytes per token times the peak count of active tokens."""
    return bytes_per_token * max_active_tokens


def decode_kv_bytes(seq_lens, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes a decode pass must read once: ``sum_s L_s * Hkv * D * 2 * e``."""
    total_tokens = int(np.asarray(seq_lens, dtype=np.int64).sum())
    return total_tokens * n_kv_heads * head_dim * 2 * elem_bytes


def decode_qo_bytes(num_seqs: int, n_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Query read plus output write: ``2 * B * H * D * e``."""
    return 2 * num_seqs * n_heads * head_dim * elem_bytes


def decode_compulsory_bytes(seq_lens, n_heads, n_kv_heads, head_dim, elem_bytes) -> int:
    """Compulsory HBM bytes of one decode batch (KV + Q + O); table reads excluded."""
    return (decode_kv_bytes(seq_lens, n_kv_heads, head_dim, elem_bytes)
            + decode_qo_bytes(len(seq_lens), n_heads, head_dim, elem_bytes))


def decode_table_bytes(seq_lens, block_size: int) -> int:
    """Block-table entries and lengths read (int32): reported, not in the headline."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return int(4 * (-(-lens // block_size)).sum() + 4 * len(lens))


def unique_kv_tokens(seq_lens, block_tables, block_size: int) -> int:
    """Distinct (physical block, offset) token slots a batch reads.

    With prefix sharing several tables point at one physical block; its tokens
    are compulsory once. The count is the union over sequences of the slots
    ``block_tables[s, j // BS] * BS + j % BS`` for ``j < L_s``.
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables, dtype=np.int64)
    slots = []
    for s, L in enumerate(lens):
        j = np.arange(int(L), dtype=np.int64)
        slots.append(bt[s, j // block_size] * block_size + j % block_size)
    if not slots:
        return 0
    return int(np.unique(np.concatenate(slots)).size)


def write_bytes(num_written: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Cache write: read k_new and v_new, write them into the pools (4 rows per token-head)."""
    return 4 * num_written * n_kv_heads * head_dim * elem_bytes


def decode_append_bytes(seq_lens_after, num_written, n_heads, n_kv_heads, head_dim, elem_bytes,
                        block_tables=None, block_size=None) -> int:
    """Compulsory bytes of one decode step that appends each sequence's new
    token and attends over all ``L + 1`` tokens: the decode bytes at the new
    lengths (the new K/V rows are read once, as part of them) plus the new rows
    stored into the pools (``2 * n * Hkv * D * e``). With the block tables, K/V
    bytes count each distinct cached slot once (shared prefix blocks)."""
    if block_tables is None:
        kv_tokens = int(np.asarray(seq_lens_after, dtype=np.int64).sum())
    else:
        kv_tokens = unique_kv_tokens(seq_lens_after, block_tables, block_size)
    return (kv_tokens * n_kv_heads * head_dim * 2 * elem_bytes
            + decode_qo_bytes(len(seq_lens_after), n_heads, head_dim, elem_bytes)
            + 2 * num_written * n_kv_heads * head_dim * elem_bytes)


def utilisation(seq_lens, block_size: int) -> float:
    """Share of allocated block slots that hold a cached token: ``sum L / (sum ceil(L/BS) * BS)``."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    alloc = (-(-lens // block_size)).sum() * block_size
    return float(lens.sum() / alloc) if alloc else 1.0
