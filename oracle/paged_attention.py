"""fp64 oracle for PagedAttention decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
library, and it shares no code with the HIP path.

What is computed (plain definition):

* The vLLM paper page ("PagedAttention" core-idea section and its block-pool
  diagram): a sequence's K/V live in fixed-size blocks scattered through one
  pool, and the attention reads them through the per-sequence block table
  (logical block i -> physical block ``block_tables[s, i]``).
* The vLLM notes page ("FlashAttention" section): tiling with an online
  softmax is exact, giving the same output as standard attention. So the
  oracle is standard attention, computed directly, over the gathered rows.
* The ICML-tutorial notes page ("architecture design" part, MQA/GQA): several
  query heads share one K/V head. Reading taken here: contiguous groups, query
  head ``h`` uses KV head ``h // (H / Hkv)``.

For one decode step of sequence ``s`` and query head ``h`` (``g = h // G``)::

    K_s[j] = k_pool[block_tables[s, j // BS], g, j % BS, :]   for j < L_s
    z_j    = scale * <q[s, h], K_s[j]>
    p_j    = exp(z_j - max z) / sum_k exp(z_k - max z)
    out[s, h] = sum_j p_j * V_s[j]

with no mask (the one query is the newest position and sees every cached
token) and ``out = 0`` for ``L_s = 0``. All arithmetic is float64 on inputs
converted exactly from their storage dtype.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def gather_tokens(pool, table_row, kv_head: int, seq_len: int, block_size: int) -> np.ndarray:
    """Rows of one sequence at one KV head in token order, read through its block table.

    Token ``j`` lives at offset ``j % BS`` of physical block
    ``table_row[j // BS]``; only the ``ceil(L / BS)`` table entries that hold a
    token are read.
    """
    n_blocks = -(-seq_len // block_size)
    if n_blocks == 0:
        return np.zeros((0, pool.shape[-1]), dtype=np.float64)
    phys = np.asarray(table_row[:n_blocks], dtype=np.int64)
    tiles = _f64(pool[phys, kv_head])                  # [n_blocks, BS, D]
    return tiles.reshape(n_blocks * block_size, -1)[:seq_len]


def attention_weights(q_rows, keys, scale: float) -> np.ndarray:
    """Softmax weights ``p`` (rows of ``q_rows`` against ``keys``), exact softmax in fp64."""
    z = float(scale) * (_f64(q_rows) @ _f64(keys).T)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _check(q, k_pool, v_pool, block_tables, seq_lens, n_heads, n_kv_heads, head_dim, block_size):
    B = len(seq_lens)
    if n_heads % n_kv_heads:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    if q.shape != (B, n_heads, head_dim):
        raise ValueError(f"q shape {q.shape}")
    if k_pool.shape[1:] != (n_kv_heads, block_size, head_dim) or v_pool.shape != k_pool.shape:
        raise ValueError(f"pool shape {k_pool.shape}")
    if block_tables.shape[0] != B:
        raise ValueError("block_tables rows != batch")
    for s, L in enumerate(seq_lens):
        if L < 0 or L > block_tables.shape[1] * block_size:
            raise ValueError(f"seq_len {L} out of range for sequence {s}")


def paged_attn_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads,
                      head_dim, block_size) -> np.ndarray:
    """``out[s, h]`` for every sequence and query head, float64 ``[B, H, D]``."""
    q = np.asarray(q)
    block_tables = np.asarray(block_tables)
    seq_lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    _check(q, k_pool, v_pool, block_tables, seq_lens, n_heads, n_kv_heads, head_dim, block_size)
    G = n_heads // n_kv_heads
    out = np.zeros((len(seq_lens), n_heads, head_dim), dtype=np.float64)
    for s, L in enumerate(seq_lens):
        if L == 0:
            continue
        for g in range(n_kv_heads):
            K = gather_tokens(k_pool, block_tables[s], g, L, block_size)
            V = gather_tokens(v_pool, block_tables[s], g, L, block_size)
            heads = slice(g * G, (g + 1) * G)
            P = attention_weights(q[s, heads], K, scale)       # [G, L]
            out[s, heads] = P @ V
    return out


def paged_attn_decode_partitioned(q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads,
                                  n_kv_heads, head_dim, block_size, partition_tokens):
    """Decode split along the sequence (the FlashDecoding idea on the ICML-tutorial page,
    kernel-optimisation part) and merged with the online-softmax rescaling of the
    vLLM notes page ("FlashAttention" section), all in fp64.

    Partition ``p`` covers tokens ``[p*P, min(L, (p+1)*P))`` and yields
    ``m_p = max z``, ``l_p = sum exp(z - m_p)``, ``acc_p = sum exp(z - m_p) v``.
    The merge takes ``M = max_p m_p`` and returns
    ``sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p``.

    Returns ``(out, partials)`` where ``partials[(s, h)]`` is the list of
    ``(m_p, l_p, acc_p)``.
    """
    q = np.asarray(q)
    block_tables = np.asarray(block_tables)
    seq_lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    _check(q, k_pool, v_pool, block_tables, seq_lens, n_heads, n_kv_heads, head_dim, block_size)
    G = n_heads // n_kv_heads
    out = np.zeros((len(seq_lens), n_heads, head_dim), dtype=np.float64)
    partials = {}
    for s, L in enumerate(seq_lens):
        if L == 0:
            continue
        for g in range(n_kv_heads):
            K = gather_tokens(k_pool, block_tables[s], g, L, block_size)
            V = gather_tokens(v_pool, block_tables[s], g, L, block_size)
            for h in range(g * G, (g + 1) * G):
                parts = []
                for start in range(0, L, partition_tokens):
                    stop = min(L, start + partition_tokens)
                    z = float(scale) * (K[start:stop] @ _f64(q[s, h]))
                    m = z.max()
                    e = np.exp(z - m)
                    parts.append((m, e.sum(), e @ V[start:stop]))
                M = max(m for m, _, _ in parts)
                num = sum(np.exp(m - M) * acc for m, _, acc in parts)
                den = sum(np.exp(m - M) * l for m, l, _ in parts)
                out[s, h] = num / den
                partials[(s, h)] = parts
    return out, partials


def paged_attn_chunk(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, scale, n_heads,
                     n_kv_heads, head_dim, block_size) -> np.ndarray:
    """Attention of a chunk of new query tokens per sequence, causal inside the chunk.

    Several new tokens of one sequence are scored in one pass. Sources:
      - Sarathi-Serve chunked prefill (PagedAttention notes page): a long
        prompt's prefill is cut into chunks interleaved with decodes.
      - Speculative decoding (vLLM notes page): the target model scores K
        draft tokens at once.
      - Continuous batching (vLLM notes page, scheduling section): sequences
        are packed into one flat token list; position indices and the
        attention mask keep each token on its own sequence.

    Readings: ``q`` is the packed ``[T, H, D]`` chunk rows; the rows of
    sequence ``s`` are ``query_start_loc[s] .. query_start_loc[s + 1] - 1``.
    These ``n_s`` tokens are the last ``n_s`` of the sequence's ``L_s`` cached
    tokens (their K/V are already written). Token ``i`` of the chunk sits at
    position ``p = L_s - n_s + i`` and, as in autoregressive decoding, sees
    every cached token at positions ``0 .. p``. ``n_s = 1`` is one decode
    step; ``n_s = L_s`` is a whole causal prefill.
    """
    q = np.asarray(q)
    block_tables = np.asarray(block_tables)
    qsl = [int(x) for x in np.asarray(query_start_loc).reshape(-1)]
    seq_lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    B = len(seq_lens)
    if len(qsl) != B + 1 or any(qsl[s + 1] < qsl[s] for s in range(B)):
        raise ValueError("query_start_loc must be [B + 1], nondecreasing")
    if q.shape != (qsl[-1], n_heads, head_dim):
        raise ValueError(f"q shape {q.shape}")
    G = n_heads // n_kv_heads
    out = np.zeros((qsl[-1], n_heads, head_dim), dtype=np.float64)
    for s, L in enumerate(seq_lens):
        n = qsl[s + 1] - qsl[s]
        if n == 0:
            continue
        if n > L or L > block_tables.shape[1] * block_size:
            raise ValueError(f"sequence {s}: {n} query tokens, {L} cached")
        for g in range(n_kv_heads):
            K = gather_tokens(k_pool, block_tables[s], g, L, block_size)
            V = gather_tokens(v_pool, block_tables[s], g, L, block_size)
            for i in range(n):
                p = L - n + i
                rows = q[qsl[s] + i, g * G:(g + 1) * G]
                P = attention_weights(rows, K[:p + 1], scale)   # [G, p + 1]
                out[qsl[s] + i, g * G:(g + 1) * G] = P @ V[:p + 1]
    return out
