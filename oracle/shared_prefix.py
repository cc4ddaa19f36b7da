"""Oracle for decode over sequences that share a prompt prefix: the grouping
of a batch by shared leading blocks, and the shared-prefix decode itself.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  - vLLM paper page, OS-paging analogy table: page sharing corresponds to
    block sharing for parallel sampling, beam search and prefix caching;
    "PagedAttention" core idea: one prompt prefix, or the samples of one
    request, can use the same KV blocks; system implementation points:
    samples of parallel sampling share the prompt's KV blocks.
  - vLLM notes page, "FlashAttention": online softmax (running max and sum)
    is exact, so attention over a token range can be split into pieces whose
    partial states (m, l, acc) are merged afterwards;
  - ICML-tutorial notes page, FlashDecoding: such a split along the sequence,
    merged with the same rescaling.

Readings (the pages fix no interface for this):
  - A group is a run of consecutive sequences whose block tables start with
    the same physical blocks. The prefix is counted in whole blocks that
    every member holds in common and that lie inside every member's length.
  - The shared-prefix decode computes, per sequence and head, the plain decode
    result: a prefix partial over tokens [0, p) read once through the group's
    first member's table, a private partial over [p, L) through the
    sequence's own table, and the two merged exactly.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import gather_tokens


def shared_prefix_groups(block_tables, seq_lens, block_size: int):
    """``(group_start, prefix_lens)`` of a batch, from its tables (host lists).

    Sequences are taken in order. A sequence joins the open group when its
    first table entry is held by the group's first member and it has at least
    one full block; the group's prefix is then the number of leading entries
    that every member shares with the first member, capped by each member's
    full blocks ``L // block_size``. A group of one sequence has prefix 0.
    """
    tables = [list(map(int, row)) for row in np.asarray(block_tables)]
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    B = len(lens)
    group_start, prefix_lens = [], [0] * B
    s = 0
    while s < B:
        first = tables[s]
        members = [s]
        shared = lens[s] // block_size
        e = s + 1
        while e < B:
            common = 0
            while (common < min(shared, lens[e] // block_size) and tables[e][common] == first[common]):
                common += 1
            if common == 0:
                break
            shared = common
            members.append(e)
            e += 1
        group_start.append(s)
        for m in members:
            prefix_lens[m] = shared * block_size if len(members) > 1 else 0
        s = e
    group_start.append(B)
    return np.array(group_start, dtype=np.int32), np.array(prefix_lens, dtype=np.int32)


def _partial(q_row, K, V, scale):
    """Partial softmax state of one query row over the rows ``K``/``V``:
    ``(m, l, acc)`` with ``m = max z``, ``l = sum e^(z - m)``,
    ``acc = sum e^(z - m) v`` (``m = -inf``, ``l = 0``, ``acc = 0`` when empty)."""
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1])
    z = float(scale) * (K @ np.asarray(q_row, dtype=np.float64))
    m = z.max()
    e = np.exp(z - m)
    return m, e.sum(), e @ V


def _merge(parts):
    """Exact merge of partial states: ``sum e^(m_i - M) acc_i / sum e^(m_i - M) l_i``."""
    live = [(m, l, acc) for m, l, acc in parts if m > -np.inf]
    M = max(m for m, _, _ in live)
    num = sum(np.exp(m - M) * acc for m, _, acc in live)
    den = sum(np.exp(m - M) * l for m, l, _ in live)
    return num / den


def paged_attn_decode_shared_prefix(q, k_pool, v_pool, block_tables, seq_lens, prefix_lens, group_start,
                                    scale, n_heads, n_kv_heads, head_dim, block_size) -> np.ndarray:
    """Decode ``out[s, h]`` (float64 ``[B, H, D]``) computed the shared-prefix
    way: per group and KV head, the prefix rows are gathered once through the
    first member's table and every member's query heads are scored against
    them; each sequence's own tokens after the prefix give a second partial;
    the two are merged. Raises on a description that breaks the sharing
    precondition (so a test can never pass on a wrong description)."""
    q = np.asarray(q)
    tables = np.asarray(block_tables)
    lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    pre = [int(x) for x in np.asarray(prefix_lens).reshape(-1)]
    gs = [int(x) for x in np.asarray(group_start).reshape(-1)]
    B = len(lens)
    if gs[0] != 0 or gs[-1] != B or any(gs[i + 1] <= gs[i] for i in range(len(gs) - 1)):
        raise ValueError("group_start must split [0, B) into consecutive non-empty groups")
    G = n_heads // n_kv_heads
    out = np.zeros((B, n_heads, head_dim), dtype=np.float64)
    for gi in range(len(gs) - 1):
        members = range(gs[gi], gs[gi + 1])
        p = pre[gs[gi]]
        nb = p // block_size
        for s in members:
            if pre[s] != p or p % block_size or p > lens[s]:
                raise ValueError(f"sequence {s}: prefix {pre[s]} breaks the group's prefix {p}")
            if list(tables[s][:nb]) != list(tables[gs[gi]][:nb]):
                raise ValueError(f"sequence {s} does not share the group's prefix blocks")
        for g in range(n_kv_heads):
            Kp = gather_tokens(k_pool, tables[gs[gi]], g, p, block_size)  # read once per group
            Vp = gather_tokens(v_pool, tables[gs[gi]], g, p, block_size)
            for s in members:
                L = lens[s]
                if L == 0:
                    continue
                K = gather_tokens(k_pool, tables[s], g, L, block_size)[p:]
                V = gather_tokens(v_pool, tables[s], g, L, block_size)[p:]
                for h in range(g * G, (g + 1) * G):
                    out[s, h] = _merge([_partial(q[s, h], Kp, Vp, scale), _partial(q[s, h], K, V, scale)])
    return out
