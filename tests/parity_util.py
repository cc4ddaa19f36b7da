"""Helpers shared by the GPU parity tests: move seeded workloads to the GPU,
run the HIP path through the C ABI binding, and run the fp64 oracle on the
same (identically rounded) inputs one KV head at a time."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_cache_260_amd import _lib

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2, torch.float16: 1e-2}


def f32np(t: torch.Tensor) -> np.ndarray:
    """Exact float32 numpy copy (bf16/fp16/fp32 all convert exactly)."""
    return t.detach().to("cpu", torch.float32).numpy()


class OnGpu:
    """Device copies of a workload's tensors."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.q = w.q.to(device)
        self.k_pool = w.k_pool.to(device)
        self.v_pool = w.v_pool.to(device)
        self.k_new = w.k_new.to(device)
        self.v_new = w.v_new.to(device)
        self.block_tables = torch.from_numpy(w.block_tables).to(device)
        self.seq_lens = torch.from_numpy(w.seq_lens).to(device)
        self.slot_mapping = torch.from_numpy(w.slot_mapping).to(device)

    def decode(self, seq_lens=None, out=None, stream=None):
        w = self.w
        sl = self.seq_lens if seq_lens is None else seq_lens
        if out is None:
            out = torch.empty_like(self.q)
        _lib.paged_attn_decode(out, self.q, self.k_pool, self.v_pool, self.block_tables, sl,
                               w.scale, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size,
                               stream=stream)
        return out

    def write(self):
        _lib.kv_cache_write(self.k_pool, self.v_pool, self.k_new, self.v_new, self.slot_mapping)


def oracle_decode(w, seq_lens, k_pool, v_pool, kv_heads=None, q=None) -> np.ndarray:
    """Oracle output ``[B, H, D]``, one KV head at a time; with ``kv_heads``
    only those heads' query rows are computed (the others hold NaN, and a
    comparison must then name the rows it covers, see ``max_abs_err``)."""
    q = w.q if q is None else q
    G = w.group
    B, H, D = q.shape
    out = np.full((B, H, D), np.nan)
    heads = range(w.n_kv_heads) if kv_heads is None else kv_heads
    qn = f32np(q)
    for g in heads:
        kp = f32np(k_pool[:, g:g + 1])
        vp = f32np(v_pool[:, g:g + 1])
        out[:, g * G:(g + 1) * G] = oracle.paged_attn_decode(
            qn[:, g * G:(g + 1) * G], kp, vp, w.block_tables, seq_lens, w.scale, G, 1, D,
            w.block_size)
    return out


def oracle_write(w, k_pool, v_pool):
    """Oracle scatter on integer views (bitwise), returns torch tensors of the pool dtype."""
    ints = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}[w.dtype]
    kp, vp = oracle.kv_cache_write(k_pool.view(ints).numpy(), v_pool.view(ints).numpy(),
                                   w.k_new.view(ints).numpy(), w.v_new.view(ints).numpy(),
                                   w.slot_mapping, w.block_size)
    return torch.from_numpy(kp).view(w.dtype), torch.from_numpy(vp).view(w.dtype)


def max_abs_err(gpu_out: torch.Tensor, ref: np.ndarray, rows=None) -> float:
    """Largest |gpu - ref| over the compared elements: all of them, or those
    ``rows`` selects (a boolean mask or index over the leading dimensions).
    The reference must be finite wherever it is compared (a NaN there is an
    oracle or fixture fault, never a reason to compare less), and so must the
    GPU output."""
    got = gpu_out.detach().to("cpu", torch.float64).numpy()
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"shape {got.shape} vs reference {ref.shape}"
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert ref.size > 0, "nothing compared"
    assert np.all(np.isfinite(ref)), "non-finite reference among the compared elements"
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)))
