"""GPU parity of multi-token (chunk) attention through the C ABI against the
fp64 oracle: decode-sized chunks, speculative-verification chunks, prefill
chunks and whole-sequence prefill, mixed batches, and invalid lengths."""
import sys

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_260_amd import _lib, workloads
from parity_util import TOL, f32np, max_abs_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def chunk_inputs(w, qlens, seed):
    qlens = np.asarray(qlens, dtype=np.int64)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(int(qsl[-1]), w.n_heads, w.head_dim, generator=g).to(w.dtype)
    return q, qsl


def run_gpu(w, q, qsl, seq_lens=None):
    dev = "cuda"
    lens = w.seq_lens if seq_lens is None else seq_lens
    out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    maxq = int(np.max(np.diff(qsl))) if len(qsl) > 1 else 0
    _lib.paged_attn_chunk(out, q.to(dev), w.k_pool.to(dev), w.v_pool.to(dev),
                          torch.from_numpy(w.block_tables).to(dev), torch.from_numpy(np.asarray(lens, np.int32)).to(dev),
                          torch.from_numpy(qsl).to(dev), w.scale, w.n_heads, w.n_kv_heads, w.head_dim,
                          w.block_size, maxq)
    torch.cuda.synchronize()
    return out


def run_oracle(w, q, qsl, seq_lens=None):
    lens = w.seq_lens if seq_lens is None else seq_lens
    G, D = w.group, w.head_dim
    out = np.zeros(tuple(q.shape))
    qn = f32np(q)
    for g in range(w.n_kv_heads):
        out[:, g * G:(g + 1) * G] = oracle.paged_attn_chunk(
            qn[:, g * G:(g + 1) * G], f32np(w.k_pool[:, g:g + 1]), f32np(w.v_pool[:, g:g + 1]), w.block_tables,
            lens, qsl, w.scale, G, 1, D, w.block_size)
    return out


def test_one_token_chunks_equal_decode():
    w = workloads.random_case(11, num_seqs=7, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                              dtype=torch.bfloat16, max_len=2000, poison=True)
    q = w.q
    qsl = np.arange(w.num_seqs + 1, dtype=np.int32)
    out = run_gpu(w, q, qsl)
    ref = oracle.paged_attn_decode(f32np(q), f32np(w.k_pool).astype(np.float64), f32np(w.v_pool), w.block_tables,
                                   w.seq_lens, w.scale, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size)
    assert max_abs_err(out, ref) <= TOL[w.dtype]


@pytest.mark.parametrize("qlen", [2, 4, 5])
def test_speculative_chunks_gqa_batch(qlen):
    """The GQA batch-128 shapes (lognormal lengths) verifying qlen draft tokens."""
    say(f"speculative chunk qlen={qlen}")
    w = workloads.make(3, poison=True)
    q, qsl = chunk_inputs(w, np.minimum(qlen, w.seq_lens), 100 + qlen)
    out = run_gpu(w, q, qsl)
    err = max_abs_err(out, run_oracle(w, q, qsl))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("H,Hkv,D,BS,dtype", [(32, 8, 128, 16, torch.bfloat16), (8, 8, 64, 32, torch.float16),
                                              (16, 2, 128, 128, torch.float16), (12, 4, 64, 16, torch.bfloat16)])
def test_prefill_chunks(H, Hkv, D, BS, dtype):
    """Chunks of tens to hundreds of tokens over contexts up to 2 900 tokens
    (several 64-block segments at block 16), with a ragged tail."""
    w = workloads.random_case(20 + D + BS, num_seqs=4, n_heads=H, n_kv_heads=Hkv, head_dim=D, block_size=BS,
                              dtype=dtype, max_len=2900, min_len=300, poison=True)
    rng = np.random.default_rng(BS)
    qlens = np.minimum(rng.integers(1, 300, size=w.num_seqs), w.seq_lens)
    q, qsl = chunk_inputs(w, qlens, D)
    out = run_gpu(w, q, qsl)
    assert max_abs_err(out, run_oracle(w, q, qsl)) <= TOL[dtype]


def test_whole_sequence_prefill_and_mixed_batch():
    """Whole-sequence chunks, decode steps and empty chunks in one batch."""
    w = workloads.random_case(31, num_seqs=6, n_heads=16, n_kv_heads=4, head_dim=128, block_size=16,
                              dtype=torch.bfloat16, max_len=400, min_len=1, poison=True)
    qlens = np.array([w.seq_lens[0], 1, 0, min(37, w.seq_lens[3]), w.seq_lens[4], 1])
    q, qsl = chunk_inputs(w, qlens, 5)
    out = run_gpu(w, q, qsl)
    assert max_abs_err(out, run_oracle(w, q, qsl)) <= TOL[w.dtype]


def test_invalid_lengths_give_nan_rows():
    w = workloads.random_case(41, num_seqs=3, n_heads=8, n_kv_heads=2, head_dim=64, block_size=16,
                              dtype=torch.float16, max_len=100, min_len=10)
    lens = w.seq_lens.copy()
    qlens = np.array([3, 4, 2])
    q, qsl = chunk_inputs(w, qlens, 6)
    bad = lens.copy()
    bad[1] = 2                                   # fewer cached tokens than chunk tokens
    out = run_gpu(w, q, qsl, seq_lens=bad).cpu().float().numpy()
    assert np.isnan(out[qsl[1]:qsl[2]]).all()
    good = np.concatenate([np.arange(qsl[0], qsl[1]), np.arange(qsl[2], qsl[3])])
    ref = run_oracle(w, q, qsl)
    assert np.abs(out[good] - ref[good]).max() <= TOL[w.dtype]
