"""GPU parity of the one-call decode step (append the newest token, then
attend) through the C ABI: the output equals the fp64 oracle's write followed
by decode, the pools equal the oracle's write byte for byte, and the result is
bit-identical to the two calls (write, then decode) on the GPU. The pools are
NaN-poisoned, so the slot of the new token holds NaN before the call: the
kernel must use the new rows, not what the slot held."""
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


@pytest.fixture(autouse=True)
def _auto_partition():
    _lib.set_partition_tokens(0)
    yield
    _lib.set_partition_tokens(0)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_append(w, lens, host_lens=None):
    """The one-call step; with host_lens, the planned call (the lengths also
    in host memory, the work order built from them)."""
    dev = "cuda"
    kp, vp = w.k_pool.to(dev), w.v_pool.to(dev)
    q = w.q.to(dev)
    out = torch.full_like(q, float("nan"))  # a row the call skips cannot pass for a result
    _lib.paged_attn_decode_append(out, q, kp, vp, w.k_new.to(dev), w.v_new.to(dev),
                                  torch.from_numpy(w.block_tables).to(dev),
                                  torch.from_numpy(np.asarray(lens, np.int32)).to(dev), w.scale, w.n_heads,
                                  w.n_kv_heads, w.head_dim, w.block_size,
                                  seq_lens_host=None if host_lens is None else np.asarray(host_lens, np.int32))
    torch.cuda.synchronize()
    return out, kp, vp


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def run_two_calls(w, lens):
    dev = "cuda"
    kp, vp = w.k_pool.to(dev), w.v_pool.to(dev)
    q = w.q.to(dev)
    out = torch.full_like(q, float("nan"))
    _lib.kv_cache_write(kp, vp, w.k_new.to(dev), w.v_new.to(dev), torch.from_numpy(w.slot_mapping).to(dev))
    _lib.paged_attn_decode(out, q, kp, vp, torch.from_numpy(w.block_tables).to(dev),
                           torch.from_numpy(np.asarray(lens, np.int32)).to(dev), w.scale, w.n_heads, w.n_kv_heads,
                           w.head_dim, w.block_size)
    torch.cuda.synchronize()
    return out, kp, vp


def oracle_step(w, lens):
    k_ref, v_ref = oracle.kv_cache_write(f32np(w.k_pool), f32np(w.v_pool), f32np(w.k_new), f32np(w.v_new),
                                         w.slot_mapping, w.block_size)
    G, D = w.group, w.head_dim
    out = np.zeros(tuple(w.q.shape))
    qn = f32np(w.q)
    for g in range(w.n_kv_heads):
        out[:, g * G:(g + 1) * G] = oracle.paged_attn_decode(
            qn[:, g * G:(g + 1) * G], k_ref[:, g:g + 1], v_ref[:, g:g + 1], w.block_tables, lens, w.scale, G, 1,
            D, w.block_size)
    return out


def check(w, partition=0):
    _lib.set_partition_tokens(partition)
    lens = w.seq_lens_after_write()
    out, kp, vp = run_append(w, lens)
    err = max_abs_err(out, oracle_step(w, lens))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    out2, kp2, vp2 = run_two_calls(w, lens)
    # the same rows in the same order: bit-identical to write-then-decode
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(kp.view(torch.int16), kp2.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), vp2.view(torch.int16))


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_append_workloads(cfg):
    say(f"append cfg{cfg}")
    check(workloads.make(cfg, poison=True))


@pytest.mark.parametrize("partition", [16, 128, 1024])
@pytest.mark.parametrize("H,Hkv,D,BS,dtype", [(32, 8, 128, 16, torch.bfloat16), (64, 2, 128, 32, torch.float16),
                                              (8, 8, 64, 64, torch.bfloat16), (12, 4, 64, 16, torch.float16)])
def test_append_shapes_and_partitions(H, Hkv, D, BS, dtype, partition):
    """Head groups of 1, 3, 4 and 32 (two head chunks per KV head), blocks of
    16 to 64 tokens, and partitions of 16 to 1024 tokens (the new token in the
    last of up to 170 partitions; both merges)."""
    say(f"append H={H} Hkv={Hkv} D={D} BS={BS} partition={partition}")
    w = workloads.random_case(500 + H + BS + partition, num_seqs=11, n_heads=H, n_kv_heads=Hkv, head_dim=D,
                              block_size=BS, dtype=dtype, max_len=2700, min_len=0, poison=True)
    check(w, partition)


def test_append_block_boundaries():
    """New tokens that open a block (L % BS == 0), fill its last slot, and a
    sequence whose only token is the new one."""
    rng = np.random.default_rng(3)
    lens = [0, 15, 16, 31, 32, 1023, 1024, 47]
    w = workloads.build(name="edges", rng=rng, seq_lens=lens, n_heads=16, n_kv_heads=4, head_dim=128,
                        block_size=16, dtype=torch.bfloat16, poison=True)
    check(w)


def test_append_invalid_length_gives_nan_and_no_write():
    w = workloads.random_case(9, num_seqs=4, n_heads=8, n_kv_heads=2, head_dim=64, block_size=16,
                              dtype=torch.float16, max_len=300, min_len=20)
    lens = w.seq_lens_after_write().copy()
    cap = w.block_tables.shape[1] * w.block_size
    lens[2] = cap + 1                                     # longer than the table
    out, kp, vp = run_append(w, lens)
    o = out.float().cpu().numpy()
    assert np.isnan(o[2]).all() and np.isfinite(o[[0, 1, 3]]).all()
    # sequence 2's slot is untouched; the others hold their new rows
    s2 = int(w.slot_mapping[2])
    blk, off = divmod(s2, w.block_size)
    assert torch.equal(kp[blk, :, off].cpu().view(torch.int16), w.k_pool[blk, :, off].view(torch.int16))
    for s in (0, 1, 3):
        blk, off = divmod(int(w.slot_mapping[s]), w.block_size)
        assert torch.equal(kp[blk, :, off].cpu().view(torch.int16), w.k_new[s].view(torch.int16))


def test_ticket_placement_repeats_across_grids():
    """Late workgroups take their places from a counter that every call
    leaves where it started. Calls with three different grids in a row (batch
    128, 40, 128 again; the later workgroups of the 128-sequence batches claim
    places, the 40-sequence batch has its own claimer count): each output
    (NaN-filled before the call) is bit-identical to the two-call path, the
    repeated batch gives the same bits as its first call, and the last call
    matches the oracle."""
    ws = [workloads.random_case(700 + b, num_seqs=b, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                                dtype=torch.bfloat16, max_len=1500, min_len=16, poison=True) for b in (128, 40)]
    outs = []
    for w in (ws[0], ws[1], ws[0]):
        say(f"tickets: batch {w.num_seqs}")
        lens = w.seq_lens_after_write()
        out, _, _ = run_append(w, lens)
        out2, _, _ = run_two_calls(w, lens)
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    lens = ws[0].seq_lens_after_write()
    err = max_abs_err(outs[2], oracle_step(ws[0], lens))
    say(f"  third call max abs err {err:.3e}")
    assert err <= TOL[ws[0].dtype]


# --- the planned call (work order built on the host) --------------------------

@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_planned_append_equals_append(cfg):
    """The planned call gives the one-call step's bits (output and pools) on
    the MHA, GQA and shared-prompt workloads; the MHA batch, whose workgroups
    take two or more items, keeps the kernel's own order."""
    say(f"planned append cfg{cfg}")
    w = workloads.make(cfg, poison=True)
    lens = w.seq_lens_after_write()
    out, kp, vp = run_append(w, lens)
    out2, kp2, vp2 = run_append(w, lens, host_lens=lens)
    assert same_bits(out, out2) and same_bits(kp, kp2) and same_bits(vp, vp2)
    if cfg == 3:
        err = max_abs_err(out2, oracle_step(w, lens))
        say(f"  max abs err {err:.3e}")
        assert err <= TOL[w.dtype]


def test_planned_append_across_grids():
    """Planned calls with three different grids in a row (batch 128, 40, 128;
    the host order with ticket claimers, then the kernel's own plan for the
    small batch), each bit-identical to the one-call step, the last also
    against the oracle."""
    ws = [workloads.random_case(700 + b, num_seqs=b, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                                dtype=torch.bfloat16, max_len=1500, min_len=16, poison=True) for b in (128, 40)]
    for w in (ws[0], ws[1], ws[0]):
        say(f"planned: batch {w.num_seqs}")
        lens = w.seq_lens_after_write()
        out, _, _ = run_append(w, lens)
        out2, _, _ = run_append(w, lens, host_lens=lens)
        assert same_bits(out, out2)
    err = max_abs_err(out2, oracle_step(ws[0], ws[0].seq_lens_after_write()))
    say(f"  last call max abs err {err:.3e}")
    assert err <= TOL[ws[0].dtype]


def test_planned_append_host_length_mismatch():
    """Host lengths that split into another partition count than the device
    lengths give NaN rows and no write for those sequences; one with the same
    count is attended over its device length; every other row keeps its bits,
    and later calls on the stream (planned and not) are unaffected."""
    w = workloads.random_case(7100, num_seqs=128, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                              dtype=torch.bfloat16, max_len=1500, min_len=16, poison=True)
    lens = w.seq_lens_after_write()
    cap = w.block_tables.shape[1] * w.block_size
    P, _ = _lib.decode_plan(w.n_heads, w.n_kv_heads, w.block_size, w.num_seqs, w.block_tables.shape[1])
    long_ = [int(s) for s in np.flatnonzero(lens > P)]
    # short[0] gets a host length one partition longer, still inside the table
    short = [int(s) for s in np.flatnonzero((lens > 64) & (lens <= P) & (lens + P <= cap))]
    assert len(long_) >= 2 and len(short) >= 3
    host = lens.copy()
    bad = [long_[0], short[0]]
    host[long_[0]] = P            # two partitions on the device, one on the host
    host[short[0]] = lens[short[0]] + P   # one on the device, two on the host
    host[short[1]] = lens[short[1]] - 32  # same count: attended over the device length
    host[short[2]] = 0                    # empty on the host, one partition either way
    say(f"mismatch: NaN rows for {bad}")
    ref, kref, vref = run_append(w, lens)
    out, kp, vp = run_append(w, lens, host_lens=host)
    o = out.float().cpu().numpy()
    good = [s for s in range(w.num_seqs) if s not in bad]
    assert np.isnan(o[bad]).all()
    assert same_bits(out[good], ref[good])
    for s in bad:  # no write: the slot keeps what it held before the call
        blk, off = divmod(int(w.slot_mapping[s]), w.block_size)
        assert same_bits(kp[blk, :, off].cpu(), w.k_pool[blk, :, off])
        assert same_bits(vp[blk, :, off].cpu(), w.v_pool[blk, :, off])
    for s in good:
        blk, off = divmod(int(w.slot_mapping[s]), w.block_size)
        assert same_bits(kp[blk, :, off], kref[blk, :, off])
    # the merge counters were left clean: both kinds of call give the bits again
    out3, _, _ = run_append(w, lens, host_lens=lens)
    out4, _, _ = run_append(w, lens)
    assert same_bits(out3, ref) and same_bits(out4, ref)


def test_planned_append_long_tables_keep_the_kernel_order():
    """Tables with more than 8 partitions per sequence merge in a separate
    kernel, so the planned call does not use the host order there: host
    lengths that disagree with the device's are not read, and the output and
    pools are the one-call step's bits."""
    w = workloads.random_case(7300, num_seqs=32, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                              dtype=torch.bfloat16, max_len=9000, min_len=16, poison=True)
    _, nparts = _lib.decode_plan(w.n_heads, w.n_kv_heads, w.block_size, w.num_seqs, w.block_tables.shape[1])
    assert nparts > 8
    lens = w.seq_lens_after_write()
    host = lens.copy()
    host[0] = lens[0] + 2048 if lens[0] + 2048 <= w.block_tables.shape[1] * w.block_size else 1
    out, kp, vp = run_append(w, lens)
    out2, kp2, vp2 = run_append(w, lens, host_lens=host)
    assert same_bits(out, out2) and same_bits(kp, kp2) and same_bits(vp, vp2)
