"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with a status before any HIP call."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from paged_kv_cache_260_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libpkv.so not built (python -m paged_kv_cache_260_amd.build)")


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*PKV_API\s+(?:int|int32_t|const char \*)\s*(pkv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pkv_paged_attn_decode", "pkv_kv_cache_write", "pkv_last_error",
                     "pkv_copy_blocks", "pkv_bm_create", "pkv_bm_append_slots"):
        assert required in names
    assert set(names) == set(_lib._SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    assert set(declared_functions()) <= exported


def _decode(**over):
    args = dict(out=16, q=16, k_pool=16, v_pool=16, block_tables=16, seq_lens=16, scale=0.125,
                n_heads=32, n_kv_heads=8, head_dim=128, block_size=16, num_seqs=4,
                max_blocks_per_seq=8, num_blocks=64, dtype=2, stream=None)
    args.update(over)
    return _lib.lib().pkv_paged_attn_decode(*args.values())


def _write(**over):
    args = dict(k_pool=16, v_pool=16, k_new=16, v_new=16, slot_mapping=16, num_tokens=4,
                n_kv_heads=8, head_dim=128, block_size=16, num_blocks=64, dtype=2, stream=None)
    args.update(over)
    return _lib.lib().pkv_kv_cache_write(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(n_heads=30), _lib.PKV_ERR_INVALID),            # not a multiple of n_kv_heads
    (dict(n_kv_heads=0), _lib.PKV_ERR_INVALID),
    (dict(head_dim=96), _lib.PKV_ERR_UNSUPPORTED),
    (dict(block_size=8), _lib.PKV_ERR_UNSUPPORTED),
    (dict(block_size=48), _lib.PKV_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.PKV_ERR_INVALID),
    (dict(q=None), _lib.PKV_ERR_INVALID),
    (dict(k_pool=24), _lib.PKV_ERR_INVALID),              # misaligned
    (dict(num_seqs=-1), _lib.PKV_ERR_INVALID),
    (dict(num_seqs=70000), _lib.PKV_ERR_INVALID),
    (dict(max_blocks_per_seq=0), _lib.PKV_ERR_INVALID),
    (dict(num_blocks=0), _lib.PKV_ERR_INVALID),
    (dict(scale=float("inf")), _lib.PKV_ERR_INVALID),
    (dict(n_heads=8 * 512), _lib.PKV_ERR_UNSUPPORTED),   # group of 512
])
def test_decode_rejects_bad_arguments(over, status):
    assert _decode(**over) == status
    assert _lib.last_error() != ""


def _planned(**over):
    args = dict(out=16, q=16, k_pool=16, v_pool=16, k_new=16, v_new=16, block_tables=16, seq_lens=16,
                seq_lens_host=16, scale=0.125, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16, num_seqs=4,
                max_blocks_per_seq=8, num_blocks=64, dtype=2, stream=None)
    args.update(over)
    return _lib.lib().pkv_paged_attn_decode_append_planned(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(seq_lens_host=None), _lib.PKV_ERR_INVALID),     # the host copy of the lengths is required
    (dict(dtype=0), _lib.PKV_ERR_UNSUPPORTED),            # float32: the one-call step is 16-bit only
    (dict(k_new=None), _lib.PKV_ERR_INVALID),
    (dict(n_heads=30), _lib.PKV_ERR_INVALID),
    (dict(v_pool=24), _lib.PKV_ERR_INVALID),              # misaligned
])
def test_planned_append_rejects_bad_arguments(over, status):
    assert _planned(**over) == status
    assert _lib.last_error() != ""


def test_fp8_planned_append_rejects_null_host_lengths():
    args = [16, 16, 16, 16, 16, 16, 16, 16, 16, 16, None, 0.125, 32, 8, 128, 16, 4, 8, 64, 2, None]
    assert _lib.lib().pkv_paged_attn_decode_append_fp8_planned(*args) == _lib.PKV_ERR_INVALID
    assert "seq_lens_host" in _lib.last_error()


def test_planned_append_empty_batch_is_noop():
    assert _planned(num_seqs=0, seq_lens_host=None, q=None, out=None) == _lib.PKV_OK


def test_decode_empty_batch_is_noop():
    assert _decode(num_seqs=0, q=None, out=None) == _lib.PKV_OK
    assert _lib.last_error() == ""


@pytest.mark.parametrize("over,status", [
    (dict(num_tokens=-1), _lib.PKV_ERR_INVALID),
    (dict(head_dim=4, dtype=2), _lib.PKV_ERR_UNSUPPORTED),   # 8-byte rows
    (dict(slot_mapping=None), _lib.PKV_ERR_INVALID),
    (dict(v_new=8), _lib.PKV_ERR_INVALID),
    (dict(dtype=-1), _lib.PKV_ERR_INVALID),
    (dict(block_size=0), _lib.PKV_ERR_INVALID),
])
def test_write_rejects_bad_arguments(over, status):
    assert _write(**over) == status


def test_write_empty_is_noop():
    assert _write(num_tokens=0, k_new=None) == _lib.PKV_OK


def test_partition_plan():
    assert _lib.decode_plan(32, 8, 16, 128, 257) == (1024, 5)     # 4112 tokens -> 5 x 1024
    assert _lib.decode_plan(4, 4, 16, 4, 7) == (112, 1)           # short tables stay whole
    assert _lib.decode_plan(32, 8, 16, 4, 8193) == (1024, 129)
    _lib.set_partition_tokens(64)
    try:
        assert _lib.decode_plan(32, 8, 16, 4, 10) == (64, 3)
        _lib.set_partition_tokens(4096)                           # capped at 64 blocks
        assert _lib.decode_plan(32, 8, 16, 4, 1000) == (1024, 16)
        _lib.set_partition_tokens(8176)                           # whole blocks, then the cap
        assert _lib.decode_plan(32, 8, 128, 4, 200) == (8064, 4)
        _lib.set_partition_tokens(48)                             # shorter than a block: kept
        assert _lib.decode_plan(32, 8, 64, 4, 3) == (48, 4)
    finally:
        _lib.set_partition_tokens(0)
    for bad in (17, -16, 8, 1 << 21):
        with pytest.raises(_lib.PkvError):
            _lib.set_partition_tokens(bad)


def test_version():
    assert _lib.version() >> 16 == 1


def _decode_noalloc(**over):
    args = dict(out=16, q=16, k_pool=16, v_pool=16, block_tables=16, seq_lens=16, scale=0.125,
                n_heads=32, n_kv_heads=8, head_dim=128, block_size=16, num_seqs=4,
                max_blocks_per_seq=8, num_blocks=64, dtype=2, stream=None)
    args.update(over)
    return _lib.lib().pkv_paged_attn_decode_noalloc(*args.values())


def test_noalloc_decode_rejects_sizes_past_its_scratch():
    """The no-allocation decode checks its fixed scratch before any HIP call:
    too many split partials (300 sequences x 32 heads x 16 partitions x 130
    floats = 80 MB > 64 MiB) or too many merge counters (3000 sequences x 8
    KV heads > 16384 - 64) give PKV_ERR_INVALID with a message naming the
    limit; the argument checks of the allocating call apply as well."""
    assert _decode_noalloc(num_seqs=300, max_blocks_per_seq=1024) == _lib.PKV_ERR_INVALID
    assert "split partials" in _lib.last_error()
    assert _decode_noalloc(num_seqs=3000, n_heads=8, max_blocks_per_seq=80) == _lib.PKV_ERR_INVALID
    assert "merge counters" in _lib.last_error()
    assert _decode_noalloc(head_dim=96) == _lib.PKV_ERR_UNSUPPORTED
    assert _decode_noalloc(num_seqs=0, q=None, out=None) == _lib.PKV_OK


def test_probe_kernels_reject_bad_arguments():
    """The read-ceiling probes check their arguments before any HIP call."""
    lib = _lib.lib()
    assert lib.pkv_probe_stream_read(None, 4096, 1, 16, None) == _lib.PKV_ERR_INVALID
    assert lib.pkv_probe_stream_read(16, 4095, 1, 16, None) == _lib.PKV_ERR_INVALID    # not whole 16-byte units
    assert lib.pkv_probe_stream_read(8, 4096, 1, 16, None) == _lib.PKV_ERR_INVALID     # misaligned
    assert lib.pkv_probe_stream_read(16, 4096, 0, 16, None) == _lib.PKV_ERR_INVALID    # empty grid
    assert lib.pkv_probe_gather_tiles(16, 8, 16, 4, 3, 1, 16, None) == _lib.PKV_ERR_UNSUPPORTED  # depth 3
    assert "depth" in _lib.last_error()
    assert lib.pkv_probe_gather_tiles(16, 0, 16, 4, 1, 1, 16, None) == _lib.PKV_ERR_INVALID     # no tiles
    assert lib.pkv_probe_gather_tiles(16, 8, None, 4, 1, 1, 16, None) == _lib.PKV_ERR_INVALID
