"""ctypes binding of ``libpkv.so`` (``include/pkv.h``, ``include/pkv_blocks.h``,
``include/pkv_fp8.h``, ``include/pkv_chunk.h``).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked and turned into the raw pointers and sizes of the C ABI, together
with the current HIP stream of the tensors' device. Every step of the
computation runs in the HIP library; there is no fallback. If the library is
missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK, PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_DEVICE, PKV_ERR_NO_BLOCKS = 0, 1, 2, 3, 4
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
PKV_FP8_E4M3 = 3  # 1-byte pool codes (torch.uint8 tensors)

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_SIGNATURES = {
    "pkv_paged_attn_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_paged_attn_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32, _i32,
                                                     _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_kv_cache_write": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64,
                                          _i32, _vp]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_set_partition_tokens": (ctypes.c_int, [_i32]),
    "pkv_decode_plan": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32),
                                       ctypes.POINTER(_i32)]),
    "pkv_release_workspace": (ctypes.c_int, []),
    "pkv_version": (_i32, []),
    # block manager and block copy (pkv_blocks.h)
    "pkv_bm_create": (ctypes.c_int, [_i64, _i32, ctypes.POINTER(_vp)]),
    "pkv_bm_destroy": (ctypes.c_int, [_vp]),
    "pkv_bm_add_sequence": (ctypes.c_int, [_vp, _i64, _i32]),
    "pkv_bm_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "pkv_bm_append_slots": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, ctypes.POINTER(_i32)]),
    "pkv_bm_free_sequence": (ctypes.c_int, [_vp, _i64]),
    "pkv_bm_num_free": (ctypes.c_int, [_vp, ctypes.POINTER(_i64)]),
    "pkv_bm_refcount": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pkv_bm_sequence": (ctypes.c_int, [_vp, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_i32), _vp, _i32]),
    "pkv_bm_build_tables": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "pkv_bm_free_queue": (ctypes.c_int, [_vp, _vp, _i64]),
    "pkv_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    # multi-token chunk attention (pkv_chunk.h)
    "pkv_paged_attn_chunk": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _i64, _i32, _i32, _vp]),
    "pkv_paged_attn_decode_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32,
                                                    _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_paged_attn_decode_append_planned": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32,
                                                            _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    # shared-prefix decode (pkv_shared_prefix.h)
    "pkv_paged_attn_decode_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32,
                                                           _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                                                           _i32, _vp]),
    "pkv_shared_prefix_groups": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "pkv_paged_attn_decode_shared_prefix_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                               _f32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                               _i32, _i64, _i32, _vp]),
    "pkv_paged_attn_chunk_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _i64, _i32, _i32, _vp]),
    # read-bandwidth probes (pkv_probe.h)
    "pkv_probe_stream_read": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "pkv_probe_gather_tiles": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i32, _i32, _vp, _vp]),
    # FP8 (e4m3) KV cache (pkv_fp8.h)
    "pkv_paged_attn_decode_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32,
                                                 _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_kv_cache_write_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                              _i64, _i32, _vp]),
    "pkv_paged_attn_decode_append_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32,
                                                        _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_paged_attn_decode_append_fp8_planned": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                                _vp, _f32, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                                                                _i32, _vp]),
}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load ``libpkv.so`` once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run `python -m paged_kv_cache_260_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def last_error() -> str:
    return lib().pkv_last_error().decode()


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, last_error())


def _stream_handle(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be on a GPU")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")


def paged_attn_decode(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                      v_pool: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                      scale: float, n_heads: int, n_kv_heads: int, head_dim: int,
                      block_size: int, stream=None) -> torch.Tensor:
    """``out[s, h] = softmax(scale * q[s, h] K_s^T) V_s`` over each sequence's paged K/V.

    Shapes: ``q``/``out`` ``[B, H, D]``; pools ``[NB, Hkv, BS, D]``;
    ``block_tables`` int32 ``[B, MB]``; ``seq_lens`` int32 ``[B]``.
    Enqueued on ``stream`` (default: the current stream of ``q``'s device).
    """
    return _decode("pkv_paged_attn_decode", out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads,
                   n_kv_heads, head_dim, block_size, stream)


def paged_attn_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                              v_pool: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                              scale: float, n_heads: int, n_kv_heads: int, head_dim: int,
                              block_size: int, stream=None) -> torch.Tensor:
    """``paged_attn_decode`` with its scratch in the library's fixed per-GPU
    array instead of an allocated workspace (``pkv_paged_attn_decode_noalloc``:
    the call allocates nothing; sizes past the array's limits raise)."""
    return _decode("pkv_paged_attn_decode_noalloc", out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                   n_heads, n_kv_heads, head_dim, block_size, stream)


def _decode(symbol, out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
            block_size, stream):
    dt = q.dtype
    _need(dt in DTYPE_CODES, f"unsupported dtype {dt}")
    for name, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, dt)
    _dev_tensor(block_tables, "block_tables", torch.int32)
    _dev_tensor(seq_lens, "seq_lens", torch.int32)
    B = q.shape[0]
    _need(q.shape == (B, n_heads, head_dim) and out.shape == q.shape, "q/out must be [B, H, D]")
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    _need(seq_lens.shape == (B,), "seq_lens must be [B]")
    devs = {t.device for t in (out, q, k_pool, v_pool, block_tables, seq_lens)}
    _need(len(devs) == 1, "all tensors must be on one device")
    with torch.cuda.device(q.device):
        _check(getattr(lib(), symbol)(
            out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
            block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), n_heads, n_kv_heads,
            head_dim, block_size, B, block_tables.shape[1], k_pool.shape[0], DTYPE_CODES[dt],
            _stream_handle(q, stream)))
    return out


def kv_cache_write(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor,
                   v_new: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Scatter ``k_new[t]``/``v_new[t]`` (``[T, Hkv, D]``) into pool slot ``slot_mapping[t]``."""
    dt = k_pool.dtype
    _need(dt in DTYPE_CODES, f"unsupported dtype {dt}")
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, name, dt)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    _need(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "pools must be [NB, Hkv, BS, D]")
    NB, Hkv, BS, D = k_pool.shape
    T = k_new.shape[0]
    _need(k_new.shape == (T, Hkv, D) and v_new.shape == k_new.shape, "k_new/v_new must be [T, Hkv, D]")
    _need(slot_mapping.shape == (T,), "slot_mapping must be [T]")
    devs = {t.device for t in (k_pool, v_pool, k_new, v_new, slot_mapping)}
    _need(len(devs) == 1, "all tensors must be on one device")
    with torch.cuda.device(k_pool.device):
        _check(lib().pkv_kv_cache_write(
            k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
            slot_mapping.data_ptr(), T, Hkv, D, BS, NB, DTYPE_CODES[dt],
            _stream_handle(k_pool, stream)))


def set_partition_tokens(tokens: int) -> None:
    """Partition length for split decode (0 = automatic). Process-wide."""
    _check(lib().pkv_set_partition_tokens(int(tokens)))


def decode_plan(n_heads: int, n_kv_heads: int, block_size: int, num_seqs: int,
                max_blocks_per_seq: int):
    """``(partition_tokens, max_partitions)`` a decode call with these sizes would use."""
    p, n = _i32(), _i32()
    _check(lib().pkv_decode_plan(n_heads, n_kv_heads, block_size, num_seqs, max_blocks_per_seq,
                                 ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def release_workspace() -> None:
    _check(lib().pkv_release_workspace())


def version() -> int:
    return int(lib().pkv_version())


def copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pairs: torch.Tensor, stream=None) -> None:
    """Copy whole pool blocks: ``pool[pairs[i, 1]] = pool[pairs[i, 0]]`` in both pools.

    ``pairs`` is int32 ``[N, 2]`` (src, dst) on the pools' device; destinations
    are distinct and are not sources (copy-on-write targets are fresh blocks).
    """
    dt = k_pool.dtype
    _need(dt in DTYPE_CODES or dt == torch.uint8, f"unsupported dtype {dt}")
    _dev_tensor(k_pool, "k_pool", dt)
    _dev_tensor(v_pool, "v_pool", dt)
    _dev_tensor(pairs, "pairs", torch.int32)
    _need(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "pools must be [NB, Hkv, BS, D]")
    _need(pairs.dim() == 2 and pairs.shape[1] == 2, "pairs must be [N, 2]")
    _need(len({k_pool.device, v_pool.device, pairs.device}) == 1, "all tensors must be on one device")
    NB, Hkv, BS, D = k_pool.shape
    code = PKV_FP8_E4M3 if dt == torch.uint8 else DTYPE_CODES[dt]
    with torch.cuda.device(k_pool.device):
        _check(lib().pkv_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), pairs.data_ptr(),
                                     pairs.shape[0], Hkv, D, BS, NB, code,
                                     _stream_handle(k_pool, stream)))


class BlockManager:
    """Host block manager of a pool of ``num_blocks`` blocks (``pkv_blocks.h``).

    A FIFO free queue, a reference count per block, and per sequence its block
    list and token count: blocks are allocated on demand, shared by forks,
    copied on write and released last block first.
    """

    def __init__(self, num_blocks: int, block_size: int):
        h = _vp()
        _check(lib().pkv_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            lib().pkv_bm_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass

    def add_sequence(self, seq_id: int, num_tokens: int) -> None:
        _check(lib().pkv_bm_add_sequence(self._h, int(seq_id), int(num_tokens)))

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pkv_bm_fork(self._h, int(parent), int(child)))

    def append_slots(self, seq_ids):
        """Reserve the next token's slot of each sequence: ``(slots, copies)``,
        numpy int32 ``[n]`` and ``[num_copies, 2]`` (src, dst)."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        slots = np.empty(n, dtype=np.int32)
        copies = np.empty((max(n, 1), 2), dtype=np.int32)
        nc = _i32()
        _check(lib().pkv_bm_append_slots(self._h, ids.ctypes.data, n, slots.ctypes.data,
                                         copies.ctypes.data, ctypes.byref(nc)))
        return slots, copies[:nc.value].copy()

    def free_sequence(self, seq_id: int) -> None:
        _check(lib().pkv_bm_free_sequence(self._h, int(seq_id)))

    def num_free(self) -> int:
        n = _i64()
        _check(lib().pkv_bm_num_free(self._h, ctypes.byref(n)))
        return n.value

    def refcount(self, block: int) -> int:
        c = _i32()
        _check(lib().pkv_bm_refcount(self._h, int(block), ctypes.byref(c)))
        return c.value

    def sequence(self, seq_id: int):
        """``(num_tokens, [block ids])`` of one sequence."""
        import numpy as np
        nt, nb = _i32(), _i32()
        _check(lib().pkv_bm_sequence(self._h, int(seq_id), ctypes.byref(nt), ctypes.byref(nb), None, 0))
        blocks = np.empty(max(nb.value, 1), dtype=np.int32)
        _check(lib().pkv_bm_sequence(self._h, int(seq_id), ctypes.byref(nt), ctypes.byref(nb),
                                     blocks.ctypes.data, nb.value))
        return nt.value, [int(b) for b in blocks[:nb.value]]

    def build_tables(self, seq_ids, max_blocks: int):
        """Host ``(block_tables [n, max_blocks], seq_lens [n])`` (int32 numpy) for decode."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        tables = np.empty((n, max_blocks), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        _check(lib().pkv_bm_build_tables(self._h, ids.ctypes.data, n, int(max_blocks),
                                         tables.ctypes.data, lens.ctypes.data))
        return tables, lens

    def free_queue(self):
        """Block ids of the free queue, front first."""
        import numpy as np
        n = self.num_free()
        out = np.empty(max(n, 1), dtype=np.int32)
        _check(lib().pkv_bm_free_queue(self._h, out.ctypes.data, n))
        return [int(b) for b in out[:n]]


def paged_attn_decode_fp8(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                          v_pool: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                          block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                          n_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                          stream=None) -> torch.Tensor:
    """Decode over FP8 pools (uint8 e4m3 codes ``[NB, Hkv, BS, D]``, float32 scales ``[Hkv]``)."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"FP8 pools need an fp16/bf16 query, got {dt}")
    _dev_tensor(out, "out", dt)
    _dev_tensor(q, "q", dt)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, torch.uint8)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev_tensor(t, name, torch.float32)
        _need(t.shape == (n_kv_heads,), f"{name} must be [Hkv]")
    _dev_tensor(block_tables, "block_tables", torch.int32)
    _dev_tensor(seq_lens, "seq_lens", torch.int32)
    B = q.shape[0]
    _need(q.shape == (B, n_heads, head_dim) and out.shape == q.shape, "q/out must be [B, H, D]")
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    _need(seq_lens.shape == (B,), "seq_lens must be [B]")
    devs = {t.device for t in (out, q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens)}
    _need(len(devs) == 1, "all tensors must be on one device")
    with torch.cuda.device(q.device):
        _check(lib().pkv_paged_attn_decode_fp8(
            out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), n_heads,
            n_kv_heads, head_dim, block_size, B, block_tables.shape[1], k_pool.shape[0],
            DTYPE_CODES[dt], _stream_handle(q, stream)))
    return out


def kv_cache_write_fp8(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor,
                       v_new: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                       slot_mapping: torch.Tensor, stream=None) -> None:
    """Quantize ``k_new``/``v_new`` (``[T, Hkv, D]``) into FP8 pools at ``slot_mapping``."""
    dt = k_new.dtype
    _need(dt in DTYPE_CODES, f"unsupported dtype {dt}")
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, torch.uint8)
    _dev_tensor(k_new, "k_new", dt)
    _dev_tensor(v_new, "v_new", dt)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32)
    _need(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "pools must be [NB, Hkv, BS, D]")
    NB, Hkv, BS, D = k_pool.shape
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev_tensor(t, name, torch.float32)
        _need(t.shape == (Hkv,), f"{name} must be [Hkv]")
    T = k_new.shape[0]
    _need(k_new.shape == (T, Hkv, D) and v_new.shape == k_new.shape, "k_new/v_new must be [T, Hkv, D]")
    _need(slot_mapping.shape == (T,), "slot_mapping must be [T]")
    devs = {t.device for t in (k_pool, v_pool, k_new, v_new, k_scale, v_scale, slot_mapping)}
    _need(len(devs) == 1, "all tensors must be on one device")
    with torch.cuda.device(k_pool.device):
        _check(lib().pkv_kv_cache_write_fp8(
            k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), slot_mapping.data_ptr(), T, Hkv, D, BS, NB, DTYPE_CODES[dt],
            _stream_handle(k_pool, stream)))


def paged_attn_chunk(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                     block_tables: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                     scale: float, n_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                     max_query_len: int, stream=None) -> torch.Tensor:
    """Causal attention of the last ``n_s`` tokens of each sequence (packed ``q``/``out`` ``[T, H, D]``,
    ``query_start_loc`` int32 ``[B + 1]``; the chunk's K/V already in the pools)."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"chunk attention needs fp16/bf16, got {dt}")
    for name, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, dt)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("query_start_loc", query_start_loc)):
        _dev_tensor(t, name, torch.int32)
    _need(seq_lens.dim() == 1, "seq_lens must be [B]")
    B = seq_lens.shape[0]
    _need(q.dim() == 3 and q.shape[1:] == (n_heads, head_dim) and out.shape == q.shape, "q/out must be [T, H, D]")
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    _need(query_start_loc.shape == (B + 1,), "query_start_loc must be [B + 1]")
    devs = {t.device for t in (out, q, k_pool, v_pool, block_tables, seq_lens, query_start_loc)}
    _need(len(devs) == 1, "all tensors must be on one device")
    with torch.cuda.device(q.device):
        _check(lib().pkv_paged_attn_chunk(
            out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), query_start_loc.data_ptr(), float(scale), n_heads, n_kv_heads, head_dim,
            block_size, B, block_tables.shape[1], k_pool.shape[0], int(max_query_len), DTYPE_CODES[dt],
            _stream_handle(q, stream)))
    return out


def paged_attn_decode_shared_prefix(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                                    v_pool: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                    prefix_lens: torch.Tensor, group_start: torch.Tensor, scale: float,
                                    n_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                                    max_group_size: int, stream=None) -> torch.Tensor:
    """Decode of a batch whose consecutive sequence groups share a prompt prefix
    (``group_start`` int32 ``[G + 1]``, ``prefix_lens`` int32 ``[B]``); same
    result as :func:`paged_attn_decode`."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"shared-prefix decode needs fp16/bf16, got {dt}")
    for name, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, dt)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("prefix_lens", prefix_lens),
                    ("group_start", group_start)):
        _dev_tensor(t, name, torch.int32)
    _need(seq_lens.dim() == 1, "seq_lens must be [B]")
    B = seq_lens.shape[0]
    _need(q.shape == (B, n_heads, head_dim) and out.shape == q.shape, "q/out must be [B, H, D]")
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    _need(prefix_lens.shape == (B,), "prefix_lens must be [B]")
    _need(group_start.dim() == 1 and group_start.shape[0] >= 2, "group_start must be [G + 1]")
    devs = {t.device for t in (out, q, k_pool, v_pool, block_tables, seq_lens, prefix_lens, group_start)}
    _need(len(devs) == 1, "all tensors must be on one device")
    with torch.cuda.device(q.device):
        _check(lib().pkv_paged_attn_decode_shared_prefix(
            out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
            seq_lens.data_ptr(), prefix_lens.data_ptr(), group_start.data_ptr(), float(scale), n_heads,
            n_kv_heads, head_dim, block_size, B, group_start.shape[0] - 1, int(max_group_size),
            block_tables.shape[1], k_pool.shape[0], DTYPE_CODES[dt], _stream_handle(q, stream)))
    return out


def shared_prefix_groups(block_tables, seq_lens, block_size: int):
    """Sharing description from host tables (numpy int32 ``[B, MB]`` and ``[B]``):
    ``(group_start [G + 1], prefix_lens [B], max_group_size)`` as numpy int32."""
    import numpy as np
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    _need(bt.ndim == 2 and sl.shape == (bt.shape[0],), "block_tables [B, MB] and seq_lens [B]")
    B = bt.shape[0]
    gs = np.zeros(B + 1, dtype=np.int32)
    pl = np.zeros(B, dtype=np.int32)
    ng = ctypes.c_int32(0)
    mg = ctypes.c_int32(0)
    _check(lib().pkv_shared_prefix_groups(bt.ctypes.data, sl.ctypes.data, B, max(1, bt.shape[1]), int(block_size),
                                          gs.ctypes.data, pl.ctypes.data, ctypes.addressof(ng),
                                          ctypes.addressof(mg)))
    return gs[:ng.value + 1].copy() if B else np.zeros(1, np.int32), pl, mg.value


def _fp8_pools(k_pool, v_pool, k_scale, v_scale, n_kv_heads, block_size, head_dim):
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, torch.uint8)
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be uint8 [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev_tensor(t, name, torch.float32)
        _need(t.shape == (n_kv_heads,), f"{name} must be float32 [n_kv_heads]")


def paged_attn_chunk_fp8(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, query_start_loc,
                         scale: float, n_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                         max_query_len: int, stream=None):
    """:func:`paged_attn_chunk` over FP8 (e4m3) pools with per-KV-head float32 scales."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"chunk attention needs fp16/bf16 queries, got {dt}")
    _dev_tensor(out, "out", dt)
    _dev_tensor(q, "q", dt)
    _fp8_pools(k_pool, v_pool, k_scale, v_scale, n_kv_heads, block_size, head_dim)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("query_start_loc", query_start_loc)):
        _dev_tensor(t, name, torch.int32)
    _need(seq_lens.dim() == 1, "seq_lens must be [B]")
    B = seq_lens.shape[0]
    _need(q.dim() == 3 and q.shape[1:] == (n_heads, head_dim) and out.shape == q.shape, "q/out must be [T, H, D]")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    _need(query_start_loc.shape == (B + 1,), "query_start_loc must be [B + 1]")
    with torch.cuda.device(q.device):
        _check(lib().pkv_paged_attn_chunk_fp8(
            out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), query_start_loc.data_ptr(),
            float(scale), n_heads, n_kv_heads, head_dim, block_size, B, block_tables.shape[1], k_pool.shape[0],
            int(max_query_len), DTYPE_CODES[dt], _stream_handle(q, stream)))
    return out


def paged_attn_decode_shared_prefix_fp8(out, q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens,
                                        prefix_lens, group_start, scale: float, n_heads: int, n_kv_heads: int,
                                        head_dim: int, block_size: int, max_group_size: int, stream=None):
    """:func:`paged_attn_decode_shared_prefix` over FP8 (e4m3) pools with per-KV-head float32 scales."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"shared-prefix decode needs fp16/bf16 queries, got {dt}")
    _dev_tensor(out, "out", dt)
    _dev_tensor(q, "q", dt)
    _fp8_pools(k_pool, v_pool, k_scale, v_scale, n_kv_heads, block_size, head_dim)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("prefix_lens", prefix_lens),
                    ("group_start", group_start)):
        _dev_tensor(t, name, torch.int32)
    _need(seq_lens.dim() == 1, "seq_lens must be [B]")
    B = seq_lens.shape[0]
    _need(q.shape == (B, n_heads, head_dim) and out.shape == q.shape, "q/out must be [B, H, D]")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    _need(prefix_lens.shape == (B,), "prefix_lens must be [B]")
    _need(group_start.dim() == 1 and group_start.shape[0] >= 2, "group_start must be [G + 1]")
    with torch.cuda.device(q.device):
        _check(lib().pkv_paged_attn_decode_shared_prefix_fp8(
            out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
            v_scale.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), prefix_lens.data_ptr(),
            group_start.data_ptr(), float(scale), n_heads, n_kv_heads, head_dim, block_size, B,
            group_start.shape[0] - 1, int(max_group_size), block_tables.shape[1], k_pool.shape[0],
            DTYPE_CODES[dt], _stream_handle(q, stream)))
    return out


def paged_attn_decode_append(out, q, k_pool, v_pool, k_new, v_new, block_tables, seq_lens, scale: float,
                             n_heads: int, n_kv_heads: int, head_dim: int, block_size: int, stream=None,
                             seq_lens_host=None):
    """One decode step: write each sequence's newest token (``k_new``/``v_new``
    ``[B, Hkv, D]``) at position ``seq_lens - 1`` of its table, then decode over
    ``seq_lens`` tokens (fp16/bf16).

    ``seq_lens_host`` (optional): the same lengths as a C-contiguous int32
    numpy array in host memory; the call is then
    ``pkv_paged_attn_decode_append_planned``, which builds the work order on
    the host."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"decode with append needs fp16/bf16, got {dt}")
    for name, t in (("out", out), ("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("k_new", k_new),
                    ("v_new", v_new)):
        _dev_tensor(t, name, dt)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens)):
        _dev_tensor(t, name, torch.int32)
    _need(seq_lens.dim() == 1, "seq_lens must be [B]")
    B = seq_lens.shape[0]
    _need(q.shape == (B, n_heads, head_dim) and out.shape == q.shape, "q/out must be [B, H, D]")
    _need(k_new.shape == (B, n_kv_heads, head_dim) and v_new.shape == k_new.shape, "k_new/v_new must be [B, Hkv, D]")
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    devs = {t.device for t in (out, q, k_pool, v_pool, k_new, v_new, block_tables, seq_lens)}
    _need(len(devs) == 1, "all tensors must be on one device")
    if seq_lens_host is not None:
        _need(isinstance(seq_lens_host, np.ndarray) and seq_lens_host.dtype == np.int32
              and seq_lens_host.shape == (B,) and seq_lens_host.flags["C_CONTIGUOUS"],
              "seq_lens_host must be a C-contiguous int32 numpy array of shape [B]")
    with torch.cuda.device(q.device):
        if seq_lens_host is None:
            _check(lib().pkv_paged_attn_decode_append(
                out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
                v_new.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), float(scale), n_heads, n_kv_heads,
                head_dim, block_size, B, block_tables.shape[1], k_pool.shape[0], DTYPE_CODES[dt],
                _stream_handle(q, stream)))
        else:
            _check(lib().pkv_paged_attn_decode_append_planned(
                out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
                v_new.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), seq_lens_host.ctypes.data,
                float(scale), n_heads, n_kv_heads, head_dim, block_size, B, block_tables.shape[1],
                k_pool.shape[0], DTYPE_CODES[dt], _stream_handle(q, stream)))
    return out


def paged_attn_decode_append_fp8(out, q, k_pool, v_pool, k_new, v_new, k_scale, v_scale, block_tables, seq_lens,
                                 scale: float, n_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                                 stream=None, seq_lens_host=None):
    """One decode step over FP8 pools (uint8 e4m3 codes ``[NB, Hkv, BS, D]``,
    float32 scales ``[Hkv]``): encode and store each sequence's newest token
    (``k_new``/``v_new`` ``[B, Hkv, D]`` in the query dtype) at position
    ``seq_lens - 1`` of its table, then decode over ``seq_lens`` tokens.

    ``seq_lens_host`` (optional): the same lengths as a C-contiguous int32
    numpy array in host memory; the call is then
    ``pkv_paged_attn_decode_append_fp8_planned``."""
    dt = q.dtype
    _need(dt in (torch.float16, torch.bfloat16), f"FP8 pools need an fp16/bf16 query, got {dt}")
    for name, t in (("out", out), ("q", q), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, name, dt)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev_tensor(t, name, torch.uint8)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev_tensor(t, name, torch.float32)
        _need(t.shape == (n_kv_heads,), f"{name} must be [Hkv]")
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens)):
        _dev_tensor(t, name, torch.int32)
    _need(seq_lens.dim() == 1, "seq_lens must be [B]")
    B = seq_lens.shape[0]
    _need(q.shape == (B, n_heads, head_dim) and out.shape == q.shape, "q/out must be [B, H, D]")
    _need(k_new.shape == (B, n_kv_heads, head_dim) and v_new.shape == k_new.shape, "k_new/v_new must be [B, Hkv, D]")
    _need(k_pool.dim() == 4 and k_pool.shape[1:] == (n_kv_heads, block_size, head_dim),
          "k_pool must be [NB, Hkv, BS, D]")
    _need(v_pool.shape == k_pool.shape, "v_pool must match k_pool")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, MB]")
    devs = {t.device for t in (out, q, k_pool, v_pool, k_new, v_new, k_scale, v_scale, block_tables, seq_lens)}
    _need(len(devs) == 1, "all tensors must be on one device")
    if seq_lens_host is not None:
        _need(isinstance(seq_lens_host, np.ndarray) and seq_lens_host.dtype == np.int32
              and seq_lens_host.shape == (B,) and seq_lens_host.flags["C_CONTIGUOUS"],
              "seq_lens_host must be a C-contiguous int32 numpy array of shape [B]")
    with torch.cuda.device(q.device):
        if seq_lens_host is None:
            _check(lib().pkv_paged_attn_decode_append_fp8(
                out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
                v_new.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), block_tables.data_ptr(),
                seq_lens.data_ptr(), float(scale), n_heads, n_kv_heads, head_dim, block_size, B,
                block_tables.shape[1], k_pool.shape[0], DTYPE_CODES[dt], _stream_handle(q, stream)))
        else:
            _check(lib().pkv_paged_attn_decode_append_fp8_planned(
                out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
                v_new.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), block_tables.data_ptr(),
                seq_lens.data_ptr(), seq_lens_host.ctypes.data, float(scale), n_heads, n_kv_heads, head_dim,
                block_size, B, block_tables.shape[1], k_pool.shape[0], DTYPE_CODES[dt],
                _stream_handle(q, stream)))
    return out


def probe_stream_read(buf: torch.Tensor, grid: int, sink: torch.Tensor, stream=None) -> None:
    """Read every 16-byte unit of ``buf`` once (``pkv_probe_stream_read``);
    ``sink`` is a uint32/int32 device tensor of at least ``grid`` entries."""
    _dev_tensor(buf, "buf")
    _dev_tensor(sink, "sink")
    _need(sink.element_size() == 4 and sink.numel() >= grid, "sink must hold grid 32-bit words")
    with torch.cuda.device(buf.device):
        _check(lib().pkv_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), int(grid),
                                           sink.data_ptr(), _stream_handle(buf, stream)))


def probe_gather_tiles(pool: torch.Tensor, tiles: torch.Tensor, depth: int, grid: int, sink: torch.Tensor,
                       stream=None) -> None:
    """Read the 4096-byte tiles of ``pool`` listed in ``tiles`` (int32), the
    decode kernel's gather pattern (``pkv_probe_gather_tiles``)."""
    _dev_tensor(pool, "pool")
    _dev_tensor(tiles, "tiles", torch.int32)
    _dev_tensor(sink, "sink")
    nbytes = pool.numel() * pool.element_size()
    _need(nbytes % 4096 == 0, "pool must be whole 4096-byte tiles")
    _need(sink.element_size() == 4 and sink.numel() >= grid, "sink must hold grid 32-bit words")
    with torch.cuda.device(pool.device):
        _check(lib().pkv_probe_gather_tiles(pool.data_ptr(), nbytes // 4096, tiles.data_ptr(), tiles.numel(),
                                            int(depth), int(grid), sink.data_ptr(), _stream_handle(pool, stream)))
