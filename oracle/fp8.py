"""Oracle for the FP8 (e4m3) KV cache: encoding, the quantizing cache write, and
decode attention over a quantized pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name KV-cache quantization as one of the further KV optimisations
(vLLM paper page, "what vLLM changed" / KV-cache directions). They also say
decode is memory-bound, so fewer bytes moved is a direct speed-up (course
page, "key insight" under prefill/decode, and the quantization item of
model compression). They fix no format. Readings taken:

  - Format: 8-bit e4m3 in the OCP layout (the FP8 format of gfx950).
      * sign, 4 exponent bits with bias 7, 3 mantissa bits;
      * exponent field 0 holds subnormals m/8 * 2^-6;
      * S.1111.111 is NaN; there is no infinity; the largest finite value is
        448 (code 0x7e).
  - One float32 scale per KV head and pool, so stored code = encode(x / scale).
  - Quantize: the value encoded is the float32 product fl32(x * fl32(1/scale)),
    the same float32 steps the kernel takes. Encoding rounds to the nearest
    representable value, ties to the even code. Magnitudes >= 448, infinity
    included, saturate to +-448. NaN stays NaN (0x7f with the sign).
  - Dequantize: decode(code) * scale, exact in float64.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import paged_attn_decode

MAX_E4M3 = 448.0


def e4m3_value(code: int) -> float:
    """The value of one e4m3 code (definition of the format)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS = _TABLE[:0x7F]  # codes 0x00 .. 0x7e: the finite non-negative values, increasing


def decode(codes) -> np.ndarray:
    """float64 values of an array of codes (uint8)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_scalar(v: float) -> int:
    """Nearest e4m3 code to ``v``, ties to the even code, saturating at +-448."""
    sign = 0x80 if np.signbit(v) else 0
    if v != v:
        return sign | 0x7F
    a = abs(v)
    if a >= MAX_E4M3:
        return sign | 0x7E
    d = np.abs(_POS - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return sign | code


def encode(values) -> np.ndarray:
    """Vectorised ``encode_scalar``: the two codes that bracket |v| in the sorted
    table of finite values, the nearer one kept (the even one on a tie)."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)  # first value >= a
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= MAX_E4M3, 0x7E, code)
    sign = np.where(np.signbit(v), 0x80, 0)
    code = np.where(np.isnan(v), 0x7F, code) | sign
    return code.astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """Codes for float32 values ``x`` (``[..., Hkv, D]``) with per-head float32 ``scale`` ([Hkv])."""
    x = np.asarray(x, dtype=np.float32)
    inv = (np.float32(1.0) / np.asarray(scale, dtype=np.float32)).astype(np.float32)
    y = (x * inv[:, None]).astype(np.float32)  # one float32 multiply per element
    return encode(y)


def kv_cache_write_fp8(k_pool, v_pool, k_new, v_new, k_scale, v_scale, slot_mapping, block_size: int):
    """Quantize each new token's K/V rows and scatter them into their slots (uint8 pools)."""
    k_out = np.array(k_pool, dtype=np.uint8, copy=True)
    v_out = np.array(v_pool, dtype=np.uint8, copy=True)
    num_slots = k_out.shape[0] * block_size
    for t, slot in enumerate(np.asarray(slot_mapping).reshape(-1)):
        slot = int(slot)
        if slot < 0:
            continue
        if slot >= num_slots:
            raise ValueError(f"slot {slot} outside a pool of {num_slots} slots")
        block, offset = divmod(slot, block_size)
        k_out[block, :, offset, :] = quantize(k_new[t], k_scale)
        v_out[block, :, offset, :] = quantize(v_new[t], v_scale)
    return k_out, v_out


def dequantize_pool(pool_codes, scale) -> np.ndarray:
    """float64 pool ``decode(code) * scale[head]`` ([NB, Hkv, BS, D])."""
    return decode(pool_codes) * np.asarray(scale, dtype=np.float64)[None, :, None, None]


def paged_attn_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens, scale,
                          n_heads, n_kv_heads, head_dim, block_size):
    """Decode attention over the dequantized pools (the plain definition)."""
    return paged_attn_decode(q, dequantize_pool(k_codes, k_scale), dequantize_pool(v_codes, v_scale),
                             block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim, block_size)
