// Device helpers shared by the paged attention kernels (decode and the
// multi-token kernel): 16-byte chunk types, MFMA steps on one chunk per lane,
// reductions across the four 16-lane rows of a wave, the transposed LDS read,
// the LDS swizzles of staged K and V tiles, and the exact FP8 (OCP e4m3)
// decode into 16-bit chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector (HIP's u32x4_t is a union struct whose copies
// become memcpy and keep values out of registers).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPerChunk = 4; };
template <> struct Elem<_Float16> { static constexpr int kPerChunk = 8; };
template <> struct Elem<__bf16> { static constexpr int kPerChunk = 8; };

// ---------------------------------------------------------------------------
// element conversions (16-byte chunk -> fp32)
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void chunk_to_float(const u32x4_t &c, float *f);

template <> __device__ __forceinline__ void chunk_to_float<__bf16>(const u32x4_t &c, float *f) {
  const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <> __device__ __forceinline__ void chunk_to_float<_Float16>(const u32x4_t &c, float *f) {
  const f16x8_t h = __builtin_bit_cast(f16x8_t, c);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(h[i]);
}

template <> __device__ __forceinline__ void chunk_to_float<float>(const u32x4_t &c, float *f) {
  f[0] = __uint_as_float(c[0]);
  f[1] = __uint_as_float(c[1]);
  f[2] = __uint_as_float(c[2]);
  f[3] = __uint_as_float(c[3]);
}

// ---------------------------------------------------------------------------
// one MFMA step over a 16-byte chunk per lane: C += A(16 x k) * B(k x 16)
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ f32x4_t mfma_chunk(u32x4_t a, u32x4_t b, f32x4_t c);

template <> __device__ __forceinline__ f32x4_t mfma_chunk<__bf16>(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <> __device__ __forceinline__ f32x4_t mfma_chunk<_Float16>(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <> __device__ __forceinline__ f32x4_t mfma_chunk<float>(u32x4_t a, u32x4_t b, f32x4_t c) {
  // 16x16x4 fp32: lane (kg, n) supplies k = kg; the four words are four k-steps.
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
  return c;
}

// Across the four 16-lane rows (lanes n, n + 16, n + 32, n + 48; every lane
// receives the result): gfx950's row swaps, v_permlane16_swap (odd rows of
// one register with even rows of the other) and v_permlane32_swap (upper
// half of one with lower half of the other), applied to two copies of x, put
// each lane's partner in one of the two registers. VALU only, no LDS round
// trip. (The second copy is made opaque to the compiler, which otherwise
// treats the two results of a swap of equal inputs as one value.)
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ float cols_max4(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("" : "+v"(b));
  swap16(a, b);
  a = b = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
  asm volatile("" : "+v"(b));
  swap32(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float cols_sum4(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("" : "+v"(b));
  swap16(a, b);
  a = b = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
  asm volatile("" : "+v"(b));
  swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

template <typename T> struct Pv;  // 4-element operand of the 16x16x16 MFMA
template <> struct Pv<__bf16> {
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4_t mfma(v4 a, v4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};
template <> struct Pv<_Float16> {
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4_t mfma(v4 a, v4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, output lane j receives
// element (j % 4) of the 8-byte chunks addressed by lanes j / 4 + 4 r,
// r = 0..3 -- one column of a 4-row block per lane.
template <typename T>
__device__ __forceinline__ typename Pv<T>::v4 lds_read_tr(const void *p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t *)(__attribute__((address_space(3))) void *)(p));
  return __builtin_bit_cast(typename Pv<T>::v4, v);
}

// FP8 (OCP e4m3) storage. Two codes (the low or the high half of a word) ->
// two values of T in one word, by gfx950's scaled conversion with scale 1:
// exact, since every e4m3 value is exact in fp16 and bf16 (one instruction
// where decoding to float32 and packing took two; 1-4% faster FP8 decode).
template <typename T> __device__ __forceinline__ uint32_t fp8x2_to(uint32_t c, bool high);
template <> __device__ __forceinline__ uint32_t fp8x2_to<__bf16>(uint32_t c, bool high) {
  return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t fp8x2_to<_Float16>(uint32_t c, bool high) {
  return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, false));
}
// 16 codes -> 16 elements of T in two 16-byte chunks (lo = elements 0..7,
// hi = 8..15).
template <typename T> __device__ __forceinline__ void fp8x16_to(const u32x4_t &c, u32x4_t &lo, u32x4_t &hi) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = fp8x2_to<T>(c[i], false);
    w[2 * i + 1] = fp8x2_to<T>(c[i], true);
  }
  lo = u32x4_t{w[0], w[1], w[2], w[3]};
  hi = u32x4_t{w[4], w[5], w[6], w[7]};
}

// Swizzled 16-byte slot of chunk `ch` of token `tr` in a staged K tile: the
// 16 tokens read together in one MFMA step land in 16 distinct bank groups.
template <int kCh> __device__ __forceinline__ int kst_slot(int tr, int ch) {
  const int sw = (kCh >= 16 ? tr : (tr >> 1)) & (kCh - 1);
  return tr * kCh + (ch ^ sw);
}
// XOR pattern of a staged V tile. Transposed reads of one 16-dim block touch
// two adjacent chunks (2b, 2b+1) of 4 consecutive tokens per 16-lane group;
// an even pattern that differs across those tokens puts the 8 chunks in 8
// distinct bank groups (and keeps chunk pairs together: (2b + h) ^ sw = (2b ^ sw) + h).
template <int kCh> __device__ __forceinline__ int vst_swz(int tr) {
  return kCh >= 16 ? (2 * tr) & 15 : 2 * ((tr >> 1) & 3);
}

}  // namespace attn
}  // namespace pkv
