// Paged decode attention for CDNA4 (gfx950).
//
// What is computed: for each sequence s and query head h, exact softmax
// attention of q[s, h] over the sequence's cached K/V rows, which live in
// fixed-size blocks of a shared pool and are reached through the sequence's
// block table (vLLM paper page, "PagedAttention" core idea and block-pool
// diagram). The softmax is streamed with a running max and running sum, which
// gives the same result as standard attention (vLLM notes page,
// "FlashAttention": tiling plus online softmax, exact). Query heads that share
// a KV head (GQA/MQA, ICML-tutorial notes page) are processed together so each
// K/V tile is read from HBM once per group. Long sequences are split along the
// sequence (FlashDecoding, same tutorial page, kernel-optimisation part) and
// the partial results are merged by a second kernel.
//
// Work decomposition (one workgroup = 4 waves):
//   blockIdx.x = KV head x query-head chunk, blockIdx.y = sequence,
//   blockIdx.z = partition of `partition_tokens` tokens.
//   Inside a workgroup the partition's 16-token tiles go round-robin to the
//   waves; each wave keeps its own running max / sum / accumulator and the
//   four are merged through LDS at the end.
//
// Per 16-token tile, per wave:
//   1. K and V tiles (16 x head_dim each) are fetched with fully coalesced
//      16-byte loads into registers, one tile ahead of the one being used
//      (register double buffering).
//   2. K goes to a wave-private LDS tile (XOR-swizzled 16-byte chunks, bank
//      conflict free both ways) and is read back in the MFMA B-operand layout:
//      lane (kg = lane/16, n = lane%16) holds token n, chunk kg + 4c.
//   3. Scores S[head][token] = Q (heads x D, rows padded to 16) * K^T come out
//      of v_mfma_f32_16x16x32_{bf16,f16} (16x16x4 for fp32): lane (kg, n)
//      receives heads 4kg..4kg+3 of token n.
//   4. Online softmax in base 2 (scale * log2 e folded into one multiply):
//      the tile max per head is a 16-lane DPP row reduction; p = exp2(z - m).
//   5. p goes through LDS to the V layout, where each lane owns one 16-byte
//      chunk of head dims and a quarter of the tokens; acc += p * v in fp32 on
//      the VALU, no cross-lane work inside the loop.
#include "kernels.h"

#include <math.h>

namespace pkv {
namespace {

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

// ---------------------------------------------------------------------------
// 16-lane (DPP row) reductions; every lane of the row receives the result
// ---------------------------------------------------------------------------
template <int kCtrl> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
// row_ror:n has control 0x120 + n; rotations by 8, 4, 2, 1 cover the row.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x122>(x));
  x = fmaxf(x, dpp_f<0x121>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x122>(x);
  x += dpp_f<0x121>(x);
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

template <typename T, int D, int GT> struct Cfg {
  static constexpr int kEpc = Elem<T>::kPerChunk;        // elements per 16-byte chunk
  static constexpr int kCh = D / kEpc;                   // chunks per token row
  static constexpr int kLoads = kTileTokens * kCh / 64;  // 16-byte loads per lane per tile
  static constexpr int kSteps = kCh / 4;                 // MFMA steps per tile
  static constexpr int kRows = 64 / kCh;                 // token rows in the V layout
  static constexpr int kNW = kDecodeWaves;
  // LDS carve-up (bytes)
  static constexpr int kKstBytes = kTileTokens * kCh * 16;            // per wave
  static constexpr int kPstBytes = kTileTokens * GT * 4;              // per wave
  static constexpr int kKstOff = 0;
  static constexpr int kPstOff = kKstOff + kNW * kKstBytes;
  static constexpr int kAccOff = kPstOff + kNW * kPstBytes;
  static constexpr int kMlOff = kAccOff + kNW * GT * D * 4;
  static constexpr int kBadOff = kMlOff + kNW * GT * 8;
  static constexpr int kSmem = kBadOff + kNW * 4;
  static_assert(kCh % 4 == 0 && 64 % kCh == 0, "head_dim must give 8, 16 or 32 chunks");
  static_assert(GT >= 1 && GT <= 16, "head tile");
};

// Swizzled 16-byte slot of chunk `ch` of token `tr` in a staged K tile: the
// 16 tokens read together in one MFMA step land in 16 distinct bank groups.
template <int kCh> __device__ __forceinline__ int kst_slot(int tr, int ch) {
  const int sw = (kCh >= 16 ? tr : (tr >> 1)) & (kCh - 1);
  return tr * kCh + (ch ^ sw);
}

template <typename T, int D, int GT>
__global__ __launch_bounds__(kDecodeWaves * 64) void paged_decode_kernel(DecodeArgs a) {
  using C = Cfg<T, D, GT>;
  constexpr int kL = C::kLoads;
  constexpr int kCh = C::kCh;
  constexpr int kEpc = C::kEpc;
  constexpr int kNW = C::kNW;
  __shared__ __attribute__((aligned(16))) char smem[C::kSmem];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x / a.head_chunks;
  const int hc = blockIdx.x - g * a.head_chunks;
  const int s = blockIdx.y;
  const int part = blockIdx.z;
  const int H = a.n_heads;
  const int head0 = g * a.group + hc * GT;
  const int nh = min(GT, a.group - hc * GT);
  T *out = static_cast<T *>(a.out);

  const int L = a.seq_lens[s];
  const bool bad_len = L < 0 || (int64_t)L > (int64_t)a.max_blocks * a.block_size;
  if (bad_len || L == 0) {
    if (part == 0) {
      const float v = bad_len ? __builtin_nanf("") : 0.f;
      for (int i = threadIdx.x; i < nh * D; i += kNW * 64)
        out[((int64_t)s * H + head0) * D + i] = static_cast<T>(v);
    }
    return;
  }
  const int P = a.partition_tokens;
  const int start = part * P;
  if (start >= L) return;
  const int end = min(L, start + P);
  const int nparts = (L + P - 1) / P;

  // ---- Q as the MFMA A operand: row n = query head (zero past nh), k = head dims
  const int kg = lane >> 4;
  const int n = lane & 15;
  u32x4_t qa[C::kSteps];
  {
    const u32x4_t *qrow = reinterpret_cast<const u32x4_t *>(
        static_cast<const T *>(a.q) + ((int64_t)s * H + head0 + min(n, nh - 1)) * D);
#pragma unroll
    for (int c = 0; c < C::kSteps; ++c) {
      const u32x4_t v = qrow[kg + 4 * c];
      qa[c] = n < nh ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // Block ids of the partition (at most 64 table entries): lane i of btv holds
  // entry jb + i. They are read back with v_readlane, so the per-tile lookup
  // issues no memory operation and never waits on the K/V loads in flight.
  const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  const int jb = start >> a.block_shift;
  const int jmax = (end - 1) >> a.block_shift;  // last table entry this partition reads
  const int64_t kv_stride_blk = (int64_t)a.n_kv_heads * a.block_size;  // rows per physical block
  const int btv = jb + lane <= jmax ? bt_row[jb + lane] : 0;
  bool bad = false;

  auto tile_offset = [&](int ti) -> int64_t {  // offset of tile ti in 16-byte chunks (uniform)
    const int tok = ti * kTileTokens;
    const int j = (tok >> a.block_shift) - jb;
    int phys = __builtin_amdgcn_readlane(btv, j);
    if (phys < 0 || (int64_t)phys >= a.num_blocks) {
      bad = true;
      phys = 0;
    }
    return ((int64_t)phys * kv_stride_blk + (int64_t)g * a.block_size +
            (tok & (a.block_size - 1))) * (D / kEpc);
  };
  const u32x4_t *kbase = static_cast<const u32x4_t *>(a.k_pool);
  const u32x4_t *vbase = static_cast<const u32x4_t *>(a.v_pool);
  struct Regs {
    u32x4_t k[kL];
    u32x4_t v[kL];
  };
  auto load_tile = [&](int ti, Regs &r) {
    const int64_t off = tile_offset(ti);
    const u32x4_t *kp = kbase + off;
    const u32x4_t *vp = vbase + off;
#pragma unroll
    for (int i = 0; i < kL; ++i) r.k[i] = kp[i * 64 + lane];
#pragma unroll
    for (int i = 0; i < kL; ++i) r.v[i] = vp[i * 64 + lane];
  };

  u32x4_t *kst = reinterpret_cast<u32x4_t *>(smem + C::kKstOff + wave * C::kKstBytes);
  float *pst = reinterpret_cast<float *>(smem + C::kPstOff + wave * C::kPstBytes);

  float m[4], l[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
  float acc[GT][kEpc];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < kEpc; ++e) acc[h][e] = 0.f;

  auto process = [&](int ti, const Regs &rg) {
    // stage K (coalesced order -> swizzled LDS tile)
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int u = i * 64 + lane;
      kst[kst_slot<kCh>(u / kCh, u % kCh)] = rg.k[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C::kSteps; ++c) sc = mfma_chunk<T>(qa[c], kst[kst_slot<kCh>(n, kg + 4 * c)], sc);

    const int valid = end - ti * kTileTokens;  // > 0; >= 16 means a full tile
    const bool tok_ok = n < valid;
    float alpha[4], p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float z = tok_ok ? sc[r] * a.scale_log2 : -INFINITY;
      const float mt = row_max16(z);
      const float mn = fmaxf(m[r], mt);
      alpha[r] = (m[r] == mn) ? 1.f : exp2f(m[r] - mn);
      m[r] = mn;
      p[r] = exp2f(z - mn);
      l[r] = l[r] * alpha[r] + p[r];
    }
    // p[token][head] -> LDS for the V layout
    if (4 * kg < GT) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * kg + r < GT) pst[n * GT + 4 * kg + r] = p[r];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // rescale by the per-head factor (uniform per head)
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float ah = readlane_f(alpha[h & 3], (h >> 2) * 16);
#pragma unroll
      for (int e = 0; e < kEpc; ++e) acc[h][e] *= ah;
    }
    const bool partial = valid < kTileTokens;
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int tok = i * C::kRows + lane / kCh;
      float pv[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) pv[h] = pst[tok * GT + h];
      float vf[kEpc];
      chunk_to_float<T>(rg.v[i], vf);
      if (partial && tok >= valid) {
#pragma unroll
        for (int e = 0; e < kEpc; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < kEpc; ++e) acc[h][e] = fmaf(pv[h], vf[e], acc[h][e]);
    }
  };

  // ---- stream this wave's tiles (tb + wave, tb + wave + NW, ...), two per
  // iteration: both tiles' loads are issued before the first is used, and no
  // load result is carried across the loop edge (so no wait ever covers a
  // load issued for a later tile).
  const int tb = start / kTileTokens;
  const int te = (end + kTileTokens - 1) / kTileTokens;
  {
    const int first = tb + wave;
    const int n_my = first < te ? (te - first + kNW - 1) / kNW : 0;
    int k = 0;
    for (; k + 1 < n_my; k += 2) {
      Regs ra, rb;
      load_tile(first + k * kNW, ra);
      load_tile(first + (k + 1) * kNW, rb);
      process(first + k * kNW, ra);
      process(first + (k + 1) * kNW, rb);
    }
    if (k < n_my) {
      Regs ra;
      load_tile(first + k * kNW, ra);
      process(first + k * kNW, ra);
    }
  }

  // ---- wave totals: row sums of l, token-row sums of acc
#pragma unroll
  for (int r = 0; r < 4; ++r) l[r] = row_sum16(l[r]);
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < kEpc; ++e)
#pragma unroll
      for (int off = kCh; off < 64; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off, 64);

  float *macc = reinterpret_cast<float *>(smem + C::kAccOff) + wave * GT * D;
  float2 *mml = reinterpret_cast<float2 *>(smem + C::kMlOff) + wave * GT;
  int *mbad = reinterpret_cast<int *>(smem + C::kBadOff);
  if (lane < kCh) {
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < kEpc; ++e) macc[h * D + lane * kEpc + e] = acc[h][e];
  }
  if (n == 0 && 4 * kg < GT) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * kg + r < GT) mml[4 * kg + r] = make_float2(m[r], l[r]);
  }
  if (lane == 0) mbad[wave] = bad ? 1 : 0;
  __syncthreads();

  // ---- merge the waves
  const float *acc_all = reinterpret_cast<const float *>(smem + C::kAccOff);
  const float2 *ml_all = reinterpret_cast<const float2 *>(smem + C::kMlOff);
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) any_bad |= mbad[w];
  for (int idx = threadIdx.x; idx < nh * D; idx += kNW * 64) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, ml_all[w * GT + h].x);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float2 ml = ml_all[w * GT + h];
      const float f = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
      den = fmaf(f, ml.y, den);
      num = fmaf(f, acc_all[(w * GT + h) * D + d], num);
    }
    if (any_bad) {
      num = den = M = __builtin_nanf("");
    }
    const int64_t row = (int64_t)s * H + head0 + h;
    if (nparts == 1) {
      out[row * D + d] = static_cast<T>(num / den);
    } else {
      const int64_t pi = row * a.max_parts + part;
      a.part_acc[pi * D + d] = num;
      if (d == 0) a.part_ml[pi] = make_float2(M, den);
    }
  }
}

// Merge of the partition partials of every split sequence:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
template <typename T, int D>
__global__ __launch_bounds__(256) void paged_decode_reduce_kernel(DecodeArgs a) {
  const int s = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int h = idx / D;
  const int d = idx - h * D;
  if (h >= a.n_heads) return;
  const int L = a.seq_lens[s];
  const int P = a.partition_tokens;
  if (L <= P || (int64_t)L > (int64_t)a.max_blocks * a.block_size) return;  // single partition or invalid
  const int nparts = (L + P - 1) / P;
  const int64_t row = (int64_t)s * a.n_heads + h;
  const float2 *ml = a.part_ml + row * a.max_parts;
  const float *acc = a.part_acc + row * a.max_parts * D + d;
  float M = -INFINITY;
  bool bad = false;
  for (int p = 0; p < nparts; ++p) {
    const float mp = ml[p].x;
    bad |= mp != mp;
    M = fmaxf(M, mp);
  }
  float num = 0.f, den = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float2 v = ml[p];
    const float f = exp2f(v.x - M);
    den = fmaf(f, v.y, den);
    num = fmaf(f, acc[(int64_t)p * D], num);
  }
  static_cast<T *>(a.out)[row * D + d] = static_cast<T>(bad ? __builtin_nanf("") : num / den);
}

template <typename T, int D, int GT>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
  dim3 grid(a.n_kv_heads * a.head_chunks, a.num_seqs, a.max_parts);
  hipLaunchKernelGGL((paged_decode_kernel<T, D, GT>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.max_parts == 1) return err;
  dim3 rgrid((a.n_heads * D + 255) / 256, a.num_seqs, 1);
  hipLaunchKernelGGL((paged_decode_reduce_kernel<T, D>), rgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(int gt, const DecodeArgs &a, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_t<T, D, 1>(a, stream);
    case 2: return launch_t<T, D, 2>(a, stream);
    case 4: return launch_t<T, D, 4>(a, stream);
    case 8: return launch_t<T, D, 8>(a, stream);
    case 16: return launch_t<T, D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_dt(int head_dim, int gt, const DecodeArgs &a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<T, 64>(gt, a, stream);
    case 128: return launch_d<T, 128>(gt, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_head_tile(int group) {
  int gt = 1;
  while (gt < group && gt < 16) gt <<= 1;
  return gt;
}

hipError_t launch_decode(DType dt, int head_dim, const DecodeArgs &a, hipStream_t stream) {
  const int gt = decode_head_tile(a.group);
  switch (dt) {
    case DType::F32: return launch_dt<float>(head_dim, gt, a, stream);
    case DType::F16: return launch_dt<_Float16>(head_dim, gt, a, stream);
    case DType::BF16: return launch_dt<__bf16>(head_dim, gt, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
