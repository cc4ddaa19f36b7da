// Paged attention of a chunk of new query tokens per sequence, causal inside
// the chunk, for CDNA4 (gfx950).
//
// What is computed: the chunk of sequence s holds its last n_s = qsl[s+1] -
// qsl[s] tokens (their K/V already in the cache, L_s tokens in all). Chunk
// token i sits at position p = L_s - n_s + i and attends, per query head,
// over the cached tokens 0 .. p. n_s = 1 is a decode step and n_s = L_s a
// whole causal prefill. Sources: chunked prefill (Sarathi-Serve, on the
// PagedAttention notes page); speculative decoding, whose target model scores
// several draft tokens at once, and continuous batching, where packed
// sequences keep to their own tokens through positions and the attention mask
// (vLLM notes page, scheduling and speculative-decoding sections).
//
// Work decomposition: one 4-wave workgroup per (KV head g, sequence s, block
// of 16 query rows). Rows are (chunk token, query head of g) pairs,
// token-major: row r is token r / G, head g * G + r % G. So a speculative
// chunk of 4 tokens with 4 heads per KV head fills exactly one MFMA row tile.
// The workgroup walks the causal context in segments of at most 64 blocks
// (their table entries sit one per lane in a VGPR). Inside a segment the
// 16-token tiles go round-robin to the waves, as in the decode kernel.
//
// Per tile, per wave:
//   1. Load the K and V tiles, one tile ahead.
//   2. Stage them in swizzled wave-private LDS.
//   3. S = Q K^T on v_mfma_f32_16x16x32 (Q, 16 rows, from LDS).
//   4. Mask tokens past each row's position.
//   5. Online softmax in base 2 with the lazy reference max.
//   6. P (hi + lo) and V^T through ds_read_b64_tr_b16 into v_mfma_f32_16x16x16.
// The four waves' states are merged through LDS at the end.
#include "attn_common.h"
#include "kernels.h"

#include <math.h>

namespace pkv {
namespace {

using namespace attn;

constexpr int kChunkWaves = 4;
constexpr int kChunkRows = 16;
constexpr int kSegBlocks = 64;

template <typename T, int D> struct ChunkCfg {
  static constexpr int kEpc = Elem<T>::kPerChunk;
  static constexpr int kCh = D / kEpc;                   // 16-byte chunks per token row
  static constexpr int kLoads = kTileTokens * kCh / 64;  // 16-byte loads per lane per tile
  static constexpr int kSteps = kCh / 4;                 // QK MFMA steps per tile
  static constexpr int kDimBlocks = D / 16;
  static constexpr int kNW = kChunkWaves;
  static constexpr int kKstBytes = kTileTokens * kCh * 16;
  static constexpr int kVstBytes = kTileTokens * kCh * 16;
  static constexpr int kPstBytes = 2 * 16 * 16 * 2;
  static constexpr int kStageBytes = kKstBytes + kVstBytes + kPstBytes;
  static constexpr int kAccBytes = kChunkRows * D * 4;
  static constexpr int kWaveBytes = kStageBytes > kAccBytes ? kStageBytes : kAccBytes;
  static constexpr int kMlOff = kNW * kWaveBytes;
  static constexpr int kBadOff = kMlOff + kNW * kChunkRows * 8;
  static constexpr int kQOff = (kBadOff + kNW * 4 + 15) / 16 * 16;
  static constexpr int kQChunks = kChunkRows * kCh;
  static constexpr int kSmem = kQOff + kQChunks * 16;
  static_assert(sizeof(T) == 2 && (kCh == 8 || kCh == 16), "16-bit types, head_dim 64 or 128");
};

template <typename T, int D>
__global__ __launch_bounds__(kChunkWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void paged_chunk_kernel(ChunkArgs a) {
  using C = ChunkCfg<T, D>;
  constexpr int kL = C::kLoads;
  constexpr int kCh = C::kCh;
  constexpr int kNW = C::kNW;
  __shared__ __attribute__((aligned(16))) char smem[C::kSmem];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = (int)(blockIdx.x % (unsigned)a.n_kv_heads);
  const int rr = (int)(blockIdx.x / (unsigned)a.n_kv_heads);
  const int rb = rr % a.row_blocks;
  const int s = rr / a.row_blocks;
  const int G = a.group;
  const int H = a.n_heads;
  const int q0 = a.query_start_loc[s];
  const int nq = a.query_start_loc[s + 1] - q0;
  const int L = a.seq_lens[s];
  const int row0 = rb * kChunkRows;
  if (nq <= 0 || q0 < 0 || row0 >= nq * G) return;
  const int nrows = min(kChunkRows, nq * G - row0);
  T *out = static_cast<T *>(a.out);
  const int kg = lane >> 4;
  const int n = lane & 15;

  auto row_token = [&](int i) { return (row0 + i) / G; };
  auto row_head = [&](int i) { return g * G + (row0 + i) % G; };

  const bool bad_len = L < nq || (int64_t)L > (int64_t)a.max_blocks * a.block_size;
  if (bad_len) {
    for (int i = threadIdx.x; i < nrows * D; i += kNW * 64) {
      const int r = i / D;
      out[((int64_t)(q0 + row_token(r)) * H + row_head(r)) * D + i % D] = static_cast<T>(__builtin_nanf(""));
    }
    return;
  }
  // positions: row i sees tokens 0 .. L - nq + token(i); the block's context
  // ends after its last row's position
  const int base_pos = L - nq;
  const int ctx_end = base_pos + row_token(nrows - 1) + 1;
  int lim[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * kg + r;
    lim[r] = i < nrows ? base_pos + row_token(i) : -1;
  }

  // Q rows -> LDS (swizzled like a K tile), zero past nrows
  {
    u32x4_t *qs = reinterpret_cast<u32x4_t *>(smem + C::kQOff);
    for (int u = threadIdx.x; u < C::kQChunks; u += kNW * 64) {
      const int i = u / kCh;
      const int c = u - i * kCh;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (i < nrows)
        v = reinterpret_cast<const u32x4_t *>(static_cast<const T *>(a.q) +
                                              ((int64_t)(q0 + row_token(i)) * H + row_head(i)) * D)[c];
      qs[kst_slot<kCh>(i, c)] = v;
    }
  }
  __syncthreads();
  const u32x4_t *qs = reinterpret_cast<const u32x4_t *>(smem + C::kQOff);

  char *wreg = smem + wave * C::kWaveBytes;
  u32x4_t *kst = reinterpret_cast<u32x4_t *>(wreg);
  char *vst = wreg + C::kKstBytes;
  char *pst = wreg + C::kKstBytes + C::kVstBytes;
  for (int i = lane; i < 2 * 16 * 16 / 8; i += 64) reinterpret_cast<uint2 *>(pst)[i] = make_uint2(0u, 0u);

  const int64_t kv_stride_blk = (int64_t)a.n_kv_heads * a.block_size;
  const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  const u32x4_t *kbase = static_cast<const u32x4_t *>(a.k_pool);
  const u32x4_t *vbase = static_cast<const u32x4_t *>(a.v_pool);
  bool bad = false;
  struct Regs {
    u32x4_t k[kL];
    u32x4_t v[kL];
  };

  float m[4], l[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
  f32x4_t acc[C::kDimBlocks];
#pragma unroll
  for (int b = 0; b < C::kDimBlocks; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int tr_tok = 4 * kg + ((lane & 15) >> 2);
  const int p_tr_off = tr_tok * 32 + (lane & 3) * 8;
  const int v_tr_base = tr_tok * kCh * 16 + (lane & 3) * 8;
  const int v_tr_swz = vst_swz<kCh>(tr_tok);
  constexpr float kLazy = 8.f;

  const int seg_tokens = kSegBlocks * a.block_size;
  for (int seg = 0; seg < ctx_end; seg += seg_tokens) {
    const int seg_end = min(ctx_end, seg + seg_tokens);
    const int jb = seg >> a.block_shift;
    const int jmax = (seg_end - 1) >> a.block_shift;
    const int btv = jb + lane <= jmax ? bt_row[jb + lane] : 0;

    auto load_tile = [&](int ti, Regs &rg) {
      const int tok = ti * kTileTokens;
      int phys = __builtin_amdgcn_readlane(btv, (tok >> a.block_shift) - jb);
      if (phys < 0 || (int64_t)phys >= a.num_blocks) {
        bad = true;
        phys = 0;
      }
      const int64_t off = ((int64_t)phys * kv_stride_blk + (int64_t)g * a.block_size +
                           (tok & (a.block_size - 1))) * kCh;
#pragma unroll
      for (int i = 0; i < kL; ++i) rg.k[i] = kbase[off + i * 64 + lane];
#pragma unroll
      for (int i = 0; i < kL; ++i) rg.v[i] = vbase[off + i * 64 + lane];
    };

    auto process = [&](int ti, Regs &rg, int next) {
      const int valid = seg_end - ti * kTileTokens;  // tokens of this tile inside the context
      u32x4_t *vs = reinterpret_cast<u32x4_t *>(vst);
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const int u = i * 64 + lane;
        const int tr = u / kCh;
        kst[kst_slot<kCh>(tr, u % kCh)] = rg.k[i];
        // rows past the context are zeroed: 0 * NaN would poison the sums
        vs[tr * kCh + ((u % kCh) ^ vst_swz<kCh>(tr))] = tr < valid ? rg.v[i] : u32x4_t{0u, 0u, 0u, 0u};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (next >= 0) load_tile(next, rg);
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::kSteps; ++c)
        sc = mfma_chunk<T>(qs[kst_slot<kCh>(n, kg + 4 * c)], kst[kst_slot<kCh>(n, kg + 4 * c)], sc);
      const int tok = ti * kTileTokens + n;
      float z[4];
      bool over = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = tok <= lim[r] ? sc[r] * a.scale_log2 : -INFINITY;
        over |= z[r] > m[r] + kLazy;
      }
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float mn = fmaxf(m[r], row_max16(z[r]));
          const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[r] - mn);
          m[r] = mn;
          l[r] *= alpha;
#pragma unroll
          for (int b = 0; b < C::kDimBlocks; ++b) acc[b][r] *= alpha;
        }
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = z[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[r] - m[r]);
        l[r] += p[r];
      }
      typename Pv<T>::v4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = static_cast<T>(p[r]);
        lo[r] = static_cast<T>(p[r] - static_cast<float>(hi[r]));
      }
      *reinterpret_cast<typename Pv<T>::v4 *>(pst + n * 32 + kg * 8) = hi;
      *reinterpret_cast<typename Pv<T>::v4 *>(pst + 512 + n * 32 + kg * 8) = lo;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const typename Pv<T>::v4 pa_hi = lds_read_tr<T>(pst + p_tr_off);
      const typename Pv<T>::v4 pa_lo = lds_read_tr<T>(pst + 512 + p_tr_off);
#pragma unroll
      for (int b = 0; b < C::kDimBlocks; ++b) {
        const typename Pv<T>::v4 vb = lds_read_tr<T>(vst + v_tr_base + (((2 * b) ^ v_tr_swz) << 4));
        acc[b] = Pv<T>::mfma(pa_hi, vb, acc[b]);
        acc[b] = Pv<T>::mfma(pa_lo, vb, acc[b]);
      }
    };

    const int tb = seg / kTileTokens;
    const int te = (seg_end + kTileTokens - 1) / kTileTokens;
    Regs rg;
    int ti = tb + wave;
    if (ti < te) load_tile(ti, rg);
    for (; ti < te; ti += kNW) process(ti, rg, ti + kNW < te ? ti + kNW : -1);
  }

  // ---- merge the four waves through LDS
#pragma unroll
  for (int r = 0; r < 4; ++r) l[r] = row_sum16(l[r]);
  __syncthreads();  // every wave is done with its staging area
  float *macc = reinterpret_cast<float *>(wreg);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int b = 0; b < C::kDimBlocks; ++b) macc[(4 * kg + r) * D + 16 * b + n] = acc[b][r];
  float2 *mml = reinterpret_cast<float2 *>(smem + C::kMlOff) + wave * kChunkRows;
  if (n == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) mml[4 * kg + r] = make_float2(m[r], l[r]);
  }
  int *mbad = reinterpret_cast<int *>(smem + C::kBadOff);
  if (lane == 0) mbad[wave] = bad ? 1 : 0;
  __syncthreads();
  const float2 *ml_all = reinterpret_cast<const float2 *>(smem + C::kMlOff);
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) any_bad |= mbad[w];
  for (int idx = threadIdx.x; idx < nrows * D; idx += kNW * 64) {
    const int i = idx / D;
    const int d = idx - i * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, ml_all[w * kChunkRows + i].x);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float2 ml = ml_all[w * kChunkRows + i];
      const float f = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
      den = fmaf(f, ml.y, den);
      num = fmaf(f, reinterpret_cast<const float *>(smem + w * C::kWaveBytes)[i * D + d], num);
    }
    out[((int64_t)(q0 + row_token(i)) * H + row_head(i)) * D + d] =
        static_cast<T>(any_bad ? __builtin_nanf("") : num / den);
  }
}

template <typename T>
hipError_t launch_chunk_t(int head_dim, const ChunkArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.n_kv_heads * a.num_seqs * a.row_blocks));
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL((paged_chunk_kernel<T, 64>), grid, dim3(kChunkWaves * 64), 0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL((paged_chunk_kernel<T, 128>), grid, dim3(kChunkWaves * 64), 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk(DType dt, int head_dim, const ChunkArgs &a, hipStream_t stream) {
  switch (dt) {
    case DType::F16: return launch_chunk_t<_Float16>(head_dim, a, stream);
    case DType::BF16: return launch_chunk_t<__bf16>(head_dim, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
