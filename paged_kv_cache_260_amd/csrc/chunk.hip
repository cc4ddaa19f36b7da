// Paged attention of a chunk of new query tokens per sequence, causal inside
// the chunk, for CDNA4 (gfx950): the kernel for long chunks (chunked prefill).
//
// What is computed: the chunk of sequence s holds its last n_s = qsl[s+1] -
// qsl[s] tokens (their K/V already in the cache, L_s tokens in all). Chunk
// token i sits at position p = L_s - n_s + i and attends, per query head,
// over the cached tokens 0 .. p. Sources: chunked prefill (Sarathi-Serve, on
// the PagedAttention notes page); continuous batching, where packed sequences
// keep to their own tokens through positions and the attention mask (vLLM
// notes page, scheduling section); the exact tiled softmax of FlashAttention
// (vLLM notes page, "FlashAttention").
//
// Long chunks make this a dense contraction: every K/V tile meets many query
// rows. One workgroup (8 waves) takes 256 query rows of one KV head: rows are
// (chunk token, query head of g) pairs, token-major, so the G heads of one
// token and 256 / G consecutive tokens share each K/V tile. The context is
// walked in 64-token stages:
//   1. The stage's K and V rows (64 x head_dim each) are loaded by the whole
//      workgroup into registers one stage ahead, then written to LDS (K
//      row-major, V for transposed reads; both XOR-swizzled) in a double
//      buffer, with one barrier per stage. Block ids come from a 64-entry
//      window of the block table held one per lane.
//   2. Each wave owns 32 rows (two 16-row MFMA tiles) and computes the
//      transposed scores S^T = K Q^T with v_mfma_f32_16x16x32: Q stays in
//      registers as the B operand, K is the A operand read from LDS. Lane
//      (kg, n) receives tokens 4 kg .. 4 kg + 3 of row n in each 16-token
//      block.
//   3. Online softmax in base 2 with a lazy reference max (raised only when a
//      score passes it by more than 8); the causal mask is applied only in
//      stages that reach past a row's position.
//   4. O^T += V^T P^T, again on v_mfma_f32_16x16x32: the eight weights a lane
//      holds for its row (two 16-token blocks) are exactly its B operand for
//      32 tokens (both operands list the tokens in the same order, which is
//      all a contraction needs), and V^T comes from LDS through
//      ds_read_b64_tr_b16.
// P is rounded to the 16-bit type for the product (accumulation is fp32).
#include "attn_common.h"
#include "kernels.h"

#include <math.h>

namespace pkv {
namespace {

using namespace attn;

constexpr int kPfWaves = 8;
constexpr int kPfRowsPerWave = 32;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // 256 query rows per workgroup
constexpr int kPfStage = 64;                         // context tokens per stage

template <typename T, int D, bool F8> struct PfCfg {
  static constexpr int kCh = D / 8;                                // 16-byte chunks per token row (in LDS)
  static constexpr int kChKV = F8 ? D / 16 : D / 8;                // 16-byte chunks per stored token row
  static constexpr int kTileChunks = kPfStage * kChKV;             // 16-byte chunks of one stored tile
  static constexpr int kSteps = kCh / 4;                           // QK MFMA steps (32 dims each)
  static constexpr int kDimBlocks = D / 16;                        // 16-dim output blocks
  static constexpr int kLoads = (kTileChunks + kPfWaves * 64 - 1) / (kPfWaves * 64);  // per thread per tile
  static constexpr int kTileBytes = kPfStage * kCh * 16;           // one K (or V) stage in LDS
  static constexpr int kBufBytes = 2 * kTileBytes;                 // K + V
  static constexpr int kSmem = 2 * kBufBytes;                      // double buffer
  static_assert(sizeof(T) == 2 && (kCh == 8 || kCh == 16), "16-bit types, head_dim 64 or 128");
};

// two floats -> two elements of T (round to nearest even) in one word; a
// vector conversion, so bf16 takes one v_cvt_pk_bf16_f32
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef T t2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), t2));
}

// F8: the pools hold OCP e4m3 codes with one scale per KV head; each 16-byte
// load (16 codes of one token) is decoded exactly into two 16-byte chunks of T
// on its way into LDS, k_scale is folded into the score scale and v_scale
// into the output.
template <typename T, int D, bool F8>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void paged_chunk_kernel(ChunkArgs a) {
  using C = PfCfg<T, D, F8>;
  constexpr int kChKV = C::kChKV;
  constexpr int kCh = C::kCh;
  constexpr int kL = C::kLoads;
  constexpr int kDB = C::kDimBlocks;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4;
  const int n = lane & 15;
  // work item: row blocks of later chunk tokens (more context) first
  const int items_per_rb = a.n_kv_heads * a.num_seqs;
  const int rb = a.row_blocks - 1 - (int)(blockIdx.x / (unsigned)items_per_rb);
  const int rem = (int)(blockIdx.x % (unsigned)items_per_rb);
  const int g = rem % a.n_kv_heads;
  const int s = rem / a.n_kv_heads;
  const int G = a.group;
  const int H = a.n_heads;
  const int q0 = a.query_start_loc[s];
  const int nq = a.query_start_loc[s + 1] - q0;
  const int L = a.seq_lens[s];
  const int row0 = rb * kPfRows;
  if (nq <= 0 || q0 < 0 || row0 >= nq * G) return;
  const int nrows = min(kPfRows, nq * G - row0);
  T *out = static_cast<T *>(a.out);
  auto out_row = [&](int r) -> int64_t {  // r: row within the item
    const int rr = row0 + r;
    return (int64_t)(q0 + rr / G) * H + g * G + rr % G;
  };

  const bool bad_len = L < nq || (int64_t)L > (int64_t)a.max_blocks * a.block_size;
  if (bad_len) {
    for (int i = tid; i < nrows * D; i += kPfWaves * 64)
      out[out_row(i / D) * D + i % D] = static_cast<T>(__builtin_nanf(""));
    return;
  }
  const int base_pos = L - nq;                                // position of chunk token 0
  const int ctx_end = base_pos + (row0 + nrows - 1) / G + 1;  // tokens the item's rows may see

  // this lane's rows (one per row tile) and their last visible positions;
  // rows past nrows (padding) take the last row's position
  const int wrow0 = wave * kPfRowsPerWave;
  int rpos[2];
  bool rvalid[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = wrow0 + 16 * rt + n;
    rvalid[rt] = r < nrows;
    rpos[rt] = base_pos + (row0 + min(r, nrows - 1)) / G;
  }
  // smallest position among the wave's rows: stages up to it need no mask
  const int wave_min_pos = base_pos + (row0 + min(wrow0, nrows - 1)) / G;

  // Q operand (B of S^T = K Q^T): lane (kg, n) holds chunk 4 c + kg of row n
  u32x4_t qb[2][C::kSteps];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = wrow0 + 16 * rt + n;
#pragma unroll
    for (int c = 0; c < C::kSteps; ++c) {
      qb[rt][c] = u32x4_t{0u, 0u, 0u, 0u};
      if (r < nrows)
        qb[rt][c] = reinterpret_cast<const u32x4_t *>(static_cast<const T *>(a.q) + out_row(r) * D)[4 * c + kg];
    }
  }

  const int64_t kv_stride_blk = (int64_t)a.n_kv_heads * a.block_size;
  const int32_t *bt_row = a.block_tables + (int64_t)s * a.max_blocks;
  const u32x4_t *kbase = static_cast<const u32x4_t *>(a.k_pool);
  const u32x4_t *vbase = static_cast<const u32x4_t *>(a.v_pool);
  const int nst = (ctx_end + kPfStage - 1) / kPfStage;
  // block-table window: lane i holds entry win + i (a stage spans at most 4
  // blocks, so it always fits one window)
  int win = 0;
  int btv = lane < a.max_blocks ? bt_row[lane] : 0;
  bool bad = false;

  struct Regs {
    u32x4_t k[kL];
    u32x4_t v[kL];
  };
  // loads of stage st into registers: thread chunk u = tid + 512 i is stored
  // chunk u % kChKV of token u / kChKV; tokens at or past ctx_end stay zero
  auto load_stage = [&](int st, Regs &rg) {
    const int t0 = st * kPfStage;
    const int last_blk = (min(t0 + kPfStage, ctx_end) - 1) >> a.block_shift;
    if (last_blk >= win + 64) {  // uniform: move the window to this stage
      win = t0 >> a.block_shift;
      btv = win + lane < a.max_blocks ? bt_row[win + lane] : 0;
    }
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int u = tid + i * kPfWaves * 64;
      const int tok = t0 + u / kChKV;
      rg.k[i] = rg.v[i] = u32x4_t{0u, 0u, 0u, 0u};
      const int j = (min(tok, ctx_end - 1) >> a.block_shift) - win;  // 0 .. 63
      int phys = __shfl(btv, j, 64);
      if (tok < ctx_end && u < C::kTileChunks) {
        if (phys < 0 || (int64_t)phys >= a.num_blocks) {
          bad = true;
          phys = 0;
        }
        const int64_t off = ((int64_t)phys * kv_stride_blk + (int64_t)g * a.block_size +
                             (tok & (a.block_size - 1))) * kChKV + u % kChKV;
        rg.k[i] = __builtin_nontemporal_load(kbase + off);
        rg.v[i] = __builtin_nontemporal_load(vbase + off);
      }
    }
  };
  auto store_stage = [&](int buf, const Regs &rg) {
    u32x4_t *ks = reinterpret_cast<u32x4_t *>(smem + buf * C::kBufBytes);
    u32x4_t *vs = reinterpret_cast<u32x4_t *>(smem + buf * C::kBufBytes + C::kTileBytes);
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      const int u = tid + i * kPfWaves * 64;
      if (u >= C::kTileChunks) continue;
      const int tr = u / kChKV;
      const int ch = u % kChKV;
      if constexpr (F8) {
        u32x4_t lo, hi;
        fp8x16_to<T>(rg.k[i], lo, hi);
        ks[kst_slot<kCh>(tr, 2 * ch)] = lo;
        ks[kst_slot<kCh>(tr, 2 * ch + 1)] = hi;
        fp8x16_to<T>(rg.v[i], lo, hi);
        vs[tr * kCh + ((2 * ch) ^ vst_swz<kCh>(tr))] = lo;
        vs[tr * kCh + ((2 * ch + 1) ^ vst_swz<kCh>(tr))] = hi;
      } else {
        ks[kst_slot<kCh>(tr, ch)] = rg.k[i];
        vs[tr * kCh + (ch ^ vst_swz<kCh>(tr))] = rg.v[i];
      }
    }
  };

  // running state per row tile: reference max (base 2), the weight sums, and
  // O^T accumulators (lane (kg, n): row n, dims 16 b + 4 kg + r)
  // lsum[rt]: every element holds row n's sum of weights
  float m[2] = {-INFINITY, -INFINITY};
  f32x4_t lsum[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  const uint32_t one2 = pack2<T>(1.f, 1.f);
  const u32x4_t ones = u32x4_t{one2, one2, one2, one2};
  f32x4_t acc[2][kDB];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int b = 0; b < kDB; ++b) acc[rt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr float kLazy = 8.f;
  float sl2 = a.scale_log2;  // scores in base-2 units
  float vsc = 1.f;           // output scale
  if constexpr (F8) {
    sl2 *= a.k_scale[g];
    vsc = a.v_scale[g];
  }
  const float inv_sl2 = 1.f / sl2;
  // transposed V reads: this lane addresses token 4 kg + (n >> 2) of a 16-token block
  const int tr_tok = 4 * kg + (n >> 2);
  const int v_tr_off = tr_tok * kCh * 16 + (lane & 3) * 8;
  const int v_tr_swz = vst_swz<kCh>(tr_tok);

  Regs rg;
  load_stage(0, rg);
  store_stage(0, rg);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage(st + 1, rg);
    const u32x4_t *ks = reinterpret_cast<const u32x4_t *>(smem + buf * C::kBufBytes);
    const char *vs = smem + buf * C::kBufBytes + C::kTileBytes;
    const int t0 = st * kPfStage;

    // S^T = K Q^T for 4 token blocks x 2 row tiles
    f32x4_t sc[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      sc[tb][0] = sc[tb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::kSteps; ++c) {
        const u32x4_t kop = ks[kst_slot<kCh>(tb * 16 + n, 4 * c + kg)];
        sc[tb][0] = mfma_chunk<T>(kop, qb[0][c], sc[tb][0]);
        sc[tb][1] = mfma_chunk<T>(kop, qb[1][c], sc[tb][1]);
      }
    }
    u32x4_t pt[2][2];  // P^T operands: [row tile][32-token half]
    // raw scores (the scale is applied inside the exponent's FMA); the causal
    // mask, only in the stages that reach past a row's position (a real
    // branch: the empty asm keeps it from becoming selects everywhere)
    if (t0 + kPfStage - 1 > wave_min_pos) {
      asm volatile("");
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[tb][rt][r] = t0 + tb * 16 + 4 * kg + r <= rpos[rt] ? sc[tb][rt][r] : -INFINITY;
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      // a raw score passes the reference by more than kLazy (base-2 units)
      // when it exceeds (m + kLazy) / sl2 (sl2 > 0)
      const float thr = (m[rt] + kLazy) * inv_sl2;
      bool over = false;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) over |= sc[tb][rt][r] > thr;
      if (__builtin_amdgcn_ballot_w64(over) != 0) {  // uniform: raise the reference
        float mx = sc[0][rt][0];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[tb][rt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m[rt], mx * sl2);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[rt] - mn);
        m[rt] = mn;
        lsum[rt] *= alpha;
#pragma unroll
        for (int b = 0; b < kDB; ++b) acc[rt][b] *= alpha;
      }
      // every row sees token 0 in the first stage, so m is finite from then
      // on and masked scores give exp2(-inf) = 0 with no test
      float p[4][4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[tb][r] = __builtin_amdgcn_exp2f(fmaf(sc[tb][rt][r], sl2, -m[rt]));
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pt[rt][h] = u32x4_t{pack2<T>(p[2 * h][0], p[2 * h][1]), pack2<T>(p[2 * h][2], p[2 * h][3]),
                            pack2<T>(p[2 * h + 1][0], p[2 * h + 1][1]), pack2<T>(p[2 * h + 1][2], p[2 * h + 1][3])};
    }
    // O^T += V^T P^T: 32 tokens (two 16-token blocks) per MFMA
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < kDB; ++b) {
        const int cofs = ((2 * b) ^ v_tr_swz) << 4;
        const auto v0 = lds_read_tr<T>(vs + (2 * h) * 16 * kCh * 16 + v_tr_off + cofs);
        const auto v1 = lds_read_tr<T>(vs + (2 * h + 1) * 16 * kCh * 16 + v_tr_off + cofs);
        const uint2 w0 = __builtin_bit_cast(uint2, v0);
        const uint2 w1 = __builtin_bit_cast(uint2, v1);
        const u32x4_t vop = u32x4_t{w0.x, w0.y, w1.x, w1.y};
        acc[0][b] = mfma_chunk<T>(vop, pt[0][h], acc[0][b]);
        acc[1][b] = mfma_chunk<T>(vop, pt[1][h], acc[1][b]);
      }
      // row sums of the rounded weights on the MFMA (V^T = ones): the same
      // weights as the numerator, and no per-element adds
      lsum[0] = mfma_chunk<T>(ones, pt[0][h], lsum[0]);
      lsum[1] = mfma_chunk<T>(ones, pt[1][h], lsum[1]);
    }
    if (st + 1 < nst) store_stage(buf ^ 1, rg);
    __syncthreads();
  }

  // ---- finalize: O = acc / sum
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float inv = vsc / lsum[rt][0];
    if (!rvalid[rt]) continue;
    T *orow = out + out_row(wrow0 + 16 * rt + n) * D;
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
      const float nan = __builtin_nanf("");
      uint2 w;
      w.x = pack2<T>(any_bad ? nan : acc[rt][b][0] * inv, any_bad ? nan : acc[rt][b][1] * inv);
      w.y = pack2<T>(any_bad ? nan : acc[rt][b][2] * inv, any_bad ? nan : acc[rt][b][3] * inv);
      *reinterpret_cast<uint2 *>(orow + 16 * b + 4 * kg) = w;
    }
  }
}

template <typename T, int D, bool F8> hipError_t launch_chunk_td(const ChunkArgs &a, hipStream_t stream) {
  constexpr int kSmem = PfCfg<T, D, F8>::kSmem;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&paged_chunk_kernel<T, D, F8>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((int64_t)a.n_kv_heads * a.num_seqs * a.row_blocks));
  hipLaunchKernelGGL((paged_chunk_kernel<T, D, F8>), grid, dim3(kPfWaves * 64), kSmem, stream, a);
  return hipGetLastError();
}

template <typename T, bool F8>
hipError_t launch_chunk_t(int head_dim, const ChunkArgs &a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_chunk_td<T, 64, F8>(a, stream);
    case 128: return launch_chunk_td<T, 128, F8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int chunk_rows_per_block() { return kPfRows; }

hipError_t launch_chunk(DType dt, int head_dim, bool fp8, const ChunkArgs &a, hipStream_t stream) {
  switch (dt) {
    case DType::F16: return fp8 ? launch_chunk_t<_Float16, true>(head_dim, a, stream)
                                : launch_chunk_t<_Float16, false>(head_dim, a, stream);
    case DType::BF16: return fp8 ? launch_chunk_t<__bf16, true>(head_dim, a, stream)
                                 : launch_chunk_t<__bf16, false>(head_dim, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
