// Slot-mapped KV cache write for CDNA4 (gfx950).
//
// Each new token's K and V rows (all KV heads) are copied into the pool slot
// the scheduler allocated for it: block slot / block_size, offset
// slot % block_size (vLLM notes page, "V1 engine": slots are allocated before
// the forward pass; vLLM paper page: a sequence grows one block at a time).
// The copy is bitwise, in 16-byte units; a negative slot (padding) or a slot
// past the pool is skipped, so the kernel never writes out of bounds.
#include "fp8_encode.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kWriteThreads = 256;

__global__ __launch_bounds__(kWriteThreads) void kv_cache_write_kernel(CacheWriteArgs a) {
  const int units = a.n_kv_heads * a.row_chunks;  // 16-byte units per token, per pool
  const uint4 *kn = static_cast<const uint4 *>(a.k_new);
  const uint4 *vn = static_cast<const uint4 *>(a.v_new);
  uint4 *kp = static_cast<uint4 *>(a.k_pool);
  uint4 *vp = static_cast<uint4 *>(a.v_pool);
  for (int t = blockIdx.x; t < a.num_tokens; t += gridDim.x) {
    // The rows are read before the slot is known (both loads in flight at
    // once); only the stores depend on it.
    for (int u = threadIdx.x; u < 2 * units; u += kWriteThreads) {
      const bool is_v = u >= units;
      const int uu = is_v ? u - units : u;
      const int64_t src = (int64_t)t * units + uu;
      int32_t slot32 = a.slot_mapping[t];
      uint4 val = is_v ? vn[src] : kn[src];
      // an empty asm that consumes both values: the compiler may not sink the
      // row load below the slot test, so one wait covers both loads
      asm volatile("" : "+v"(slot32), "+v"(val.x), "+v"(val.y), "+v"(val.z), "+v"(val.w));
      const int64_t slot = slot32;
      if (slot < 0 || slot >= a.num_slots) continue;
      const int64_t blk = slot / a.block_size;
      const int64_t off = slot - blk * a.block_size;
      const int head = uu / a.row_chunks;
      const int c = uu - head * a.row_chunks;
      const int64_t dst = ((blk * a.n_kv_heads + head) * a.block_size + off) * a.row_chunks + c;
      (is_v ? vp : kp)[dst] = val;
    }
  }
}

// --------------------------------------------------------------------------
// FP8 (OCP e4m3) pools: each new row is quantized with its KV head's scale.
// The value encoded is the float32 product x * (1 / scale) (both correctly
// rounded), and the encoding rounds to the nearest e4m3 value, ties to the
// even code, saturating at +-448; NaN stays NaN. KV-cache quantization is
// one of the further KV optimisations the vLLM paper page lists; the format
// and rounding are this library's (the pages fix none).
// --------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ float elem_to_float(T v) { return static_cast<float>(v); }

// 16 consecutive input elements of one row -> 16 floats
template <typename T> __device__ __forceinline__ void load16(const T *p, float *f) {
  constexpr int kLoads = 16 * (int)sizeof(T) / 16;
  constexpr int kPer = 16 / kLoads;
  const u32x4_t *q = reinterpret_cast<const u32x4_t *>(p);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const u32x4_t c = q[i];
    const T *e = reinterpret_cast<const T *>(&c);
#pragma unroll
    for (int j = 0; j < kPer; ++j) f[i * kPer + j] = elem_to_float<T>(e[j]);
  }
}

template <typename T>
__global__ __launch_bounds__(kWriteThreads) void kv_cache_write_fp8_kernel(CacheWriteFp8Args a) {
  const int row_units = a.head_dim / 16;        // 16-element units per row
  const int units = a.n_kv_heads * row_units;   // per token, per pool
  for (int t = blockIdx.x; t < a.num_tokens; t += gridDim.x) {
    for (int u = threadIdx.x; u < 2 * units; u += kWriteThreads) {
      const bool is_v = u >= units;
      const int uu = is_v ? u - units : u;
      const int head = uu / row_units;
      const int c = uu - head * row_units;
      const T *src = static_cast<const T *>(is_v ? a.v_new : a.k_new) +
                     ((int64_t)t * a.n_kv_heads + head) * a.head_dim + 16 * c;
      int32_t slot32 = a.slot_mapping[t];
      float f[16];
      load16<T>(src, f);
      const float sc = (is_v ? a.v_scale : a.k_scale)[head];
      asm volatile("" : "+v"(slot32));
      const int64_t slot = slot32;
      if (slot < 0 || slot >= a.num_slots) continue;
      const float inv = __fdiv_rn(1.0f, sc);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = f32_to_e4m3(__fmul_rn(f[4 * i], inv)) | (f32_to_e4m3(__fmul_rn(f[4 * i + 1], inv)) << 8) |
               (f32_to_e4m3(__fmul_rn(f[4 * i + 2], inv)) << 16) |
               (f32_to_e4m3(__fmul_rn(f[4 * i + 3], inv)) << 24);
      }
      const int64_t blk = slot / a.block_size;
      const int64_t off = slot - blk * a.block_size;
      uint8_t *dst = (is_v ? a.v_pool : a.k_pool) +
                     ((blk * a.n_kv_heads + head) * a.block_size + off) * a.head_dim + 16 * c;
      *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

}  // namespace

hipError_t launch_cache_write_fp8(DType in_dtype, const CacheWriteFp8Args &a, hipStream_t stream) {
  const int grid = a.num_tokens < 65536 ? a.num_tokens : 65536;
  switch (in_dtype) {
    case DType::F32:
      hipLaunchKernelGGL(kv_cache_write_fp8_kernel<float>, dim3(grid), dim3(kWriteThreads), 0, stream, a);
      break;
    case DType::F16:
      hipLaunchKernelGGL(kv_cache_write_fp8_kernel<_Float16>, dim3(grid), dim3(kWriteThreads), 0, stream, a);
      break;
    case DType::BF16:
      hipLaunchKernelGGL(kv_cache_write_fp8_kernel<__bf16>, dim3(grid), dim3(kWriteThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream) {
  const int grid = a.num_tokens < 65536 ? a.num_tokens : 65536;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3(grid), dim3(kWriteThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
