// Slot-mapped KV cache write for CDNA4 (gfx950).
//
// Each new token's K and V rows (all KV heads) are copied into the pool slot
// the scheduler allocated for it: block slot / block_size, offset
// slot % block_size (vLLM notes page, "V1 engine": slots are allocated before
// the forward pass; vLLM paper page: a sequence grows one block at a time).
// The copy is bitwise, in 16-byte units; a negative slot (padding) or a slot
// past the pool is skipped, so the kernel never writes out of bounds.
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

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream) {
  const int grid = a.num_tokens < 65536 ? a.num_tokens : 65536;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3(grid), dim3(kWriteThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
