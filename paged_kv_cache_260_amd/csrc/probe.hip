// Read-bandwidth probes: what the chip delivers to kernels that only read,
// measured beside the decode kernel so its roofline fraction has a measured
// ceiling next to the datasheet peak (declared in pkv_probe.h).
//
//   stream_read_kernel   every 16-byte unit of one buffer, in address order,
//                        with non-temporal loads, UNROLL units in flight per
//                        thread (grid-stride).
//   gather_tiles_kernel  4 KiB tiles (one 16-token block of one KV head in
//                        bf16 at head_dim 128) taken from a pool in the order
//                        of a tile list: the decode kernel's access pattern.
//                        Each wave owns a run of 64 list entries, held one per
//                        lane and read back with v_readlane (as the decode
//                        kernel holds a partition's block-table entries), and
//                        keeps DEPTH tiles of non-temporal loads in flight.
// Neither writes anything but one word per workgroup when the xor of all it
// read equals a value no input produces in practice, which keeps the loads
// alive without adding traffic.
#include "kernels.h"
#include "pkv_probe.h"
#include "status.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kTileUnits = 4096 / 16;          // 16-byte units per tile
constexpr int kTileLoads = kTileUnits / 64;    // loads per lane per tile
constexpr uint32_t kNever = 0x9e3779b9u;

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <int UNROLL>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t *buf, int64_t units,
                                                                     uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < units; i += UNROLL * stride) {
    u32x4_t v[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) acc ^= fold(v[k]);
  }
  for (; i < units; i += stride) acc ^= fold(__builtin_nontemporal_load(buf + i));
  if (acc == kNever) sink[blockIdx.x] = acc;
}

template <int DEPTH>
__global__ __launch_bounds__(kProbeThreads) void gather_tiles_kernel(const u32x4_t *pool, int64_t pool_tiles,
                                                                      const int32_t *tiles, int64_t num_tiles,
                                                                      uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kProbeThreads / 64);
  const int64_t wave = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t runs = (num_tiles + 63) / 64;
  uint32_t acc = 0;
  for (int64_t r = wave; r < runs; r += waves) {
    const int64_t base = r * 64;
    const int n = (int)min<int64_t>(64, num_tiles - base);
    const int ids = lane < n ? tiles[base + lane] : 0;
    for (int t = 0; t < n; t += DEPTH) {
      u32x4_t v[DEPTH][kTileLoads];
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        // ids outside the pool are clamped into it (never read out of bounds)
        const int64_t tile = min<int64_t>(max(__builtin_amdgcn_readlane(ids, min(t + d, n - 1)), 0), pool_tiles - 1);
        const u32x4_t *p = pool + (int64_t)tile * kTileUnits + lane;
#pragma unroll
        for (int k = 0; k < kTileLoads; ++k) v[d][k] = __builtin_nontemporal_load(p + k * 64);
      }
#pragma unroll
      for (int d = 0; d < DEPTH; ++d)
#pragma unroll
        for (int k = 0; k < kTileLoads; ++k) acc ^= t + d < n ? fold(v[d][k]) : 0u;
    }
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

template <int DEPTH>
hipError_t launch_gather(const void *pool, int64_t pool_tiles, const int32_t *tiles, int64_t num_tiles, int32_t grid,
                         uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL((gather_tiles_kernel<DEPTH>), dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4_t *>(pool), pool_tiles, tiles, num_tiles, sink);
  return hipGetLastError();
}

}  // namespace
}  // namespace pkv

extern "C" {

int pkv_probe_stream_read(const void *buf, int64_t bytes, int32_t grid, uint32_t *sink, void *stream) {
  if (!buf || !sink) return pkv::set_error(PKV_ERR_INVALID, "null pointer");
  if (bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return pkv::set_error(PKV_ERR_INVALID, "buffer of %lld bytes: want a positive multiple of 16, 16-byte aligned",
                          (long long)bytes);
  if (grid < 1 || grid > (1 << 20)) return pkv::set_error(PKV_ERR_INVALID, "grid %d outside [1, 2^20]", grid);
  hipLaunchKernelGGL((pkv::stream_read_kernel<8>), dim3((unsigned)grid), dim3(pkv::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pkv::u32x4_t *>(buf), bytes / 16, sink);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::set_error(PKV_ERR_DEVICE, "stream read probe: %s", hipGetErrorString(e));
  return pkv::clear_error();
}

int pkv_probe_gather_tiles(const void *pool, int64_t pool_tiles, const int32_t *tiles, int64_t num_tiles,
                           int32_t depth, int32_t grid, uint32_t *sink, void *stream) {
  if (!pool || !tiles || !sink) return pkv::set_error(PKV_ERR_INVALID, "null pointer");
  if (pool_tiles < 1 || num_tiles < 1 || (reinterpret_cast<uintptr_t>(pool) & 15u) != 0)
    return pkv::set_error(PKV_ERR_INVALID, "need tiles in the pool and the list, and a 16-byte aligned pool");
  if (grid < 1 || grid > (1 << 20)) return pkv::set_error(PKV_ERR_INVALID, "grid %d outside [1, 2^20]", grid);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (depth) {
    case 1: e = pkv::launch_gather<1>(pool, pool_tiles, tiles, num_tiles, grid, sink, st); break;
    case 2: e = pkv::launch_gather<2>(pool, pool_tiles, tiles, num_tiles, grid, sink, st); break;
    case 4: e = pkv::launch_gather<4>(pool, pool_tiles, tiles, num_tiles, grid, sink, st); break;
    default: return pkv::set_error(PKV_ERR_UNSUPPORTED, "depth %d: built for 1, 2 and 4", depth);
  }
  if (e != hipSuccess) return pkv::set_error(PKV_ERR_DEVICE, "gather probe: %s", hipGetErrorString(e));
  return pkv::clear_error();
}

}  // extern "C"
