/*
 * pkv_probe.h -- read-bandwidth probes of libpkv.so (C ABI, next to pkv.h).
 *
 * Decode is bound by HBM bandwidth (the course page's key insight: decoding
 * reads the whole KV cache per generated token; vLLM paper page: the KV
 * cache dominates memory traffic), so its roofline is bytes per second. These
 * two kernels measure what the chip delivers to a kernel that only reads, as
 * a ceiling beside the datasheet peak:
 *
 *   pkv_probe_stream_read   reads every 16-byte unit of `buf` once, in
 *                           address order (non-temporal loads, 8 per thread
 *                           in flight, grid-stride over `grid` workgroups of
 *                           256 threads).
 *   pkv_probe_gather_tiles  reads 4096-byte tiles of `pool` in the order of
 *                           `tiles` (int32 tile indices; a shuffled list is
 *                           the paged decode's pattern: one tile = one
 *                           16-token block of one KV head, bf16, head_dim
 *                           128). Each 64-lane wave holds 64 list entries one
 *                           per lane and keeps `depth` tiles (1, 2 or 4) of
 *                           non-temporal loads in flight.
 *
 * Neither writes memory except, in practice never, one word of `sink` per
 * workgroup (sink: device uint32 [grid]). Bytes read per call: `bytes`, or
 * num_tiles * 4096. Tile indices outside [0, pool_tiles) are clamped into
 * the pool. Arguments are device pointers; work goes to `stream`. Invalid
 * sizes return PKV_ERR_INVALID, an unbuilt depth PKV_ERR_UNSUPPORTED.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

PKV_API int pkv_probe_stream_read(const void *buf, int64_t bytes, int32_t grid, uint32_t *sink, void *stream);

PKV_API int pkv_probe_gather_tiles(const void *pool, int64_t pool_tiles, const int32_t *tiles, int64_t num_tiles,
                                   int32_t depth, int32_t grid, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
