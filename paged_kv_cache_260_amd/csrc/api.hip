// C-ABI layer: argument validation, planning, workspace, kernel dispatch.
//
// Every check that can be made from host-side sizes and pointers happens
// before the first HIP call, so a bad call returns a status without touching
// the device (and can be exercised on a machine with no GPU).
#include "pkv.h"
#include "pkv_blocks.h"
#include "pkv_fp8.h"
#include "pkv_chunk.h"
#include "pkv_shared_prefix.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "kernels.h"
#include "status.h"

namespace pkv {

thread_local std::string g_error;

int set_error(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return status;
}

int clear_error() {
  g_error.clear();
  return PKV_OK;
}

}  // namespace pkv

namespace {

template <typename... Args> int fail(int status, const char *fmt, Args... args) {
  return pkv::set_error(status, fmt, args...);
}

int ok() { return pkv::clear_error(); }

int hip_fail(hipError_t e, const char *what) {
  return fail(PKV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return (1 << s) == v ? s : -1;
}

std::atomic<int32_t> g_partition_override{0};

// Automatic partition length: sequences up to 1024 tokens stay whole; longer
// ones are cut into 1024-token partitions, so one long sequence spreads over
// many CUs while merge traffic stays under 1% of the KV bytes. (Measured on
// MI355X: 1024 is as fast as or faster than 512 on every batch shape tried;
// shorter partitions lose to per-workgroup startup cost.)
constexpr int64_t kAutoPartition = 1024;

// Chunk attention takes the decode kernel's work items while a chunk fills at
// most this many 16-row blocks per KV head (chunk length x query heads per KV
// head <= 64 rows); longer chunks go to the chunk kernel.
#ifndef PKV_CHUNK_ROWS_MAX_BLOCKS
#define PKV_CHUNK_ROWS_MAX_BLOCKS 4
#endif
constexpr int64_t kChunkRowsMaxBlocks = PKV_CHUNK_ROWS_MAX_BLOCKS;

void plan(int32_t block_size, int32_t max_blocks, int32_t *ptok, int32_t *nparts) {
  const int64_t max_tokens = (int64_t)max_blocks * block_size;
  int64_t p = g_partition_override.load();
  if (p <= 0) p = max_tokens <= kAutoPartition ? ((max_tokens + 15) / 16) * 16 : kAutoPartition;
  // Longer than a block: whole blocks, so every partition starts on a block
  // boundary. At most 64 blocks (the kernel keeps their ids in one VGPR).
  if (p > block_size) p = (p / block_size) * block_size;
  const int64_t cap = (int64_t)pkv::kMaxPartitionBlocks * block_size;
  if (p > cap) p = cap;
  *ptok = (int32_t)p;
  *nparts = (int32_t)((max_tokens + p - 1) / p);
}

// Split-partial workspace, one per (device, stream), grown on demand:
//   [part_acc: rows x D floats][part_ml: rows x float2], rows = num_seqs * n_heads * max_parts.
struct Workspace {
  void *ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int get_workspace(hipStream_t stream, size_t bytes, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace &ws = g_ws[{dev, stream}];
  if (ws.bytes < bytes) {
    if (ws.ptr) {
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      hipFree(ws.ptr);
      ws.ptr = nullptr;
      ws.bytes = 0;
    }
    const size_t grow = bytes + bytes / 2;
    e = hipMalloc(&ws.ptr, grow);
    if (e != hipSuccess) {
      ws.ptr = nullptr;
      return hip_fail(e, "hipMalloc (decode workspace)");
    }
    ws.bytes = grow;
  }
  *out = ws.ptr;
  return PKV_OK;
}

// Counters of the decode-kernel family, one buffer per (device, stream),
// zeroed when allocated: the late workgroups' ticket counter in the first
// kTicketInts ints (any value works, tickets.h), then the arrival counters of
// the in-kernel partition merge, which every call leaves at zero again (the
// partitions of a row set agree on their count; shared-prefix calls whose
// description is broken count nothing).
std::map<std::pair<int, hipStream_t>, Workspace> g_arrivals;
constexpr int64_t kTicketInts = 64;

int get_arrivals(hipStream_t stream, int64_t count, int32_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace &ws = g_arrivals[{dev, stream}];
  const size_t bytes = (size_t)count * sizeof(int32_t);
  if (ws.bytes < bytes) {
    if (ws.ptr) {
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      hipFree(ws.ptr);
      ws.ptr = nullptr;
      ws.bytes = 0;
    }
    const size_t grow = (bytes + bytes / 2 + 255) & ~(size_t)255;
    e = hipMalloc(&ws.ptr, grow);
    if (e != hipSuccess) {
      ws.ptr = nullptr;
      return hip_fail(e, "hipMalloc (decode arrival counters)");
    }
    e = pkv::launch_zero_i32(static_cast<int32_t *>(ws.ptr), (int64_t)(grow / sizeof(int32_t)), stream);
    if (e != hipSuccess) return hip_fail(e, "clearing decode arrival counters");
    ws.bytes = grow;
  }
  *out = static_cast<int32_t *>(ws.ptr);
  return PKV_OK;
}

// Scratch of pkv_paged_attn_decode_noalloc: a fixed device array in this
// library's code object, one copy per GPU that loads it, held until the
// process ends. Its first PKV_NOALLOC_COUNTERS int32 are the ticket and
// arrival counters (zero before a call, and every call leaves the arrival
// counters at zero again); the PKV_NOALLOC_WORKSPACE_BYTES after them take
// the split partials. In host code `scratch` names a host-side stand-in, never
// the device memory: kernels and copies get the address hipGetSymbolAddress
// returns for the current device (scratch_base).
constexpr size_t kScratchCounterBytes = (size_t)PKV_NOALLOC_COUNTERS * sizeof(int32_t);
constexpr size_t kScratchBytes = kScratchCounterBytes + (size_t)PKV_NOALLOC_WORKSPACE_BYTES;
static_assert(kScratchCounterBytes % 256 == 0, "workspace part stays 256-byte aligned");
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch. The first call on a device
// looks it up and clears the counters with a fill kernel on `stream`, ahead
// of that call's own kernels (no allocation, no memset node).
int scratch_base(hipStream_t stream, char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(PKV_ERR_DEVICE, "device %d: no scratch slot", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress (decode scratch)");
    e = pkv::launch_zero_i32(static_cast<int32_t *>(p), PKV_NOALLOC_COUNTERS, stream);
    if (e != hipSuccess) return hip_fail(e, "clearing the decode scratch counters");
    g_scratch_ptr[dev] = static_cast<char *>(p);
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

const char *pkv_last_error(void) { return pkv::g_error.c_str(); }

int32_t pkv_version(void) { return (1 << 16) | 0; }

int pkv_set_partition_tokens(int32_t tokens) {
  if (tokens != 0 && (tokens < 16 || tokens > (1 << 20) || tokens % 16 != 0))
    return fail(PKV_ERR_INVALID, "partition length %d: want 0 or a multiple of 16 in [16, 2^20]",
                tokens);
  g_partition_override.store(tokens);
  return ok();
}

int pkv_decode_plan(int32_t n_heads, int32_t n_kv_heads, int32_t block_size, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t *partition_tokens,
                    int32_t *max_partitions) {
  (void)n_heads;
  (void)n_kv_heads;
  (void)num_seqs;
  if (block_size < 1 || max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID, "block_size and max_blocks_per_seq must be >= 1");
  int32_t p, np;
  plan(block_size, max_blocks_per_seq, &p, &np);
  if (partition_tokens) *partition_tokens = p;
  if (max_partitions) *max_partitions = np;
  return ok();
}

}  // extern "C"

namespace {

// Shared by the 16/32-bit and the FP8 decode entry points (fp8: pools hold
// e4m3 codes, k_scale / v_scale are device float32 [n_kv_heads]).
int decode_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                const int32_t *block_tables, const int32_t *seq_lens, float scale, int32_t n_heads,
                int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_seqs,
                int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype, void *stream, bool fp8,
                const float *k_scale, const float *v_scale, const void *k_new = nullptr,
                const void *v_new = nullptr, bool no_alloc = false, const int32_t *host_seq_lens = nullptr) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (fp8 && dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "FP8 pools need a float16 or bfloat16 query and output");
  const bool append = k_new != nullptr || v_new != nullptr;
  if (append && dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "decode with append is built for float16 and bfloat16");
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PKV_ERR_INVALID, "num_seqs %d outside [0, 65535]", num_seqs);
  if (n_heads < 1 || n_kv_heads < 1)
    return fail(PKV_ERR_INVALID, "n_heads %d and n_kv_heads %d must be >= 1", n_heads, n_kv_heads);
  if (n_heads % n_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "n_heads %d is not a multiple of n_kv_heads %d", n_heads,
                n_kv_heads);
  const int group = n_heads / n_kv_heads;
  if (group > 256) return fail(PKV_ERR_UNSUPPORTED, "n_heads / n_kv_heads = %d > 256", group);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: built for 64 and 128", head_dim);
  const int bshift = log2_exact(block_size);
  if (block_size < 16 || block_size > 128 || bshift < 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d: built for 16, 32, 64, 128", block_size);
  if (max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq %d must be >= 1", max_blocks_per_seq);
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "num_blocks %lld must be >= 1", (long long)num_blocks);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale is not finite");
  if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq * block_size exceeds int32");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens)
    return fail(PKV_ERR_INVALID, "null array pointer");
  if (fp8 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVALID, "null scale pointer");
  if (append && (!k_new || !v_new)) return fail(PKV_ERR_INVALID, "null k_new or v_new");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_ERR_INVALID, "q, out, k_pool and v_pool must be 16-byte aligned");
  if (append && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(PKV_ERR_INVALID, "k_new and v_new must be 16-byte aligned");

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.num_seqs = num_seqs;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.group = group;
  const int gt = pkv::decode_head_tile(group);
  a.head_chunks = (group + gt - 1) / gt;
  a.block_size = block_size;
  a.block_shift = bshift;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  plan(block_size, max_blocks_per_seq, &a.partition_tokens, &a.max_parts);
  if ((int64_t)num_seqs * a.max_parts * n_kv_heads * a.head_chunks > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "%d sequences x %d partitions x %d heads: too many workgroups",
                num_seqs, a.max_parts, n_kv_heads);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // counters: the ticket counter of the late workgroups first, then (in-kernel
  // merge) the arrival counters; split partials: [acc rows x D | (m, l) rows]
  const bool fused_merge = a.max_parts > 1 && a.max_parts <= pkv::kFusedMergeParts;
  // A host-built order only where partitions are merged inside the kernel (or
  // there is one per sequence): a sequence whose host and device lengths
  // disagree then writes its NaN rows and no partials, and no merge kernel can
  // later combine stale partials of it into those rows.
  a.host_seq_lens = a.max_parts == 1 || fused_merge ? host_seq_lens : nullptr;
  const int64_t counter_ints = kTicketInts + (fused_merge ? (int64_t)num_seqs * n_kv_heads * a.head_chunks : 0);
  const size_t rows = a.max_parts > 1 ? (size_t)num_seqs * n_heads * a.max_parts : 0;
  const size_t acc_bytes = rows * head_dim * sizeof(float);
  const size_t ws_bytes = acc_bytes + rows * sizeof(float2);
  int32_t *counters = nullptr;
  void *ws = nullptr;
  if (no_alloc) {
    if (counter_ints > PKV_NOALLOC_COUNTERS)
      return fail(PKV_ERR_INVALID,
                  "no-allocation decode: %lld merge counters needed (sequences x KV heads x head chunks + %lld), "
                  "the scratch holds %d",
                  (long long)counter_ints, (long long)kTicketInts, PKV_NOALLOC_COUNTERS);
    if (ws_bytes > (size_t)PKV_NOALLOC_WORKSPACE_BYTES)
      return fail(PKV_ERR_INVALID,
                  "no-allocation decode: %zu bytes of split partials needed (%zu rows x (head_dim + 2) x 4), "
                  "the scratch holds %zu",
                  ws_bytes, rows, (size_t)PKV_NOALLOC_WORKSPACE_BYTES);
    char *base = nullptr;
    int rc = scratch_base(st, &base);
    if (rc != PKV_OK) return rc;
    counters = reinterpret_cast<int32_t *>(base);
    ws = base + kScratchCounterBytes;
  } else {
    int rc = get_arrivals(st, counter_ints, &counters);
    if (rc != PKV_OK) return rc;
    if (rows) {
      rc = get_workspace(st, ws_bytes, &ws);
      if (rc != PKV_OK) return rc;
    }
  }
  a.tickets = reinterpret_cast<uint32_t *>(counters);
  if (rows) {
    a.part_acc = static_cast<float *>(ws);
    a.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(ws) + acc_bytes);
    if (fused_merge) a.arrivals = counters + kTicketInts;
  }
  hipError_t e = append ? pkv::launch_decode_append(static_cast<pkv::DType>(dtype), head_dim, fp8, a, st)
                 : fp8  ? pkv::launch_decode_fp8(static_cast<pkv::DType>(dtype), head_dim, a, st)
                        : pkv::launch_decode(static_cast<pkv::DType>(dtype), head_dim, a, st);
  if (e != hipSuccess) return hip_fail(e, "paged decode launch");
  return ok();
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *block_tables, const int32_t *seq_lens, float scale,
                          int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                          int64_t num_blocks, int32_t dtype, void *stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, false, nullptr,
                     nullptr);
}

int pkv_paged_attn_decode_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                                  const int32_t *block_tables, const int32_t *seq_lens, float scale,
                                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                  void *stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, false, nullptr,
                     nullptr, nullptr, nullptr, true);
}

int pkv_paged_attn_decode_append(void *out, const void *q, void *k_pool, void *v_pool, const void *k_new,
                                 const void *v_new, const int32_t *block_tables, const int32_t *seq_lens,
                                 float scale, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int32_t dtype, void *stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, false, nullptr, nullptr,
                     k_new, v_new);
}

int pkv_paged_attn_decode_append_planned(void *out, const void *q, void *k_pool, void *v_pool, const void *k_new,
                                         const void *v_new, const int32_t *block_tables, const int32_t *seq_lens,
                                         const int32_t *seq_lens_host, float scale, int32_t n_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_seqs,
                                         int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                         void *stream) {
  if (num_seqs > 0 && !seq_lens_host) return fail(PKV_ERR_INVALID, "null seq_lens_host");
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, false, nullptr, nullptr,
                     k_new, v_new, false, seq_lens_host);
}

int pkv_paged_attn_decode_append_fp8(void *out, const void *q, void *k_pool, void *v_pool, const void *k_new,
                                     const void *v_new, const float *k_scale, const float *v_scale,
                                     const int32_t *block_tables, const int32_t *seq_lens, float scale,
                                     int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t dtype, void *stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, true, k_scale, v_scale,
                     k_new, v_new);
}

int pkv_paged_attn_decode_append_fp8_planned(void *out, const void *q, void *k_pool, void *v_pool,
                                             const void *k_new, const void *v_new, const float *k_scale,
                                             const float *v_scale, const int32_t *block_tables,
                                             const int32_t *seq_lens, const int32_t *seq_lens_host, float scale,
                                             int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                                             int64_t num_blocks, int32_t dtype, void *stream) {
  if (num_seqs > 0 && !seq_lens_host) return fail(PKV_ERR_INVALID, "null seq_lens_host");
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, true, k_scale, v_scale,
                     k_new, v_new, false, seq_lens_host);
}

int pkv_paged_attn_decode_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                              const float *k_scale, const float *v_scale, const int32_t *block_tables,
                              const int32_t *seq_lens, float scale, int32_t n_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype, void *stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads, head_dim,
                     block_size, num_seqs, max_blocks_per_seq, num_blocks, dtype, stream, true, k_scale,
                     v_scale);
}

}  // extern "C"

namespace {

// Shared by the 16-bit and the FP8 chunk entry points.
int chunk_impl(void *out, const void *q, const void *k_pool, const void *v_pool, const int32_t *block_tables,
               const int32_t *seq_lens, const int32_t *query_start_loc, float scale, int32_t n_heads,
               int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_seqs,
               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_query_len, int32_t dtype, void *stream,
               bool fp8, const float *k_scale, const float *v_scale) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (dtype == PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "chunk attention is built for float16 and bfloat16");
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs %d < 0", num_seqs);
  if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "n_heads %d must be a positive multiple of n_kv_heads %d", n_heads, n_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: built for 64 and 128", head_dim);
  const int bshift = log2_exact(block_size);
  if (block_size < 16 || block_size > 128 || bshift < 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d: built for 16, 32, 64, 128", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq and num_blocks must be >= 1");
  if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq * block_size exceeds int32");
  if (max_query_len < 0) return fail(PKV_ERR_INVALID, "max_query_len %d < 0", max_query_len);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale is not finite");
  const int group = n_heads / n_kv_heads;
  const int64_t row_blocks = ((int64_t)max_query_len * group + 15) / 16;
  if (num_seqs == 0 || row_blocks == 0) return ok();
  if ((int64_t)n_kv_heads * num_seqs * row_blocks > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "too many work items");
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens || !query_start_loc)
    return fail(PKV_ERR_INVALID, "null array pointer");
  if (fp8 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVALID, "null scale pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_ERR_INVALID, "q, out, k_pool and v_pool must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (row_blocks <= kChunkRowsMaxBlocks) {
    // short chunks (speculative verification, small chunked-prefill pieces):
    // the decode kernel's split, longest-first work items with 16 chunk rows each
    pkv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.query_start_loc = query_start_loc;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.num_seqs = num_seqs;
    a.n_heads = n_heads;
    a.n_kv_heads = n_kv_heads;
    a.group = group;
    a.head_chunks = (int32_t)row_blocks;
    a.block_size = block_size;
    a.block_shift = bshift;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    plan(block_size, max_blocks_per_seq, &a.partition_tokens, &a.max_parts);
    const int64_t items = (int64_t)num_seqs * n_kv_heads * row_blocks;
    if (items * a.max_parts > (int64_t)INT32_MAX) return fail(PKV_ERR_INVALID, "too many work items");
    // the late workgroups' ticket counter first, then the arrival counters
    // (as in decode)
    const bool fused_merge = a.max_parts > 1 && a.max_parts <= pkv::kFusedMergeParts;
    int32_t *counters = nullptr;
    int rc = get_arrivals(st, kTicketInts + (fused_merge ? items : 0), &counters);
    if (rc != PKV_OK) return rc;
    a.tickets = reinterpret_cast<uint32_t *>(counters);
    if (a.max_parts > 1) {
      const size_t rows = (size_t)items * 16 * a.max_parts;
      const size_t acc_bytes = rows * head_dim * sizeof(float);
      void *ws = nullptr;
      rc = get_workspace(st, acc_bytes + rows * sizeof(float2), &ws);
      if (rc != PKV_OK) return rc;
      a.part_acc = static_cast<float *>(ws);
      a.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(ws) + acc_bytes);
      if (fused_merge) a.arrivals = counters + kTicketInts;
    }
    hipError_t e = pkv::launch_chunk_rows(static_cast<pkv::DType>(dtype), head_dim, fp8, a, st);
    if (e != hipSuccess) return hip_fail(e, "chunk attention launch");
    return ok();
  }
  pkv::ChunkArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.num_seqs = num_seqs;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.group = group;
  a.block_size = block_size;
  a.block_shift = bshift;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.row_blocks = (int32_t)(((int64_t)max_query_len * group + pkv::chunk_rows_per_block() - 1) /
                           pkv::chunk_rows_per_block());
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  hipError_t e = pkv::launch_chunk(static_cast<pkv::DType>(dtype), head_dim, fp8, a, st);
  if (e != hipSuccess) return hip_fail(e, "chunk attention launch");
  return ok();
}

}  // namespace

extern "C" {

int pkv_paged_attn_chunk(void *out, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *block_tables, const int32_t *seq_lens, const int32_t *query_start_loc,
                         float scale, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_query_len,
                         int32_t dtype, void *stream) {
  return chunk_impl(out, q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, scale, n_heads, n_kv_heads,
                    head_dim, block_size, num_seqs, max_blocks_per_seq, num_blocks, max_query_len, dtype, stream,
                    false, nullptr, nullptr);
}

int pkv_paged_attn_chunk_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                             const float *k_scale, const float *v_scale, const int32_t *block_tables,
                             const int32_t *seq_lens, const int32_t *query_start_loc, float scale, int32_t n_heads,
                             int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_seqs,
                             int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_query_len, int32_t dtype,
                             void *stream) {
  return chunk_impl(out, q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, scale, n_heads, n_kv_heads,
                    head_dim, block_size, num_seqs, max_blocks_per_seq, num_blocks, max_query_len, dtype, stream,
                    true, k_scale, v_scale);
}

}  // extern "C"

namespace {

// Shared by the 16-bit and the FP8 shared-prefix entry points.
int shared_prefix_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *seq_lens, const int32_t *prefix_lens,
                       const int32_t *group_start, float scale, int32_t n_heads, int32_t n_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_seqs, int32_t num_groups,
                       int32_t max_group_size, int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                       void *stream, bool fp8, const float *k_scale, const float *v_scale) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode is built for float16 and bfloat16");
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PKV_ERR_INVALID, "num_seqs %d outside [0, 65535]", num_seqs);
  if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "n_heads %d must be a positive multiple of n_kv_heads %d", n_heads, n_kv_heads);
  const int group = n_heads / n_kv_heads;
  if (group > 256) return fail(PKV_ERR_UNSUPPORTED, "n_heads / n_kv_heads = %d > 256", group);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: built for 64 and 128", head_dim);
  const int bshift = log2_exact(block_size);
  if (block_size < 16 || block_size > 128 || bshift < 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d: built for 16, 32, 64, 128", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq and num_blocks must be >= 1");
  if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq * block_size exceeds int32");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale is not finite");
  if (num_seqs == 0) return ok();
  if (num_groups < 1 || num_groups > num_seqs)
    return fail(PKV_ERR_INVALID, "num_groups %d outside [1, num_seqs = %d]", num_groups, num_seqs);
  if (max_group_size < 1 || max_group_size > num_seqs)
    return fail(PKV_ERR_INVALID, "max_group_size %d outside [1, num_seqs = %d]", max_group_size, num_seqs);
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens || !prefix_lens || !group_start)
    return fail(PKV_ERR_INVALID, "null array pointer");
  if (fp8 && (!k_scale || !v_scale)) return fail(PKV_ERR_INVALID, "null scale pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_ERR_INVALID, "q, out, k_pool and v_pool must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);

  // suffix launch: plain decode items over each sequence's private tokens
  pkv::DecodeArgs suf{};
  suf.out = out;
  suf.q = q;
  suf.k_pool = k_pool;
  suf.v_pool = v_pool;
  suf.block_tables = block_tables;
  suf.seq_lens = seq_lens;
  suf.scale_log2 = (float)((double)scale * 1.4426950408889634);
  suf.num_seqs = num_seqs;
  suf.n_heads = n_heads;
  suf.n_kv_heads = n_kv_heads;
  suf.group = group;
  const int gt = pkv::decode_head_tile(group);
  suf.head_chunks = (group + gt - 1) / gt;
  suf.block_size = block_size;
  suf.block_shift = bshift;
  suf.max_blocks = max_blocks_per_seq;
  suf.num_blocks = num_blocks;
  suf.prefix_lens = prefix_lens;
  suf.member_seqs = num_seqs;
  suf.k_scale = k_scale;
  suf.v_scale = v_scale;
  plan(block_size, max_blocks_per_seq, &suf.partition_tokens, &suf.max_parts);

  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  const int64_t slots = 2 * (int64_t)pkv::kDecodeWgsPerCu * pkv::device_cus();

  // One launch for both kinds of work item when every group's rows fit one
  // 16-row block per KV head and the partial slots per (sequence, head) fit
  // the in-kernel merge.
  // The kernel's longest-first plan checks the sharing description (a broken
  // one must not unbalance the arrival counts), so the one-launch path is
  // taken only for batches that plan covers.
  pkv::DecodeArgs ent = suf;
  ent.num_seqs = num_groups + num_seqs;
  if (group <= 16 && (group & (group - 1)) == 0 && (int64_t)max_group_size * group <= 16 &&
      num_groups + num_seqs <= 65535 && pkv::decode_compact_plan(ent)) {
    int64_t p_pre = suf.partition_tokens, n_pre = suf.max_parts;
    if (g_partition_override.load() <= 0) {
      // shortest prefix partition whose count fits the slots the private
      // parts leave; the kernel lengthens it to the longest private part
      const int64_t want = pkv::kFusedMergeParts - suf.max_parts;
      if (want >= 1) {
        p_pre = (max_tokens + want - 1) / want;
        p_pre = p_pre > block_size ? (p_pre + block_size - 1) / block_size * block_size : (p_pre + 15) / 16 * 16;
        p_pre = std::min<int64_t>(p_pre, (int64_t)pkv::kMaxPartitionBlocks * block_size);
        n_pre = (max_tokens + p_pre - 1) / p_pre;
      } else {
        n_pre = pkv::kFusedMergeParts;  // no room: two launches
      }
    }
    if (n_pre + suf.max_parts <= pkv::kFusedMergeParts) {
      pkv::DecodeArgs a = suf;
      a.num_seqs = num_groups + num_seqs;  // entities
      a.num_groups = num_groups;
      a.query_start_loc = group_start;
      a.head_chunks = 1;
      a.prefix_partition_tokens = (int32_t)p_pre;
      a.prefix_partition_fixed = g_partition_override.load() > 0;
      a.max_parts = (int32_t)(n_pre + suf.max_parts);  // slot stride
      const size_t rows = (size_t)num_seqs * n_heads * a.max_parts;
      const size_t acc_bytes = rows * head_dim * sizeof(float);
      void *ws = nullptr;
      int rc = get_workspace(st, acc_bytes + rows * sizeof(float2), &ws);
      if (rc != PKV_OK) return rc;
      a.part_acc = static_cast<float *>(ws);
      a.part_ml = reinterpret_cast<float2 *>(static_cast<char *>(ws) + acc_bytes);
      int32_t *counters = nullptr;
      rc = get_arrivals(st, kTicketInts + (int64_t)num_seqs * n_kv_heads, &counters);
      if (rc != PKV_OK) return rc;
      a.arrivals = counters + kTicketInts;
      hipError_t e = pkv::launch_shared_fused(static_cast<pkv::DType>(dtype), head_dim, fp8, a, st);
      if (e != hipSuccess) return hip_fail(e, "shared-prefix decode launch");
      return ok();
    }
  }

  // prefix launch: rows of (member, head) over each group's shared prefix
  pkv::DecodeArgs pre = suf;
  pre.query_start_loc = group_start;
  pre.num_seqs = num_groups;
  const int64_t row_blocks = ((int64_t)max_group_size * group + 15) / 16;
  pre.head_chunks = (int32_t)row_blocks;
  const int64_t pre_items = (int64_t)num_groups * n_kv_heads * row_blocks;
  // Few groups give few prefix items, each walking a long prefix: split the
  // prefix so that the items fill about two rounds of the chip's resident
  // workgroups (at most kFusedMergeParts partitions, whole blocks, at most
  // kMaxPartitionBlocks blocks each, at least one 16-token tile).
  if (g_partition_override.load() <= 0) {
    const int64_t want = std::min<int64_t>(pkv::kFusedMergeParts, std::max<int64_t>(1, (slots + pre_items - 1) / pre_items));
    int64_t p = (max_tokens + want - 1) / want;
    p = p > block_size ? (p + block_size - 1) / block_size * block_size : (p + 15) / 16 * 16;
    p = std::min<int64_t>(p, (int64_t)pkv::kMaxPartitionBlocks * block_size);
    pre.partition_tokens = (int32_t)p;
    pre.max_parts = (int32_t)((max_tokens + p - 1) / p);
  }
  const int64_t suf_units = (int64_t)n_kv_heads * suf.head_chunks;
  if (pre_items * pre.max_parts > (int64_t)INT32_MAX ||
      (int64_t)num_seqs * suf.max_parts * suf_units > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "too many work items");

  // workspace: [split acc | split ml] (shared by the two launches, which run
  // one after the other) then [prefix acc | prefix ml] per (sequence, head)
  const size_t split_rows = std::max(pre.max_parts > 1 ? (size_t)pre_items * 16 * pre.max_parts : 0,
                                     suf.max_parts > 1 ? (size_t)num_seqs * n_heads * suf.max_parts : 0);
  const size_t pre_rows = (size_t)num_seqs * n_heads;
  const size_t split_acc = split_rows * head_dim * sizeof(float);
  const size_t split_ml = split_rows * sizeof(float2);
  const size_t pre_acc = pre_rows * head_dim * sizeof(float);
  void *ws = nullptr;
  int rc = get_workspace(st, split_acc + split_ml + pre_acc + pre_rows * sizeof(float2), &ws);
  if (rc != PKV_OK) return rc;
  char *w = static_cast<char *>(ws);
  if (split_rows) {
    suf.part_acc = pre.part_acc = reinterpret_cast<float *>(w);
    suf.part_ml = pre.part_ml = reinterpret_cast<float2 *>(w + split_acc);
  }
  suf.pre_acc = pre.pre_acc = reinterpret_cast<float *>(w + split_acc + split_ml);
  suf.pre_ml = pre.pre_ml = reinterpret_cast<float2 *>(w + split_acc + split_ml + pre_acc);
  const bool pre_fused = pre.max_parts > 1 && pre.max_parts <= pkv::kFusedMergeParts;
  const bool suf_fused = suf.max_parts > 1 && suf.max_parts <= pkv::kFusedMergeParts;
  if (pre_fused || suf_fused) {
    // one counter set serves both launches: each leaves its counters at zero
    int32_t *arr = nullptr;
    rc = get_arrivals(st, kTicketInts + std::max(pre_fused ? pre_items : 0, suf_fused ? (int64_t)num_seqs * suf_units : 0),
                      &arr);
    if (rc != PKV_OK) return rc;
    if (pre_fused) pre.arrivals = arr + kTicketInts;
    if (suf_fused) suf.arrivals = arr + kTicketInts;
  }
  hipError_t e = pkv::launch_shared_prefix(static_cast<pkv::DType>(dtype), head_dim, fp8, pre, suf, st);
  if (e != hipSuccess) return hip_fail(e, "shared-prefix decode launch");
  return ok();
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode_shared_prefix(void *out, const void *q, const void *k_pool, const void *v_pool,
                                        const int32_t *block_tables, const int32_t *seq_lens,
                                        const int32_t *prefix_lens, const int32_t *group_start, float scale,
                                        int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                        void *stream) {
  return shared_prefix_impl(out, q, k_pool, v_pool, block_tables, seq_lens, prefix_lens, group_start, scale,
                            n_heads, n_kv_heads, head_dim, block_size, num_seqs, num_groups, max_group_size,
                            max_blocks_per_seq, num_blocks, dtype, stream, false, nullptr, nullptr);
}

int pkv_paged_attn_decode_shared_prefix_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                            const float *k_scale, const float *v_scale,
                                            const int32_t *block_tables, const int32_t *seq_lens,
                                            const int32_t *prefix_lens, const int32_t *group_start, float scale,
                                            int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t num_seqs, int32_t num_groups,
                                            int32_t max_group_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                                            int32_t dtype, void *stream) {
  return shared_prefix_impl(out, q, k_pool, v_pool, block_tables, seq_lens, prefix_lens, group_start, scale,
                            n_heads, n_kv_heads, head_dim, block_size, num_seqs, num_groups, max_group_size,
                            max_blocks_per_seq, num_blocks, dtype, stream, true, k_scale, v_scale);
}

int pkv_kv_cache_write_fp8(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                           const float *k_scale, const float *v_scale, const int32_t *slot_mapping,
                           int32_t num_tokens, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, int32_t dtype, void *stream) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  if (n_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "n_kv_heads, head_dim, block_size, num_blocks must be >= 1");
  if (head_dim % 16 != 0) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 16", head_dim);
  if ((int64_t)n_kv_heads * (head_dim / 16) * 2 > (int64_t)INT32_MAX) return fail(PKV_ERR_INVALID, "row too large");
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping || !k_scale || !v_scale)
    return fail(PKV_ERR_INVALID, "null pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID, "pools and new rows must be 16-byte aligned");
  pkv::CacheWriteFp8Args a{};
  a.k_pool = static_cast<uint8_t *>(k_pool);
  a.v_pool = static_cast<uint8_t *>(v_pool);
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_slots = num_blocks * block_size;
  hipError_t e = pkv::launch_cache_write_fp8(static_cast<pkv::DType>(dtype), a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 cache write launch");
  return ok();
}

int pkv_kv_cache_write(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                       const int32_t *slot_mapping, int32_t num_tokens, int32_t n_kv_heads,
                       int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                       void *stream) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  if (n_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "n_kv_heads, head_dim, block_size, num_blocks must be >= 1");
  const int64_t row_bytes = (int64_t)head_dim * pkv::dtype_bytes(static_cast<pkv::DType>(dtype));
  if (row_bytes % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim * element size = %lld bytes, not a multiple of 16",
                (long long)row_bytes);
  if ((int64_t)n_kv_heads * (row_bytes / 16) * 2 > (int64_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "row too large");
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID, "null array pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID, "pools and new rows must be 16-byte aligned");
  pkv::CacheWriteArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.n_kv_heads = n_kv_heads;
  a.row_chunks = (int32_t)(row_bytes / 16);
  a.block_size = block_size;
  a.num_slots = num_blocks * block_size;
  hipError_t e = pkv::launch_cache_write(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache write launch");
  return ok();
}

int pkv_copy_blocks(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                    int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                    int32_t dtype, void *stream) {
  if (!valid_dtype(dtype) && dtype != PKV_FP8_E4M3) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (num_pairs < 0) return fail(PKV_ERR_INVALID, "num_pairs %d < 0", num_pairs);
  if (n_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "n_kv_heads, head_dim, block_size and num_blocks must be >= 1");
  const int64_t block_bytes = (int64_t)n_kv_heads * block_size * head_dim *
                              (dtype == PKV_FP8_E4M3 ? 1 : pkv::dtype_bytes(static_cast<pkv::DType>(dtype)));
  if (block_bytes % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "block of %lld bytes is not a multiple of 16", (long long)block_bytes);
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !pairs) return fail(PKV_ERR_INVALID, "null pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool)) return fail(PKV_ERR_INVALID, "pools must be 16-byte aligned");
  if (block_bytes / 16 > (int64_t)65535 * 2048)
    return fail(PKV_ERR_UNSUPPORTED, "block of %lld bytes is too large", (long long)block_bytes);
  pkv::CopyBlocksArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.block_units = block_bytes / 16;
  a.num_blocks = num_blocks;
  hipError_t e = pkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return ok();
}

int pkv_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int rc = PKV_OK;
  for (auto *m : {&g_ws, &g_arrivals}) {
    for (auto &kv : *m) {
      if (!kv.second.ptr) continue;
      int prev = 0;
      hipGetDevice(&prev);
      hipSetDevice(kv.first.first);
      hipError_t e = hipStreamSynchronize(kv.first.second);
      if (e == hipSuccess) e = hipFree(kv.second.ptr);
      hipSetDevice(prev);
      if (e != hipSuccess) rc = hip_fail(e, "releasing workspace");
      kv.second = Workspace{};
    }
    m->clear();
  }
  return rc == PKV_OK ? ok() : rc;
}

}  // extern "C"
