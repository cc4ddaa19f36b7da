// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

inline int dtype_bytes(DType t) { return t == DType::F32 ? 4 : 2; }

// Tokens per decode tile: one MFMA column block (16 tokens of one KV head).
constexpr int kTileTokens = 16;
// Waves per decode workgroup.
constexpr int kDecodeWaves = 4;
// A decode partition spans at most this many blocks: their ids sit one per
// lane in a single VGPR.
constexpr int kMaxPartitionBlocks = 64;

// Host-built work order (pkv_paged_attn_decode_append_planned): at most this
// many items per unit, for batches of at most kHostPlanSeqs sequences.
constexpr int kHostPlanItems = 1024;
constexpr int kHostPlanSeqs = 256;

struct DecodeArgs {
  void *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *seq_lens;
  float scale_log2;        // softmax scale * log2(e): scores live in base-2 units
  int32_t num_seqs;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t group;           // n_heads / n_kv_heads
  int32_t head_chunks;     // ceil(group / head tile)
  int32_t block_size;
  int32_t block_shift;     // log2(block_size)
  int32_t max_blocks;      // block_tables row width
  int64_t num_blocks;
  int32_t partition_tokens;
  int32_t max_parts;
  int32_t wgs_per_unit;    // decode workgroups per unit (set by launch_decode)
  float *part_acc;         // [num_seqs * n_heads * max_parts, head_dim] (only when max_parts > 1)
  float2 *part_ml;         // [num_seqs * n_heads * max_parts] (max in base-2 units, sum)
  // Arrival counters [num_seqs * n_kv_heads * head_chunks], zero between calls;
  // set when the partitions of a sequence are merged by the last of them to
  // finish (max_parts <= kFusedMergeParts), null when a merge kernel runs.
  int32_t *arrivals;
  // Longest-first plans: workgroups past the first static_wgs (those the chip
  // starts at once) take their place in the order from a ticket counter, so
  // the later items go to whichever XCD frees a slot first. The counter wraps
  // to zero after the call's last ticket (null: fixed places).
  uint32_t *tickets;
  int32_t static_wgs;      // set by the launch
  // FP8 pools only: per-KV-head scales of the stored codes (null otherwise)
  const float *k_scale;
  const float *v_scale;
  // Chunk rows only (launch_chunk_rows): [num_seqs + 1] offsets of each
  // sequence's query tokens; head_chunks then counts 16-row blocks per KV head
  // and partial rows are indexed per item: ((s * units + unit) * 16 + row).
  // Prefix launch of the shared-prefix decode: the groups' sequence ranges.
  const int32_t *query_start_loc;
  // Shared-prefix decode (launch_shared_prefix). prefix_lens [member_seqs]:
  // shared prefix tokens of each sequence. The prefix launch (num_seqs =
  // groups) writes un-normalised partials per (sequence, head) row into
  // pre_acc [member_seqs * n_heads, head_dim] and pre_ml; the suffix launch
  // (num_seqs = sequences) walks tokens [prefix_lens[s], seq_lens[s]) and folds
  // them in.
  const int32_t *prefix_lens;
  int32_t member_seqs;
  float *pre_acc;
  float2 *pre_ml;
  // Shared-prefix decode in one launch (launch_shared_fused): num_seqs counts
  // entities (num_groups prefixes, then member_seqs private parts); prefix
  // entities are split into partitions of prefix_partition_tokens, private
  // ones of partition_tokens; max_parts is the slot stride per (sequence,
  // head) row (prefix slots first), at most kFusedMergeParts.
  int32_t num_groups;
  int32_t prefix_partition_tokens;  // the shortest allowed (the kernel may lengthen it)
  int32_t prefix_partition_fixed;   // nonzero: use prefix_partition_tokens as given
  // Decode with append (launch_decode_append): the newest token's K and V
  // rows, [num_seqs, n_kv_heads, head_dim] of the query type (FP8 pools:
  // encoded with k_scale / v_scale on their way in)
  const void *k_new;
  const void *v_new;
  // Host memory, read by the launch only (null: none): the lengths seq_lens
  // holds on the device, from which the launch may build the work order.
  const int32_t *host_seq_lens;
  // Work order built on the host (hp_items > 0): item j of a unit is sequence
  // hp[j] & 255, partition hp[j] >> 8, and the workgroups skip the
  // longest-first plan; hp_np[s] is the partition count the host derived
  // for sequence s, which every item of s checks against the device length.
  int32_t hp_items;
  uint16_t hp[kHostPlanItems];
  uint8_t hp_np[kHostPlanSeqs];
};

// Largest partition count merged inside the decode kernel; longer tables use
// a separate merge kernel.
constexpr int kFusedMergeParts = 8;

// Decode workgroups resident per compute unit (the kernel's register budget
// allows three), and the compute units of the current device.
constexpr int kDecodeWgsPerCu = 3;
int device_cus();

// Head tile: query heads of one KV head processed by one workgroup (1, 2, 4, 8 or 16).
int decode_head_tile(int group);

hipError_t launch_decode(DType dt, int head_dim, const DecodeArgs &a, hipStream_t stream);

// True when a launch with these arguments takes the longest-first item order
// that every workgroup builds from the lengths (a.num_seqs counts entities).
bool decode_compact_plan(const DecodeArgs &a);

// Multi-token (chunk) attention: the last n_s tokens of each sequence, causal.
struct ChunkArgs {
  void *out;                       // [T, n_heads, head_dim]
  const void *q;                   // [T, n_heads, head_dim]
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *seq_lens;
  const int32_t *query_start_loc;  // [num_seqs + 1]
  float scale_log2;
  int32_t num_seqs;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t group;
  int32_t block_size;
  int32_t block_shift;
  int32_t max_blocks;
  int64_t num_blocks;
  int32_t row_blocks;              // ceil(max_query_len * group / chunk_rows_per_block())
  // FP8 (e4m3) pools only (launch_chunk with fp8): per-KV-head scales
  const float *k_scale;
  const float *v_scale;
};

// Query rows (chunk token x query head pairs) per chunk-kernel workgroup.
int chunk_rows_per_block();

// fp8: pools of e4m3 codes with a.k_scale / a.v_scale; dt (q, out) F16 or BF16.
hipError_t launch_chunk(DType dt, int head_dim, bool fp8, const ChunkArgs &a, hipStream_t stream);

// Chunk attention on the decode kernel's work items (16 rows of (token, head)
// pairs per item, split along the sequence and merged like decode); dt is
// F16 or BF16; fp8 selects e4m3 pools with a.k_scale / a.v_scale.
hipError_t launch_chunk_rows(DType dt, int head_dim, bool fp8, const DecodeArgs &a, hipStream_t stream);

// Shared-prefix decode: the prefix launch (pre: rows mode over groups, head
// tile 16) then the suffix launch (suf: decode of the private tokens with the
// prefix partials folded in); dt is F16 or BF16.
hipError_t launch_shared_prefix(DType dt, int head_dim, bool fp8, const DecodeArgs &pre, const DecodeArgs &suf,
                                hipStream_t stream);

// Shared-prefix decode in one launch: prefix and private partitions are work
// items of one grid, merged per (sequence, KV head) by the last to finish.
// Needs n_heads / n_kv_heads in {1, 2, 4, 8, 16} and every group's members x
// heads per KV head <= 16; dt is F16 or BF16; fp8 selects e4m3 pools with
// a.k_scale / a.v_scale (also for launch_shared_prefix).
hipError_t launch_shared_fused(DType dt, int head_dim, bool fp8, const DecodeArgs &a, hipStream_t stream);

// Decode that first appends each sequence's newest token (position
// seq_lens[s] - 1) from a.k_new / a.v_new into its slot; dt is F16 or BF16;
// fp8: the pools hold e4m3 codes (a.k_scale / a.v_scale).
hipError_t launch_decode_append(DType dt, int head_dim, bool fp8, const DecodeArgs &a, hipStream_t stream);

// Same over FP8 (OCP e4m3) pools with a.k_scale / a.v_scale; dt (query and
// output) must be F16 or BF16.
hipError_t launch_decode_fp8(DType dt, int head_dim, const DecodeArgs &a, hipStream_t stream);

// Sets n int32 words to zero with a kernel (no memset node, so it may be captured).
hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t stream);

struct CacheWriteArgs {
  void *k_pool;
  void *v_pool;
  const void *k_new;
  const void *v_new;
  const int32_t *slot_mapping;
  int32_t num_tokens;
  int32_t n_kv_heads;
  int32_t row_chunks;      // head_dim * elem_bytes / 16
  int32_t block_size;
  int64_t num_slots;       // num_blocks * block_size
};

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t stream);

// Quantizing write into FP8 (OCP e4m3) pools: one float32 scale per KV head.
struct CacheWriteFp8Args {
  uint8_t *k_pool;
  uint8_t *v_pool;
  const void *k_new;       // [num_tokens, n_kv_heads, head_dim] of the input dtype
  const void *v_new;
  const float *k_scale;    // [n_kv_heads]
  const float *v_scale;
  const int32_t *slot_mapping;
  int32_t num_tokens;
  int32_t n_kv_heads;
  int32_t head_dim;        // multiple of 16
  int32_t block_size;
  int64_t num_slots;
};

hipError_t launch_cache_write_fp8(DType in_dtype, const CacheWriteFp8Args &a, hipStream_t stream);

struct CopyBlocksArgs {
  void *k_pool;
  void *v_pool;
  const int32_t *pairs;    // [num_pairs, 2] (src, dst)
  int32_t num_pairs;
  int64_t block_units;     // 16-byte units per block of one pool
  int64_t num_blocks;
};

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t stream);

}  // namespace pkv
