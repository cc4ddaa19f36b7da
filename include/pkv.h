/*
 * pkv.h -- C ABI of the MI355X (gfx950) paged KV-cache library.
 *
 * Two operations make up the decode hot path of PagedAttention:
 *
 *   pkv_paged_attn_decode  one query token per sequence attends over a KV cache
 *                          that lives in fixed-size blocks of a shared pool,
 *                          reached through a per-sequence block table (vLLM
 *                          paper page, "PagedAttention" core-idea section and
 *                          its block-pool diagram; vLLM notes page, "KV Cache
 *                          and PagedAttention" section, default block of 16
 *                          tokens).
 *   pkv_kv_cache_write     appends each new token's K and V into the pool slot
 *                          the scheduler allocated for it (vLLM notes page,
 *                          "V1 engine": allocate_slots before the forward pass;
 *                          vLLM paper page: blocks grow on demand).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers on the current HIP device, dense
 *   and row-major, 16-byte aligned, except the one host array a function
 *   names as such (seq_lens_host of pkv_paged_attn_decode_append_planned).
 *   The caller owns every array; the library keeps no pointer after a call
 *   returns.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means the
 *   null stream). The caller keeps the arrays alive until the stream reaches
 *   that point. Nothing synchronises the host.
 * - Every function returns a pkv_status. On a non-OK status nothing was
 *   launched and pkv_last_error() returns a message (thread-local). No C++
 *   exception crosses this boundary.
 * - Floating-point arrays of one call share a dtype (pkv_dtype). Index arrays
 *   are int32.
 *
 * Tensor layouts (the pages fix none; these are this library's):
 *   q, out          [num_seqs, n_heads, head_dim]
 *   k_pool, v_pool  [num_blocks, n_kv_heads, block_size, head_dim]
 *                   (one block of one KV head is a contiguous block_size*head_dim run)
 *   block_tables    int32 [num_seqs, max_blocks_per_seq]; logical block i of
 *                   sequence s is physical block block_tables[s, i]
 *   seq_lens        int32 [num_seqs]; tokens already cached for each sequence
 *   k_new, v_new    [num_tokens, n_kv_heads, head_dim]
 *   slot_mapping    int32 [num_tokens]; slot = physical_block * block_size + offset
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

/* Exported from libpkv.so (built with hidden visibility by default). */
#define PKV_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,      /* bad argument: null pointer, shape, alignment, size */
  PKV_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim, block_size or dtype */
  PKV_ERR_DEVICE = 3,       /* a HIP call failed (launch, allocation, device query) */
  PKV_ERR_NO_BLOCKS = 4     /* the block manager's free queue is too short (pkv_blocks.h) */
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3  /* 1-byte OCP e4m3 pool codes (pkv_fp8.h); copy_blocks only here */
} pkv_dtype;

/*
 * Paged decode attention (vLLM paper page, "PagedAttention": attention reads
 * K/V through the block table; vLLM notes page, "FlashAttention": the online
 * softmax is exact; ICML-tutorial notes page, MQA/GQA: query heads share KV
 * heads).
 *
 * For sequence s, query head h and its KV head g = h / (n_heads / n_kv_heads):
 *   K_s[j] = k_pool[block_tables[s, j / block_size], g, j % block_size, :], j < seq_lens[s]
 *   out[s, h] = sum_j softmax_j(scale * <q[s, h], K_s[j]>) * V_s[j]
 * computed in fp32 from the stored dtype and rounded to nearest-even into
 * `out`. seq_lens[s] == 0 gives a zero row.
 *
 * Arguments:
 *   out                 written, [num_seqs, n_heads, head_dim], dtype
 *   q                   read, [num_seqs, n_heads, head_dim], dtype
 *   k_pool, v_pool      read, [num_blocks, n_kv_heads, block_size, head_dim], dtype
 *   block_tables        read, int32 [num_seqs, max_blocks_per_seq]; only the
 *                       first ceil(seq_lens[s] / block_size) entries of a row are
 *                       read, the rest may hold anything (e.g. -1)
 *   seq_lens            read, int32 [num_seqs]
 *   scale               softmax scale (commonly 1/sqrt(head_dim))
 *   n_heads, n_kv_heads n_heads % n_kv_heads == 0, n_heads / n_kv_heads <= 256
 *   head_dim            64 or 128
 *   block_size          16, 32, 64 or 128
 *   num_seqs            >= 0 (0: no-op), <= 65535
 *   max_blocks_per_seq  >= 1, row width of block_tables
 *   num_blocks          >= 1, pool size in blocks
 *   dtype               pkv_dtype of q, out and both pools
 *   stream              hipStream_t
 *
 * Device-side values are not checked on the host. Instead the kernels never
 * touch memory outside the arrays: a sequence whose length is negative or
 * exceeds max_blocks_per_seq * block_size, or whose table holds an id outside
 * [0, num_blocks) among its used entries, gets NaN in its output rows.
 *
 * Long sequences are split into partitions whose partial results (fp32) go to
 * a workspace owned by the library (grown on demand per device and stream,
 * released by pkv_release_workspace). Up to 8 partitions per sequence are
 * merged by the last of them to finish, inside the decode kernel; longer
 * tables use a second kernel on the same stream. Two calls that run at the
 * same time on one stream are not supported; different streams get
 * different workspaces.
 */
PKV_API int pkv_paged_attn_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *block_tables, const int32_t *seq_lens, float scale,
                          int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                          int64_t num_blocks, int32_t dtype, void *stream);

/*
 * Slot-mapped KV cache write (vLLM notes page, "V1 engine" step: slots are
 * allocated for the step's new tokens; vLLM paper page: a sequence grows one
 * block at a time on demand).
 *
 * For every t < num_tokens with 0 <= slot_mapping[t] < num_blocks * block_size:
 *   k_pool[slot / block_size, :, slot % block_size, :] = k_new[t, :, :]
 *   v_pool[slot / block_size, :, slot % block_size, :] = v_new[t, :, :]
 * as a bitwise copy. A negative slot marks padding and is skipped; a slot past
 * the pool is skipped too (never written out of bounds). Every other pool byte
 * is left unchanged. Two tokens with the same slot race: the caller must not
 * pass duplicates.
 *
 * Arguments:
 *   k_pool, v_pool   written in place, [num_blocks, n_kv_heads, block_size, head_dim]
 *   k_new, v_new     read, [num_tokens, n_kv_heads, head_dim]
 *   slot_mapping     read, int32 [num_tokens]
 *   num_tokens       >= 0 (0: no-op)
 *   n_kv_heads       >= 1
 *   head_dim         > 0 with head_dim * element size a multiple of 16 bytes
 *   block_size       >= 1
 *   num_blocks       >= 1
 *   dtype            pkv_dtype of all four float arrays
 *   stream           hipStream_t
 */
PKV_API int pkv_kv_cache_write(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                       const int32_t *slot_mapping, int32_t num_tokens, int32_t n_kv_heads,
                       int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                       void *stream);

/*
 * One decode step in one call: append each sequence's newest token, then
 * attend. Equivalent to pkv_kv_cache_write of k_new / v_new into the slots
 * of positions seq_lens[s] - 1 (slot = block_tables[s, (L - 1) / block_size] *
 * block_size + (L - 1) % block_size) followed by pkv_paged_attn_decode with
 * seq_lens, which here count the new token. The vLLM notes page's engine
 * step (allocate the slots, then run the forward pass that writes the new
 * K/V and attends) is the sequence these two calls follow; one kernel does
 * both: the work item that holds a sequence's newest token writes it to the
 * pool and uses it from on-chip memory instead of reading it back, which
 * removes the separate write kernel and its launch from every step.
 *
 * Arguments: as in pkv_paged_attn_decode, plus
 *   k_pool, v_pool  read and written (the new rows are stored)
 *   k_new, v_new    read, [num_seqs, n_kv_heads, head_dim] of dtype, 16-byte aligned
 *   seq_lens        read, tokens per sequence including the new one (>= 1; 0 =
 *                   empty sequence: zero output, nothing written)
 *   dtype           PKV_F16 or PKV_BF16 (PKV_F32 gives PKV_ERR_UNSUPPORTED)
 * Device-side checks as in pkv_paged_attn_decode; a sequence with an invalid
 * length or table entry gets NaN rows and no write.
 */
PKV_API int pkv_paged_attn_decode_append(void *out, const void *q, void *k_pool, void *v_pool, const void *k_new,
                                         const void *v_new, const int32_t *block_tables, const int32_t *seq_lens,
                                         float scale, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                                         int64_t num_blocks, int32_t dtype, void *stream);

/*
 * pkv_paged_attn_decode_append with the lengths also given in host memory.
 * The vLLM notes page's engine step has the scheduler, on the host, decide
 * each step's batch and lengths before the forward pass runs; a caller that
 * holds them there passes them here, and the library builds the work order
 * (which workgroup takes which sequence partition, longest first) on the host
 * and hands it to the kernel with the launch. The workgroups then start their
 * first items at once instead of first loading every length and building
 * that order themselves.
 *
 * Arguments: as in pkv_paged_attn_decode_append, plus
 *   seq_lens_host   host memory, [num_seqs] int32, the values seq_lens holds
 *                   on the device; read during the call only, owned by the
 *                   caller (PKV_ERR_INVALID if null while num_seqs > 0)
 * Results are those of pkv_paged_attn_decode_append, bit for bit. The order
 * is used when the batch has at most 256 sequences, every workgroup takes
 * one item and a sequence has at most 8 partitions (pkv_decode_plan; they
 * are then merged inside the kernel); other batches take the kernel's own
 * order and read seq_lens_host no further. Where the order is used, a
 * sequence whose device length splits into a different number of
 * partitions than its host length gets NaN rows and its new token is not
 * stored (one with the same count is attended over its device length);
 * other sequences are unaffected.
 */
PKV_API int pkv_paged_attn_decode_append_planned(void *out, const void *q, void *k_pool, void *v_pool,
                                                 const void *k_new, const void *v_new, const int32_t *block_tables,
                                                 const int32_t *seq_lens, const int32_t *seq_lens_host, float scale,
                                                 int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                                 int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                                                 int64_t num_blocks, int32_t dtype, void *stream);

/*
 * pkv_paged_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, result, checks and kernels as
 * pkv_paged_attn_decode (outputs are bit-identical); the only difference is
 * where the kernels keep their scratch (the split partials and the merge
 * counters): a fixed array compiled into the library, one per GPU, held until
 * the process ends, instead of a workspace grown on demand. The call makes no
 * allocation: the first call on a device looks up that device's array and
 * clears its counters with a small kernel on `stream`.
 *
 * Limits (PKV_ERR_INVALID beyond them, before anything is launched):
 *   split partials  num_seqs * n_heads * P * (head_dim + 2) * 4 bytes
 *                   <= PKV_NOALLOC_WORKSPACE_BYTES, with P the partition count
 *                   pkv_decode_plan reports (no partials when P = 1);
 *   merge counters  num_seqs * n_kv_heads * ceil(n_heads / n_kv_heads / 16)
 *                   + 64 <= PKV_NOALLOC_COUNTERS when 1 < P <= 8.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams or host threads) race and must not be issued.
 */
#define PKV_NOALLOC_WORKSPACE_BYTES (64u << 20)
#define PKV_NOALLOC_COUNTERS 16384
PKV_API int pkv_paged_attn_decode_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                                          const int32_t *block_tables, const int32_t *seq_lens, float scale,
                                          int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                                          int64_t num_blocks, int32_t dtype, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
PKV_API const char *pkv_last_error(void);

/*
 * Sequence-partition length (tokens) used by pkv_paged_attn_decode.
 * 0 restores the automatic choice; otherwise a multiple of 16 in [16, 1<<20].
 * A call rounds a length above block_size down to whole blocks and caps it
 * at 64 blocks (64 * block_size tokens). Process-wide; meant
 * for tests and tuning. Returns PKV_ERR_INVALID for any other value.
 */
PKV_API int pkv_set_partition_tokens(int32_t tokens);

/*
 * Partition length and count the next pkv_paged_attn_decode with these sizes
 * would use (written to *partition_tokens and *max_partitions; either may be
 * NULL). Pure host arithmetic, no device access.
 */
PKV_API int pkv_decode_plan(int32_t n_heads, int32_t n_kv_heads, int32_t block_size, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t *partition_tokens,
                    int32_t *max_partitions);

/* Free every workspace the library holds (waits for their streams first). */
PKV_API int pkv_release_workspace(void);

/* ABI version, (major << 16) | minor. */
PKV_API int32_t pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
