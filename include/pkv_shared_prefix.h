/*
 * pkv_shared_prefix.h -- decode attention for batches whose sequences share
 * a prompt prefix (C ABI of libpkv.so, next to pkv.h).
 *
 * Samples of one prompt (parallel sampling, beam search) and requests with a
 * common system prompt reference the same physical KV blocks for the shared
 * prefix (vLLM paper page: the OS-paging analogy table pairs page sharing
 * with block sharing for parallel sampling, beam search and prefix caching;
 * "PagedAttention" core idea, block-level sharing; system implementation
 * points, prefix sharing). Plain decode reads those blocks once per sequence.
 * This call reads them once per group instead: the group's query heads of one
 * KV head (members x heads per KV head, e.g. 4 samples x 4 heads = 16 rows,
 * one MFMA tile) are scored together against each shared tile. Each
 * sequence's private tokens are then walked alone, and the two partial
 * softmax states are merged exactly as split partitions are (online softmax:
 * running max and sum, vLLM notes page "FlashAttention"; partition merge,
 * ICML-tutorial notes page, FlashDecoding).
 *
 * Result: the same definition as pkv_paged_attn_decode, for every sequence:
 *   out[s, h] = sum_{j < seq_lens[s]} softmax_j(scale * <q[s, h], K_s[j]>) V_s[j].
 * Only the order of the float32 sums differs.
 *
 * Sharing description (device int32 arrays):
 *   group_start  [num_groups + 1]: group i is sequences group_start[i] ..
 *                group_start[i + 1] - 1. The groups are consecutive and
 *                cover the batch: group_start[0] = 0, strictly increasing,
 *                group_start[num_groups] = num_seqs.
 *   prefix_lens  [num_seqs]: shared prefix tokens of each sequence, equal
 *                within a group, a multiple of block_size, at most
 *                seq_lens[s]; 0 = nothing shared (a group of one sequence
 *                may use any valid value; 0 is the natural one).
 * Precondition: the members of a group hold the same physical block ids in
 * their first prefix_lens / block_size table entries (the prefix is read
 * through the group's first member's table). pkv_shared_prefix_groups
 * derives such a description from host copies of the tables.
 *
 * Arguments:
 *   out, q, k_pool, v_pool, block_tables, seq_lens, scale, n_heads,
 *   n_kv_heads, head_dim, block_size, num_seqs, max_blocks_per_seq,
 *   num_blocks, stream: as in pkv_paged_attn_decode (head_dim 64 or 128,
 *                    block_size 16..128)
 *   num_groups       >= 1 when num_seqs > 0
 *   max_group_size   >= every group's size (host value; sizes the launch)
 *   dtype            PKV_F16 or PKV_BF16 (PKV_F32 gives PKV_ERR_UNSUPPORTED)
 * Kernels run on `stream`. When n_heads / n_kv_heads is 1, 2, 4, 8 or 16,
 * every group has at most 16 / (n_heads / n_kv_heads) members, and the
 * table is short enough for the partial slots to fit the in-kernel merge
 * (at most 8 per row), prefix partitions and private-token partitions are
 * work items of one launch, and the last of them to finish for a (sequence,
 * KV head) merges that row set. Otherwise the prefix runs in one launch and
 * the private tokens in a second, which folds the prefix partials in. The
 * partial states go through the library's workspace for (device, stream), so
 * calls that overlap on one stream's workspace from several host threads
 * race, as for pkv_paged_attn_decode.
 * Device-side checks: a sequence whose prefix_lens value is negative, not a
 * multiple of block_size or larger than seq_lens[s], or whose length exceeds
 * the table, gets NaN rows. Group ranges that do not cut the batch into
 * consecutive groups, or prefix lengths that differ within a group, break the
 * precondition. The one-launch path checks the whole description in the
 * kernel and then writes NaN to every output row; the two-launch path leaves
 * the results of the offending sequences undefined. Either way no memory
 * outside the arguments and the workspace is accessed, and later calls on the
 * stream are unaffected.
 */
#ifndef PKV_SHARED_PREFIX_H
#define PKV_SHARED_PREFIX_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

PKV_API int pkv_paged_attn_decode_shared_prefix(void *out, const void *q, const void *k_pool, const void *v_pool,
                                                const int32_t *block_tables, const int32_t *seq_lens,
                                                const int32_t *prefix_lens, const int32_t *group_start,
                                                float scale, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t num_seqs, int32_t num_groups,
                                                int32_t max_group_size, int32_t max_blocks_per_seq,
                                                int64_t num_blocks, int32_t dtype, void *stream);

/*
 * pkv_paged_attn_decode_shared_prefix over FP8 pools (the format and scales of
 * pkv_fp8.h): the same result definition with the dequantized rows
 * decode(code) * scale[KV head]. k_pool and v_pool are uint8 [num_blocks,
 * n_kv_heads, block_size, head_dim]; k_scale and v_scale are device float32
 * [n_kv_heads]; dtype (of q and out) is PKV_F16 or PKV_BF16. Other arguments,
 * paths and checks as in pkv_paged_attn_decode_shared_prefix.
 */
PKV_API int pkv_paged_attn_decode_shared_prefix_fp8(void *out, const void *q, const void *k_pool,
                                                    const void *v_pool, const float *k_scale, const float *v_scale,
                                                    const int32_t *block_tables, const int32_t *seq_lens,
                                                    const int32_t *prefix_lens, const int32_t *group_start,
                                                    float scale, int32_t n_heads, int32_t n_kv_heads,
                                                    int32_t head_dim, int32_t block_size, int32_t num_seqs,
                                                    int32_t num_groups, int32_t max_group_size,
                                                    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                                    void *stream);

/*
 * Host helper: a sharing description for pkv_paged_attn_decode_shared_prefix
 * from host copies of the block tables and lengths. Consecutive sequences
 * join one group while they hold the same first table entry (and each has at
 * least one full block); a group's prefix is the longest run of leading
 * entries that all members hold in common, counted in whole blocks and
 * capped at every member's full blocks (floor(seq_lens / block_size)). A
 * group of one sequence gets prefix 0.
 *
 * Arguments (host memory):
 *   block_tables     read, int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens         read, int32 [num_seqs], each in [0, max_blocks_per_seq * block_size]
 *   group_start      written, int32 [num_seqs + 1] (the first *num_groups + 1 entries are used)
 *   prefix_lens      written, int32 [num_seqs]
 *   num_groups       written: the number of groups (0 when num_seqs = 0)
 *   max_group_size   written (may be NULL): the largest group's size
 * Returns PKV_ERR_INVALID for null pointers, negative sizes or a length
 * outside the table.
 */
PKV_API int pkv_shared_prefix_groups(const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                     int32_t max_blocks_per_seq, int32_t block_size, int32_t *group_start,
                                     int32_t *prefix_lens, int32_t *num_groups, int32_t *max_group_size);

#ifdef __cplusplus
}
#endif

#endif /* PKV_SHARED_PREFIX_H */
