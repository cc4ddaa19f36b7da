/*
 * pkv_blocks.h -- block manager and block copy of the paged KV cache
 * (C ABI of libpkv.so, next to pkv.h).
 *
 * The pool of KV blocks is allocated once, up front. A host-side manager
 * hands blocks to sequences on demand and takes them back. Blocks can be
 * shared between sequences through a reference count, and a shared block is
 * copied before it is written (copy-on-write). Sources:
 *   - vLLM paper page, "PagedAttention" core idea: blocks are taken from a
 *     pool as a sequence grows and returned when it ends. Its OS-paging
 *     table pairs fork and copy-on-write with block sharing for parallel
 *     sampling and beam search. Its "system implementation points" list a
 *     pre-allocated pool and reference-counted sharing.
 *   - vLLM notes page, "KV Cache and PagedAttention": a block may be
 *     referenced by several requests (ref_count) and is copied on write. The
 *     KV cache manager keeps a free-block queue.
 *   - vLLM notes page, "Prefix Caching", eviction paragraph: a finished
 *     request's blocks join the free queue in reverse order, so its last
 *     blocks are the first to be reused.
 *
 * Manager semantics (host only; no device memory is touched):
 *   - The free queue starts as blocks 0, 1, ..., num_blocks - 1. Allocation
 *     takes the front; a block whose count drops to zero joins the back.
 *   - A sequence owns a list of blocks and a token count. Its token j lives
 *     in slot block_list[j / block_size] * block_size + j % block_size.
 *   - add_sequence allocates ceil(num_tokens / block_size) blocks.
 *   - fork gives the child the parent's block list and token count, and
 *     raises every shared block's count by one.
 *   - append_slot reserves the slot of the next token:
 *       * position % block_size == 0: a new block is allocated;
 *       * the last block is shared (count > 1): copy-on-write. A new block
 *         replaces it in this sequence's list, the old block's count drops
 *         by one, and (src = old, dst = new) is reported. The caller copies
 *         the block (pkv_copy_blocks) before writing the slot.
 *   - free_sequence drops the count of each of its blocks, last block first;
 *     blocks reaching zero join the back of the free queue in that order.
 *   - Every operation either completes or changes nothing: it returns
 *     PKV_ERR_NO_BLOCKS when the free queue is too short, and
 *     PKV_ERR_INVALID for an unknown or duplicate sequence id.
 *   - A manager may be used from several threads (one mutex per manager).
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* New manager over a pool of num_blocks (>= 1, < 2^31 / block_size) blocks of
 * block_size (>= 1) tokens; *out receives the handle. */
PKV_API int pkv_bm_create(int64_t num_blocks, int32_t block_size, pkv_block_manager **out);

/* Frees the manager and everything it tracks (NULL is a no-op). */
PKV_API int pkv_bm_destroy(pkv_block_manager *bm);

/* Registers sequence seq_id (not yet known) with num_tokens (>= 0) tokens
 * already in the cache and allocates their ceil(num_tokens / block_size)
 * blocks. */
PKV_API int pkv_bm_add_sequence(pkv_block_manager *bm, int64_t seq_id, int32_t num_tokens);

/* Registers child (not yet known) as a copy of parent: same blocks (their
 * counts + 1) and token count. */
PKV_API int pkv_bm_fork(pkv_block_manager *bm, int64_t parent, int64_t child);

/* Reserves the slot of the next token of each of the n sequences in
 * seq_ids (distinct ids; n >= 0), in order, and grows each token count by
 * one. slots[i] receives the slot of seq_ids[i]. Copy-on-write copies needed
 * before those slots are written go to copies as (src, dst) pairs, int32
 * [2 * n] capacity; *num_copies receives their count. All-or-nothing: if the
 * free queue cannot cover every new and copied block, nothing changes and
 * PKV_ERR_NO_BLOCKS is returned. */
PKV_API int pkv_bm_append_slots(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                                int32_t *slots, int32_t *copies, int32_t *num_copies);

/* Forgets sequence seq_id and releases its blocks (see above). */
PKV_API int pkv_bm_free_sequence(pkv_block_manager *bm, int64_t seq_id);

/* Blocks in the free queue. */
PKV_API int pkv_bm_num_free(pkv_block_manager *bm, int64_t *num_free);

/* Reference count of one block (0 when free). */
PKV_API int pkv_bm_refcount(pkv_block_manager *bm, int32_t block, int32_t *count);

/* Token count and block list of one sequence: *num_tokens, *num_blocks, and
 * the first min(*num_blocks, capacity) block ids into blocks (may be NULL
 * when capacity is 0). */
PKV_API int pkv_bm_sequence(pkv_block_manager *bm, int64_t seq_id, int32_t *num_tokens,
                            int32_t *num_blocks, int32_t *blocks, int32_t capacity);

/* Host arrays for pkv_paged_attn_decode over the n sequences in seq_ids:
 * block_tables int32 [n, max_blocks] (entries past a sequence's blocks are
 * set to -1) and seq_lens int32 [n]. PKV_ERR_INVALID if a sequence has more
 * than max_blocks blocks. The copies to the device are the caller's. */
PKV_API int pkv_bm_build_tables(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                                int32_t max_blocks, int32_t *block_tables, int32_t *seq_lens);

/* Block indices of the free queue, front first: the first
 * min(num_free, capacity) go to blocks. For checks of the allocation order. */
PKV_API int pkv_bm_free_queue(pkv_block_manager *bm, int32_t *blocks, int64_t capacity);

/*
 * Copy of whole pool blocks on the GPU (the copy that copy-on-write asks
 * for; vLLM paper page, block sharing with copy-on-write).
 *
 * For every i < num_pairs with both ids in [0, num_blocks):
 *   k_pool[pairs[2i + 1]] = k_pool[pairs[2i]], and the same for v_pool,
 * copying all n_kv_heads * block_size * head_dim elements of the block,
 * bitwise. A pair with an id outside the pool is skipped. Destinations must
 * be distinct and must not be the source of another pair in the same call
 * (copy-on-write destinations are fresh blocks); otherwise the result is
 * undefined.
 *
 * Arguments:
 *   k_pool, v_pool   device, in place, [num_blocks, n_kv_heads, block_size, head_dim]
 *   pairs            device, int32 [num_pairs, 2] (src, dst)
 *   num_pairs        >= 0 (0: no-op)
 *   n_kv_heads, head_dim, block_size, num_blocks >= 1, with
 *                    n_kv_heads * block_size * head_dim * element size a
 *                    multiple of 16 bytes
 *   dtype            pkv_dtype of both pools
 *   stream           hipStream_t
 */
PKV_API int pkv_copy_blocks(void *k_pool, void *v_pool, const int32_t *pairs, int32_t num_pairs,
                            int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int32_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
