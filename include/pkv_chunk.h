/*
 * pkv_chunk.h -- paged attention of a chunk of new query tokens per sequence,
 * causal inside the chunk (C ABI of libpkv.so, next to pkv.h).
 *
 * This is the attention of chunked prefill and of speculative verification.
 *   - Chunked prefill (Sarathi-Serve, PagedAttention notes page): a long
 *     prompt's prefill runs in chunks interleaved with decode steps.
 *   - Speculative decoding (vLLM notes page): the target model scores K
 *     draft tokens in one pass.
 *   - Continuous batching (vLLM notes page, scheduling section): the
 *     sequences of a step are packed into one token list, and positions plus
 *     the attention mask keep every token on its own sequence.
 *
 * For sequence s the chunk is its last n_s = query_start_loc[s + 1] -
 * query_start_loc[s] tokens. Their K/V must already be in the pool (written
 * with pkv_kv_cache_write), and seq_lens[s] counts every cached token,
 * chunk included. Chunk token i sits at position p = seq_lens[s] - n_s + i,
 * and for each query head h (KV head g = h / (n_heads / n_kv_heads)):
 *   out[query_start_loc[s] + i, h] = sum_{j <= p} softmax_j(scale * <q[., h], K_s[j]>) V_s[j]
 * in float32 from 16-bit inputs, rounded to nearest-even. n_s = 1 is a decode
 * step; n_s = seq_lens[s] is a whole causal prefill.
 *
 * Arguments:
 *   out              written, [T, n_heads, head_dim], T = query_start_loc[num_seqs]
 *   q                read, [T, n_heads, head_dim]
 *   k_pool, v_pool, block_tables, seq_lens, scale, n_heads, n_kv_heads,
 *   head_dim, block_size, max_blocks_per_seq, num_blocks: as in
 *                    pkv_paged_attn_decode (head_dim 64 or 128, block_size
 *                    16..128)
 *   query_start_loc  read, int32 [num_seqs + 1], nondecreasing, starting at 0
 *   num_seqs         >= 0 (0: no-op)
 *   max_query_len    >= every n_s (host value; sizes the launch)
 *   dtype            PKV_F16 or PKV_BF16 (PKV_F32 gives PKV_ERR_UNSUPPORTED)
 *   stream           hipStream_t
 * Device-side values are not checked on the host. A sequence with n_s >
 * seq_lens[s], or seq_lens[s] > max_blocks_per_seq * block_size, or a used
 * table entry outside the pool gets NaN rows; chunk rows past max_query_len
 * are not computed. Cached K/V rows must be finite: long chunks multiply
 * whole 64-token stages with a weight of exactly zero for the tokens a row
 * may not see, so a NaN or infinity stored at a cached token can also reach
 * earlier rows of the same chunk (slots past seq_lens[s] are never read).
 */
#ifndef PKV_CHUNK_H
#define PKV_CHUNK_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

PKV_API int pkv_paged_attn_chunk(void *out, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_tables, const int32_t *seq_lens,
                                 const int32_t *query_start_loc, float scale, int32_t n_heads,
                                 int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_query_len,
                                 int32_t dtype, void *stream);

/*
 * pkv_paged_attn_chunk over FP8 pools (the format and scales of pkv_fp8.h):
 * the same result definition, with K and V rows the dequantized values
 * decode(code) * scale[KV head]. k_pool and v_pool are uint8 [num_blocks,
 * n_kv_heads, block_size, head_dim]; k_scale and v_scale are device float32
 * [n_kv_heads]; dtype (of q and out) is PKV_F16 or PKV_BF16. Other arguments
 * and device-side checks as in pkv_paged_attn_chunk.
 */
PKV_API int pkv_paged_attn_chunk_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                     const float *k_scale, const float *v_scale, const int32_t *block_tables,
                                     const int32_t *seq_lens, const int32_t *query_start_loc, float scale,
                                     int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t max_query_len, int32_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_CHUNK_H */
