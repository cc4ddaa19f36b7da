/*
 * pkv_fp8.h -- FP8 KV cache: pools of 8-bit OCP e4m3 codes with one float32
 * scale per KV head (C ABI of libpkv.so, next to pkv.h).
 *
 * KV-cache quantization is one of the further KV optimisations the vLLM
 * paper page lists ("what vLLM changed", KV-cache directions). The course
 * page explains the payoff: decode is memory-bound, so moving fewer bytes
 * speeds it up directly. The pages fix no format; this library's is:
 *   - code: OCP e4m3 (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *     exponent 0 = subnormals m/8 * 2^-6; S.1111.111 = NaN; no infinity;
 *     largest finite value 448), one byte per element;
 *   - value of a stored element = decode(code) * scale[kv head], with a
 *     separate k_scale and v_scale per KV head (float32, device, [n_kv_heads]);
 *   - writing x: code = encode(x * (1 / scale)), both float32 operations
 *     correctly rounded; encode rounds to the nearest e4m3 value, ties to the
 *     even code, saturates to +-448 (infinity too), and keeps NaN as NaN.
 * Pools have the layout of pkv.h with 1-byte elements:
 *   [num_blocks, n_kv_heads, block_size, head_dim] uint8.
 * pkv_copy_blocks copies FP8 blocks with dtype PKV_FP8_E4M3.
 */
#ifndef PKV_FP8_H
#define PKV_FP8_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_paged_attn_decode over FP8 pools: the same result definition, with
 * K_s[j] and V_s[j] the dequantized rows decode(code) * scale. The kernel
 * decodes codes exactly into the query's 16-bit type, folds k_scale into the
 * softmax scale and applies v_scale to the output. Accumulation is float32.
 *
 * Arguments are those of pkv_paged_attn_decode, plus:
 *   k_pool, v_pool   read, uint8 [num_blocks, n_kv_heads, block_size, head_dim]
 *   k_scale, v_scale read, float32 [n_kv_heads]
 *   dtype            of q and out: PKV_F16 or PKV_BF16 (PKV_F32 gives
 *                    PKV_ERR_UNSUPPORTED)
 * Device-side checks, workspace and merge behave as in pkv_paged_attn_decode.
 */
PKV_API int pkv_paged_attn_decode_fp8(void *out, const void *q, const void *k_pool, const void *v_pool,
                                      const float *k_scale, const float *v_scale,
                                      const int32_t *block_tables, const int32_t *seq_lens, float scale,
                                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t dtype, void *stream);

/*
 * pkv_kv_cache_write into FP8 pools. Each element of k_new / v_new (dtype
 * F32, F16 or BF16) is quantized with its KV head's scale as described above
 * and stored in the slot; padding (slot < 0) and slots past the pool are
 * skipped, every other pool byte is unchanged.
 *
 * Arguments:
 *   k_pool, v_pool   written in place, uint8 [num_blocks, n_kv_heads, block_size, head_dim]
 *   k_new, v_new     read, [num_tokens, n_kv_heads, head_dim] of dtype
 *   k_scale, v_scale read, float32 [n_kv_heads] (device)
 *   slot_mapping     read, int32 [num_tokens]
 *   head_dim         a multiple of 16
 *   other sizes      as in pkv_kv_cache_write
 */
PKV_API int pkv_kv_cache_write_fp8(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                                   const float *k_scale, const float *v_scale, const int32_t *slot_mapping,
                                   int32_t num_tokens, int32_t n_kv_heads, int32_t head_dim,
                                   int32_t block_size, int64_t num_blocks, int32_t dtype, void *stream);

/*
 * pkv_paged_attn_decode_append over FP8 pools: one decode step in one launch.
 * Equivalent to pkv_kv_cache_write_fp8 of k_new / v_new into the slot of
 * position seq_lens[s] - 1 (slot = block_tables[s, (L - 1) / block_size] *
 * block_size + (L - 1) % block_size) followed by pkv_paged_attn_decode_fp8
 * with seq_lens, which here count the new token: the stored codes are those
 * of the FP8 write, and the output equals the two calls' bit for bit. The
 * work item that holds a sequence's newest token encodes and stores its rows
 * and attends over their decoded codes from on-chip memory (engine step on
 * the vLLM notes page: slots first, then the pass that writes the new K/V and
 * attends; KV quantization as a KV-cache optimisation on the vLLM paper page).
 *
 * Arguments: as in pkv_paged_attn_decode_fp8, plus
 *   k_pool, v_pool   read and written (uint8 e4m3 codes; the new rows are stored)
 *   k_new, v_new     read, [num_seqs, n_kv_heads, head_dim] of dtype, 16-byte aligned
 *   seq_lens         read, tokens per sequence including the new one (0 = empty
 *                    sequence: zero output, nothing written)
 *   dtype            of q, out, k_new and v_new: PKV_F16 or PKV_BF16
 * A sequence with an invalid length or table entry gets NaN rows and no write.
 */
PKV_API int pkv_paged_attn_decode_append_fp8(void *out, const void *q, void *k_pool, void *v_pool,
                                             const void *k_new, const void *v_new, const float *k_scale,
                                             const float *v_scale, const int32_t *block_tables,
                                             const int32_t *seq_lens, float scale, int32_t n_heads,
                                             int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                             int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_blocks,
                                             int32_t dtype, void *stream);

/*
 * pkv_paged_attn_decode_append_fp8 with the lengths also in host memory, as
 * pkv_paged_attn_decode_append_planned (pkv.h) is to the 16-bit step: the
 * library builds the longest-first work order on the host from
 * seq_lens_host (host memory, [num_seqs] int32, the values seq_lens holds on
 * the device; read during the call only, owned by the caller;
 * PKV_ERR_INVALID if null while num_seqs > 0) and the kernel skips its own.
 * Used for batches of at most 256 sequences, at most 1024 work items per KV
 * head and at most 8 partitions per sequence (merged inside the kernel),
 * where a workgroup may take more than one item; other batches take the
 * kernel's own order. Results are those of pkv_paged_attn_decode_append_fp8
 * bit for bit; where the order is used, a sequence whose device length
 * splits into a different number of partitions than its host length gets
 * NaN rows and no write, other sequences are unaffected.
 */
PKV_API int pkv_paged_attn_decode_append_fp8_planned(void *out, const void *q, void *k_pool, void *v_pool,
                                                     const void *k_new, const void *v_new, const float *k_scale,
                                                     const float *v_scale, const int32_t *block_tables,
                                                     const int32_t *seq_lens, const int32_t *seq_lens_host,
                                                     float scale, int32_t n_heads, int32_t n_kv_heads,
                                                     int32_t head_dim, int32_t block_size, int32_t num_seqs,
                                                     int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_FP8_H */
