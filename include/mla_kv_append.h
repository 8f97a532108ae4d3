/*
 * mla_kv_append.h - paged latent-cache append, the step before decode.
 *
 * Before a decode step reads the cache, the new tokens' cache rows (the
 * latent c_KV of 512 values and the pre-rotated positional part of 64 values,
 * 576 BF16 per token; page "MLA 和 MHA 的 Kernel 区别", section
 * "内存布局和 KV Cache 大小": the cache keeps only the compressed vector)
 * are written into the paged cache (FlashMLA overview page: pages of 64
 * tokens, addressed through a block table). The long-text inference page
 * ("Unlocking GPU Potential ...") names managing this cache as the step
 * that serving must get right.
 *
 * Placement rule (the same one the decode call's causal mask assumes): the
 * s_new new tokens of sequence b are the last s_new of its N_b tokens, so
 * new token i goes to position
 *
 *   p = N_b - s_new + i,   stored at row p mod 64 of page block_table[b][p / 64].
 *
 * A token with p < 0 (a sequence shorter than s_new) has no place and is not
 * written; such tokens are not counted as skipped. A token whose table entry
 * lies outside the row (p / 64 >= max_blocks_per_seq) or names no page
 * (entry < 0 or >= num_pages) is not written and is counted in
 * *skipped_rows. Nothing else in the cache changes.
 *
 * Conventions as in mla_decode.h: caller-owned buffers, enqueued on `stream`,
 * host-side argument checks return a status and enqueue nothing.
 */
#ifndef MLA_KV_APPEND_H
#define MLA_KV_APPEND_H

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_kv_append - scatter new cache rows into the paged cache.
 *
 *   new_rows       device bf16 [batch][s_new][576], contiguous, 16-byte aligned
 *   batch          >= 1
 *   s_new          new tokens per sequence, >= 1
 *   seqlens        device int32 [batch]: N_b, the cache length after the append
 *   block_table    device int32 [batch][max_blocks_per_seq], 4-byte aligned
 *   max_blocks_per_seq  row stride of block_table, >= 1
 *   kv_cache       device bf16 [num_pages][64][1][576], 16-byte aligned; the
 *                  rows named by the rule above are overwritten
 *   num_pages      >= 1
 *   skipped_rows   device int32 or NULL: incremented once per token that has
 *                  p >= 0 but no valid page (the call does not reset it)
 *   stream         hipStream_t
 *
 * Limits: batch * s_new * 72 < 2^31 (MLA_ERR_UNSUPPORTED otherwise).
 * Preconditions: new_rows does not overlap kv_cache; no two tokens of the call
 * map to the same cache row (distinct pages across block-table rows), else
 * which one lands there is unspecified.
 */
mla_status mla_kv_append(const void* new_rows, int batch, int s_new, const int32_t* seqlens,
                         const int32_t* block_table, int max_blocks_per_seq, void* kv_cache,
                         int num_pages, int32_t* skipped_rows, void* stream);

/*
 * mla_kv_append_fp8 - the same append into an FP8 cache (page layout of
 * mla_decode_fp8.h): each placed token's 512 latent values are quantised
 * with one FP32 scale, its 64 rotary values copied as BF16, and the scale
 * stored in its group. Quantisation of a row x (BF16 values, exact in FP32):
 *
 *   scale = fl32(amax / 448), the FP32 number nearest amax / 448
 *           (amax = max |x_d|; 1 for an all-zero row)
 *   byte  = the E4M3 value nearest the exact quotient |x_d| / scale, ties
 *           to the even mantissa, magnitudes past 448 saturating to 448;
 *           sign bit of x_d
 *
 * (the exact quotient, not its FP32 rounding: where fl32(x_d / scale) lands
 * on a midpoint between two E4M3 values the exact quotient usually does
 * not, and the nearer value is the one on its side)
 *
 * Arguments as for mla_kv_append, with kv_pages device bytes
 * [num_pages][MLA_FP8_PAGE_BYTES], 16-byte aligned, in place of kv_cache.
 * Limits: batch * s_new * 72 < 2^31.
 */
mla_status mla_kv_append_fp8(const void* new_rows, int batch, int s_new, const int32_t* seqlens,
                             const int32_t* block_table, int max_blocks_per_seq, void* kv_pages,
                             int num_pages, int32_t* skipped_rows, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_KV_APPEND_H */
