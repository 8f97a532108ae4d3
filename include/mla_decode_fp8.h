/*
 * mla_decode_fp8.h - MLA decode over an FP8 latent cache.
 *
 * The cache of MLA holds only the compressed latent row (page "MLA 和 MHA 的
 * Kernel 区别", section "内存布局和 KV Cache 大小"), and decode is bound by
 * the bytes it streams from it, so storing the latent part in 8 bits makes
 * decode about 1.8x lighter. The page also remarks that quantising in the
 * latent space is well tolerated.
 *
 * Number format: OCP FP8 E4M3 (the gfx950 native FP8; sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest
 * finite 448). One FP32 scale per token: the value of latent coordinate d of
 * token t is e4m3(byte[t][d]) * scale[t]. The 64 rotary values stay BF16.
 *
 * Page layout (64 tokens, MLA_FP8_PAGE_BYTES = 41,216 bytes, contiguous):
 * four groups of 16 tokens, group k (tokens 16k .. 16k+15) at 10,304 k,
 * each holding, for its tokens r = 0..15,
 *
 *   bytes [0, 8192)         latent: token r's 512 E4M3 bytes at 512 r
 *   bytes [8192, 10240)     rotary: token r's 64 BF16 values at 8192 + 128 r
 *   bytes [10240, 10304)    scales: token r's FP32 scale at 10240 + 4 r
 *
 * (a group is what one wave of the kernel streams, scales included)
 *
 * Everything else (metadata, query, output, lse, workspace, split plan,
 * calling pattern, masking, empty rows, errors) is exactly as for
 * mla_decode_fwd in mla_decode.h, computed over the dequantised rows
 * [e4m3(bytes) * scale ; rope].
 */
#ifndef MLA_DECODE_FP8_H
#define MLA_DECODE_FP8_H

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_FP8_PAGE_BYTES 41216

/*
 * mla_get_split_metadata_fp8 - the split plan for mla_decode_fwd_fp8.
 *
 * Same arguments, layout and semantics as mla_get_split_metadata. The FP8
 * decode uses score/value blocks of 16, 32 or 64 rows (the smallest that
 * holds a sequence's rows, 64 beyond), while the BF16 decode uses 16-row
 * blocks below 64 rows, so the two calls' plans can differ (at 32 rows, for
 * example); mla_metadata_bytes and mla_workspace_bytes cover both.
 */
mla_status mla_get_split_metadata_fp8(const int32_t* seqlens, int batch, int h_q, int s_q,
                                      int num_partitions, int32_t* metadata, size_t metadata_bytes,
                                      void* stream);

/*
 * mla_decode_fwd_fp8 - mla_decode_fwd over FP8 pages.
 *
 *   kv_cache   device bytes [num_pages][MLA_FP8_PAGE_BYTES] in the layout
 *              above, 16-byte aligned
 *   metadata   from mla_get_split_metadata_fp8 (or NULL: computed in-call)
 *   (all other arguments as for mla_decode_fwd)
 *
 * Supported: h_q * s_q up to MLA_MAX_ROWS, as for mla_decode_fwd. The
 * score/value kernel keeps each half page in LDS as it is in memory and
 * widens E4M3 to BF16 in registers as its two products read it. A process
 * whose kernel choice was forced to the 16-row organisation
 * (mla_set_plan_override: each wave converts its own key stripe into BF16
 * first) gets MLA_ERR_UNSUPPORTED above 64 rows; the fused-wave override
 * does not apply to FP8. Latent bytes of used tokens must not be NaN
 * patterns; scales must be finite.
 */
mla_status mla_decode_fwd_fp8(const void* q, const void* kv_cache, const int32_t* block_table,
                              int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q, int h_q,
                              int num_pages, float softmax_scale, int causal, int32_t* metadata,
                              int num_partitions, void* workspace, size_t workspace_bytes, void* out,
                              float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_FP8_H */
