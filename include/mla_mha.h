/*
 * mla_mha.h - paged grouped-query MHA decode, the contrast case to MLA.
 *
 * The page "MLA 和 MHA 的 Kernel 区别" sets MLA against standard multi-head
 * attention (sections "内存布局和 KV Cache 大小" and "Decode 阶段的 HBM 访问
 * 模式" / "MHA Decode"): MHA caches a key and a value vector per KV head and
 * token and decode reads both for every cached token, where MLA reads one
 * latent row. This call runs that MHA decode over a paged cache of the same
 * page size, so the two can be measured on the same GPU and sequences.
 *
 * For sequence b, query token i and query head h (KV head h / (H_q / H_kv)):
 *
 *   L     = N_b, or under the causal mask clamp(N_b - s_q + i + 1, 0, N_b)
 *   s_t   = softmax_scale * <q[b,i,h,:], K[t, kv, :]>,   t < L
 *   out   = sum_t softmax(s)_t V[t, kv, :]     (BF16, round to nearest even)
 *   lse   = ln sum_t exp(s_t)                  (FP32; -inf and zero output when L = 0)
 *
 * where K[t] and V[t] are row t mod 64 of page block_table[b][t / 64].
 *
 *   q            device bf16 [batch][s_q][h_q][128], 16-byte aligned
 *   k_cache      device bf16 [num_pages][64][h_kv][128], 16-byte aligned
 *   v_cache      device bf16 [num_pages][64][h_kv][128], 16-byte aligned
 *   block_table  device int32 [batch][max_blocks_per_seq]
 *   seqlens      device int32 [batch]
 *   h_q, h_kv    h_q a multiple of h_kv; (h_q / h_kv) * s_q <= 16
 *   out          device bf16 [batch][s_q][h_q][128], 8-byte aligned (written)
 *   lse          device fp32 [batch][s_q][h_q] (written)
 *
 * One workgroup per (sequence, KV head) streams that head's keys and values
 * of the whole sequence (no split plan, no workspace). Preconditions and
 * conventions as for mla_decode_fwd in mla_decode.h.
 */
#ifndef MLA_MHA_H
#define MLA_MHA_H

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_MHA_HEAD_DIM 128

mla_status mla_mha_decode_fwd(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q, int h_q,
                              int h_kv, int num_pages, float softmax_scale, int causal, void* out, float* lse,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_MHA_H */
