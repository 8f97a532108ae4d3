/*
 * mla_absorb.h - the weight-absorption steps on either side of MLA decode.
 *
 * On the page "MLA 和 MHA 的 Kernel 区别" (MLA vs MHA kernel differences),
 * section "内存布局和 KV Cache 大小" and its MLA decode pseudo-code, every
 * head's key and value are up-projections of the cached latent row,
 * K_h = c_KV W_UK_h and V_h = c_KV W_UV_h (W_UK_h: 512 x d_nope,
 * W_UV_h: 512 x d_v). Decode (mla_decode.h) works in the latent space
 * instead: the query has W_UK_h folded in and W_UV_h is applied to the
 * latent output. These two calls are those folds, per token t and head h:
 *
 *   mla_absorb_q:  q_abs[t,h,0:512]   = W_UK_h q_nope[t,h,:]
 *                  q_abs[t,h,512:576] = q_rope[t,h,:]       (copied)
 *   mla_absorb_o:  o[t,h,:]           = o_lat[t,h,:] W_UV_h
 *
 * BF16 in, FP32 accumulation on the matrix cores, BF16 out (round to nearest
 * even). q_abs is written in the layout mla_decode_fwd reads for q
 * ([batch][s_q][h][576] with t = b * s_q + i), and o_lat is read in the
 * layout it writes for out.
 *
 * Weight layouts are chosen so that both products read their contraction
 * dimension contiguously: W_UK as [h][512][d_nope] (W_UK_h row by row) and
 * W_UV TRANSPOSED, as [h][d_v][512] (row v of W_UV_h^T holds column v of
 * W_UV_h). Weights are static, so the transpose is done once at load time.
 *
 * Conventions as in mla_decode.h: caller-owned device buffers, enqueued on
 * `stream`, host-side argument checks return a status and enqueue nothing.
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_absorb_q - absorbed query for decode.
 *
 *   q_nope   device bf16 [tokens][h][d_nope], contiguous, 16-byte aligned
 *   q_rope   device bf16 [tokens][h][64], contiguous, 16-byte aligned
 *   w_uk     device bf16 [h][512][d_nope], contiguous, 16-byte aligned
 *   tokens   >= 1 (batch * s_q)
 *   h        >= 1
 *   d_nope   multiple of 32, 32..512
 *   q_abs    device bf16 [tokens][h][576], 16-byte aligned; written
 *   stream   hipStream_t
 *
 * Limits: tokens * h * 576 < 2^31 (MLA_ERR_UNSUPPORTED otherwise).
 */
mla_status mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int h,
                        int d_nope, void* q_abs, void* stream);

/*
 * mla_absorb_o - head outputs from the latent decode output.
 *
 *   o_lat    device bf16 [tokens][h][512], contiguous, 16-byte aligned
 *            (the out buffer of mla_decode_fwd)
 *   w_uv_t   device bf16 [h][d_v][512], contiguous, 16-byte aligned
 *            (W_UV_h transposed, per head)
 *   tokens   >= 1
 *   h        >= 1
 *   d_v      multiple of 32, 32..512
 *   out      device bf16 [tokens][h][d_v], 8-byte aligned; written
 *   stream   hipStream_t
 *
 * Limits: tokens * h * 512 < 2^31 (MLA_ERR_UNSUPPORTED otherwise).
 */
mla_status mla_absorb_o(const void* o_lat, const void* w_uv_t, int tokens, int h, int d_v, void* out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
