/*
 * mla_decode.h - C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * What it computes. Multi-head Latent Attention decode over a paged,
 * compressed KV cache, as described on the FlashMLA overview page
 * (nullthought.net, "FlashMLA Overview": BF16, a paged KV cache with 64-token
 * blocks, variable-length sequences) and on the page "MLA 和 MHA 的 Kernel
 * 区别" (MLA vs MHA kernel differences), sections "内存布局和 KV Cache 大小"
 * (the cache holds only the latent c_KV) and "Decode 阶段的 HBM 访问模式" /
 * "MLA Decode" (score every cached token, softmax, weighted sum of values).
 *
 * The query arrives in absorbed form (W_UK folded in), so each cache row of
 * 576 BF16 values is the key, and its first 512 values are the value. The
 * last 64 values are a pre-rotated positional part that enters scores only.
 * For sequence b, query token i and head h (row r = i*h_q + h):
 *
 *   L      = N_b                         (causal == 0)
 *          = clamp(N_b - s_q + i + 1, 0, N_b)   (causal == 1)
 *   s_t    = softmax_scale * <q[b,i,h,:], K_t>,   t < L
 *   out    = sum_t softmax(s)_t * K_t[0:512]      (BF16, round to nearest even)
 *   lse    = ln sum_t exp(s_t)                    (FP32; -inf when L == 0)
 *
 * where K_t is row t mod 64 of physical page block_table[b][t / 64]. A row
 * with L == 0 outputs zeros.
 *
 * Calling pattern (FlashMLA overview page, flash_api.cpp walk-through: the
 * metadata call is made once, then the attention call once per layer):
 *
 *   once per decode step:  mla_get_split_metadata(...)
 *   once per layer:        mla_decode_fwd(...)
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device memory on the current HIP device;
 *    "host" pointers are ordinary host memory. The caller owns every buffer;
 *    the library keeps no per-call state and allocates nothing.
 *  - `stream` is a hipStream_t (NULL = the default stream). All device work
 *    is enqueued on it; no call synchronises the host.
 *  - Arguments are validated on the host before any HIP call. A failed check
 *    returns a status and enqueues nothing. Exceptions never cross the ABI.
 *  - Conditions that cannot be checked without reading device memory are
 *    preconditions (listed per call); breaking them is undefined behaviour.
 *  - Calls on different streams may run concurrently as long as they do not
 *    share workspace or metadata buffers.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed geometry: one latent KV head, rows of 576 BF16 (512 latent + 64
 * positional), values = first 512 entries, pages of 64 tokens. */
#define MLA_HEAD_DIM 576
#define MLA_HEAD_DIM_V 512
#define MLA_PAGE_SIZE 64
/* Largest supported rows per sequence, M = h_q * s_q. */
#define MLA_MAX_ROWS 1024

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,          /* null pointer, bad size, bad flag        */
    MLA_ERR_UNSUPPORTED = 2,          /* shape outside what the kernels cover   */
    MLA_ERR_MISALIGNED = 3,           /* pointer alignment requirement broken   */
    MLA_ERR_WORKSPACE_TOO_SMALL = 4,  /* metadata or workspace buffer too small */
    MLA_ERR_HIP = 5,                  /* a HIP runtime call or launch failed    */
    MLA_ERR_SCRATCH_LIMIT = 6         /* beyond mla_decode_fwd_noalloc's scratch */
} mla_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(int status);

/* ABI version of this header, (major << 16) | minor. */
int mla_abi_version(void);

/* Number of partitions the split scheduler uses by default for this shape on
 * the current device (a function of the device's compute-unit count and of
 * M = h_q * s_q). Returns <= 0 with no device. Host-only query. */
int mla_default_num_partitions(int h_q, int s_q);

/* Bytes of the metadata buffer for `batch` sequences and `num_partitions`
 * partitions (num_partitions <= 0 means the default). 0 on invalid input. */
size_t mla_metadata_bytes(int batch, int h_q, int s_q, int num_partitions);

/* Bytes of scratch workspace mla_decode_fwd needs (split partial results, and
 * the metadata when the call computes it itself). 0 on invalid input. */
size_t mla_workspace_bytes(int batch, int h_q, int s_q, int num_partitions);

/*
 * mla_get_split_metadata - split-KV work plan for one decode step.
 *
 * The work of a step is the list of (sequence, page) pairs. It is cut into
 * `num_partitions` contiguous ranges of near-equal cost (a range may start or
 * end inside a sequence; a sequence cut into several ranges is recombined by
 * its log-sum-exp). This spreads small-batch, long-context decode over all
 * compute units (motivation: the long-text inference page, "Unlocking GPU
 * Potential ...", on decode starving the GPU when batch < SM count).
 * The plan depends only on seqlens, h_q, s_q and num_partitions, so it can be
 * reused by every layer of the step.
 *
 *   seqlens         device int32[batch], N_b >= 0 (cached tokens per sequence,
 *                   including the s_q new ones)
 *   batch           >= 1
 *   h_q, s_q        query heads (>= 1) and new tokens per sequence (>= 1);
 *                   h_q * s_q <= MLA_MAX_ROWS
 *   num_partitions  <= 0 for the default, else 1..65536
 *   metadata        device int32 buffer, 4-byte aligned, of at least
 *                   mla_metadata_bytes(batch, h_q, s_q, num_partitions) bytes;
 *                   written by the call
 *   stream          hipStream_t
 *
 * Precondition: total pages sum_b ceil(N_b/64) < 2^30.
 */
mla_status mla_get_split_metadata(const int32_t* seqlens, int batch, int h_q, int s_q,
                                  int num_partitions, int32_t* metadata,
                                  size_t metadata_bytes, void* stream);

/*
 * Same plan computed on the host from host seqlens into a host buffer of the
 * same layout (for callers that already hold lengths on the host, and for
 * tests). Uses no GPU.
 */
mla_status mla_get_split_metadata_host(const int32_t* seqlens, int batch, int h_q, int s_q,
                                       int num_partitions, int32_t* metadata,
                                       size_t metadata_bytes);

/*
 * mla_check_metadata_host - whether a host copy of a plan (`metadata`,
 * `metadata_bytes` bytes, from mla_get_split_metadata_host or copied back
 * from the device) was built for these arguments: its header (magic, batch,
 * partition count, per-segment cost, row blocks) against the plan that
 * mla_decode_fwd (fp8 = 0) or mla_decode_fwd_fp8 (fp8 = 1) builds for
 * batch, h_q, s_q and num_partitions. The decode kernels run the same test
 * on the device copy before they read anything else of it.
 * Returns MLA_OK on a match; MLA_ERR_INVALID_ARG on a mismatch, a NULL or
 * misaligned buffer, or fp8 not 0/1; MLA_ERR_WORKSPACE_TOO_SMALL when the
 * buffer is shorter than the header; MLA_ERR_UNSUPPORTED for a shape with no
 * plan. Uses no GPU (with num_partitions <= 0 the default partition count
 * comes from the current device's CU count, 256 when there is none).
 */
mla_status mla_check_metadata_host(const int32_t* metadata, size_t metadata_bytes, int batch, int h_q,
                                   int s_q, int num_partitions, int fp8);

/*
 * mla_decode_fwd - MLA decode attention for one layer (see top of file).
 *
 *   q              device bf16 [batch][s_q][h_q][576], contiguous, 16-byte aligned
 *   kv_cache       device bf16 [num_pages][64][1][576], contiguous, 16-byte aligned
 *   block_table    device int32 [batch][max_blocks_per_seq], 4-byte aligned
 *   max_blocks_per_seq  row stride of block_table, >= 1
 *   seqlens        device int32 [batch]
 *   batch, s_q, h_q     as for mla_get_split_metadata (must match it)
 *   num_pages      number of physical pages in kv_cache, >= 1
 *   softmax_scale  finite, > 0 (e.g. 1/sqrt(576))
 *   causal         0 or 1 (bottom-right mask over the s_q new tokens)
 *   metadata       device buffer from mla_get_split_metadata for the same
 *                  seqlens/batch/h_q/s_q/num_partitions, or NULL to have this
 *                  call compute it inside `workspace` first. The kernels
 *                  check the plan's header against the call's arguments
 *                  before using it (mla_check_metadata_host); a plan built
 *                  for other arguments makes the call write NaN into every
 *                  lse entry and store nothing else (the call itself still
 *                  returns MLA_OK: the check runs on the device). The plan is
 *                  only read, except for its partial counters (one int per
 *                  sequence and row block, zero as the metadata call writes
 *                  them): when the decode kernel merges split sequences
 *                  itself it counts the partials there and leaves every
 *                  counter at zero again when the call completes. So one
 *                  metadata buffer serves any number of calls in stream
 *                  order, but not two calls that overlap in time (on one
 *                  stream or several); a call that does not complete (its
 *                  context lost) leaves the plan unusable until
 *                  mla_get_split_metadata rewrites it
 *   num_partitions the value given to mla_get_split_metadata (<= 0: default)
 *   workspace      device scratch, 16-byte aligned, of at least
 *                  mla_workspace_bytes(batch, h_q, s_q, num_partitions) bytes;
 *                  contents on entry are ignored
 *   out            device bf16 [batch][s_q][h_q][512], 16-byte aligned (written)
 *   lse            device fp32 [batch][s_q][h_q], 4-byte aligned (written)
 *   stream         hipStream_t
 *
 * Preconditions: 0 <= block_table[b][n] < num_pages for n < ceil(N_b/64);
 * N_b <= 64 * max_blocks_per_seq. Entries past a sequence's last page and
 * page rows past N_b are never used and may hold anything (NaN included).
 * Buffers must not overlap, except q/kv_cache/block_table/seqlens which are
 * only read.
 */
mla_status mla_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q,
                          int h_q, int num_pages, float softmax_scale, int causal,
                          int32_t* metadata, int num_partitions, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * mla_check_decode_inputs - checks on the device the preconditions of
 * mla_decode_fwd (and of the FP8 and allocation-free variants) that the host
 * cannot see: the paged cache of the "FlashMLA Overview" page, variable-length
 * sequences in 64-token blocks looked up through a per-sequence block table.
 * Counts into *violations (written, not added to) every way the inputs break
 * them: a sequence length below 0 or above 64 * max_blocks_per_seq (counted
 * once; that sequence's entries are then not checked), and every entry
 * block_table[b][n] with n < ceil(seqlens[b] / 64) outside [0, num_pages).
 * Entries past a sequence's last page are never read by the decode and are
 * not checked. 0 means the decode's device preconditions hold.
 *
 *   block_table          device int32 [batch][max_blocks_per_seq], 4-byte aligned
 *   max_blocks_per_seq   row stride of block_table, >= 1
 *   seqlens              device int32 [batch], 4-byte aligned
 *   batch                >= 1
 *   num_pages            number of physical pages of the cache, >= 1
 *   violations           device int32, 4-byte aligned (written)
 *   stream               hipStream_t
 *
 * Enqueues one small single-workgroup kernel on `stream` and returns without
 * waiting; the caller reads *violations back after the stream reaches it.
 * It reads the used part of the whole table, so it is meant for debugging
 * and tests, not for every decode step. Returns MLA_OK;
 * MLA_ERR_INVALID_ARG for a NULL pointer or a size below 1;
 * MLA_ERR_UNSUPPORTED when batch * max_blocks_per_seq exceeds 2^31 - 1;
 * MLA_ERR_MISALIGNED; MLA_ERR_HIP if the launch fails.
 */
mla_status mla_check_decode_inputs(const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens,
                                   int batch, int num_pages, int32_t* violations, void* stream);

/*
 * mla_decode_fwd_noalloc - mla_decode_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without
 * `workspace`, the same results, bit for bit. It calls no hipMalloc,
 * hipFree or other allocating routine; the split partials (and the plan,
 * when `metadata` is NULL) live in a scratch array of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory from
 * its first call there until the process ends.
 *
 * Limit: a call whose workspace need exceeds MLA_NOALLOC_SCRATCH_BYTES
 * returns MLA_ERR_SCRATCH_LIMIT and enqueues nothing; every call with
 * mla_workspace_bytes(batch, h_q, s_q, num_partitions) <=
 * MLA_NOALLOC_SCRATCH_BYTES is accepted (with the default partition count
 * that covers, for example, 128 sequences at 128 heads and 132 sequences of
 * two tokens at 128 heads).
 *
 * All calls on one GPU share its scratch and leave their contents in it;
 * nothing there needs to start at zero (a plan computed in the scratch is
 * written whole by each call). Calls that overlap in time on one GPU (on
 * different streams, or different host threads) race on the scratch and
 * give undefined results: order them on one stream. The first call on a
 * device looks up the scratch's address (not an allocation; it may load
 * the library's code object on that device).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (72u << 20)

mla_status mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                  int max_blocks_per_seq, const int32_t* seqlens, int batch, int s_q, int h_q,
                                  int num_pages, float softmax_scale, int causal, int32_t* metadata,
                                  int num_partitions, void* out, float* lse, void* stream);

/*
 * mla_set_plan_override - testing and benchmarking hook (not part of the
 * attention semantics): forces the decode organisation of every plan built
 * after the call, process-wide, for BF16 caches.
 *
 *   kernel  -1 the default choice, 0 always the 16-row organisation (each
 *           wave its own key stripe), 1 always the score/value-wave
 *           organisation (blocks of 16, 32 or 64 rows, the smallest that
 *           holds the rows), 2 always the fused-wave organisation (blocks of
 *           128 rows, each wave scoring and accumulating 32 of them)
 *   merge   -1 the default choice, 0 split sequences are merged by a combine
 *           kernel after decode, 1 by the last decode workgroup of each
 *           (the fused-wave organisation always uses the combine kernel)
 *
 * The plan (metadata, size queries) and the decode call it serves must be
 * made under the same setting: a plan built under another kernel choice no
 * longer matches the call (see mla_check_metadata_host). Returns
 * MLA_ERR_INVALID_ARG for kernel outside -1..2 or merge outside -1..1.
 */
mla_status mla_set_plan_override(int kernel, int merge);

/*
 * Kernel timing for benchmarks (not part of the attention semantics).
 *
 * mla_timing_enable(1) makes every following mla_decode_fwd call on this
 * process record HIP events on its own stream around its decode kernel and
 * around its combine kernel; mla_timing_enable(0) stops recording and drops
 * what was recorded. Events are created by the library on first use and
 * reused; at most 4096 calls are recorded, later calls are not timed.
 * Returns MLA_OK, or MLA_ERR_HIP if an event cannot be created.
 *
 * mla_timing_collect: once every recorded call has completed (the caller
 * synchronises the streams first), writes the summed milliseconds of the
 * decode kernels and of the combine kernels and the number of calls, then
 * clears the record. Any output pointer may be NULL. Returns MLA_ERR_HIP if
 * an event has not completed or cannot be read.
 */
mla_status mla_timing_enable(int enable);
mla_status mla_timing_collect(double* decode_ms, double* combine_ms, int* calls);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
