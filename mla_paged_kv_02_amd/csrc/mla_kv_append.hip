// mla_kv_append.hip - paged latent-cache append (include/mla_kv_append.h).
//
// A pure scatter: every new token's 1152-byte row is copied into its page
// slot, p = N_b - s_new + i (FlashMLA overview page: 64-token pages behind a
// block table; the new tokens are the last s_new of the sequence, as the
// decode call's causal mask reads them). The work is one 16-byte chunk per
// thread step, numbered token-major so that a wave's loads read consecutive
// source bytes and its stores fill consecutive bytes of a page row (rows of
// consecutive positions in one page are adjacent too). No LDS, no MFMA: the
// kernel is bound by HBM and, for one decode step's few rows, by launch
// latency.
#include "../../include/mla_kv_append.h"

#include <hip/hip_runtime.h>

#include "mla_common.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr int kAppendUnroll = 4;   // chunks per thread, kAppendThreads apart
constexpr int kAppendChunksPerBlock = kAppendThreads * kAppendUnroll;

struct AppendArgs {
    const u32x4* src;        // new rows, 72 chunks each
    u32x4* kv;               // cache, 72 chunks per row
    const int32_t* seqlens;
    const int32_t* block_table;
    int32_t* skipped;        // may be null
    int batch, s_new, max_blocks, num_pages;
    int total_chunks;        // batch * s_new * 72
};

// Destination chunk index of source chunk g, or -1 when its token is not
// written. Counts a token without a page once (at its first chunk).
__device__ __forceinline__ long long append_target(const AppendArgs& a, int g) {
    const int row = g / kRowChunks;
    const int c = g - row * kRowChunks;
    const int b = row / a.s_new;
    const int i = row - b * a.s_new;
    const int p = a.seqlens[b] - a.s_new + i;
    if (p < 0) return -1;
    const int blk = p >> 6;
    int page = -1;
    if (blk < a.max_blocks) page = a.block_table[(size_t)b * a.max_blocks + blk];
    if (page < 0 || page >= a.num_pages) {
        if (c == 0 && a.skipped) atomicAdd(a.skipped, 1);
        return -1;
    }
    return ((long long)page * kPageRows + (p & (kPageRows - 1))) * kRowChunks + c;
}

__global__ __launch_bounds__(kAppendThreads) void mla_kv_append_kernel(AppendArgs a) {
    const int g0 = blockIdx.x * kAppendChunksPerBlock + threadIdx.x;
    long long dst[kAppendUnroll];
    u32x4 v[kAppendUnroll] = {};
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        const int g = g0 + u * kAppendThreads;
        dst[u] = g < a.total_chunks ? append_target(a, g) : -1;
        if (dst[u] >= 0) v[u] = __builtin_nontemporal_load(a.src + g);
    }
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u)
        if (dst[u] >= 0) a.kv[dst[u]] = v[u];
}

bool aligned_to(const void* p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace
}  // namespace mla

extern "C" mla_status mla_kv_append(const void* new_rows, int batch, int s_new, const int32_t* seqlens,
                                    const int32_t* block_table, int max_blocks_per_seq, void* kv_cache,
                                    int num_pages, int32_t* skipped_rows, void* stream) {
    using namespace mla;
    if (!new_rows || !seqlens || !block_table || !kv_cache) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || s_new < 1 || max_blocks_per_seq < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
    const long long chunks = (long long)batch * s_new * kRowChunks;
    if (chunks >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * batch > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
    if (!aligned_to(new_rows, 16) || !aligned_to(kv_cache, 16)) return MLA_ERR_MISALIGNED;
    if (!aligned_to(seqlens, 4) || !aligned_to(block_table, 4) || (skipped_rows && !aligned_to(skipped_rows, 4)))
        return MLA_ERR_MISALIGNED;
    AppendArgs a{};
    a.src = static_cast<const u32x4*>(new_rows);
    a.kv = static_cast<u32x4*>(kv_cache);
    a.seqlens = seqlens;
    a.block_table = block_table;
    a.skipped = skipped_rows;
    a.batch = batch;
    a.s_new = s_new;
    a.max_blocks = max_blocks_per_seq;
    a.num_pages = num_pages;
    a.total_chunks = (int)chunks;
    const unsigned grid = (unsigned)((chunks + kAppendChunksPerBlock - 1) / kAppendChunksPerBlock);
    hipLaunchKernelGGL(mla_kv_append_kernel, dim3(grid), dim3(kAppendThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
