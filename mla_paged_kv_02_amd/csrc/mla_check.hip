// mla_check.hip - device-side check of the decode preconditions that the
// host cannot see without reading device memory (include/mla_decode.h,
// mla_check_decode_inputs).
//
// The decode reads, for every sequence b with N_b = seqlens[b] tokens, the
// block-table entries n < ceil(N_b / 64) (the paged cache of the
// "FlashMLA Overview" page: variable-length sequences in 64-token blocks
// looked up through a per-sequence table) and trusts them to name pages of
// the cache. This kernel counts the ways a call could break that trust:
// a length below zero or above 64 * max_blocks_per_seq (counted once, the
// sequence's entries then unchecked), and every entry the decode would read
// that lies outside [0, num_pages). Entries past a sequence's last page are
// never read and are not checked.
//
// One workgroup walks the whole table (wave w takes sequences w, w + 16, ...,
// its lanes the entries), sums the counts through LDS and stores the total
// once: no atomics across workgroups, no counter to clear beforehand, and the
// same answer on every run. It reads the used part of the table once, so it
// is a debugging and testing aid, not a per-step call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void mla_check_inputs_kernel(const int32_t* block_table, int max_blocks,
                                                                         const int32_t* seqlens, int batch,
                                                                         int num_pages, int32_t* violations) {
    __shared__ int wave_counts[kCheckThreads / 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int bad = 0;
    for (int b = wave; b < batch; b += kCheckThreads / 64) {
        const int n_tok = seqlens[b];
        if (n_tok < 0 || (long long)n_tok > 64LL * max_blocks) {
            bad += lane == 0 ? 1 : 0;
            continue;
        }
        const int pages = (n_tok + 63) / 64;
        const int32_t* row = block_table + (size_t)b * max_blocks;
        for (int n = lane; n < pages; n += 64) {
            const int32_t e = row[n];
            bad += (e < 0 || e >= num_pages) ? 1 : 0;
        }
    }
    // wave sum, then the workgroup's
    for (int m = 32; m >= 1; m >>= 1) bad += __shfl_xor(bad, m, 64);
    if (lane == 0) wave_counts[wave] = bad;
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = 0;
        for (int w = 0; w < kCheckThreads / 64; ++w) total += wave_counts[w];
        *violations = total;
    }
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_check_decode_inputs(const int32_t* block_table, int max_blocks_per_seq,
                                              const int32_t* seqlens, int batch, int num_pages,
                                              int32_t* violations, void* stream) {
    using namespace mla;
    if (!block_table || !seqlens || !violations) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || max_blocks_per_seq < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
    if ((long long)max_blocks_per_seq * batch > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(block_table) % 4 || reinterpret_cast<uintptr_t>(seqlens) % 4 ||
        reinterpret_cast<uintptr_t>(violations) % 4)
        return MLA_ERR_MISALIGNED;
    hipLaunchKernelGGL(mla_check_inputs_kernel, dim3(1), dim3(kCheckThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), block_table, max_blocks_per_seq, seqlens, batch,
                       num_pages, violations);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
