// mla_sched_kernel.hip - builds the split-KV plan (see mla_sched.h) on the
// device in one workgroup, and the identical plan on the host.
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {

namespace {

constexpr int kSchedThreads = 1024;
constexpr int kLdsBatch = 8192;   // 32 KB of cost-line starts

// floor(a / b) through one correctly rounded double division. Exact for the
// two quotients the plan needs: the numerator stays below 2^47 (a partition
// index < 2^16 times a cost < 2^31) and the exact quotient q = n - k/b with
// k >= 1 sits at least 1/b >= 2^-31 below the next integer, while the
// rounding error is at most half an ulp of a quotient below 2^31 (<= 2^-22)
// when b <= 2^16, or of a quotient below 2^16 (<= 2^-37) when b < 2^31.
// The 64-bit integer division it replaces is a long instruction sequence.
__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
    return (int64_t)__builtin_floor((double)a / (double)b);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the last lane of
// row 0 and of row 2 into rows 1 and 3, then the last lane of row 1 into rows
// 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum over the workgroup; *total receives the sum. `sums`
// holds the wave totals (kSchedThreads / 64 ints); a caller that scans again
// before every wave is past this call's barrier passes another buffer.
__device__ int block_exclusive_scan(int v, int* total, int* sums) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) sums[wave] = incl;
    __syncthreads();
    constexpr int kWaves = kSchedThreads / 64;
    const int ws = wave_inclusive_scan(lane < kWaves ? sums[lane] : 0);
    *total = __builtin_amdgcn_readlane(ws, kWaves - 1);
    const int offset = wave > 0 ? __builtin_amdgcn_readlane(ws, wave - 1) : 0;
    return offset + incl - v;
}

__global__ __launch_bounds__(kSchedThreads) void mla_split_meta_kernel(const int32_t* seqlens,
                                                                       int batch, int P, int cseg,
                                                                       int R, int32_t* meta) {
    // cost-line starts stay in LDS for the boundary searches when they fit
    // (every batch up to kLdsBatch sequences); larger batches search the copy
    // in the metadata itself
    __shared__ int32_t s_start[kLdsBatch];
    __shared__ int32_t s_len[kLdsBatch];   // lengths, so no record waits on a second global read
    __shared__ int wave_sums[4][kSchedThreads / 64];   // scan totals, by call
    const bool in_lds = batch <= kLdsBatch;
    int32_t* seq = meta + kMetaHeader + kPartInts * P;
    const int tid = threadIdx.x;

    // cost-line start of every sequence
    int carry = 0, nscan = 0;
    for (int base = 0; base < batch; base += kSchedThreads) {
        const int b = base + tid;
        const int32_t len = b < batch ? seqlens[b] : 0;
        const int v = b < batch ? (int)cost_len(len, cseg) : 0;
        int chunk_total;
        const int ex = block_exclusive_scan(v, &chunk_total, wave_sums[nscan++ & 3]);
        if (b < batch) {
            seq[4 * b + 3] = carry + ex;
            if (in_lds) {
                s_start[b] = carry + ex;
                s_len[b] = len;
            }
        }
        carry += chunk_total;
    }
    const int64_t total = carry;
    const int32_t pa = active_partitions(total, P);

    // partitions holding each sequence's pages; split-partial slots
    int slots = 0;
    for (int base = 0; base < batch; base += kSchedThreads) {
        const int b = base + tid;
        int first = -1, count = 0;
        if (b < batch) {
            // both written by this thread above
            const int32_t st = in_lds ? s_start[b] : seq[4 * b + 3];
            const int32_t np = pages_of(in_lds ? s_len[b] : seqlens[b]);
            if (np > 0) {   // seq_partitions with the divisions above
                first = (int32_t)floor_div((int64_t)(st + cseg + 1) * pa - 1, total);
                const int32_t z = (int32_t)floor_div((int64_t)(st + cseg + np) * pa - 1, total);
                count = z - first + 1;
            }
        }
        const int v = count > 1 ? count : 0;
        int chunk_total;
        const int ex = block_exclusive_scan(v, &chunk_total, wave_sums[nscan++ & 3]);
        if (b < batch) {
            seq[4 * b + 0] = count > 1 ? slots + ex : -1;
            seq[4 * b + 1] = first;
            seq[4 * b + 2] = count;
        }
        slots += chunk_total;
    }
    __syncthreads();

    // partition boundaries (boundary_at). With the starts in LDS both
    // boundaries of a partition are found together by radix-4 lifting for the
    // largest b with start[b] <= x: per level three probes per boundary, the
    // six LDS reads issued at once (indexes clamped into the batch, the test
    // keeps j < batch), one round trip per level instead of two chains of
    // binary-search steps. Larger batches search the copy in the metadata.
    int s4 = 1;   // largest power of 4 <= batch - 1 (1 for batch <= 4)
    while ((int64_t)s4 * 4 <= batch - 1) s4 *= 4;
    for (int p = tid; p < P; p += kSchedThreads) {
        int32_t* e = meta + kMetaHeader + kPartInts * p;
        if (p < pa) {
            // partition_start(p) = floor(p * total / pa)
            int32_t v[4];
            const int64_t x0 = floor_div((int64_t)p * total, pa);
            const int64_t x1 = floor_div((int64_t)(p + 1) * total, pa);
            if (in_lds) {
                // s_start[0] = 0 <= x, and the probes reach 4 * s4 - 1 >= batch - 1
                int lo0 = 0, lo1 = 0;
                for (int st = s4; st > 0; st >>= 2) {
                    int c0 = 0, c1 = 0;
#pragma unroll
                    for (int i = 1; i <= 3; ++i) {
                        const int j0 = lo0 + i * st, j1 = lo1 + i * st;
                        const int32_t a0 = s_start[j0 < batch ? j0 : batch - 1];
                        const int32_t a1 = s_start[j1 < batch ? j1 : batch - 1];
                        c0 += (j0 < batch && a0 <= x0) ? 1 : 0;
                        c1 += (j1 < batch && a1 <= x1) ? 1 : 0;
                    }
                    lo0 += c0 * st;
                    lo1 += c1 * st;
                }
                // x0 < total; x1 = total for the last active partition
                const int64_t off0 = x0 - s_start[lo0] - cseg;
                const int64_t off1 = x1 - s_start[lo1] - cseg;
                v[0] = lo0;
                v[1] = off0 < 0 ? 0 : (int32_t)off0;
                v[2] = x1 >= total ? batch : lo1;
                v[3] = x1 >= total ? 0 : (off1 < 0 ? 0 : (int32_t)off1);
            } else {
                boundary_at(x0, seq + 3, 4, batch, total, cseg, &v[0], &v[1]);
                boundary_at(x1, seq + 3, 4, batch, total, cseg, &v[2], &v[3]);
            }
            e[0] = v[0]; e[1] = v[1]; e[2] = v[2]; e[3] = v[3];
            e[4] = v[0] < batch ? (in_lds ? s_len[v[0]] : seqlens[v[0]]) : 0;
        } else {
            e[0] = batch; e[1] = 0; e[2] = batch; e[3] = 0;
            e[4] = 0;
        }
        e[5] = 0; e[6] = 0; e[7] = 0;
    }
    // partial counters start at zero
    for (int i = tid; i < R * batch; i += kSchedThreads) meta[meta_counters(batch, P) + i] = 0;
    if (tid < kMetaHeader) {
        int32_t h = 0;
        switch (tid) {
            case 0: h = kMetaMagic; break;
            case 1: h = batch; break;
            case 2: h = P; break;
            case 3: h = cseg; break;
            case 4: h = pa > 0 ? (int32_t)((total + pa - 1) / pa) : 0; break;
            case 5: h = slots; break;
            case 6: h = (int32_t)total; break;
            case 7: h = pa; break;
            case 8: h = R; break;
            default: h = 0;
        }
        meta[tid] = h;
    }
}

}  // namespace

hipError_t launch_split_metadata(const int32_t* seqlens, int batch, int num_partitions, int cseg,
                                 int row_blocks, int32_t* meta, hipStream_t stream) {
    hipLaunchKernelGGL(mla_split_meta_kernel, dim3(1), dim3(kSchedThreads), 0, stream, seqlens,
                       batch, num_partitions, cseg, row_blocks, meta);
    return hipGetLastError();
}

void split_metadata_host(const int32_t* seqlens, int batch, int P, int cseg, int R, int32_t* meta) {
    int32_t* seq = meta + kMetaHeader + kPartInts * P;
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) {
        seq[4 * b + 3] = (int32_t)total;
        total += cost_len(seqlens[b], cseg);
    }
    const int32_t pa = active_partitions(total, P);
    int slots = 0;
    for (int b = 0; b < batch; ++b) {
        int first, count;
        seq_partitions(seq[4 * b + 3], pages_of(seqlens[b]), cseg, total, pa, &first, &count);
        seq[4 * b + 0] = count > 1 ? slots : -1;
        seq[4 * b + 1] = first;
        seq[4 * b + 2] = count;
        if (count > 1) slots += count;
    }
    for (int p = 0; p < P; ++p) {
        int32_t* e = meta + kMetaHeader + kPartInts * p;
        if (p < pa) {
            boundary_at(partition_start(p, total, pa), seq + 3, 4, batch, total, cseg, &e[0], &e[1]);
            boundary_at(partition_start(p + 1, total, pa), seq + 3, 4, batch, total, cseg, &e[2], &e[3]);
            e[4] = e[0] < batch ? seqlens[e[0]] : 0;
        } else {
            e[0] = batch; e[1] = 0; e[2] = batch; e[3] = 0;
            e[4] = 0;
        }
        e[5] = 0; e[6] = 0; e[7] = 0;
    }
    for (int i = 0; i < kMetaHeader; ++i) meta[i] = 0;
    meta[0] = kMetaMagic;
    meta[1] = batch;
    meta[2] = P;
    meta[3] = cseg;
    meta[4] = pa > 0 ? (int32_t)((total + pa - 1) / pa) : 0;
    meta[5] = slots;
    meta[6] = (int32_t)total;
    meta[7] = pa;
    meta[8] = R;
    for (int i = 0; i < R * batch; ++i) meta[meta_counters(batch, P) + i] = 0;
}

}  // namespace mla
