// mla_fused_combine.h - the LSE combine run by the last workgroup of a
// split sequence, inside the decode kernel.
//
// Same rule as the combine kernel (o = sum_s exp(lse_s - lse) o_s with
// lse = log sum_s exp(lse_s): one softmax over the union of the partitions'
// key sets; flash-decoding page). Used when sequences have few partials, so
// that a decode call needs no second kernel: every workgroup that writes a
// partial for (sequence b, row block rb) counts itself in counters[b * R + rb]
// once its partial has reached the device-coherent level (the partial stores
// are written through, so waiting for their completion is the release); the
// one that brings the count to the number of partitions holding the sequence
// invalidates its caches (the acquire), merges all partials and resets the
// counter to zero for the next call. No workgroup writes back or invalidates
// a whole L2 except the merging ones.
#pragma once

#include "mla_common.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {

__device__ __forceinline__ int32_t ld_plan_word(const int32_t* p, int i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p))[i];
}

// The plan check every decode kernel runs before it reads anything else of
// the plan: true if the header matches the call. Otherwise the workgroups
// write NaN into every lse entry between them (the visible sign of a plan
// built for other arguments) and the kernel stores nothing else.
template <int kThreads>
__device__ __forceinline__ bool plan_matches_or_poison(const DecodeArgs& a) {
    const bool ok = plan_header_matches(ld_plan_word(a.meta, 0), ld_plan_word(a.meta, 1), ld_plan_word(a.meta, 2),
                                        ld_plan_word(a.meta, 3), ld_plan_word(a.meta, 8), a.batch, a.P, a.cseg,
                                        a.R);
    if (ok) return true;
    const size_t n = (size_t)a.batch * a.M;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
        a.lse[i] = __builtin_nanf("");
    return false;
}

// Merges the partials of rows row0 .. row0 + nrows - 1 (< M) of sequence b,
// slots base .. base + cnt - 1, into out and lse. All kThreads threads of
// the workgroup call it; each owns one row and 512 / (kThreads / nrows)
// consecutive columns.
template <int kThreads, int kRows>
__device__ __forceinline__ void combine_rows(const DecodeArgs& a, int b, int row0, int base, int cnt) {
    constexpr int kTpr = kThreads / kRows;           // threads per row
    constexpr int kCols = kHeadDimV / kTpr;          // columns per thread
    constexpr int kVec = kCols / 4;                  // 16-byte loads per partial
    const int r = threadIdx.x / kTpr;
    const int row = row0 + r;
    if (row >= a.M) return;
    const int col = (threadIdx.x % kTpr) * kCols;
    const float* lp = a.part_lse + (size_t)row * a.lse_stride + base;
    float m = -INFINITY;
    for (int s = 0; s < cnt; ++s) m = fmaxf(m, lp[s]);
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float tot = 0.f;
    f32x4 acc[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* pp = a.part_o + ((size_t)base * a.M + row) * kHeadDimV + col;
    for (int s = 0; s < cnt; ++s) {
        const float w = __builtin_amdgcn_exp2f((lp[s] - m_use) * kLog2e);
        tot += w;
        const f32x4* src = reinterpret_cast<const f32x4*>(pp + (size_t)s * a.M * kHeadDimV);
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
            const f32x4 x = src[v];
            acc[v][0] += w * x[0]; acc[v][1] += w * x[1]; acc[v][2] += w * x[2]; acc[v][3] += w * x[3];
        }
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + col;
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
        f32x4 x = acc[v];
        x[0] *= inv; x[1] *= inv; x[2] *= inv; x[3] *= inv;
        *reinterpret_cast<bf16x4*>(op + 4 * v) = pack_bf16x4(x);
    }
    if (threadIdx.x % kTpr == 0)
        a.lse[(size_t)b * a.M + row] = tot > 0.f ? m_use + __log2f(tot) * kLn2 : -INFINITY;
}

// After this workgroup stored its partial for (b, rb): count it, and merge
// the sequence's partials when it is the last. `flag` is an int in LDS that
// no wave touches around the call. Every thread calls it; the first
// kMergeThreads of them (a multiple of kRows dividing 512 columns evenly)
// do the merge.
template <int kThreads, int kRows, int kMergeThreads = kThreads>
__device__ __forceinline__ void count_partial_and_combine(const DecodeArgs& a, int b, int rb, int* flag) {
    const int32_t* si = a.meta + kMetaHeader + kPartInts * a.P + 4 * b;
    const int base = si[0];
    const int cnt = si[2];
    // this thread's partial stores (device-coherent) have completed
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) *flag = atomicAdd(&a.counters[b * a.R + rb], 1) == cnt - 1;
    __syncthreads();
    const bool last = *flag != 0;
    __syncthreads();   // every wave has read the flag before it is reused
    if (!last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // no stale copies of the partials
    if (kMergeThreads == kThreads || threadIdx.x < kMergeThreads)
        combine_rows<kMergeThreads, kRows>(a, b, rb * kRows, base, cnt);
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[b * a.R + rb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Empty sequences (no pages, so no partition visits them): zero output and
// lse = -inf, spread over the workgroups. Every thread calls it.
template <int kThreads>
__device__ __forceinline__ void write_empty_sequences(const DecodeArgs& a) {
    for (int e = blockIdx.x; e < a.batch; e += gridDim.x) {
        if (a.seqlens[e] > 0) continue;
        uint16_t* op = a.out + (size_t)e * a.M * kHeadDimV;
        for (int i = threadIdx.x; i < a.M * (kHeadDimV / 8); i += kThreads)
            *reinterpret_cast<uint4*>(op + 8 * i) = uint4{0u, 0u, 0u, 0u};
        for (int i = threadIdx.x; i < a.M; i += kThreads) a.lse[(size_t)e * a.M + i] = -INFINITY;
    }
}

}  // namespace mla
