// mla_combine_kernel.hip - merges the partials of sequences whose pages were
// cut between partitions, and writes the result of empty sequences.
//
// Partial s of a row holds o_s (softmax-weighted value sum over its pages,
// normalised within them) and lse_s. The whole-sequence result is
// lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s: an exact
// rewrite of one softmax over all keys (softmax over a union of disjoint key
// sets). Splitting the key range this way is what lets decode with a small
// batch use the whole GPU (long-text inference page, "Unlocking GPU
// Potential ...").
//
// The work is pure streaming of FP32 partial rows (2 KB per row and
// partial). An item is one half row (256 columns, 16 bytes per lane) of one
// sequence. With few partials per sequence a block of four waves takes four
// items, one wave each; with many (long sequences on a small batch) the 4 or
// 16 waves of a block share one item's partials and sum them through LDS, so
// that each wave has only a round trip or two of loads to wait for (giving
// a wave four items, their loads all issued before the first reduction,
// was slower: 26.5 vs 19.6 us on 132 sequences of 256 rows, 8.8 vs 5.5 us
// on 64 sequences of 16 rows, with fewer waves in flight).
//
// The grid covers the sequences that can need it. With at least as many
// partition boundaries as sequences, one group of blocks per sequence
// (unsplit sequences exit at once). With fewer boundaries than sequences
// (many sequences, few partitions), one group per boundary p = 1..P-1: a
// sequence is split exactly when a boundary falls inside its pages, and the
// group of boundary p merges sequence b when partition p starts inside b
// and b's first partition is p - 1 (its first cut), so each split sequence
// is merged once and unsplit ones cost nothing; a few blocks after those
// groups write the results of empty sequences.
#include "mla_common.h"
#include "mla_fused_combine.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {

namespace {

constexpr int kCombineUnroll = 8;   // partial rows in flight per wave

__device__ __forceinline__ float ld_const_f32(const float* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) float*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

template <int kWPI>   // waves per item
__global__ __launch_bounds__(64 * (kWPI > 4 ? kWPI : 4)) void mla_combine_kernel(DecodeArgs a, int by_boundary) {
    constexpr int kWaves = kWPI > 4 ? kWPI : 4;
    constexpr int kItems = kWaves / kWPI;
    __shared__ f32x4 red[kWPI > 1 ? kWaves : 1][64];
    // a plan built for other arguments: the decode kernel has written NaN
    // into every lse entry and nothing else; neither does this kernel
    if (!plan_header_matches(ld_plan_word(a.meta, 0), ld_plan_word(a.meta, 1), ld_plan_word(a.meta, 2),
                             ld_plan_word(a.meta, 3), ld_plan_word(a.meta, 8), a.batch, a.P, a.cseg, a.R))
        return;
    // one-dimensional grid, the blocks of a sequence (or boundary) consecutive
    const int per_b = __builtin_amdgcn_readfirstlane((2 * a.M + kItems - 1) / kItems);
    const int slot = blockIdx.x / per_b;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int item = (blockIdx.x - slot * per_b) * kItems + w / kWPI;   // row * 2 + half
    const int sub = w % kWPI;
    const int row = item >> 1;
    const int half = item & 1;
    const bool live = row < a.M;

    // sequence records {slot base, first partition, partition count, cost start}
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const __attribute__((address_space(4))) i32x4* seqrec = reinterpret_cast<const __attribute__((address_space(4))) i32x4*>(
        reinterpret_cast<uintptr_t>(a.meta + kMetaHeader + kPartInts * a.P));
    int b = slot;
    if (by_boundary) {
        const int nbound = a.P - 1;
        if (slot >= nbound) {
            // empty sequences: wave w of block k writes sequence 4k + w
            const int e = 4 * (blockIdx.x - nbound * per_b) + w;
            if (w >= 4 || e >= a.batch || seqrec[e].z != 0) return;
            uint16_t* eo = a.out + (size_t)e * a.M * kHeadDimV + lane * 8;
            for (int r = 0; r < a.M; ++r) *reinterpret_cast<uint4*>(eo + (size_t)r * kHeadDimV) = uint4{0u, 0u, 0u, 0u};
            for (int r = lane; r < a.M; r += 64) a.lse[(size_t)e * a.M + r] = -INFINITY;
            return;
        }
        // partition p = slot + 1 starts at (b, n): a cut inside sequence b
        // when n > 0; this group merges b if it is b's first cut
        const int p = slot + 1;
        b = ld_plan_word(a.meta, kMetaHeader + kPartInts * p + 0);
        const int n = ld_plan_word(a.meta, kMetaHeader + kPartInts * p + 1);
        if (n == 0 || b >= a.batch || seqrec[b].y != p - 1) return;
    }
    const i32x4 si = seqrec[b];
    const int cnt = si.z;
    if (cnt == 1) return;   // the decode kernel wrote this sequence's result
    const int col = half * 256 + lane * 4;
    uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + col;
    if (cnt == 0) {   // no pages: empty sequence
        if (live && sub == 0) {
            *reinterpret_cast<uint2*>(op) = uint2{0u, 0u};
            if (half == 0 && lane == 0) a.lse[(size_t)b * a.M + row] = -INFINITY;
        }
        return;
    }
    const int base = si.x;
    const int rr = live ? row : 0;
    const float* lp = a.part_lse + (size_t)rr * a.lse_stride + base;   // lp[s]: partial s

    const float* pbase = a.part_o + ((size_t)base * a.M + rr) * kHeadDimV + col;
    const size_t pstride = (size_t)a.M * kHeadDimV;
    // this wave's partials are s = sub, sub + kWPI, ...; the first group is
    // loaded before the lse reduction so that the two latencies overlap
    f32x4 x[kCombineUnroll];
    float wt[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
        const int su = sub + u * kWPI;
        if (su < cnt) {
            x[u] = *reinterpret_cast<const f32x4*>(pbase + (size_t)su * pstride);
            wt[u] = ld_const_f32(lp, su);
        }
    }

    // combined lse (every wave of the item computes it). A wave that owns
    // all of an item's partials (one wave per item, at most one group of
    // them) already holds every lse_s in wt[]: no loads, no lane exchange.
    // Otherwise the lanes load the lse_s a few apiece and reduce.
    float m = -INFINITY, tot = 0.f, m_use = 0.f;
    if (kWPI == 1 && cnt <= kCombineUnroll) {
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u)
            if (u < cnt) m = fmaxf(m, wt[u]);
        m_use = (m == -INFINITY) ? 0.f : m;
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u)
            if (u < cnt) tot += __builtin_amdgcn_exp2f((wt[u] - m_use) * kLog2e);
    } else {
        for (int s = lane; s < cnt; s += 64) m = fmaxf(m, lp[s]);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, wave_xor(m, d));
        m_use = (m == -INFINITY) ? 0.f : m;
        for (int s = lane; s < cnt; s += 64) tot += __builtin_amdgcn_exp2f((lp[s] - m_use) * kLog2e);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) tot += wave_xor(tot, d);
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto accumulate = [&](const f32x4& xv, float lse_s) {
        const float wu = __builtin_amdgcn_exp2f((lse_s - m_use) * kLog2e);
        acc[0] += wu * xv[0]; acc[1] += wu * xv[1]; acc[2] += wu * xv[2]; acc[3] += wu * xv[3];
    };
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u)
        if (sub + u * kWPI < cnt) accumulate(x[u], wt[u]);
    // further groups, a partly filled last one included: one round trip each
    for (int s = sub + kCombineUnroll * kWPI; s < cnt; s += kCombineUnroll * kWPI) {
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const int su = s + u * kWPI;
            if (su < cnt) {
                x[u] = *reinterpret_cast<const f32x4*>(pbase + (size_t)su * pstride);
                wt[u] = ld_const_f32(lp, su);
            }
        }
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u)
            if (s + u * kWPI < cnt) accumulate(x[u], wt[u]);
    }
    if constexpr (kWPI > 1) {
        red[w][lane] = acc;
        __syncthreads();
        if (sub != 0) return;
#pragma unroll
        for (int k = 1; k < kWPI; ++k) {
            const f32x4 y = red[w + k][lane];
            acc[0] += y[0]; acc[1] += y[1]; acc[2] += y[2]; acc[3] += y[3];
        }
    }
    if (!live) return;
    acc[0] *= inv; acc[1] *= inv; acc[2] *= inv; acc[3] *= inv;
    *reinterpret_cast<bf16x4*>(op) = pack_bf16x4(acc);
    if (half == 0 && lane == 0)
        a.lse[(size_t)b * a.M + row] = tot > 0.f ? m_use + __log2f(tot) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    // Partials per split sequence average about P / batch + 1; the waves
    // sharing an item grow with that figure, so that a wave's share of an
    // item (its partials s = sub, sub + waves, ...) usually fits in the one
    // group of loads issued before the lse reduction.
    // Consecutive blocks go to different XCDs, and a sequence's blocks are
    // consecutive, so a long sequence's work spreads over all of them.
    // With fewer partition boundaries than sequences the grid follows the
    // boundaries (at most P - 1 sequences can be split), plus one block per
    // four sequences for the empty ones.
    const int per_seq = plan.P / plan.batch;
    const int items = 2 * plan.M;
    const int by_boundary = plan.P - 1 < plan.batch ? 1 : 0;
    const unsigned nb = (unsigned)(by_boundary ? plan.P - 1 : plan.batch);
    const unsigned extra = by_boundary ? (unsigned)((plan.batch + 3) / 4) : 0u;
    if (per_seq >= 4 * kCombineUnroll) {
        hipLaunchKernelGGL(mla_combine_kernel<16>, dim3(nb * items + extra), dim3(64 * 16), 0, stream, args,
                           by_boundary);
    } else if (per_seq >= kCombineUnroll) {
        hipLaunchKernelGGL(mla_combine_kernel<4>, dim3(nb * items + extra), dim3(64 * 4), 0, stream, args,
                           by_boundary);
    } else {
        hipLaunchKernelGGL(mla_combine_kernel<1>, dim3(nb * ((items + 3) / 4) + extra), dim3(64 * 4), 0, stream,
                           args, by_boundary);
    }
    return hipGetLastError();
}

}  // namespace mla
