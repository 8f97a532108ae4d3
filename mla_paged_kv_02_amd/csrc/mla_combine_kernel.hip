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
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {

namespace {

constexpr int kCombineRows = 4;  // one wave per row

__global__ __launch_bounds__(64 * kCombineRows) void mla_combine_kernel(DecodeArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.y * kCombineRows + (threadIdx.x >> 6);
    if (row >= a.M) return;
    const int32_t* si = a.meta + kMetaHeader + 4 * a.P + 4 * b;
    const int cnt = si[2];
    uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + lane * 8;

    if (cnt <= 1) {
        if (cnt == 0) {  // no pages: empty sequence
            *reinterpret_cast<uint4*>(op) = uint4{0u, 0u, 0u, 0u};
            if (lane == 0) a.lse[(size_t)b * a.M + row] = -INFINITY;
        }
        return;
    }
    const int base = si[0];
    const float* lp = a.part_lse + (size_t)base * a.M + row;

    float m = -INFINITY;
    for (int s = lane; s < cnt; s += 64) m = fmaxf(m, lp[(size_t)s * a.M]);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, wave_xor(m, d));
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float tot = 0.f;
    for (int s = lane; s < cnt; s += 64) tot += __builtin_amdgcn_exp2f((lp[(size_t)s * a.M] - m_use) * kLog2e);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) tot += wave_xor(tot, d);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < cnt; ++s) {
        const float w = __builtin_amdgcn_exp2f((lp[(size_t)s * a.M] - m_use) * kLog2e) * inv;
        const float* pp = a.part_o + ((size_t)(base + s) * a.M + row) * kHeadDimV + lane * 8;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(pp);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(pp + 4);
        acc[0] += w * x0[0]; acc[1] += w * x0[1]; acc[2] += w * x0[2]; acc[3] += w * x0[3];
        acc[4] += w * x1[0]; acc[5] += w * x1[1]; acc[6] += w * x1[2]; acc[7] += w * x1[3];
    }
    bf16x8 v;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (__bf16)acc[k];
    *reinterpret_cast<bf16x8*>(op) = v;
    if (lane == 0) a.lse[(size_t)b * a.M + row] = tot > 0.f ? (m_use + __log2f(tot) * kLn2) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    const dim3 grid(plan.batch, (plan.M + kCombineRows - 1) / kCombineRows);
    hipLaunchKernelGGL(mla_combine_kernel, grid, dim3(64 * kCombineRows), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mla
