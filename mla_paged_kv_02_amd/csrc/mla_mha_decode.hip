// mla_mha_decode.hip - paged grouped-query MHA decode (include/mla_mha.h),
// the contrast case to MLA on the page "MLA 和 MHA 的 Kernel 区别" (section
// "Decode 阶段的 HBM 访问模式": MHA reads a key and a value vector per KV head
// for every cached token).
//
// One workgroup per (sequence, KV head), four waves; wave w owns keys
// 16w..16w+15 of every page and streams that stripe of the head's keys and
// values (4 KB each: 16 rows of 256 bytes, 2 KB apart in the page) through a
// private LDS double buffer, the next page's stripe in flight while the
// current one is used, no barrier in the page loop. The query rows of the
// head's group (at most 16: heads x new tokens) sit in registers.
//
//  * scores S^T = K Q^T: one 16-key x 16-row tile per page, four MFMAs of
//    depth 32; key rows are stored with chunk c of row r at c ^ (r & 15)
//    (a row is exactly one LDS bank period), so a fragment read is
//    conflict-free;
//  * online softmax per row (the lane holds row i16, keys 4g..4g+3): the
//    running maximum rescales the row's sum and accumulators;
//  * O^T += V^T P^T: eight MFMAs of depth 16 per page, each V^T operand one
//    transposing LDS read (value rows swizzled c ^ (r & 7));
//  * the four waves' (m, l, O) are merged through LDS at the end.
#include "../../include/mla_mha.h"

#include <hip/hip_runtime.h>

#include "mla_common.h"

namespace mla {
namespace {

constexpr int kMD = 128;                     // head dim
constexpr int kMRow = kMD * 2;               // 256 bytes per (token, head) row
constexpr int kMStripe = 16 * kMRow;         // 4 KB of keys (or values) per wave per page
constexpr int kMLoads = 8;                   // 4 key + 4 value wave loads per stripe
constexpr int kMTiles = kMD / 16;            // 8 output tiles of 16 dims

constexpr int mwait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kMWaitStripe = mwait_vm_lgkm0(kMLoads);
constexpr int kMWaitAll = mwait_vm_lgkm0(0);

template <int kImm>
__device__ __forceinline__ void mwait() {
    __builtin_amdgcn_s_waitcnt(kImm);
    asm volatile("" ::: "memory");
}

struct MhaArgs {
    const uint16_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const int32_t* block_table;
    const int32_t* seqlens;
    uint16_t* out;
    float* lse;
    int max_blocks, s_q, h_q, h_kv, group_rows, heads_per_group;
    float scale_log2;
    int causal;
};

__device__ __forceinline__ int ld_scalar(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p))[i];
}

__global__ __launch_bounds__(256, 2) void mla_mha_decode_kernel(MhaArgs a) {
    // per wave: two slots of [keys 4 KB][values 4 KB]
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][2][2 * kMStripe];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;
    const int b = blockIdx.x / a.h_kv;
    const int kvh = blockIdx.x - b * a.h_kv;

    // query row i16 of the group: token i16 / heads_per_group, head
    // kvh * heads_per_group + i16 % heads_per_group (rows past the group
    // repeat row 0 and are never stored)
    const int row = i16 < a.group_rows ? i16 : 0;
    const int tok = row / a.heads_per_group;
    const int head = kvh * a.heads_per_group + (row - tok * a.heads_per_group);
    const size_t qrow = ((size_t)b * a.s_q + tok) * a.h_q + head;
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + qrow * kMD + 32 * ks + 8 * g);

    const int nseq = ld_scalar(a.seqlens, b);
    const int npages = (nseq + kPageRows - 1) / kPageRows;
    const int L = a.causal ? min(max(nseq - a.s_q + tok + 1, 0), nseq) : nseq;
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
    const size_t page_bytes = (size_t)kPageRows * a.h_kv * kMRow;

    // Stripe loads: load j (0..3) of keys and of values covers stripe rows
    // 4j .. 4j+3; the lane takes row r = 4j + g, LDS chunk i16, and fetches
    // the logical chunk stored there. Rows past the sequence end read token 0
    // of the page (always valid), with weight zero.
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + g;
        const uint32_t rowoff = (uint32_t)(((wave * 16 + r) * a.h_kv + kvh) * kMRow);
        koff[j] = rowoff + (uint32_t)((i16 ^ (r & 15)) * 16);
        voff[j] = rowoff + (uint32_t)((i16 ^ (r & 7)) * 16);
    }
    const uint32_t row0 = (uint32_t)(kvh * kMRow);
    auto issue = [&](int pn, int slot) {
        const int phys = ld_scalar(bt_row, pn);
        const uint8_t* kp = a.k + (size_t)phys * page_bytes;
        const uint8_t* vp = a.v + (size_t)phys * page_bytes;
        const int valid = nseq - pn * kPageRows - wave * 16;
        const uint32_t dst = lds_addr_of(&lds[wave][slot][0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + g;
            const bool ok = r < valid;
            load_lds16_untracked(kp, ok ? koff[j] : row0 + (uint32_t)((i16 ^ (r & 15)) * 16), dst + j * 1024);
            load_lds16_untracked(vp, ok ? voff[j] : row0 + (uint32_t)((i16 ^ (r & 7)) * 16),
                                 dst + kMStripe + j * 1024);
        }
    };

    int vofs[4];
    {
        const int vr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vofs[i] = vr * kMRow + ((i16 & 1) << 3) + (((i * 2 + ((i16 & 3) >> 1)) ^ (vr & 7)) << 4);
    }

    f32x4 o[kMTiles];
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    if (npages > 0) issue(0, 0);
    for (int pn = 0; pn < npages; ++pn) {
        const int slot = pn & 1;
        if (pn + 1 < npages) {
            issue(pn + 1, slot ^ 1);
            mwait<kMWaitStripe>();
        } else {
            mwait<kMWaitAll>();
        }
        const uint8_t* kb = &lds[wave][slot][0];
        const uint8_t* vb = kb + kMStripe;

        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s = mfma16(lds_read16(kb + i16 * kMRow + (((4 * ks + g) ^ i16) << 4)), qf[ks], s);

        const int key0 = pn * kPageRows + wave * 16 + 4 * g;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] = (key0 + j < L) ? s[j] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        mx = max_over_kgroups(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        f32x4 p;
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(s[j] - m_use);
        l_run = l_run * alpha + (p[0] + p[1] + p[2] + p[3]);
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < kMTiles; ++t) {
            o[t][0] *= alpha; o[t][1] *= alpha; o[t][2] *= alpha; o[t][3] *= alpha;
        }
        const bf16x4 pf = pack_bf16x4(p);
#pragma unroll
        for (int t = 0; t < kMTiles; ++t)
            o[t] = mfma16k16(lds_read_tr(vb + vofs[t & 3] + (t >> 2) * 128), pf, o[t]);
    }
    mwait<kMWaitAll>();

    // ---- merge the four waves through LDS: wave w's tiles at its own slots,
    // m and l after them; wave w then finalises tiles 2w, 2w+1
    const float lsum = sum_over_kgroups(l_run);
    {
        float* wbuf = reinterpret_cast<float*>(&lds[wave][0][0]);
#pragma unroll
        for (int t = 0; t < kMTiles; ++t) *reinterpret_cast<f32x4*>(wbuf + t * 256 + lane * 4) = o[t];
        if (g == 0) {
            wbuf[kMTiles * 256 + i16] = m_run;
            wbuf[kMTiles * 256 + 16 + i16] = lsum;
        }
    }
    __syncthreads();
    float mw[4], lw[4], mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float* ml = reinterpret_cast<const float*>(&lds[w][0][0]) + kMTiles * 256;
        mw[w] = ml[i16];
        lw[w] = ml[16 + i16];
        mmax = fmaxf(mmax, lw[w] > 0.f ? mw[w] : -INFINITY);
    }
    const float mref = mmax == -INFINITY ? 0.f : mmax;
    float ltot = 0.f, sc[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        sc[w] = lw[w] > 0.f ? __builtin_amdgcn_exp2f(mw[w] - mref) : 0.f;
        ltot += lw[w] * sc[w];
    }
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (i16 >= a.group_rows) return;
    const size_t orow = qrow;   // row i16 < group_rows: row == i16
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * wave + tt;
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(&lds[w][0][0]) +
                                                            t * 256 + lane * 4);
            const float f = sc[w] * inv;
            r[0] += f * v[0]; r[1] += f * v[1]; r[2] += f * v[2]; r[3] += f * v[3];
        }
        *reinterpret_cast<bf16x4*>(a.out + orow * kMD + 16 * t + 4 * g) = pack_bf16x4(r);
    }
    if (wave == 0 && g == 0) a.lse[orow] = ltot > 0.f ? (mref + __log2f(ltot)) * kLn2 : -INFINITY;
}

bool aligned_to(const void* p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace
}  // namespace mla

extern "C" mla_status mla_mha_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens,
                                         int batch, int s_q, int h_q, int h_kv, int num_pages, float softmax_scale,
                                         int causal, void* out, float* lse, void* stream) {
    using namespace mla;
    if (!q || !k_cache || !v_cache || !block_table || !seqlens || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || s_q < 1 || h_q < 1 || h_kv < 1 || max_blocks_per_seq < 1 || num_pages < 1)
        return MLA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
    // finite and > 0, the contract shared with mla_decode_fwd (NaN and -0.0 fail it)
    if (!(softmax_scale > 0.f) || softmax_scale > 3.4028235e38f) return MLA_ERR_INVALID_ARG;
    if (h_q % h_kv) return MLA_ERR_INVALID_ARG;
    if ((h_q / h_kv) * s_q > 16) return MLA_ERR_UNSUPPORTED;
    if ((long long)batch * h_kv > 0x7fffffffLL || (long long)max_blocks_per_seq * batch > (1LL << 31) - 1 ||
        (long long)kPageRows * h_kv * kMRow * num_pages > (1LL << 46))
        return MLA_ERR_UNSUPPORTED;
    if (!aligned_to(q, 16) || !aligned_to(k_cache, 16) || !aligned_to(v_cache, 16) || !aligned_to(out, 8) ||
        !aligned_to(lse, 4) || !aligned_to(block_table, 4) || !aligned_to(seqlens, 4))
        return MLA_ERR_MISALIGNED;
    MhaArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint8_t*>(k_cache);
    a.v = static_cast<const uint8_t*>(v_cache);
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.max_blocks = max_blocks_per_seq;
    a.s_q = s_q;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.heads_per_group = h_q / h_kv;
    a.group_rows = a.heads_per_group * s_q;
    a.scale_log2 = softmax_scale * kLog2e;
    a.causal = causal;
    hipLaunchKernelGGL(mla_mha_decode_kernel, dim3((unsigned)(batch * h_kv)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
