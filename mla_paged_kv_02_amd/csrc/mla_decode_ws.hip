// mla_decode_ws.hip - split-KV MLA decode for blocks of 64 query rows with
// separate score and value waves.
//
// Method as in the other decode kernels (page "MLA 和 MHA 的 Kernel 区别",
// section "MLA 的 FlashAttention": stream latent-cache tiles through on-chip
// memory, score the query block against them, one-pass softmax; absorbed
// form). This organisation is for query blocks wide enough that the two
// products and the LDS traffic that feeds them are the work:
//
//  * eight waves, two per SIMD. Score waves 0..3 own query rows 16s..16s+15
//    (query in registers) and compute S^T = K Q^T, the mask and the softmax
//    weights of every half page; value waves 4..7 own output columns
//    128v..128v+127 of all 64 rows (O^T accumulators) and compute
//    O^T += V^T P^T. P crosses over through LDS in exactly the MFMA operand
//    layout, so each V^T fragment (two transposing LDS reads) feeds four row
//    tiles instead of one. While a score wave waits on LDS or runs its exps,
//    the value wave on the same SIMD keeps the matrix core busy;
//  * the cache streams through a ring of four half-page slots (32 keys,
//    36 KB): the value waves load them with 16-byte direct loads, two half
//    pages ahead, while the score waves compute scores; a workgroup barrier
//    starts each step (publishing a slot and the previous weights, freeing
//    the slot the value waves finished) and one splits it in halves, so
//    that 16-byte K reads and transposing V reads never share the LDS. Step
//    c scores half page c and accumulates half page c-1;
//  * softmax reference fixed per row at its first visible maximum plus a
//    margin; a score beyond the headroom raises a flag that every wave reads
//    after the next barrier, and the workgroup redoes the segment with raised
//    references (exact; never triggered by scores of realistic range).
//
// The direct-to-LDS loads are issued untracked by the compiler and every
// wait for them is explicit. The two roles are separate code paths with the
// same barrier sequence, so the score waves' query registers and the value
// waves' accumulators share the register file and two waves fit per SIMD.
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_sched.h"
#include "mla_store_asm.h"

namespace mla {

namespace {

__device__ __forceinline__ int ld_const_ws(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

constexpr int kScoreWaves = 4;
constexpr int kCRows = 32;                      // keys per ring slot (half page)
constexpr int kCBytes = kCRows * kRowBytes;     // 36864
constexpr int kWLoads = 9;                      // a value wave's wave-loads per slot (8 rows)
constexpr int kKS = kHeadDim / 32;              // 18 k-steps of the score product
constexpr int kVTiles = 8;                      // value tiles (16 columns) per value wave
constexpr float kRefMargin = 32.f;
constexpr float kHeadroom = 64.f;

constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
// a slot's loads are followed by one more slot's loads before it is read
constexpr int kWaitSlot = wait_vm_lgkm0(kWLoads);
constexpr int kWaitAll = wait_vm_lgkm0(0);

template <int kImm>
__device__ __forceinline__ void wait_then_fence() {
    __builtin_amdgcn_s_waitcnt(kImm);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

__global__ __launch_bounds__(512) void mla_decode_ws_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kCBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kCBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[kCBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[kCBytes];
    // weights of a half page for the value waves: row tile rt at 1 KB * rt,
    // lane l at 16 l (the B operand of O^T += V^T P^T); two buffers by parity
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][4 * 1024];
    // per row of the block: softmax reference and sum, for the epilogue
    __shared__ float row_ml[64][2];
    // overflow flags by step parity: set during step c in flag[c & 1], read
    // by every wave after the next barrier
    __shared__ int restart_flag[2];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool scorer = wid < kScoreWaves;
    const int sw = wid & 3;   // score wave: row tile; value wave: column block
    const int g = lane >> 4;
    const int i16 = lane & 15;

    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    const int b0 = ld_const_ws(a.meta, kMetaHeader + 4 * p + 0);
    const int n0 = ld_const_ws(a.meta, kMetaHeader + 4 * p + 1);
    const int b_end = ld_const_ws(a.meta, kMetaHeader + 4 * p + 2);
    const int n_end = ld_const_ws(a.meta, kMetaHeader + 4 * p + 3);
    const int32_t* seqinfo = a.meta + kMetaHeader + 4 * a.P;

    if (threadIdx.x == 0) {
        restart_flag[0] = 0;
        restart_flag[1] = 0;
    }
    uint8_t* const slots[4] = {ring0, ring1, ring2, ring3};
    const uint32_t slot_lds[4] = {lds_addr_of(ring0), lds_addr_of(ring1), lds_addr_of(ring2),
                                  lds_addr_of(ring3)};

    // value wave v gathers rows 8v..8v+7 of every half page: LDS 16-byte
    // chunk k of its 9 KB holds row k/72, slot k%72 = logical chunk
    // slot^swz(row); goff[j] is the lane's source offset for load j
    int goff[kWLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
        const int k = j * 64 + lane;
        const int r = k / kRowChunks;
        const int c = k - r * kRowChunks;
        goff[j] = r * kRowBytes + ((c ^ lds_swizzle(r)) << 4);
    }
    // Rows at or past the sequence end read the page's first kilobyte (row
    // 0, always valid): finite data whose softmax weight is zero.
    auto issue_half = [&](const uint8_t* page, int half, int valid, uint32_t dst) {
        const int base = half * kCBytes + sw * 9216;
        const uint32_t d = dst + sw * 9216;
        if (valid >= half * kCRows + sw * 8 + 8) {
            const uint8_t* src = page + base;
#pragma unroll
            for (int j = 0; j < kWLoads; ++j) load_lds16_untracked(src, (uint32_t)goff[j], d + j * 1024);
        } else {
#pragma unroll
            for (int j = 0; j < kWLoads; ++j) {
                const int r = half * kCRows + sw * 8 + (j * 64 + lane) / kRowChunks;
                const uint32_t lo_off = r < valid ? (uint32_t)(base + goff[j]) : (uint32_t)(lane * 16);
                load_lds16_untracked(page, lo_off, d + j * 1024);
            }
        }
    };

    // per-lane LDS offsets inside a slot: K fragment of k-step ks for key row
    // i16 (and 16+i16) at kofs[ks & 1] + 128 (ks >> 1); V^T fragment of value
    // tile dt for key rows vr = 4g + i16/4 (and 16+vr) at vofs[dt & 3] + 128 (dt >> 2)
    int kofs[2], vofs[4];
    {
        const int vr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int i = 0; i < 2; ++i) kofs[i] = i16 * kRowBytes + (((i * 4 + g) ^ lds_swizzle(i16)) << 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vofs[i] = vr * kRowBytes + ((i16 & 1) << 3) + (((i * 2 + ((i16 & 3) >> 1)) ^ lds_swizzle(vr)) << 4);
    }

    // The two roles run the same segment, step and barrier sequence in
    // separate code, so that the score waves' query registers and the value
    // waves' accumulators never live at the same program point.
    auto run = [&](auto role) {
        constexpr bool kScorer = decltype(role)::value;
        const int srow = rb * 64 + sw * 16 + i16;   // score wave's query row
        const bool srow_ok = srow < a.M;
        const int stok = srow_ok ? srow / a.h_q : 0;
        bf16x8 qf[kScorer ? kKS : 1];
        f32x4 o[kScorer ? 1 : 4][kScorer ? 1 : kVTiles];

        int b = b0, n = n0;
        while (b < b_end || (b == b_end && n < n_end)) {
            const int nseq = ld_const_ws(a.seqlens, b);
            const int npages = pages_of(nseq);
            const int hi = (b == b_end) ? n_end : npages;
            if (n >= hi) { ++b; n = 0; continue; }
            const int lo = n;
            const int nch = 2 * (hi - lo);   // half pages of the segment

            const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
            auto page_of_chunk = [&](int c) {
                const int pn = lo + (c < nch ? c : nch - 1) / 2;
                return reinterpret_cast<const uint8_t*>(a.kv) +
                       (size_t)ld_const_ws(bt_row, pn) * kPageBytes;
            };
            auto issue_chunk = [&](int c, const uint8_t* page, uint32_t dst) {
                const int cc = c < nch ? c : nch - 1;
                issue_half(page, cc & 1, nseq - (lo + cc / 2) * kPageRows, dst);
            };

            const int L = a.causal ? min(max(nseq - a.s_q + stok + 1, 0), nseq) : nseq;
            float m_ref = -INFINITY, l_run = 0.f;
            if constexpr (kScorer) {
                const uint16_t* qp =
                    a.q + ((size_t)b * a.M + (srow_ok ? srow : rb * 64)) * kHeadDim + g * 8;
#pragma unroll
                for (int ks = 0; ks < kKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
            }

            bool restart = false;
            do {
                // value waves fill slots 0 and 1; the score waves' query
                // loads are the compiler's own and waited for where used
                const uint8_t* page2 = nullptr;
                if constexpr (!kScorer) {
                    issue_chunk(0, page_of_chunk(0), slot_lds[0]);
                    issue_chunk(1, page_of_chunk(1), slot_lds[1]);
                    page2 = page_of_chunk(2);
                    wait_then_fence<kWaitAll>();
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                        for (int t = 0; t < kVTiles; ++t) o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                } else {
                    l_run = 0.f;
                }
                block_barrier();   // every wave is past the previous use of the ring
                if (restart && wid == 0 && lane == 0) {
                    restart_flag[0] = 0;
                    restart_flag[1] = 0;
                }
                bool skip = false;   // overflow seen: no more weights until the restart

                // Step c, first half: the value waves issue half page c+2
                // into slot (S+2) % 4 (its previous contents, half page c-2,
                // were accumulated in step c-1) while the score waves compute
                // S^T for half page c from slot S = c % 4. Second half: the
                // score waves turn the scores into weights while the value
                // waves accumulate half page c-1 from slot (S+3) % 4. The
                // 16-byte K reads and the transposing V reads stay in
                // separate halves: concurrent transposing reads starve the
                // others in the LDS.
                int c = 0;
                auto step = [&](auto sc) -> bool {
                    constexpr int S = decltype(sc)::value;
                    const uint8_t* page_next = nullptr;
                    if constexpr (!kScorer) {
                        wait_then_fence<kWaitSlot>();   // my part of half page c
                        page_next = page_of_chunk(c + 3);
                    } else {
                        // weights and flags of step c-1 are written
                        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
                        asm volatile("" ::: "memory");
                    }
                    block_barrier();
                    const int flag = restart_flag[(S + 1) & 1];   // raised in step c-1; acted on below
                    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (!kScorer) {
                        issue_chunk(c + 2, page2, slot_lds[(S + 2) % 4]);
                        page2 = page_next;
                    } else if (c < nch) {
                        const uint8_t* cur = slots[S];
                        // ---- S^T = K Q^T, key tiles 0 and 1, two chains each
                        f32x4 sp[2][2];
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                            for (int pp = 0; pp < 2; ++pp) sp[kt][pp] = f32x4{0.f, 0.f, 0.f, 0.f};
                        constexpr int KD = 4;
                        auto k_off = [&](int ks) { return kofs[ks & 1] + (ks >> 1) * 128; };
                        bf16x8 k0[KD], k1[KD];
#pragma unroll
                        for (int d = 0; d < KD; ++d) {
                            k0[d] = lds_read16(cur + k_off(d));
                            k1[d] = lds_read16(cur + 16 * kRowBytes + k_off(d));
                        }
#pragma unroll
                        for (int ks = 0; ks < kKS; ++ks) {
                            sp[0][ks & 1] = mfma16(k0[ks % KD], qf[ks], sp[0][ks & 1]);
                            sp[1][ks & 1] = mfma16(k1[ks % KD], qf[ks], sp[1][ks & 1]);
                            if (ks + KD < kKS) {
                                k0[ks % KD] = lds_read16(cur + k_off(ks + KD));
                                k1[ks % KD] = lds_read16(cur + 16 * kRowBytes + k_off(ks + KD));
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        s0 = sp[0][0];
                        s1 = sp[1][0];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            s0[j] += sp[0][1][j];
                            s1[j] += sp[1][1][j];
                        }
                    }
                    block_barrier();   // the K reads of this step are done
                    if (flag != 0) return false;
                    if constexpr (kScorer) {
                        if (c < nch) {
                            // ---- mask + reference check; lane holds keys
                            // 4g+j of key tile 0 and 16+4g+j of key tile 1
                            const int key0 = (lo + c / 2) * kPageRows + (c & 1) * kCRows + 4 * g;
                            float mx = -INFINITY;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float v0 = (key0 + j < L) ? s0[j] * a.scale_log2 : -INFINITY;
                                const float v1 = (key0 + 16 + j < L) ? s1[j] * a.scale_log2 : -INFINITY;
                                s0[j] = v0;
                                s1[j] = v1;
                                mx = fmaxf(mx, fmaxf(v0, v1));
                            }
                            mx = max_over_kgroups(mx);
                            if (m_ref == -INFINITY) m_ref = mx == -INFINITY ? -INFINITY : mx + kRefMargin;
                            const bool over = mx > m_ref + kHeadroom;
                            if (__ballot(over) != 0) {
                                if (over) m_ref = mx + kRefMargin;
                                if (lane == 0) restart_flag[S & 1] = 1;
                                skip = true;
                            }
                            if (!skip) {
                                const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    s0[j] = __builtin_amdgcn_exp2f(s0[j] - m_use);
                                    s1[j] = __builtin_amdgcn_exp2f(s1[j] - m_use);
                                    l_run += s0[j] + s1[j];
                                }
                                // B = P^T: k-slot j <-> key 4g+j, 4+j <-> key 16+4g+j
                                *reinterpret_cast<bf16x8*>(&pbuf[S & 1][sw * 1024 + lane * 16]) =
                                    cat_bf16x4(pack_bf16x4(s0), pack_bf16x4(s1));
                            }
                        }
                    } else if (c >= 1) {
                        // ---- O^T += V^T P^T for half page c-1: four row tiles
                        // share each V^T fragment (two transposing reads)
                        const uint8_t* cur = slots[(S + 3) % 4];
                        const uint8_t* pb = &pbuf[(S + 1) & 1][lane * 16];
                        bf16x8 pf[4];
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt) pf[rt] = lds_read16(pb + rt * 1024);
                        constexpr int VD = 5;
                        auto v_frag = [&](int t) {
                            const int dt = sw * kVTiles + t;
                            const int off = vofs[dt & 3] + (dt >> 2) * 128;
                            return cat_bf16x4(lds_read_tr(cur + off), lds_read_tr(cur + 16 * kRowBytes + off));
                        };
                        bf16x8 vf[VD];
#pragma unroll
                        for (int d = 0; d < VD; ++d) vf[d] = v_frag(d);
#pragma unroll
                        for (int t = 0; t < kVTiles; ++t) {
#pragma unroll
                            for (int rt = 0; rt < 4; ++rt) o[rt][t] = mfma16(vf[t % VD], pf[rt], o[rt][t]);
                            if (t + VD < kVTiles) vf[t % VD] = v_frag(t + VD);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    ++c;
                    return c <= nch;
                };
                using S0 = std::integral_constant<int, 0>;
                using S1 = std::integral_constant<int, 1>;
                using S2 = std::integral_constant<int, 2>;
                using S3 = std::integral_constant<int, 3>;
                while (step(S0{}) && step(S1{}) && step(S2{}) && step(S3{})) {
                }
                // drain the half pages still in flight; after the barrier
                // every wave sees an overflow raised in the last step too
                wait_then_fence<kWaitAll>();
                block_barrier();
                restart = (restart_flag[0] | restart_flag[1]) != 0;
                if (restart) block_barrier();   // every wave has read the flag before it is cleared
            } while (restart);

            // ---- epilogue: score waves publish (reference, sum) per row and
            // the lse; value waves normalise and store their columns
            const bool full = (lo == 0) && (hi == npages);
            int slotno = 0;
            if (!full) slotno = ld_const_ws(seqinfo, 4 * b + 0) + (p - ld_const_ws(seqinfo, 4 * b + 1));
            if constexpr (kScorer) {
                const float lsum = sum_over_kgroups(l_run);
                if (g == 0) {
                    row_ml[sw * 16 + i16][0] = m_ref;
                    row_ml[sw * 16 + i16][1] = lsum;
                    const float lse_v = lsum > 0.f ? (m_ref + __log2f(lsum)) * kLn2 : -INFINITY;
                    if (srow_ok) {
                        if (full) a.lse[(size_t)b * a.M + srow] = lse_v;
                        else a.part_lse[(size_t)slotno * a.M + srow] = lse_v;
                    }
                }
            }
            block_barrier();
            if constexpr (!kScorer) {
                const int col0 = sw * 128 + 4 * g;   // tile t covers columns col0 + 16 t .. +3
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int row = rb * 64 + rt * 16 + i16;
                    const float lsum = row_ml[rt * 16 + i16][1];
                    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
                    if (row >= a.M) continue;
                    if (full) {
                        uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + col0;
                        bf16x4 v[kVTiles];
#pragma unroll
                        for (int t = 0; t < kVTiles; ++t) {
                            f32x4 x = o[rt][t];
                            x[0] *= inv; x[1] *= inv; x[2] *= inv; x[3] *= inv;
                            v[t] = pack_bf16x4(x);
                        }
                        TileStores<kVTiles>::out(op, v);
                    } else {
                        float* pp = a.part_o + ((size_t)slotno * a.M + row) * kHeadDimV + col0;
                        f32x4 v[kVTiles];
#pragma unroll
                        for (int t = 0; t < kVTiles; ++t) {
                            v[t] = o[rt][t];
                            v[t][0] *= inv; v[t][1] *= inv; v[t][2] *= inv; v[t][3] *= inv;
                        }
                        TileStores<kVTiles>::part(pp, v);
                    }
                }
            }
            block_barrier();   // row_ml and the buffers are free again
            ++b;
            n = 0;
        }
    };
    if (scorer) run(std::true_type{});
    else run(std::false_type{});
}

hipError_t launch_decode_ws(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_ws_kernel, dim3(plan.P * plan.R), dim3(512), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mla
