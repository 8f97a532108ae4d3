// mla_decode_ws.hip - split-KV MLA decode for blocks of 64 query rows with
// separate score and value waves.
//
// Method as in the other decode kernels (page "MLA 和 MHA 的 Kernel 区别",
// section "MLA 的 FlashAttention": stream latent-cache tiles through on-chip
// memory, score the query block against them, one-pass softmax; absorbed
// form). This organisation is for query blocks wide enough that the two
// products and the LDS traffic that feeds them are the work:
//
//  * eight waves, two per SIMD. Score wave s owns key tile s & 1 (keys
//    16(s&1)..+15 of every half page) for the 32 query rows of row tiles
//    2(s>>1) and 2(s>>1)+1 (query in registers): each K fragment it reads
//    from LDS feeds two row tiles. It computes S^T = K Q^T, the mask and the
//    softmax weights of its keys. Value waves 4..7 own output columns
//    128v..128v+127 of all 64 rows (O^T accumulators) and compute
//    O^T += V^T P^T. P crosses over through LDS in exactly the MFMA operand
//    layout, so each V^T fragment (two transposing LDS reads) feeds four row
//    tiles instead of one. While a score wave waits on LDS or runs its exps,
//    the value wave on the same SIMD keeps the matrix core busy;
//  * the cache streams through a ring of four half-page slots (32 keys,
//    36 KB): the value waves load them with 16-byte direct loads, two half
//    pages ahead. Step c scores half page c and accumulates half page c-1;
//    one workgroup barrier per step publishes half page c, the weights of
//    half page c-1 and the overflow flags, and frees the slot the value
//    waves finished;
//  * the softmax reference of each row is fixed at its maximum over the
//    first half page of the segment plus a margin: on that half page the
//    score waves score both key tiles, so the two waves of a row pair take
//    the same value without talking (the visible keys of a row are a prefix
//    of the segment, so a row has no visible key later unless it has one
//    there). A score beyond the headroom raises a flag that every wave reads
//    after the next barrier; the workgroup merges the raised references of
//    the two key tiles and redoes the segment (exact; never triggered by
//    scores of realistic range).
//
// The direct-to-LDS loads are issued untracked by the compiler and every
// wait for them is explicit. The two roles are separate code paths with the
// same barrier sequence, so the score waves' query registers and the value
// waves' accumulators share the register file and two waves fit per SIMD.
#include "mla_common.h"
#include "mla_fused_combine.h"
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

// Workgroup barrier that publishes this wave's LDS writes: they have
// completed (lgkmcnt(0)) before the wave arrives. Loads into LDS in flight
// are not waited for here; their own waits precede the barrier that
// publishes them.
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
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
    // per row of the block: softmax reference, and the sums of the two key
    // tiles, for the epilogue
    __shared__ float row_m[64];
    __shared__ float row_l[2][64];
    // overflow flags by step parity: set during step c in flag[c & 1], read
    // by every wave after the next barrier
    __shared__ int restart_flag[2];
    __shared__ int last_flag;   // this workgroup merges a split sequence

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool scorer = wid < kScoreWaves;
    // score wave sw: key tile sw & 1 of row pair sw >> 1; value wave sw:
    // column block sw (and rows 8 sw..8 sw+7 of every half page it loads)
    const int sw = wid & 3;
    const int g = lane >> 4;
    const int i16 = lane & 15;

    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    // partition record: its range and the length of its first sequence,
    // so that the first segment starts without another dependent load
    const int32_t* part = a.meta + kMetaHeader + kPartInts * p;
    const int b0 = ld_const_ws(part, 0);
    const int n0 = ld_const_ws(part, 1);
    const int b_end = ld_const_ws(part, 2);
    const int n_end = ld_const_ws(part, 3);
    const int len0 = ld_const_ws(part, 4);
    const int32_t* seqinfo = a.meta + kMetaHeader + kPartInts * a.P;

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
    // Load j (of kWLoads) of this value wave's part of a half page. Rows at
    // or past the sequence end read the page's first kilobyte (row 0, always
    // valid): finite data whose softmax weight is zero.
    auto issue_one = [&](const uint8_t* page, int half, int valid, uint32_t dst, int j) {
        const int base = half * kCBytes + sw * 9216;
        const int r = half * kCRows + sw * 8 + (j * 64 + lane) / kRowChunks;
        const uint32_t off = r < valid ? (uint32_t)(base + goff[j]) : (uint32_t)(lane * 16);
        load_lds16_untracked(page, off, dst + sw * 9216 + j * 1024);
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
        // score wave: key tile kt, block rows lrow[r] = 32 rp + 16 r + i16
        constexpr int NR = kScorer ? 2 : 1;
        const int kt = sw & 1;
        const int rp = sw >> 1;
        int lrow[NR], stok[NR];
        bool srow_ok[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lrow[r] = 32 * rp + 16 * r + i16;
            srow_ok[r] = rb * 64 + lrow[r] < a.M;
            stok[r] = srow_ok[r] ? (rb * 64 + lrow[r]) / a.h_q : 0;
        }
        bf16x8 qf[NR][kScorer ? kKS : 1];
        f32x4 o[kScorer ? 1 : 4][kScorer ? 1 : kVTiles];

        int b = b0, n = n0;
        while (b < b_end || (b == b_end && n < n_end)) {
            const int nseq = b == b0 ? len0 : ld_const_ws(a.seqlens, b);
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
            // load j of half page c (past the segment end: the last one again,
            // so that every step issues the same number of loads)
            auto issue_part = [&](int c, const uint8_t* page, uint32_t dst, int j) {
                const int cc = c < nch ? c : nch - 1;
                issue_one(page, cc & 1, nseq - (lo + cc / 2) * kPageRows, dst, j);
            };
            auto issue_chunk = [&](int c, const uint8_t* page, uint32_t dst) {
#pragma unroll
                for (int j = 0; j < kWLoads; ++j) issue_part(c, page, dst, j);
            };

            int L[NR];
            float m_ref[NR], l_run[NR];
            const float inv_scale = 1.f / a.scale_log2;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                L[r] = a.causal ? min(max(nseq - a.s_q + stok[r] + 1, 0), nseq) : nseq;
                m_ref[r] = -INFINITY;
                l_run[r] = 0.f;
            }
            // a segment holding the whole sequence writes the output itself;
            // otherwise its partial goes to slot slot_base + (p - first partition)
            const bool full = (lo == 0) && (hi == npages);
            const int slotno =
                full ? 0 : ld_const_ws(seqinfo, 4 * b + 0) + (p - ld_const_ws(seqinfo, 4 * b + 1));
            if constexpr (kScorer) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const uint16_t* qp = a.q +
                        ((size_t)b * a.M + (srow_ok[r] ? rb * 64 + lrow[r] : rb * 64)) * kHeadDim + g * 8;
#pragma unroll
                    for (int ks = 0; ks < kKS; ++ks) qf[r][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
                }
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
#pragma unroll
                    for (int r = 0; r < NR; ++r) l_run[r] = 0.f;
                }
                block_barrier();   // every wave is past the previous use of the ring
                if (restart && wid == 0 && lane == 0) {
                    restart_flag[0] = 0;
                    restart_flag[1] = 0;
                }
                bool skip = false;   // overflow seen: no more weights until the restart

                // Step c: the value waves issue half page c+2 into slot
                // (S+2) % 4 (its previous contents, half page c-2, were
                // accumulated in step c-1) and accumulate half page c-1 from
                // slot (S+3) % 4, while the score waves turn half page c
                // (slot S = c % 4) into weights.
                int c = 0;
                auto step = [&](auto sc) -> bool {
                    constexpr int S = decltype(sc)::value;
                    const uint8_t* page_next = nullptr;
                    if constexpr (!kScorer) {
                        wait_then_fence<kWaitSlot>();   // my part of half page c
                        page_next = page_of_chunk(c + 3);
                    }
                    block_barrier();   // publishes the weights and flags of step c-1
                    if (restart_flag[(S + 1) & 1] != 0) return false;   // raised in step c-1
                    // value waves: half page c+2 into slot (S+2) % 4, which held
                    // half page c-2 (accumulated in step c-1); spread over the
                    // value products below, so the address unit that takes
                    // the loads never backs the wave up for long
                    const uint8_t* const page_c2 = page2;
                    if constexpr (!kScorer) {
                        page2 = page_next;
                        if (c == 0) issue_chunk(c + 2, page_c2, slot_lds[(S + 2) % 4]);
                    } else if (c < nch) {
                        // ---- S^T = K Q^T for key tile `tile` of half page c,
                        // both row tiles; one K fragment feeds both. Lane
                        // holds keys key0 + j (j < 4) of rows lrow[r], -inf
                        // where masked; lm[r] = the lane's maximum of them.
                        auto score_tile = [&](int tile, f32x4 (&sv)[NR], float (&lm)[NR]) {
                            const uint8_t* kb = slots[S] + tile * 16 * kRowBytes;
                            f32x4 sp[NR][2];
#pragma unroll
                            for (int r = 0; r < NR; ++r)
#pragma unroll
                                for (int pp = 0; pp < 2; ++pp) sp[r][pp] = f32x4{0.f, 0.f, 0.f, 0.f};
                            constexpr int KD = 4;
                            auto k_off = [&](int ks) { return kofs[ks & 1] + (ks >> 1) * 128; };
                            bf16x8 kf[KD];
#pragma unroll
                            for (int d = 0; d < KD; ++d) kf[d] = lds_read16(kb + k_off(d));
#pragma unroll
                            for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
                                for (int r = 0; r < NR; ++r) sp[r][ks & 1] = mfma16(kf[ks % KD], qf[r][ks], sp[r][ks & 1]);
                                if (ks + KD < kKS) kf[ks % KD] = lds_read16(kb + k_off(ks + KD));
                                __builtin_amdgcn_sched_barrier(0);
                            }
                            const int key0 = (lo + c / 2) * kPageRows + (c & 1) * kCRows + tile * 16 + 4 * g;
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                float m = -INFINITY;
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const float v = (key0 + j < L[r]) ? sp[r][0][j] + sp[r][1][j] : -INFINITY;
                                    sv[r][j] = v;
                                    m = fmaxf(m, v);
                                }
                                lm[r] = m;
                            }
                        };
                        // row maximum in the log2 domain (scale > 0: the
                        // maximum commutes with it)
                        auto row_max = [&](float m) { return max_over_kgroups(m) * a.scale_log2; };
                        f32x4 sv[NR];
                        float lm[NR];
                        score_tile(kt, sv, lm);
                        if (c == 0) {
                            // the reference comes from both key tiles
                            f32x4 so[NR];
                            float lo2[NR];
                            score_tile(kt ^ 1, so, lo2);
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                const float mx = row_max(fmaxf(lm[r], lo2[r]));
                                if (m_ref[r] == -INFINITY) m_ref[r] = mx == -INFINITY ? -INFINITY : mx + kRefMargin;
                            }
                        }
                        // overflow: a score above the reference plus the
                        // headroom, tested on raw scores against the limit
                        // divided back by the scale (a bound, not a rounding
                        // decision: weights stay below 2^64 either way)
                        bool over = false;
#pragma unroll
                        for (int r = 0; r < NR; ++r) over = over || (lm[r] > (m_ref[r] + kHeadroom) * inv_scale);
                        if (__ballot(over) != 0) {
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                const float mx = row_max(lm[r]);
                                if (mx > m_ref[r] + kHeadroom) m_ref[r] = mx + kRefMargin;
                            }
                            if (lane == 0) restart_flag[S & 1] = 1;
                            skip = true;
                        }
                        if (!skip) {
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                const float neg_m = (m_ref[r] == -INFINITY) ? 0.f : -m_ref[r];
                                f32x4 pw;
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    // masked scores are -inf: weight 0
                                    pw[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r][j], a.scale_log2, neg_m));
                                    l_run[r] += pw[j];
                                }
                                // B = P^T of row tile 2 rp + r: k-slot 4 kt + j <-> key 16 kt + 4 g + j
                                *reinterpret_cast<bf16x4*>(&pbuf[S & 1][(2 * rp + r) * 1024 + lane * 16 + kt * 8]) =
                                    pack_bf16x4(pw);
                            }
                        }
                    }
                    if (!kScorer && c >= 1) {
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
                            issue_part(c + 2, page_c2, slot_lds[(S + 2) % 4], t);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        static_assert(kVTiles + 1 == kWLoads, "one load per value tile and one after");
                        issue_part(c + 2, page_c2, slot_lds[(S + 2) % 4], kVTiles);
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
                if (restart) {
                    // the two key tiles of a row pair raised their references
                    // on their own scores: both take the larger one
                    if constexpr (kScorer) {
                        if (g == 0 && kt == 1)
#pragma unroll
                            for (int r = 0; r < NR; ++r) row_m[lrow[r]] = m_ref[r];
                    }
                    block_barrier();
                    if constexpr (kScorer) {
                        if (kt == 0) {
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                m_ref[r] = fmaxf(m_ref[r], row_m[lrow[r]]);
                                if (g == 0) row_m[lrow[r]] = m_ref[r];
                            }
                        }
                    }
                    block_barrier();
                    if constexpr (kScorer) {
#pragma unroll
                        for (int r = 0; r < NR; ++r) m_ref[r] = row_m[lrow[r]];
                    }
                    block_barrier();   // every wave has read the flags and row_m
                }
            } while (restart);

            // ---- epilogue: score waves publish (reference, sum) per row and
            // the lse; value waves normalise and store their columns
            if constexpr (kScorer) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float lsum = sum_over_kgroups(l_run[r]);
                    if (g == 0) {
                        row_l[kt][lrow[r]] = lsum;
                        if (kt == 0) row_m[lrow[r]] = m_ref[r];
                    }
                }
            }
            block_barrier();
            if constexpr (!kScorer) {
                const int col0 = sw * 128 + 4 * g;   // tile t covers columns col0 + 16 t .. +3
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int row = rb * 64 + rt * 16 + i16;
                    const float lsum = row_l[0][rt * 16 + i16] + row_l[1][rt * 16 + i16];
                    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
                    if (row >= a.M) continue;
                    if (sw == 0 && g == 0) {
                        const float mr = row_m[rt * 16 + i16];
                        const float lse_v = lsum > 0.f ? (mr + __log2f(lsum)) * kLn2 : -INFINITY;
                        if (full) a.lse[(size_t)b * a.M + row] = lse_v;
                        else   // device-coherent, as the partial tiles
                            __hip_atomic_store(&a.part_lse[(size_t)row * a.lse_stride + slotno], lse_v,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
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
                        TileStores<kVTiles>::part(pp, v, a.counters != nullptr);
                    }
                }
            }
            block_barrier();   // row_m, row_l and the buffers are free again
            if (!full && a.counters) count_partial_and_combine<512, 64>(a, b, rb, &last_flag);
            ++b;
            n = 0;
        }
        if (a.counters) write_empty_sequences<512>(a);
    };
    if (scorer) run(std::true_type{});
    else run(std::false_type{});
}

hipError_t launch_decode_ws(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_ws_kernel, dim3(plan.P * plan.R), dim3(512), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mla
