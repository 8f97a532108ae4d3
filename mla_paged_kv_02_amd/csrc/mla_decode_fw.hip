// mla_decode_fw.hip - split-KV MLA decode for 128-row query blocks, every
// wave scoring and accumulating its own rows.
//
// Method (page "MLA 和 MHA 的 Kernel 区别", section "MLA 的 FlashAttention":
// stream latent-cache tiles through on-chip memory, score the query block
// against them, one-pass softmax; absorbed form, so keys are the cache rows
// and values their first 512 entries). The organisation lets each page cross
// into a compute unit once per 128 rows:
//
//  * four waves, one per SIMD; wave w owns row tiles 2w, 2w + 1 (16 rows
//    each) of the block: their query in VGPRs and their output accumulators
//    O^T (all 512 columns, FP32) in the 256 AGPRs;
//  * per 32-key half page a wave computes S^T = K Q^T over both 16-key tiles
//    (each K fragment feeds both row tiles), the mask and the softmax
//    weights, then O^T += V^T P^T with its own weights as the B operand: the
//    layout the score product leaves a lane's weights in is exactly the
//    operand layout of the value product when the value operand reads keys
//    4g..4g+3 and 16+4g..16+4g+3 (two transposing reads), so P never leaves
//    the registers and the waves never exchange data;
//  * the pages stream through a ring of four half-page slots (36 KB each)
//    with 16-byte direct loads; a half page is scored and accumulated in the
//    same step, so three are in flight while one is used. The stream is the
//    partition's whole page list: the last steps of a segment already load
//    the next segment's first half pages;
//  * each row's softmax reference is fixed at its maximum over the
//    segment's first half page plus a margin; a score beyond the headroom
//    sets a flag that every wave reads after the next barrier, and the
//    workgroup redoes the segment from its first page with the raised
//    references (exact; never triggered by scores of realistic range).
//
// Measured limit: every wave reads the whole half page from LDS (68 KB per
// step), and with one wave per SIMD too few of those reads are in flight to
// cover their latency; at 128 heads this organisation is 13-15% slower than
// two 64-row score/value blocks, so plans use it only when forced.
//
// The direct-to-LDS loads are issued untracked by the compiler and every
// wait for them is explicit; the query loads are the compiler's own (it
// waits for everything in flight before their first use, once per segment).
#include "mla_common.h"
#include "mla_fused_combine.h"
#include "mla_internal.h"
#include "mla_sched.h"
#include "mla_store_asm.h"

namespace mla {

namespace {

__device__ __forceinline__ int ld_const_fw(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

constexpr int kCRows = 32;                      // keys per ring slot (half page)
constexpr int kCBytes = kCRows * kRowBytes;     // 36864
// A slot holds its 32 cache rows in two regions: the latent part (the first
// 512 entries, 1 KB) of row r at r * 1 KB, the rope part (128 B) of row r at
// kRopeOff + r * 128. 16-byte chunk c of a row sits at position c ^ swz(r)
// of its region (swz_main / swz_rope), so that every LDS read below touches
// 128 distinct bytes per group of lanes served together: the eight rows of a
// K fragment group, and the four rows times two chunks of a transposing V
// read group.
constexpr int kMainRow = 1024;
constexpr int kRopeRow = 128;
constexpr int kRopeOff = kCRows * kMainRow;     // 32768
static_assert(kRopeOff + kCRows * kRopeRow == kCBytes, "slot regions");
__device__ __forceinline__ constexpr int swz_main(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ constexpr int swz_rope(int r) { return r & 7; }
constexpr int kWLoads = 9;                      // a wave's wave-loads per slot (8 rows)
constexpr int kKS = kHeadDim / 32;              // 18 k-steps of the score product
constexpr int kDT = kHeadDimV / 16;             // 32 value tiles of 16 columns
constexpr float kRefMargin = 32.f;
constexpr float kHeadroom = 64.f;

constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

template <int kImm>
__device__ __forceinline__ void wait_then_fence() {
    __builtin_amdgcn_s_waitcnt(kImm);
    asm volatile("" ::: "memory");
}

// The score product accumulates in VGPRs: the value accumulators of a wave's
// 32 rows (all 512 columns, FP32) take every AGPR, and the compiler, which
// keeps every MFMA accumulator it selects in AGPRs here, would spill. It
// inserts no wait states around inline asm: accumulating into the same
// registers needs none, and after a chain's last product score_chain_done
// gives 24 before the results are read (an 8-pass product's result needs
// at most 12).
__device__ __forceinline__ void mfma16_v_first(f32x4& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_v_acc(f32x4& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_chain_done(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Workgroup barrier that publishes this wave's LDS writes (lgkmcnt(0)).
// Loads into LDS in flight are not waited for here.
__device__ __forceinline__ void block_barrier_fw() {
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace

template <int kWRT>   // row tiles per wave
__global__ __launch_bounds__(256) void mla_decode_fw_kernel(DecodeArgs a) {
    // the register budget (query 144 VGPRs, accumulators 256 AGPRs) is set
    // for two row tiles per wave
    static_assert(kWRT == 2, "128-row blocks only");
    constexpr int kRows = 64 * kWRT;
    __shared__ __attribute__((aligned(16))) uint8_t ring[4 * kCBytes];
    // overflow flags by step parity: set during step c in flag[c & 1], read
    // by every wave after the next barrier
    __shared__ int restart_flag[2];

    if (!plan_matches_or_poison<256>(a)) return;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;

    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    // partition record: its range and the length of its first sequence
    const int32_t* part = a.meta + kMetaHeader + kPartInts * p;
    const int b0 = ld_const_fw(part, 0);
    const int n0 = ld_const_fw(part, 1);
    const int b_end = ld_const_fw(part, 2);
    const int n_end = ld_const_fw(part, 3);
    const int len0 = ld_const_fw(part, 4);
    const int32_t* seqinfo = a.meta + kMetaHeader + kPartInts * a.P;

    if (threadIdx.x == 0) {
        restart_flag[0] = 0;
        restart_flag[1] = 0;
    }
    const uint32_t ring_lds = lds_addr_of(ring);

    // The partition's segments: (sequence, page range) in order, each
    // holding at least one page; b < 0 past the partition's end.
    struct Seg {
        int b, lo, hi, nseq;
    };
    auto find_seg = [&](int b, int n) {
        while (b < b_end || (b == b_end && n < n_end)) {
            const int nseq = b == b0 ? len0 : ld_const_fw(a.seqlens, b);
            const int hi = (b == b_end) ? n_end : pages_of(nseq);
            if (n < hi) return Seg{b, n, hi, nseq};
            ++b;
            n = 0;
        }
        return Seg{-1, 0, 0, 0};
    };

    // ---- the fetch stream: the partition's half pages in order. fseg/fc
    // name the next half page to take; fpage is its page. Wave w gathers
    // rows 8w..8w+7 of every half page: load j < 8 the latent part of row
    // 8w + j (lane l: its chunk l ^ swz_main(j)), load 8 their rope parts
    // (lane l: row 8w + l/8, chunk (l % 8) ^ (l / 8)).
    Seg fseg = find_seg(b0, n0);
    int fc = 0;
    auto fpage_of = [&]() {
        const int32_t* bt_row = a.block_table + (size_t)fseg.b * a.max_blocks;
        return reinterpret_cast<const uint8_t*>(a.kv) + (size_t)ld_const_fw(bt_row, fseg.lo + fc / 2) * kPageBytes;
    };
    const uint8_t* fpage = fseg.b >= 0 ? fpage_of() : nullptr;
    const uint8_t* t_src = nullptr;
    int t_half = 0, t_rows = 0;
    auto take = [&]() -> bool {
        if (fseg.b < 0) return false;
        t_src = fpage;
        t_half = fc & 1;
        t_rows = fseg.nseq - (fseg.lo + fc / 2) * kPageRows;
        if (++fc == 2 * (fseg.hi - fseg.lo)) {
            fseg = find_seg(fseg.b + 1, 0);
            fc = 0;
        }
        if (fseg.b >= 0 && (fc & 1) == 0) fpage = fpage_of();
        return true;
    };
    // load j of the taken half page into the slot at `dst`. Rows at or past
    // the sequence end read row 0 of the page (always valid): finite data
    // whose softmax weight is zero.
    auto issue_one = [&](uint32_t dst, int j) {
        if (j < 8) {
            const int prow = t_half * kCRows + w * 8 + j;   // wave-uniform
            const uint8_t* src = t_src + (prow < t_rows ? prow : 0) * kRowBytes;
            load_lds16_untracked(src, (uint32_t)((lane ^ swz_main(j)) << 4), dst + (w * 8 + j) * kMainRow);
        } else {
            const int prow = t_half * kCRows + w * 8 + (lane >> 3);
            const int srow = prow < t_rows ? prow : 0;
            const uint32_t off = (uint32_t)(srow * kRowBytes + kMainRow + (((lane & 7) ^ (lane >> 3)) << 4));
            load_lds16_untracked(t_src, off, dst + kRopeOff + w * 8 * kRopeRow);
        }
    };
    auto issue_all = [&](uint32_t dst) {
#pragma unroll
        for (int j = 0; j < kWLoads; ++j) issue_one(dst, j);
    };
    // half pages in flight beyond the one being waited for: 0, 1 or 2
    int ahead = 0;
    auto fill = [&](int soff) {
        ahead = 0;
        if (take()) issue_all(ring_lds + soff * kCBytes);
        if (take()) {
            issue_all(ring_lds + ((soff + 1) & 3) * kCBytes);
            ++ahead;
        }
        if (take()) {
            issue_all(ring_lds + ((soff + 2) & 3) * kCBytes);
            ++ahead;
        }
    };

    // per-lane LDS offsets inside a slot, key row i16 of key tile t: K
    // fragment of k-step ks < 16 at kofs[ks & 1] + 128 (ks >> 1) + 16 KB t,
    // of k-step 16 + e at kofs_r[e] + 2 KB t; V^T fragment of value tile dt
    // for key rows vr = 4g + i16/4 (and 16 + vr) at vofs[dt & 3] + 128 (dt >> 2)
    int kofs[2], kofs_r[2], vofs[4];
    {
        const int vr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            kofs[i] = i16 * kMainRow + (((i * 4 + g) ^ swz_main(i16)) << 4);
            kofs_r[i] = kRopeOff + i16 * kRopeRow + (((i * 4 + g) ^ swz_rope(i16)) << 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vofs[i] = vr * kMainRow + ((i16 & 1) << 3) + (((i * 2 + ((i16 & 3) >> 1)) ^ swz_main(vr)) << 4);
    }

    // this wave's rows: block row 16 (kWRT w + r) + i16
    int stok[kWRT];
    bool srow_ok[kWRT];
#pragma unroll
    for (int r = 0; r < kWRT; ++r) {
        const int row = rb * kRows + 16 * (kWRT * w + r) + i16;
        srow_ok[r] = row < a.M;
        stok[r] = srow_ok[r] ? row / a.h_q : 0;
    }
    bf16x8 qf[kWRT][kKS];
    f32x4 o[kWRT][kDT];

    fill(0);
    int soff = 0;   // ring slot of the segment's first half page (0 or 2)
    Seg seg = find_seg(b0, n0);
    // per row: the softmax reference, kept when a segment is redone
    float m_ref[kWRT];
    bool redo = false;
    while (seg.b >= 0) {
        const int b = seg.b, lo = seg.lo, hi = seg.hi, nseq = seg.nseq;
        const int nch = 2 * (hi - lo);   // half pages of the segment
#pragma unroll
        for (int r = 0; r < kWRT; ++r) {
            // rows past M read the block's first row (always a row of the sequence)
            const int row = srow_ok[r] ? rb * kRows + 16 * (kWRT * w + r) + i16 : rb * kRows;
            const uint16_t* qp = a.q + ((size_t)b * a.M + row) * kHeadDim + g * 8;
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) qf[r][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
        }
        // The query has landed before the step loop starts, so the compiler
        // places no wait of its own inside the loop (its waits would count
        // only the query loads and stall on the cache loads in flight).
        // Loads complete in order: this also waits for the half pages
        // already in flight for this segment.
        wait_then_fence<wait_vm_lgkm0(0)>();
        int L[kWRT];
        float l_run[kWRT];
#pragma unroll
        for (int r = 0; r < kWRT; ++r) {
            L[r] = a.causal ? min(max(nseq - a.s_q + stok[r] + 1, 0), nseq) : nseq;
            if (!redo) m_ref[r] = -INFINITY;
            l_run[r] = 0.f;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) o[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        {
            bool skip = false;   // overflow seen: no more weights until the restart
            int c = 0;
            // Step c: wait for my part of half page c, barrier (every wave's
            // part visible; every wave done with half page c-1, whose slot
            // then takes the stream's next half page), then score and
            // accumulate half page c.
            auto step = [&](auto sc) -> bool {
                constexpr int S = decltype(sc)::value;
                if (ahead == 2) wait_then_fence<wait_vm_lgkm0(2 * kWLoads)>();
                else if (ahead == 1) wait_then_fence<wait_vm_lgkm0(kWLoads)>();
                else wait_then_fence<wait_vm_lgkm0(0)>();
                block_barrier_fw();
                if (restart_flag[(S + 1) & 1] != 0) return false;   // raised in step c-1
                const uint8_t* cur = ring + ((S + soff) & 3) * kCBytes;
                // the stream's next half page into the slot of half page c-1
                const bool issue_now = take();
                const uint32_t dst = ring_lds + ((S + soff + 3) & 3) * kCBytes;

                // ---- S^T = K Q^T for both key tiles of half page c, every row
                // tile; lane holds keys 16 t + 4 g + j of row i16 in sp[r][t][j]
                f32x4 sp[kWRT][2];
                {
                    constexpr int KD = 4;   // K fragments in flight (both tiles of two k-steps)
                    auto k_frag = [&](int i) {   // i = 2 ks + tile
                        const int ks = i >> 1, t = i & 1;
                        return ks < 16 ? lds_read16(cur + t * 16 * kMainRow + kofs[ks & 1] + (ks >> 1) * 128)
                                       : lds_read16(cur + t * 16 * kRopeRow + kofs_r[ks - 16]);
                    };
                    bf16x8 kf[KD];
#pragma unroll
                    for (int d = 0; d < KD; ++d) kf[d] = k_frag(d);
#pragma unroll
                    for (int i = 0; i < 2 * kKS; ++i) {
#pragma unroll
                        for (int r = 0; r < kWRT; ++r) {
                            if (i < 2) mfma16_v_first(sp[r][i & 1], kf[i % KD], qf[r][i >> 1]);
                            else mfma16_v_acc(sp[r][i & 1], kf[i % KD], qf[r][i >> 1]);
                        }
                        if (i + KD < 2 * kKS) kf[i % KD] = k_frag(i + KD);
                        // the stream's loads, spread over the products
                        if (issue_now && (i & 3) == 3 && (i >> 2) < kWLoads) issue_one(dst, i >> 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    score_chain_done(sp[0][0], sp[0][1], sp[kWRT - 1][0], sp[kWRT - 1][1]);
                }
                // ---- mask, reference, overflow check, weights (log2 domain)
                const int kbase = (lo + c / 2) * kPageRows + (c & 1) * kCRows + 4 * g;
                float lm[kWRT];
#pragma unroll
                for (int r = 0; r < kWRT; ++r) {
                    float m = -INFINITY;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float v = (kbase + 16 * t + j < L[r]) ? sp[r][t][j] : -INFINITY;
                            sp[r][t][j] = v;
                            m = fmaxf(m, v);
                        }
                    lm[r] = m;
                }
                if (c == 0) {
                    // the reference: the first half page's maximum plus a margin
#pragma unroll
                    for (int r = 0; r < kWRT; ++r) {
                        const float mx = max_over_kgroups(lm[r]) * a.scale_log2;
                        if (m_ref[r] == -INFINITY) m_ref[r] = mx == -INFINITY ? -INFINITY : mx + kRefMargin;
                    }
                }
                // overflow: a scaled score above the reference plus the
                // headroom. The lane's maximum times the scale is the maximum of
                // its scaled scores (scale > 0), and the row maximum is at least
                // the lane's, so a lane that reports overflow always raises its
                // row's reference: every restart strictly raises some reference
                // to a score of the segment plus the margin, and the restarts end.
                bool over = false;
#pragma unroll
                for (int r = 0; r < kWRT; ++r) over = over || (lm[r] * a.scale_log2 > m_ref[r] + kHeadroom);
                if (__ballot(over) != 0) {
#pragma unroll
                    for (int r = 0; r < kWRT; ++r) {
                        const float mx = max_over_kgroups(lm[r]) * a.scale_log2;
                        if (mx > m_ref[r] + kHeadroom) m_ref[r] = mx + kRefMargin;
                    }
                    if (lane == 0) restart_flag[S & 1] = 1;
                    skip = true;
                }
                if (!skip) {
                    // P^T of row tile r: k-slot 8 g + 4 t + j <-> key 16 t + 4 g + j
                    bf16x8 pt[kWRT];
#pragma unroll
                    for (int r = 0; r < kWRT; ++r) {
                        const float neg_m = (m_ref[r] == -INFINITY) ? 0.f : -m_ref[r];
                        f32x4 pw[2];
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                // masked scores are -inf: weight 0
                                pw[t][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[r][t][j], a.scale_log2, neg_m));
                                l_run[r] += pw[t][j];
                            }
                        pt[r] = cat_bf16x4(pack_bf16x4(pw[0]), pack_bf16x4(pw[1]));
                    }
                    // ---- O^T += V^T P^T: each V^T fragment (two transposing
                    // reads: keys 4g..4g+3 and 16+4g..16+4g+3) feeds every row tile
                    constexpr int VD = 4;
                    auto v_frag = [&](int dt) {
                        const int off = vofs[dt & 3] + (dt >> 2) * 128;
                        return cat_bf16x4(lds_read_tr(cur + off), lds_read_tr(cur + 16 * kMainRow + off));
                    };
                    bf16x8 vf[VD];
#pragma unroll
                    for (int d = 0; d < VD; ++d) vf[d] = v_frag(d);
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
                        for (int r = 0; r < kWRT; ++r) o[r][dt] = mfma16(vf[dt % VD], pt[r], o[r][dt]);
                        if (dt + VD < kDT) vf[dt % VD] = v_frag(dt + VD);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                static_assert(2 * kKS / 4 == kWLoads, "one load per four K fragments");
                if (issue_now) ahead = ahead < 2 ? ahead + 1 : 2;
                else ahead = ahead > 0 ? ahead - 1 : 0;
                ++c;
                return c < nch;
            };
            using S0 = std::integral_constant<int, 0>;
            using S1 = std::integral_constant<int, 1>;
            using S2 = std::integral_constant<int, 2>;
            using S3 = std::integral_constant<int, 3>;
            while (step(S0{}) && step(S1{}) && step(S2{}) && step(S3{})) {
            }
        }
        // after the barrier every wave sees an overflow raised in the last step
        block_barrier_fw();
        redo = (restart_flag[0] | restart_flag[1]) != 0;
        if (redo) {
            // drain the ring and refill it from this segment's start; the
            // raised references stay, and the segment runs again
            wait_then_fence<wait_vm_lgkm0(0)>();
            block_barrier_fw();   // every wave has read the flags
            if (threadIdx.x == 0) {
                restart_flag[0] = 0;
                restart_flag[1] = 0;
            }
            fseg = seg;
            fc = 0;
            fpage = fpage_of();
            fill(soff);
            continue;
        }

        // ---- epilogue: normalise and store this wave's rows
        const bool full = (lo == 0) && (hi == pages_of(nseq));
        const int slotno = full ? 0 : ld_const_fw(seqinfo, 4 * b + 0) + (p - ld_const_fw(seqinfo, 4 * b + 1));
#pragma unroll
        for (int r = 0; r < kWRT; ++r) {
            const int row = rb * kRows + 16 * (kWRT * w + r) + i16;
            const float lsum = sum_over_kgroups(l_run[r]);
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            if (row < a.M) {
                if (g == 0) {
                    const float lse_v = lsum > 0.f ? (m_ref[r] + __log2f(lsum)) * kLn2 : -INFINITY;
                    if (full) a.lse[(size_t)b * a.M + row] = lse_v;
                    else a.part_lse[(size_t)row * a.lse_stride + slotno] = lse_v;
                }
                // tile dt covers columns 16 dt + 4 g .. +3 of the row
#pragma unroll
                for (int q4 = 0; q4 < kDT / 8; ++q4) {
                    if (full) {
                        uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + q4 * 128 + 4 * g;
                        bf16x4 v[8];
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            f32x4 x = o[r][q4 * 8 + t];
                            x[0] *= inv; x[1] *= inv; x[2] *= inv; x[3] *= inv;
                            v[t] = pack_bf16x4(x);
                        }
                        TileStores<8>::out(op, v);
                    } else {
                        float* pp = a.part_o + ((size_t)slotno * a.M + row) * kHeadDimV + q4 * 128 + 4 * g;
                        f32x4 v[8];
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            v[t] = o[r][q4 * 8 + t];
                            v[t][0] *= inv; v[t][1] *= inv; v[t][2] *= inv; v[t][3] *= inv;
                        }
                        TileStores<8>::part(pp, v, false);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        soff = (soff + nch) & 3;
        seg = find_seg(b + 1, 0);
    }
}

template <int kWRT>
static hipError_t launch_fw(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_fw_kernel<kWRT>, dim3(plan.P * plan.R), dim3(256), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_decode_fw(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    if (plan.tm == 128) return launch_fw<2>(plan, args, stream);
    return hipErrorInvalidValue;
}

}  // namespace mla
