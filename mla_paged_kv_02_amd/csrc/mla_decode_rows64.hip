// mla_decode_rows64.hip - split-KV MLA decode for blocks of 64 or 128 query
// rows.
//
// Method as in the other decode kernels (page "MLA 和 MHA 的 Kernel 区别",
// section "MLA 的 FlashAttention": stream latent-cache tiles through on-chip
// memory, score the query block against them, one-pass softmax; absorbed
// form), organised for query blocks large enough that the two products are
// the work: every page is brought into LDS once per workgroup and used by
// all its query rows.
//
//  * four waves, wave w owns RT 16-row tiles of the block (RT = 1: 64 rows
//    per workgroup, RT = 2: 128); the query stays in registers and the O^T
//    accumulators (RT x 16 rows x 512 columns) in AGPRs;
//  * the cache streams through a ring of four half-page slots (32 keys,
//    36 KB each); wave w loads rows 8w..8w+7 of every half page with 16-byte
//    direct loads, three half pages ahead of the one in use, and one
//    workgroup barrier per half page makes the slot visible to all waves and
//    frees the slot of the previous half page;
//  * per half page a wave computes S^T = K Q^T for 32 keys x RT row tiles
//    (2 x RT x 18 MFMA 16x16x32, each K fragment read once and used for all
//    RT row tiles) and O^T += V^T P^T with depth 32 (32 x RT MFMA): a lane's
//    eight softmax weights (4 keys of each 16-key tile) are exactly its B
//    operand and the matching V^T operand is two transposing LDS reads,
//    again shared by the RT row tiles. With RT = 2 each LDS byte feeds twice
//    the MFMA work, which is what the LDS bandwidth needs;
//  * softmax reference fixed per row at its first visible maximum plus a
//    margin; if a later score would exceed it by more than the headroom, the
//    wave raises a flag, every wave sees it after the next barrier and the
//    workgroup redoes the segment with raised references (exact; never
//    triggered by scores of realistic range);
//  * no cross-wave merge: each wave finishes its own rows.
//
// The direct-to-LDS loads are issued untracked by the compiler and every
// wait for them is explicit.
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_sched.h"
#include "mla_store_asm.h"

namespace mla {

namespace {

__device__ __forceinline__ int ld_const_w(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

constexpr int kWaves = 4;
constexpr int kCRows = 32;                      // keys per ring slot (half page)
constexpr int kCBytes = kCRows * kRowBytes;     // 36864
constexpr int kWLoads = 9;                      // a wave's wave-loads per slot (8 rows)
constexpr int kKS = kHeadDim / 32;              // 18 k-steps of the score product
constexpr int kNDT = kHeadDimV / 16;            // 32 output tiles of 16 columns
constexpr int kQReg = kKS - 1;                  // k-steps 0..16: query in registers
                                                // k-step 17 (last RoPE dims): query in LDS
constexpr float kRefMargin = 32.f;
constexpr float kHeadroom = 64.f;

constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
// a slot's loads are followed by two more slots' loads before it is read
constexpr int kWaitSlot = wait_vm_lgkm0(2 * kWLoads);
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

template <int RT>
__global__ __launch_bounds__(256) void mla_decode_wide_kernel(DecodeArgs a) {
    constexpr int kRowsWG = 64 * RT;
    constexpr int KD = RT == 1 ? 3 : 2;   // K prefetch depth (k-steps)
    constexpr int VD = RT == 1 ? 4 : 3;   // V^T prefetch depth (tiles)

    __shared__ __attribute__((aligned(16))) uint8_t ring0[kCBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kCBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[kCBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[kCBytes];
    // the query block's last k-step (RoPE dims 544..575) in MFMA operand
    // order: row tile (wave, rt) owns 1 KB, lane l at +16 l
    __shared__ __attribute__((aligned(16))) uint8_t qlast[kWaves * RT * 1024];
    // overflow flags by half-page parity: set during step c in flag[c & 1],
    // read by every wave after the next barrier
    __shared__ int restart_flag[2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;

    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    int b = ld_const_w(a.meta, kMetaHeader + 4 * p + 0);
    int n = ld_const_w(a.meta, kMetaHeader + 4 * p + 1);
    const int b_end = ld_const_w(a.meta, kMetaHeader + 4 * p + 2);
    const int n_end = ld_const_w(a.meta, kMetaHeader + 4 * p + 3);
    const int32_t* seqinfo = a.meta + kMetaHeader + 4 * a.P;

    int row[RT], tok[RT];
    bool row_ok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        row[rt] = rb * kRowsWG + wave * 16 * RT + rt * 16 + i16;
        row_ok[rt] = row[rt] < a.M;
        tok[rt] = row_ok[rt] ? row[rt] / a.h_q : 0;
    }

    if (threadIdx.x == 0) {
        restart_flag[0] = 0;
        restart_flag[1] = 0;
    }
    const uint32_t slot_lds[4] = {lds_addr_of(ring0), lds_addr_of(ring1), lds_addr_of(ring2),
                                  lds_addr_of(ring3)};

    // Slot gather: wave w loads rows 8w..8w+7 of the half page with 9 wave
    // loads of 1 KB; LDS 16-byte chunk k of the wave's 9 KB holds row k/72,
    // slot k%72 = logical chunk slot^swz(row). goff[j] is the lane's source
    // offset for load j from the wave's first row.
    int goff[kWLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
        const int k = j * 64 + lane;
        const int r = k / kRowChunks;
        const int c = k - r * kRowChunks;
        goff[j] = r * kRowBytes + ((c ^ lds_swizzle(r)) << 4);
    }
    // Rows at or past the sequence end read the page's first kilobyte (row
    // 0, always valid): finite data whose softmax weight is zero. Only the
    // last page of a sequence takes that path.
    auto issue_half = [&](const uint8_t* page, int half, int valid, uint32_t dst) {
        const int base = half * kCBytes + wave * 9216;
        const uint32_t d = dst + wave * 9216;
        if (valid >= half * kCRows + wave * 8 + 8) {
            const uint8_t* src = page + base;
#pragma unroll
            for (int j = 0; j < kWLoads; ++j) load_lds16_untracked(src, (uint32_t)goff[j], d + j * 1024);
        } else {
#pragma unroll
            for (int j = 0; j < kWLoads; ++j) {
                const int r = half * kCRows + wave * 8 + (j * 64 + lane) / kRowChunks;
                const uint32_t lo_off = r < valid ? (uint32_t)(base + goff[j]) : (uint32_t)(lane * 16);
                load_lds16_untracked(page, lo_off, d + j * 1024);
            }
        }
    };

    // LDS byte offsets inside a slot, precomputed per lane: the K fragment of
    // k-step ks for key row i16 (and 16+i16) is at kofs[ks & 1] + 128 (ks >> 1);
    // the V^T fragment of value tile dt for key rows vr = 4g + i16/4 (and
    // 16+vr) at vofs[dt & 3] + 128 (dt >> 2).
    int kofs[2], vofs[4];
    {
        const int vr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            kofs[i] = i16 * kRowBytes + (((i * 4 + g) ^ lds_swizzle(i16)) << 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vofs[i] = vr * kRowBytes + ((i16 & 1) << 3) + (((i * 2 + ((i16 & 3) >> 1)) ^ lds_swizzle(vr)) << 4);
    }

    f32x4 o[RT][kNDT];
    bf16x8 qf[RT][kQReg];
    const uint8_t* const ql_frag = qlast + wave * RT * 1024 + lane * 16;

    while (b < b_end || (b == b_end && n < n_end)) {
        const int nseq = ld_const_w(a.seqlens, b);
        const int npages = pages_of(nseq);
        const int hi = (b == b_end) ? n_end : npages;
        if (n >= hi) { ++b; n = 0; continue; }
        const int lo = n;
        const int nch = 2 * (hi - lo);   // half pages of the segment

        const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
        auto page_of_chunk = [&](int c) {
            const int pn = lo + (c < nch ? c : nch - 1) / 2;
            return reinterpret_cast<const uint8_t*>(a.kv) +
                   (size_t)ld_const_w(bt_row, pn) * kPageBytes;
        };
        // issue half page c (clamped to the last one) into its ring slot
        auto issue_chunk = [&](int c, const uint8_t* page, uint32_t dst) {
            const int cc = c < nch ? c : nch - 1;
            issue_half(page, cc & 1, nseq - (lo + cc / 2) * kPageRows, dst);
        };

        int L[RT];
        float m_ref[RT], l_run[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            L[rt] = a.causal ? min(max(nseq - a.s_q + tok[rt] + 1, 0), nseq) : nseq;
            m_ref[rt] = -INFINITY;
        }

        // the wave's query rows (rows past M repeat the block's first row;
        // their results are never stored)
        {
            const uint16_t* q_blk = a.q + ((size_t)b * a.M + rb * kRowsWG) * kHeadDim;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int r_in = row_ok[rt] ? row[rt] - rb * kRowsWG : 0;
                const uint16_t* qp = q_blk + r_in * kHeadDim + g * 8;
#pragma unroll
                for (int ks = 0; ks < kQReg; ++ks) qf[rt][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
                load_lds16_untracked(q_blk, (uint32_t)((r_in * kHeadDim + g * 8 + kQReg * 32) * 2),
                                     lds_addr_of(qlast) + (wave * RT + rt) * 1024);
            }
        }

        bool restart = false;
        do {
            // fill slots 0..2, then drain: the query loads and the first
            // three half pages are in, and every wave is past the previous
            // use of the ring
            issue_chunk(0, page_of_chunk(0), slot_lds[0]);
            issue_chunk(1, page_of_chunk(1), slot_lds[1]);
            issue_chunk(2, page_of_chunk(2), slot_lds[2]);
            const uint8_t* page3 = page_of_chunk(3);
            wait_then_fence<kWaitAll>();
            block_barrier();
            if (restart && wave == 0 && lane == 0) {
                restart_flag[0] = 0;
                restart_flag[1] = 0;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int dt = 0; dt < kNDT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
                l_run[rt] = 0.f;
            }
            bool skip = false;   // this wave saw an overflow; PV is pointless until the restart

            // One half page: chunk c sits in slot S = c % 4; chunk c+3 is
            // issued into slot (S+3) % 4, whose previous chunk c-1 every
            // wave finished before the barrier. Returns false when the
            // segment is done or a restart is due.
            int c = 0;
            auto step = [&](auto sc) -> bool {
                constexpr int S = decltype(sc)::value;
                uint8_t* cur = S == 0 ? ring0 : S == 1 ? ring1 : S == 2 ? ring2 : ring3;
                const uint8_t* page_next = page_of_chunk(c + 4);   // a step ahead
                wait_then_fence<kWaitSlot>();
                block_barrier();
                if (restart_flag[(S + 1) & 1] != 0) return false;   // raised in step c-1
                issue_chunk(c + 3, page3, slot_lds[(S + 3) % 4]);
                page3 = page_next;

                // ---- S^T = K Q^T: key tiles 0 and 1 of the slot, all row
                // tiles. With one row tile the k-steps alternate between two
                // accumulators per key tile, so four independent MFMA chains
                // cover the MFMA latency; they are summed at the end.
                constexpr int NP = RT == 1 ? 2 : 1;
                f32x4 s[2][RT], sp[2][RT][NP];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) {
                        sp[0][rt][pp] = f32x4{0.f, 0.f, 0.f, 0.f};
                        sp[1][rt][pp] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                {
                    auto k_off = [&](int ks) { return kofs[ks & 1] + (ks >> 1) * 128; };
                    bf16x8 ql[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) ql[rt] = lds_read16(ql_frag + rt * 1024);
                    bf16x8 k0[KD], k1[KD];
#pragma unroll
                    for (int d = 0; d < KD; ++d) {
                        k0[d] = lds_read16(cur + k_off(d));
                        k1[d] = lds_read16(cur + 16 * kRowBytes + k_off(d));
                    }
#pragma unroll
                    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            const bf16x8 qb = ks < kQReg ? qf[rt][ks] : ql[rt];
                            sp[0][rt][ks % NP] = mfma16(k0[ks % KD], qb, sp[0][rt][ks % NP]);
                            sp[1][rt][ks % NP] = mfma16(k1[ks % KD], qb, sp[1][rt][ks % NP]);
                        }
                        if (ks + KD < kKS) {
                            k0[ks % KD] = lds_read16(cur + k_off(ks + KD));
                            k1[ks % KD] = lds_read16(cur + 16 * kRowBytes + k_off(ks + KD));
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        s[kt][rt] = sp[kt][rt][0];
                        if constexpr (NP == 2) {
                            s[kt][rt][0] += sp[kt][rt][1][0]; s[kt][rt][1] += sp[kt][rt][1][1];
                            s[kt][rt][2] += sp[kt][rt][1][2]; s[kt][rt][3] += sp[kt][rt][1][3];
                        }
                    }

                // ---- mask + reference check; lane holds row i16 of each
                // row tile, keys 4g+j of key tile 0 and 16+4g+j of key tile 1
                const int key0 = (lo + c / 2) * kPageRows + (c & 1) * kCRows + 4 * g;
                bool over_any = false;
                float mx[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    mx[rt] = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float v0 = (key0 + j < L[rt]) ? s[0][rt][j] * a.scale_log2 : -INFINITY;
                        const float v1 = (key0 + 16 + j < L[rt]) ? s[1][rt][j] * a.scale_log2 : -INFINITY;
                        s[0][rt][j] = v0;
                        s[1][rt][j] = v1;
                        mx[rt] = fmaxf(mx[rt], fmaxf(v0, v1));
                    }
                    mx[rt] = max_over_kgroups(mx[rt]);
                    if (m_ref[rt] == -INFINITY)
                        m_ref[rt] = mx[rt] == -INFINITY ? -INFINITY : mx[rt] + kRefMargin;
                    over_any |= mx[rt] > m_ref[rt] + kHeadroom;
                }
                if (__ballot(over_any) != 0) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        if (mx[rt] > m_ref[rt] + kHeadroom) m_ref[rt] = mx[rt] + kRefMargin;
                    if (lane == 0) restart_flag[S & 1] = 1;
                    skip = true;
                }
                if (!skip) {
                    // B = P^T per row tile: k-slot j <-> key 4g+j, k-slot 4+j
                    // <-> key 16+4g+j
                    bf16x8 pf[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const float m_use = (m_ref[rt] == -INFINITY) ? 0.f : m_ref[rt];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            s[0][rt][j] = __builtin_amdgcn_exp2f(s[0][rt][j] - m_use);
                            s[1][rt][j] = __builtin_amdgcn_exp2f(s[1][rt][j] - m_use);
                            l_run[rt] += s[0][rt][j] + s[1][rt][j];
                        }
                        pf[rt] = cat_bf16x4(pack_bf16x4(s[0][rt]), pack_bf16x4(s[1][rt]));
                    }

                    // ---- O^T += V^T P^T, depth 32: A = V^T for keys
                    // 4g..4g+3 and 16+4g..16+4g+3, two transposing reads,
                    // shared by the row tiles
                    auto v_off = [&](int dt) { return vofs[dt & 3] + (dt >> 2) * 128; };
                    auto v_frag = [&](int dt) {
                        return cat_bf16x4(lds_read_tr(cur + v_off(dt)),
                                          lds_read_tr(cur + 16 * kRowBytes + v_off(dt)));
                    };
                    bf16x8 vf[VD];
#pragma unroll
                    for (int d = 0; d < VD; ++d) vf[d] = v_frag(d);
#pragma unroll
                    for (int dt = 0; dt < kNDT; ++dt) {
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) o[rt][dt] = mfma16(vf[dt % VD], pf[rt], o[rt][dt]);
                        if (dt + VD < kNDT) vf[dt % VD] = v_frag(dt + VD);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                ++c;
                return c < nch;
            };
            using S0 = std::integral_constant<int, 0>;
            using S1 = std::integral_constant<int, 1>;
            using S2 = std::integral_constant<int, 2>;
            using S3 = std::integral_constant<int, 3>;
            while (step(S0{}) && step(S1{}) && step(S2{}) && step(S3{})) {
            }
            // drain the half pages still in flight; after the barrier every
            // wave sees an overflow raised in the last half page too
            wait_then_fence<kWaitAll>();
            block_barrier();
            restart = (restart_flag[0] | restart_flag[1]) != 0;
            if (restart) block_barrier();   // every wave has read the flag before it is cleared
        } while (restart);

        // ---- epilogue: this wave's rows
        const bool full = (lo == 0) && (hi == npages);
        const int col0 = 4 * g;   // tile dt covers columns col0 + 16 dt .. +3
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float lsum = l_run[rt];
            lsum = sum_over_kgroups(lsum);
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            const float lse_v = lsum > 0.f ? (m_ref[rt] + __log2f(lsum)) * kLn2 : -INFINITY;
            if (!row_ok[rt]) continue;
            if (full) {
                uint16_t* op = a.out + ((size_t)b * a.M + row[rt]) * kHeadDimV + col0;
                bf16x4 v[kNDT];
#pragma unroll
                for (int dt = 0; dt < kNDT; ++dt) {
                    f32x4 t = o[rt][dt];
                    t[0] *= inv; t[1] *= inv; t[2] *= inv; t[3] *= inv;
                    v[dt] = pack_bf16x4(t);
                }
                TileStores<kNDT>::out(op, v);
                if (g == 0) a.lse[(size_t)b * a.M + row[rt]] = lse_v;
            } else {
                const int slotno = ld_const_w(seqinfo, 4 * b + 0) + (p - ld_const_w(seqinfo, 4 * b + 1));
                float* pp = a.part_o + ((size_t)slotno * a.M + row[rt]) * kHeadDimV + col0;
                f32x4 v[kNDT];
#pragma unroll
                for (int dt = 0; dt < kNDT; ++dt) {
                    v[dt] = o[rt][dt];
                    v[dt][0] *= inv; v[dt][1] *= inv; v[dt][2] *= inv; v[dt][3] *= inv;
                }
                TileStores<kNDT>::part(pp, v);
                if (g == 0) a.part_lse[(size_t)row[rt] * a.lse_stride + slotno] = lse_v;
            }
        }
        ++b;
        n = 0;
    }
}

hipError_t launch_decode_rows64(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    const dim3 grid(plan.P * plan.R);
    if (plan.tm == 64) {
        hipLaunchKernelGGL(mla_decode_wide_kernel<1>, grid, dim3(256), 0, stream, args);
    } else if (plan.tm == 128) {
        hipLaunchKernelGGL(mla_decode_wide_kernel<2>, grid, dim3(256), 0, stream, args);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mla
