// mla_decode_rows16.hip - split-KV MLA decode for blocks of 16 query rows.
//
// Same method as the multi-row kernel (page "MLA 和 MHA 的 Kernel 区别",
// section "MLA 的 FlashAttention": stream latent-cache tiles through on-chip
// memory and score the query block against them; absorbed form; one-pass
// softmax), organised for small query blocks, where the kernel is bound by
// HBM bytes rather than by arithmetic:
//
//  * each of the four waves owns a 16-key stripe of every 64-token page
//    (keys 16w..16w+15), so all waves do the same amount of distinct work;
//  * a wave loads only its own stripe (16 rows, 18 KB) with 16-byte direct
//    loads into a private double buffer and waits for its own loads only:
//    the next page's stripe is in flight while the current one is used, and
//    the page loop has no workgroup barrier;
//  * scores S^T = K Q^T are one 16x16 tile per page (18 MFMAs of depth 32,
//    the query block's latent part read from LDS, its RoPE part held in
//    registers); the value product O^T += V^T P^T has depth 16, so a lane's
//    four softmax weights are exactly its MFMA operand and each value operand
//    is a single transposing LDS read;
//  * the softmax reference of each row is fixed when the row first sees a
//    visible key (its maximum there plus a margin), so the O accumulators are
//    never rescaled inside the loop. Should a later score exceed the
//    reference by more than the headroom (which bounds every weight by 2^64),
//    the wave raises the reference and redoes its part of the segment from
//    the first page: exact, and for real score ranges it never happens;
//  * at the end of a sequence segment the four waves' (reference, sum, O) are
//    merged through LDS by the log-sum-exp rule and written once.
//
// The direct-to-LDS loads are issued so that the compiler does not track
// them; every wait for them is explicit below (vmcnt counts are per wave, and
// the wave issues nothing else to vector memory while a stripe is in flight).
#include "mla_common.h"
#include "mla_fused_combine.h"
#include "mla_internal.h"
#include "mla_sched.h"
#include "mla_store_asm.h"

namespace mla {

namespace {

__device__ __forceinline__ int ld_const_s(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

constexpr int kWaves = 4;
constexpr int kSRows = 16;                      // keys per stripe
constexpr int kSBytes = kSRows * kRowBytes;     // 18432
constexpr int kSLoads = kSBytes / 1024;         // 18 wave loads per stripe
constexpr int kKS = kHeadDim / 32;              // 18 k-steps of the score product
constexpr int kNDT = kHeadDimV / 16;            // 32 output tiles of 16 columns
constexpr int kQLatSteps = kHeadDimV / 32;      // 16 k-steps over the latent dims (query in LDS)
constexpr int kQRopeSteps = kKS - kQLatSteps;   // 2 k-steps over the RoPE dims (query in VGPRs)
// log2-domain margin added to a row's first maximum, and the headroom above
// the reference a score may reach before the wave restarts the segment
constexpr float kRefMargin = 32.f;
constexpr float kHeadroom = 64.f;

// gfx9 s_waitcnt immediates (expcnt never waited on)
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kWaitStripe = wait_vm_lgkm0(kSLoads);   // vmcnt(18) lgkmcnt(0)
constexpr int kWaitAll = wait_vm_lgkm0(0);            // vmcnt(0) lgkmcnt(0)

template <int kImm>
__device__ __forceinline__ void wait_then_fence() {
    __builtin_amdgcn_s_waitcnt(kImm);
    asm volatile("" ::: "memory");
}

}  // namespace

// One workgroup: 4 waves, 16 query rows (row block rb), one partition of the
// page list. Lane (g = lane/16, i16 = lane%16) holds query row i16 in the
// MFMA layouts; scores S^T[key][row] and output O^T[dim][row] keep the row
// in the lane, so all per-row softmax state is lane-local.
__global__ __launch_bounds__(256) void mla_decode_rows16_kernel(DecodeArgs a) {
    // Two LDS objects, one per buffer of every wave's double buffer.
    __shared__ __attribute__((aligned(16))) uint8_t buf0[kWaves][kSBytes];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[kWaves][kSBytes];
    // Latent part of the 16 query rows (dims 0..511), in MFMA operand order:
    // k-step ks occupies bytes [1024 ks, 1024 ks + 1024), lane l at 16 l.
    // With the stripe buffers this fills the 160 KB of LDS exactly.
    __shared__ __attribute__((aligned(16))) uint8_t qlds[kQLatSteps * 1024];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int g = lane >> 4;
    const int i16 = lane & 15;

    if (!plan_matches_or_poison<256>(a)) return;
    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    // partition record: its range and the length of its first sequence,
    // so that the first segment starts without another dependent load
    const int32_t* part = a.meta + kMetaHeader + kPartInts * p;
    int b = ld_const_s(part, 0);
    int n = ld_const_s(part, 1);
    const int b_end = ld_const_s(part, 2);
    const int n_end = ld_const_s(part, 3);
    const int len0 = ld_const_s(part, 4);
    const int b_first = b;
    const int32_t* seqinfo = a.meta + kMetaHeader + kPartInts * a.P;

    const int row = rb * 16 + i16;
    const bool row_ok = row < a.M;
    const int tok = row_ok ? row / a.h_q : 0;

    uint8_t* const mine0 = buf0[wave];
    uint8_t* const mine1 = buf1[wave];
    const uint32_t mine0_lds = lds_addr_of(mine0);
    const uint32_t mine1_lds = lds_addr_of(mine1);
    const uint32_t qlds_lds = lds_addr_of(qlds);

    // Stripe gather: 18 wave loads of 1 KB; LDS 16-byte chunk k holds stripe
    // row k/72, slot k%72 = logical chunk slot^swz(row). Nine loads cover
    // eight rows, so the lane's nine source offsets repeat for rows 8..15.
    int goff[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) {
        const int k = j * 64 + lane;
        const int r = k / kRowChunks;
        const int c = k - r * kRowChunks;
        goff[j] = r * kRowBytes + ((c ^ lds_swizzle(r)) << 4);
    }
    // Rows at or past the sequence end read the page's first kilobyte (row 0,
    // always valid): finite data whose softmax weight is zero. Only the last
    // page of a sequence takes that path.
    auto issue_stripe = [&](const uint8_t* page, int valid, uint32_t dst) {
        if (valid >= kSRows) {
            const uint8_t* src = page + wave * kSBytes;
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int j = 0; j < 9; ++j)
                    load_lds16_untracked(src, (uint32_t)(grp * 9216 + goff[j]), dst + grp * 9216 + j * 1024);
        } else {
#pragma unroll
            for (int grp = 0; grp < 2; ++grp) {
#pragma unroll
                for (int j = 0; j < 9; ++j) {
                    const int r = grp * 8 + (j * 64 + lane) / kRowChunks;
                    const uint32_t lo_off = r < valid ? (uint32_t)(wave * kSBytes + grp * 9216 + goff[j])
                                                     : (uint32_t)(lane * 16);
                    load_lds16_untracked(page, lo_off, dst + grp * 9216 + j * 1024);
                }
            }
        }
    };

    // LDS byte offsets inside a stripe, precomputed per lane: the K fragment
    // of k-step ks for key row i16 is at kofs[ks & 1] + 128 (ks >> 1); the
    // V^T fragment of value tile dt for key rows vr = 4g + i16/4 at
    // vofs[dt & 3] + 128 (dt >> 2).
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

    f32x4 o[kNDT];
    const uint8_t* const q_frag = qlds + lane * 16;

    while (b < b_end || (b == b_end && n < n_end)) {
        const int nseq = b == b_first ? len0 : ld_const_s(a.seqlens, b);
        const int npages = pages_of(nseq);
        const int hi = (b == b_end) ? n_end : npages;
        if (n >= hi) { ++b; n = 0; continue; }
        const int lo = n;

        const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
        auto page_ptr = [&](int phys) {
            return reinterpret_cast<const uint8_t*>(a.kv) + (size_t)phys * kPageBytes;
        };
        auto stripe_valid = [&](int pn) { return nseq - pn * kPageRows - wave * kSRows; };

        // Query rows rb*16..+15 (rows past M repeat row rb*16; their results
        // are never stored): wave w brings latent k-steps 4w..4w+3 into the
        // shared query buffer and the two RoPE k-steps into its own second
        // stripe buffer, then the first page's stripe follows.
        {
            const uint16_t* q_blk = a.q + ((size_t)b * a.M + rb * 16) * kHeadDim;
            const uint32_t q_off = (uint32_t)(((row_ok ? i16 : 0) * kHeadDim + g * 8) * 2);
#pragma unroll
            for (int i = 0; i < kQLatSteps / kWaves; ++i) {
                const int ks = wave * (kQLatSteps / kWaves) + i;
                load_lds16_untracked(q_blk, q_off + ks * 64, qlds_lds + ks * 1024);
            }
#pragma unroll
            for (int i = 0; i < kQRopeSteps; ++i)
                load_lds16_untracked(q_blk, q_off + (kQLatSteps + i) * 64, mine1_lds + i * 1024);
        }
        issue_stripe(page_ptr(ld_const_s(bt_row, lo)), stripe_valid(lo), mine0_lds);
        int phys1 = ld_const_s(bt_row, lo + 1 < hi ? lo + 1 : lo);
        // the query loads (issued before the stripe) have landed; after the
        // barrier every wave's share of the latent query is visible
        wait_then_fence<kWaitStripe>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        bf16x8 qr[kQRopeSteps];
#pragma unroll
        for (int i = 0; i < kQRopeSteps; ++i) qr[i] = lds_read16(mine1 + i * 1024 + lane * 16);
        // the RoPE query must be in registers before the first step
        // overwrites its buffer
        wait_then_fence<kWaitStripe>();

        const int L = a.causal ? min(max(nseq - a.s_q + tok + 1, 0), nseq) : nseq;
        float m_ref = -INFINITY, l_run = 0.f;
        // a segment holding the whole sequence writes the output itself;
        // otherwise its partial goes to slot slot_base + (p - first partition)
        const bool full = (lo == 0) && (hi == npages);
        const int slotno = full ? 0 : ld_const_s(seqinfo, 4 * b + 0) + (p - ld_const_s(seqinfo, 4 * b + 1));

        // One page: the stripe of page pn sits in `cur`; the next page's
        // stripe, if the segment has one, is issued into `nxt` first, so one
        // stripe is in flight while this one is used. Returns the next page
        // to process.
        auto page_step = [&](int pn, uint8_t* cur, uint32_t nxt_lds) -> int {
            const bool more = pn + 1 < hi;
            if (more) issue_stripe(page_ptr(phys1), stripe_valid(pn + 1), nxt_lds);
            phys1 = ld_const_s(bt_row, pn + 2 < hi ? pn + 2 : hi - 1);
            // this page's stripe and the table entry
            if (more) wait_then_fence<kWaitStripe>();
            else wait_then_fence<kWaitAll>();

            // ---- S^T[key][row] = K Q^T over the stripe's 16 keys
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            {
                constexpr int KD = 4;
                auto k_off = [&](int ks) { return kofs[ks & 1] + (ks >> 1) * 128; };
                bf16x8 kf[KD], qf[KD];
#pragma unroll
                for (int d = 0; d < KD; ++d) {
                    kf[d] = lds_read16(cur + k_off(d));
                    qf[d] = lds_read16(q_frag + d * 1024);
                }
#pragma unroll
                for (int ks = 0; ks < kKS; ++ks) {
                    const bf16x8 qb = ks < kQLatSteps ? qf[ks % KD] : qr[ks - kQLatSteps];
                    s = mfma16(kf[ks % KD], qb, s);
                    if (ks + KD < kKS) kf[ks % KD] = lds_read16(cur + k_off(ks + KD));
                    if (ks + KD < kQLatSteps) qf[ks % KD] = lds_read16(q_frag + (ks + KD) * 1024);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // ---- mask, reference check (log2 domain). Lane holds row i16,
            // keys 4g+j of the stripe.
            const int key0 = pn * kPageRows + wave * kSRows + 4 * g;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = (key0 + j < L) ? s[j] * a.scale_log2 : -INFINITY;
                s[j] = v;
                mx = fmaxf(mx, v);
            }
            mx = max_over_kgroups(mx);
            // A row with no visible key so far has O = 0 and l = 0, so its
            // reference can be set freely.
            if (m_ref == -INFINITY) m_ref = mx == -INFINITY ? -INFINITY : mx + kRefMargin;
            const bool over = mx > m_ref + kHeadroom;
            if (__ballot(over) != 0) {
                // raise the reference of the rows that overflowed; the
                // caller restarts the segment
                if (over) m_ref = mx + kRefMargin;
                return -1;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[j] = __builtin_amdgcn_exp2f(s[j] - m_use);
                l_run += s[j];
            }
            // P^T operand: k-slot 4g+j <-> key 4g+j of the stripe
            const bf16x4 pf = pack_bf16x4(s);

            // ---- O^T[dim][row] += V^T[dim][key] P^T[key][row], depth 16:
            // the V^T operand of a lane is keys 4g..4g+3 of one dim, one
            // transposing read.
            {
                constexpr int VD = 8;
                auto v_off = [&](int dt) { return vofs[dt & 3] + (dt >> 2) * 128; };
                bf16x4 vf[VD];
#pragma unroll
                for (int d = 0; d < VD; ++d) vf[d] = lds_read_tr(cur + v_off(d));
#pragma unroll
                for (int dt = 0; dt < kNDT; ++dt) {
                    o[dt] = mfma16k16(vf[dt % VD], pf, o[dt]);
                    if (dt + VD < kNDT) vf[dt % VD] = lds_read_tr(cur + v_off(dt + VD));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            return pn + 1;
        };

        // Buffers alternate by position in the two-step body. A restart
        // (per wave, no barrier involved) drains the stripe in flight and
        // starts over from page lo with cleared accumulators.
        bool restart;
        do {
#pragma unroll
            for (int dt = 0; dt < kNDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            l_run = 0.f;
            int pn = lo;
            while (true) {
                pn = page_step(pn, mine0, mine1_lds);
                if (pn < 0 || pn >= hi) break;
                pn = page_step(pn, mine1, mine0_lds);
                if (pn < 0 || pn >= hi) break;
            }
            restart = pn < 0;
            // after a restart the stripe issued for the next page must land
            // before the buffers are reused
            wait_then_fence<kWaitAll>();
            if (restart) {
                issue_stripe(page_ptr(ld_const_s(bt_row, lo)), stripe_valid(lo), mine0_lds);
                phys1 = ld_const_s(bt_row, lo + 1 < hi ? lo + 1 : lo);
            }
        } while (restart);

        // ---- merge the four waves' (m, l, O) through LDS. Wave w's O^T
        // tiles 0..15 go to its own buf0 entry, 16..31 to its buf1 entry,
        // one kilobyte per tile (lane-contiguous, conflict-free); m and l
        // follow the tiles in buf0. Only this wave has touched its entries
        // since the last barrier, so no barrier is needed before writing.
        float lsum = l_run;
        lsum = sum_over_kgroups(lsum);
        {
            float* w0 = reinterpret_cast<float*>(mine0);
            float* w1 = reinterpret_cast<float*>(mine1);
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<f32x4*>(w0 + dt * 256 + lane * 4) = o[dt];
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<f32x4*>(w1 + dt * 256 + lane * 4) = o[16 + dt];
            if (g == 0) {
                w0[4096 + i16] = m_ref;
                w0[4096 + 16 + i16] = lsum;
            }
        }
        __syncthreads();
        // this wave finalises columns 128*wave .. +127 = tiles 8*wave .. +7
        float mw[kWaves], lw[kWaves];
        float mmax = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* ml = reinterpret_cast<const float*>(buf0[w]) + 4096;
            mw[w] = ml[i16];
            lw[w] = ml[16 + i16];
            mmax = fmaxf(mmax, lw[w] > 0.f ? mw[w] : -INFINITY);
        }
        const float mref = mmax == -INFINITY ? 0.f : mmax;
        float ltot = 0.f, sc[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            sc[w] = lw[w] > 0.f ? __builtin_amdgcn_exp2f(mw[w] - mref) : 0.f;
            ltot += lw[w] * sc[w];
        }
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        const float lse_v = ltot > 0.f ? (mref + __log2f(ltot)) * kLn2 : -INFINITY;
        f32x4 res[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) res[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile0 = (wave & 1) * 8;   // first tile in the buffer holding tiles 8*wave..
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* src = reinterpret_cast<const float*>(wave < 2 ? buf0[w] : buf1[w]) + tile0 * 256 + lane * 4;
            const float f = sc[w] * inv;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(src + t * 256);
                res[t][0] += f * v[0]; res[t][1] += f * v[1]; res[t][2] += f * v[2]; res[t][3] += f * v[3];
            }
        }
        if (row_ok) {
            const int col0 = wave * 128 + 4 * g;   // tile t covers columns col0 + 16 t .. +3
            if (full) {
                uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + col0;
                bf16x4 v[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = pack_bf16x4(res[t]);
                TileStores<8>::out(op, v);
                if (wave == 0 && g == 0) a.lse[(size_t)b * a.M + row] = lse_v;
            } else {
                float* pp = a.part_o + ((size_t)slotno * a.M + row) * kHeadDimV + col0;
                TileStores<8>::part(pp, res, a.counters != nullptr);
                if (wave == 0 && g == 0)   // device-coherent, as the partial tiles
                    __hip_atomic_store(&a.part_lse[(size_t)row * a.lse_stride + slotno], lse_v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();   // buffers and the query block are free again
        // the query buffer holds the flag: the next segment's query loads
        // come after the helper's last barrier
        if (!full && a.counters) count_partial_and_combine<256, 16>(a, b, rb, reinterpret_cast<int*>(qlds));
        ++b;
        n = 0;
    }
    if (a.counters) write_empty_sequences<256>(a);
}

hipError_t launch_decode_rows16(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_rows16_kernel, dim3(plan.P * plan.R), dim3(256), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mla
