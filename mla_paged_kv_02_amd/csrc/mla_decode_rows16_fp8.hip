// mla_decode_rows16_fp8.hip - split-KV MLA decode over an FP8 latent cache,
// blocks of 16 query rows.
//
// The cache keeps only the latent row (page "MLA 和 MHA 的 Kernel 区别",
// section "内存布局和 KV Cache 大小"), so storing it in 8 bits cuts the
// bytes decode must stream, which is what bounds it. Page layout (64 tokens,
// 41,216 bytes): four groups of 16 tokens, 10,304 bytes each, holding the 16
// latent rows as OCP E4M3 bytes (512 each), then their rotary parts in BF16
// (128 bytes each), then their 16 FP32 scales. The value of latent
// coordinate d of token t is e4m3(byte) * scale[t]. A group is exactly one
// wave's stripe, so its scales arrive with its rows.
//
// Same organisation as the BF16 16-row kernel (four waves, each streaming
// its own 16-key stripe of every page through a private double buffer, no
// barrier in the page loop), with three changes:
//
//  * a stripe is one group: 8 KB of E4M3 latent rows, 2 KB of rotary rows
//    and the 64-byte scale block (a four-lane load);
//  * after its stripe lands, a wave converts the latent bytes to BF16 into a
//    private 16 KB buffer (row stride 1 KB, chunk c of row r at c ^ (r & 7))
//    with the hardware's packed FP8->BF16 conversion; E4M3 values are exact
//    in BF16, so nothing is rounded there. The score and value products then
//    read that buffer exactly as the BF16 kernel reads its stripes;
//  * the scale multiplies the latent half of a key's score (kept in its own
//    accumulator; the rotary half is unscaled) and is folded into the key's
//    softmax weight before the value product, O = sum_t p_t * scale_t * V_t,
//    while the normaliser sums p_t alone.
#include "mla_common.h"
#include "mla_fused_combine.h"
#include "mla_internal.h"
#include "mla_sched.h"
#include "mla_store_asm.h"

namespace mla {

namespace {

__device__ __forceinline__ int ld_const_i(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kSRows = 16;                          // keys per stripe
constexpr int kLatBytes = 512;                      // E4M3 latent row
constexpr int kRopeBytes = 128;                     // BF16 rotary row
constexpr int kStripeLat = kSRows * kLatBytes;      // 8192: latent rows of a group
constexpr int kStripeRope = kSRows * kRopeBytes;    // 2048: rotary rows
constexpr int kScaleOffG = kStripeLat + kStripeRope;           // 10240: scales
constexpr int kStripeBytes = kScaleOffG + kSRows * 4;          // 10304 per group / LDS slot
constexpr int kF8PageBytes = 4 * kStripeBytes;      // 41216
constexpr int kSLoads = 11;                         // 10 wave loads of 1 KB + the scale block
constexpr int kCvtRow = 1024;                       // BF16 latent row in LDS
constexpr int kCvtBytes = kSRows * kCvtRow;         // 16384
constexpr int kWaveLds = 2 * kStripeBytes + kCvtBytes;         // 36992
constexpr int kNDT = kHeadDimV / 16;                // 32 output tiles of 16 columns
constexpr int kQLatSteps = kHeadDimV / 32;          // 16
constexpr int kQLdsSteps = kQLatSteps - 1;          // 15 latent k-steps in LDS, the last in VGPRs
constexpr int kQRopeSteps = 2;
constexpr float kRefMargin = 32.f;
constexpr float kHeadroom = 64.f;

constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kWaitStripe = wait_vm_lgkm0(kSLoads);
constexpr int kWaitAll = wait_vm_lgkm0(0);
constexpr int kWaitLgkm = wait_vm_lgkm0(63);                   // lgkmcnt(0) only

template <int kImm>
__device__ __forceinline__ void wait_then_fence() {
    __builtin_amdgcn_s_waitcnt(kImm);
    asm volatile("" ::: "memory");
}

// 16 E4M3 values (one 16-byte chunk) -> 16 BF16 values, exact.
__device__ __forceinline__ void e4m3x16_to_bf16(const uint32_t (&w)[4], bf16x8& lo, bf16x8& hi) {
    bf16x2 p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
        p[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[2 * i] = p[i][0];
        lo[2 * i + 1] = p[i][1];
        hi[2 * i] = p[4 + i][0];
        hi[2 * i + 1] = p[4 + i][1];
    }
}

}  // namespace

__global__ __launch_bounds__(256) void mla_decode_rows16_fp8_kernel(DecodeArgs a) {
    // per wave: two stripe buffers, then the 16 KB BF16 latent buffer; the
    // query's latent k-steps 0..14 (its last latent k-step and its rotary
    // part are held in registers), which makes room for the scale blocks
    __shared__ __attribute__((aligned(16))) uint8_t wlds[kWaves][kWaveLds];
    __shared__ __attribute__((aligned(16))) uint8_t qlds[kQLdsSteps * 1024];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int i16 = lane & 15;

    if (!plan_matches_or_poison<256>(a)) return;
    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    const int32_t* part = a.meta + kMetaHeader + kPartInts * p;
    int b = ld_const_i(part, 0);
    int n = ld_const_i(part, 1);
    const int b_end = ld_const_i(part, 2);
    const int n_end = ld_const_i(part, 3);
    const int len0 = ld_const_i(part, 4);
    const int b_first = b;
    const int32_t* seqinfo = a.meta + kMetaHeader + kPartInts * a.P;

    const int row = rb * 16 + i16;
    const bool row_ok = row < a.M;
    const int tok = row_ok ? row / a.h_q : 0;

    uint8_t* const mine0 = wlds[wave];
    uint8_t* const mine1 = wlds[wave] + kStripeBytes;
    uint8_t* const cvt = wlds[wave] + 2 * kStripeBytes;
    const uint32_t mine0_lds = lds_addr_of(mine0);
    const uint32_t mine1_lds = lds_addr_of(mine1);
    const uint32_t qlds_lds = lds_addr_of(qlds);

    // Stripe gather (the wave's group, a copy of its layout): wave load
    // j < 8 brings latent bytes 1024 j .. (rows 2j, 2j+1), loads 8 and 9 the
    // rotary rows 8(j-8) .. +7, and lanes 0..3 bring the 64-byte scale block.
    // Rows at or past the sequence end read token 0 of the page (always
    // valid): finite data whose softmax weight is zero. Their scales are
    // read as stored and never used.
    auto issue_stripe = [&](const uint8_t* page, int valid, uint32_t dst) {
        const uint32_t g0 = (uint32_t)(wave * kStripeBytes);
        if (valid >= kSRows) {
#pragma unroll
            for (int j = 0; j < 10; ++j) load_lds16_untracked(page, g0 + j * 1024 + lane * 16, dst + j * 1024);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 2 * j + (lane >> 5);
                const uint32_t off = r < valid ? g0 + j * 1024 + lane * 16 : (uint32_t)((lane & 31) * 16);
                load_lds16_untracked(page, off, dst + j * 1024);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = 8 * j + (lane >> 3);
                const uint32_t off = r < valid ? g0 + kStripeLat + j * 1024 + lane * 16
                                               : (uint32_t)(kStripeLat + (lane & 7) * 16);
                load_lds16_untracked(page, off, dst + kStripeLat + j * 1024);
            }
        }
        if (lane < 4) load_lds16_untracked(page, g0 + kScaleOffG + lane * 16, dst + kScaleOffG);
    };

    // Conversion of the stripe's latent bytes: pass it (0..7) takes row
    // 2 it + lane/32, E4M3 chunk lane%32 (16 values), and writes BF16 chunks
    // 2c, 2c+1 of that row, each at its swizzled slot.
    auto convert_stripe = [&](const uint8_t* src) {
        // all eight reads first, so their latencies overlap
        u32x4 raw[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) raw[it] = *(const MLA_AS3 u32x4*)(src + it * 1024 + lane * 16);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 2 * it + (lane >> 5);
            const int c = lane & 31;
            const u32x4 v = raw[it];
            const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
            bf16x8 lo, hi;
            e4m3x16_to_bf16(w, lo, hi);
            uint8_t* rowp = cvt + r * kCvtRow;
            *(MLA_AS3 bf16x8*)(rowp + (((2 * c) ^ lds_swizzle(r)) << 4)) = lo;
            *(MLA_AS3 bf16x8*)(rowp + (((2 * c + 1) ^ lds_swizzle(r)) << 4)) = hi;
        }
    };

    // LDS offsets: K fragment of latent k-step ks for key row i16 at
    // kofs[ks & 1] + 128 (ks >> 1) in the BF16 buffer; rotary k-step i at
    // rofs + 64 i in the stripe; V^T fragment of value tile dt at
    // vofs[dt & 3] + 128 (dt >> 2) in the BF16 buffer.
    int kofs[2], vofs[4];
    const int rofs = kStripeLat + i16 * kRopeBytes + g * 16;
    {
        const int vr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int i = 0; i < 2; ++i) kofs[i] = i16 * kCvtRow + (((i * 4 + g) ^ lds_swizzle(i16)) << 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vofs[i] = vr * kCvtRow + ((i16 & 1) << 3) + (((i * 2 + ((i16 & 3) >> 1)) ^ lds_swizzle(vr)) << 4);
    }

    f32x4 o[kNDT];
    const uint8_t* const q_frag = qlds + lane * 16;

    while (b < b_end || (b == b_end && n < n_end)) {
        const int nseq = b == b_first ? len0 : ld_const_i(a.seqlens, b);
        const int npages = pages_of(nseq);
        const int hi = (b == b_end) ? n_end : npages;
        if (n >= hi) { ++b; n = 0; continue; }
        const int lo = n;

        const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
        auto page_ptr = [&](int phys) {
            return reinterpret_cast<const uint8_t*>(a.kv) + (size_t)phys * kF8PageBytes;
        };
        auto stripe_valid = [&](int pn) { return nseq - pn * kPageRows - wave * kSRows; };

        {
            const uint16_t* q_blk = a.q + ((size_t)b * a.M + rb * 16) * kHeadDim;
            const uint32_t q_off = (uint32_t)(((row_ok ? i16 : 0) * kHeadDim + g * 8) * 2);
            // latent k-steps 4w .. 4w+3 below 15 into the shared buffer; the
            // last latent k-step and the two rotary ones into this wave's
            // second stripe buffer, to be read into registers
#pragma unroll
            for (int i = 0; i < kQLatSteps / kWaves; ++i) {
                const int ks = wave * (kQLatSteps / kWaves) + i;
                if (ks < kQLdsSteps) load_lds16_untracked(q_blk, q_off + ks * 64, qlds_lds + ks * 1024);
            }
#pragma unroll
            for (int i = 0; i < 1 + kQRopeSteps; ++i)
                load_lds16_untracked(q_blk, q_off + (kQLdsSteps + i) * 64, mine1_lds + i * 1024);
        }
        // Two stripes are in flight while a page is computed: a page's stripe
        // buffer is free once its latent bytes are converted and its rotary
        // rows and scales are in registers, so the stripe two pages ahead
        // goes into it then. The second buffer holds the query's last latent
        // and rotary k-steps until they are in registers.
        issue_stripe(page_ptr(ld_const_i(bt_row, lo)), stripe_valid(lo), mine0_lds);
        int phys2 = ld_const_i(bt_row, lo + 1 < hi ? lo + 1 : lo);
        wait_then_fence<kWaitStripe>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const bf16x8 qlast = lds_read16(mine1 + lane * 16);
        bf16x8 qr[kQRopeSteps];
#pragma unroll
        for (int i = 0; i < kQRopeSteps; ++i) qr[i] = lds_read16(mine1 + (1 + i) * 1024 + lane * 16);
        wait_then_fence<kWaitLgkm>();
        if (lo + 1 < hi) issue_stripe(page_ptr(phys2), stripe_valid(lo + 1), mine1_lds);
        phys2 = ld_const_i(bt_row, lo + 2 < hi ? lo + 2 : hi - 1);

        const int L = a.causal ? min(max(nseq - a.s_q + tok + 1, 0), nseq) : nseq;
        float m_ref = -INFINITY, l_run = 0.f;
        const bool full = (lo == 0) && (hi == npages);
        const int slotno = full ? 0 : ld_const_i(seqinfo, 4 * b + 0) + (p - ld_const_i(seqinfo, 4 * b + 1));

        // Page pn: its stripe is in `cur` (stripe pn+1, if any, behind it).
        auto page_step = [&](int pn, uint8_t* cur, uint32_t cur_lds) -> int {
            if (pn + 1 < hi) wait_then_fence<kWaitStripe>();
            else wait_then_fence<kWaitAll>();
            // rotary K fragments and the lane's four key scales to registers,
            // the latent bytes converted; then the buffer takes stripe pn+2
            bf16x8 kr[kQRopeSteps];
#pragma unroll
            for (int i = 0; i < kQRopeSteps; ++i) kr[i] = lds_read16(cur + rofs + i * 64);
            const f32x4 sc4 = *(const MLA_AS3 f32x4*)(cur + kScaleOffG + 16 * g);
            convert_stripe(cur);
            wait_then_fence<kWaitLgkm>();
            if (pn + 2 < hi) issue_stripe(page_ptr(phys2), stripe_valid(pn + 2), cur_lds);
            phys2 = ld_const_i(bt_row, pn + 3 < hi ? pn + 3 : hi - 1);

            // ---- S^T = K Q^T: latent (scaled below) and rotary parts apart
            f32x4 s_lat = {0.f, 0.f, 0.f, 0.f}, s_rope = {0.f, 0.f, 0.f, 0.f};
            {
                constexpr int KD = 4;
                auto k_off = [&](int ks) { return kofs[ks & 1] + (ks >> 1) * 128; };
                bf16x8 kf[KD], qf[KD];
#pragma unroll
                for (int d = 0; d < KD; ++d) {
                    kf[d] = lds_read16(cvt + k_off(d));
                    qf[d] = lds_read16(q_frag + d * 1024);
                }
#pragma unroll
                for (int ks = 0; ks < kQLatSteps; ++ks) {
                    s_lat = mfma16(kf[ks % KD], ks < kQLdsSteps ? qf[ks % KD] : qlast, s_lat);
                    if (ks + KD < kQLatSteps) kf[ks % KD] = lds_read16(cvt + k_off(ks + KD));
                    if (ks + KD < kQLdsSteps) qf[ks % KD] = lds_read16(q_frag + (ks + KD) * 1024);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < kQRopeSteps; ++i) s_rope = mfma16(kr[i], qr[i], s_rope);
            }

            // ---- mask, per-token scale, reference check (log2 domain)
            const int key0 = pn * kPageRows + wave * kSRows + 4 * g;
            // lane group g holds keys 4g..4g+3 of the stripe
            float sck[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sck[j] = (key0 + j < L) ? sc4[j] : 0.f;
            f32x4 s;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = (key0 + j < L) ? fmaf(s_lat[j], sck[j], s_rope[j]) * a.scale_log2 : -INFINITY;
                s[j] = v;
                mx = fmaxf(mx, v);
            }
            mx = max_over_kgroups(mx);
            if (m_ref == -INFINITY) m_ref = mx == -INFINITY ? -INFINITY : mx + kRefMargin;
            const bool over = mx > m_ref + kHeadroom;
            if (__ballot(over) != 0) {
                if (over) m_ref = mx + kRefMargin;
                return -1;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
            f32x4 pw;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = __builtin_amdgcn_exp2f(s[j] - m_use);
                l_run += e;
                pw[j] = e * sck[j];     // the value product sees p_t * scale_t
            }
            const bf16x4 pf = pack_bf16x4(pw);

            // ---- O^T += V^T P^T from the BF16 latent buffer
            {
                constexpr int VD = 8;
                auto v_off = [&](int dt) { return vofs[dt & 3] + (dt >> 2) * 128; };
                bf16x4 vf[VD];
#pragma unroll
                for (int d = 0; d < VD; ++d) vf[d] = lds_read_tr(cvt + v_off(d));
#pragma unroll
                for (int dt = 0; dt < kNDT; ++dt) {
                    o[dt] = mfma16k16(vf[dt % VD], pf, o[dt]);
                    if (dt + VD < kNDT) vf[dt % VD] = lds_read_tr(cvt + v_off(dt + VD));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            return pn + 1;
        };

        bool restart;
        do {
#pragma unroll
            for (int dt = 0; dt < kNDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            l_run = 0.f;
            int pn = lo;
            while (true) {
                pn = page_step(pn, mine0, mine0_lds);
                if (pn < 0 || pn >= hi) break;
                pn = page_step(pn, mine1, mine1_lds);
                if (pn < 0 || pn >= hi) break;
            }
            restart = pn < 0;
            // after a restart the stripes in flight must land before the
            // buffers are reused
            wait_then_fence<kWaitAll>();
            if (restart) {
                issue_stripe(page_ptr(ld_const_i(bt_row, lo)), stripe_valid(lo), mine0_lds);
                if (lo + 1 < hi) issue_stripe(page_ptr(ld_const_i(bt_row, lo + 1)), stripe_valid(lo + 1), mine1_lds);
                phys2 = ld_const_i(bt_row, lo + 2 < hi ? lo + 2 : hi - 1);
            }
        } while (restart);

        // ---- merge the four waves' (m, l, O) through LDS: tiles 0..15 and
        // m, l in the stripe buffers (20 KB), tiles 16..31 in the BF16 buffer
        float lsum = l_run;
        lsum = sum_over_kgroups(lsum);
        {
            float* w0 = reinterpret_cast<float*>(mine0);
            float* w1 = reinterpret_cast<float*>(cvt);
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
        float mw[kWaves], lw[kWaves];
        float mmax = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* ml = reinterpret_cast<const float*>(wlds[w]) + 4096;
            mw[w] = ml[i16];
            lw[w] = ml[16 + i16];
            mmax = fmaxf(mmax, lw[w] > 0.f ? mw[w] : -INFINITY);
        }
        const float mref = mmax == -INFINITY ? 0.f : mmax;
        float ltot = 0.f, scw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            scw[w] = lw[w] > 0.f ? __builtin_amdgcn_exp2f(mw[w] - mref) : 0.f;
            ltot += lw[w] * scw[w];
        }
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        const float lse_v = ltot > 0.f ? (mref + __log2f(ltot)) * kLn2 : -INFINITY;
        f32x4 res[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) res[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile0 = (wave & 1) * 8;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint8_t* base = wave < 2 ? wlds[w] : wlds[w] + 2 * kStripeBytes;
            const float* src = reinterpret_cast<const float*>(base) + tile0 * 256 + lane * 4;
            const float f = scw[w] * inv;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(src + t * 256);
                res[t][0] += f * v[0]; res[t][1] += f * v[1]; res[t][2] += f * v[2]; res[t][3] += f * v[3];
            }
        }
        if (row_ok) {
            const int col0 = wave * 128 + 4 * g;
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
                if (wave == 0 && g == 0)
                    __hip_atomic_store(&a.part_lse[(size_t)row * a.lse_stride + slotno], lse_v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
        if (!full && a.counters) count_partial_and_combine<256, 16>(a, b, rb, reinterpret_cast<int*>(qlds));
        ++b;
        n = 0;
    }
    if (a.counters) write_empty_sequences<256>(a);
}

hipError_t launch_decode_rows16_fp8(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(mla_decode_rows16_fp8_kernel, dim3(plan.P * plan.R), dim3(256), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mla
