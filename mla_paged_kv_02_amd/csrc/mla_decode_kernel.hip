// mla_decode_kernel.hip - split-KV MLA decode over a paged latent cache, gfx950.
//
// Method (page "MLA 和 MHA 的 Kernel 区别", section "FlashAttention 适配的差异" /
// "MLA 的 FlashAttention"): stream the latent cache through on-chip memory
// one tile of tokens at a time and score the query against the tile. Here a
// tile is one 64-token page of the paged cache (FlashMLA overview page:
// block size 64), and the query is in absorbed form, so the page rows are the
// keys and their first 512 values are the values; no up-projection happens
// in the loop. All h_q*s_q query rows of a sequence share the page, which is
// what makes both products dense matrix products (same page, same section:
// the decompressed tile stays on chip and is reused by many queries).
//
// Per workgroup: a partition of the page list (from the split plan) and one
// block of query rows. Per half page (32 keys):
//   1. gather: the page named by the block table streams HBM -> LDS with
//      16-byte direct loads into a 4-slot ring, three half pages ahead of
//      the one in use; rows are XOR-swizzled against bank conflicts;
//   2. S^T = K Q^T on BF16 MFMA (16x16x32), Q resident in registers;
//   3. mask + online softmax in the exp2 domain (running max m and sum l per
//      row, wavefront shuffles for the row max);
//   4. O^T += V^T P^T on MFMA, V read from the same LDS page with transposing
//      reads, P taken from the score registers without any data movement;
//   5. at the end of a sequence's run of pages: the final BF16 output and
//      log-sum-exp, or FP32 partials for the combine kernel when the
//      sequence was cut between partitions.
// The one-pass (online) softmax replaces the page's two-pass pseudo-code,
// which reads the latent cache a second time for the weighted sum
// ("Decode 阶段的 HBM 访问模式" / "MLA Decode"); both give the same result.
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_sched.h"
#include "mla_store_asm.h"

#include <type_traits>

namespace mla {

// Read-only metadata through the scalar path: the constant address space
// tells the compiler these words are never written while the kernel runs, so
// uniform loads become scalar loads (they must not count as vector memory
// operations, which the ring's wait counts rely on).
__device__ __forceinline__ int ld_const(const int32_t* p, size_t i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        reinterpret_cast<uintptr_t>(p))[i];
}

// Waits until at most N of this wave's vector memory loads are outstanding
// and its LDS operations are done, then meets the other waves at a barrier.
// The wait is the compiler's own s_waitcnt, so its wait-count tracking knows
// the older loads (earlier ring chunks) are complete and adds no wait of its
// own before reading them; the empty asm keeps memory accesses from moving
// across the barrier.
template <int N>
__device__ __forceinline__ void ring_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 encoding: vmcnt[3:0] | expcnt[6:4]=7 (no wait) | lgkmcnt[11:8]=0 | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wave layout: NW waves; wave w owns query rows 16*(w / NC) .. +15 of the
// workgroup's row block and value columns (w % NC) * 512/NC .. +512/NC.
// Each wave computes the scores of its 16 rows for every key (waves that
// share rows repeat that product) and the output of its own columns.
//
// Pipeline: keys stream through LDS in 32-row half pages ("chunks") held in
// a ring of 4 slots; while a chunk is consumed the next three are in flight,
// which keeps enough bytes outstanding per CU to cover HBM latency. Every
// chunk is exactly 9 16-byte wave loads per wave and every step issues one
// chunk, so the wait for chunk k is "at most 18 loads outstanding".
template <int NW, int NC>
__global__ __launch_bounds__(NW * 64) void mla_decode_kernel(DecodeArgs a) {
    constexpr int RG = NW / NC;           // row groups per workgroup
    constexpr int TM = 16 * RG;           // query rows per workgroup
    constexpr int DCOLS = kHeadDimV / NC; // value columns per wave
    constexpr int NDT = DCOLS / 16;       // 16-column output tiles per wave
    constexpr int KS = kHeadDim / 32;     // 18 k-steps of the score product
    constexpr int CROWS = 32;             // keys per chunk
    constexpr int CBYTES = CROWS * kRowBytes;  // 36864
    constexpr int NSLOT = 4;
    constexpr int LOADS = (CBYTES / 1024) / NW;  // 16-byte wave loads per wave per chunk
    static_assert(NW == 4 && LOADS == 9, "one 8-row group of a chunk per wave");
    constexpr float kRescaleLog2 = 8.f;   // lazy rescale threshold (p <= 2^8)
    constexpr int KD = 4;                 // K operand prefetch depth (k-steps)
    constexpr int VD = 8;                 // V operand prefetch depth (tiles)

    // One LDS object per ring slot. Reads of the slot in use and the direct
    // loads into the slot being refilled then touch provably distinct
    // objects, so the compiler does not make the reads wait for the loads.
    __shared__ __attribute__((aligned(16))) uint8_t ring0[CBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[CBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[CBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[CBYTES];
    auto ring = [&](auto sc) -> uint8_t* {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0) return ring0;
        else if constexpr (S == 1) return ring1;
        else if constexpr (S == 2) return ring2;
        else return ring3;
    };

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = wave / NC;
    const int cg = wave % NC;
    const int g = lane >> 4;      // k-group of the MFMA operand layout
    const int i16 = lane & 15;    // row (query) index inside the 16-row tile

    // Block id -> (partition, row block). Blocks are dispatched round-robin
    // over the 8 XCDs; the R row blocks of one partition get ids 8 apart so
    // they share an XCD and its L2 while reading the same pages.
    const int bid = blockIdx.x;
    const int rb = (bid >> 3) % a.R;
    const int p = ((bid >> 3) / a.R) * 8 + (bid & 7);

    const int b_end = ld_const(a.meta, kMetaHeader + 4 * p + 2);
    const int n_end = ld_const(a.meta, kMetaHeader + 4 * p + 3);
    const int32_t* seqinfo = a.meta + kMetaHeader + 4 * a.P;

    auto seqlen = [&](int bb) { return ld_const(a.seqlens, bb); };
    auto inside = [&](int bb, int nn) { return bb < b_end || (bb == b_end && nn < n_end); };
    auto seg_hi = [&](int bb) { return bb == b_end ? n_end : pages_of(seqlen(bb)); };

    // chunk cursor: sequence b, page n, half h (keys 64n + 32h ..)
    struct Cur { int b, n, h; };
    auto exists = [&](const Cur& c) { return inside(c.b, c.n); };
    auto advance = [&](const Cur& c) {
        if (c.h == 0 && seqlen(c.b) - c.n * kPageRows > CROWS) return Cur{c.b, c.n, 1};
        int nb = c.b, nn = c.n + 1;
        while (inside(nb, nn) && nn >= seg_hi(nb)) { ++nb; nn = 0; }
        return Cur{nb, nn, 0};
    };

    Cur cur{ld_const(a.meta, kMetaHeader + 4 * p), ld_const(a.meta, kMetaHeader + 4 * p + 1), 0};
    while (inside(cur.b, cur.n) && cur.n >= seg_hi(cur.b)) { ++cur.b; cur.n = 0; }
    if (!exists(cur)) return;

    const int row = rb * TM + rg * 16 + i16;   // query row within the sequence
    const bool row_ok = row < a.M;
    const int tok = row_ok ? row / a.h_q : 0;  // which new token the row belongs to

    // Chunk gather: wave w loads rows 8w..8w+7 of the chunk. LDS chunk slot k
    // (16 B) of the wave's 9 KB holds row k/72, slot k%72 = that row's logical
    // chunk slot^swz(row). Rows at or past the sequence end read the page's
    // first kilobyte instead (row 0, always valid when the chunk is used):
    // finite data whose softmax weight is zero, so tails never inject NaN/Inf
    // and every chunk costs the same number of loads.
    int goff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int k = j * 64 + lane;
        const int r = k / kRowChunks;
        const int c = k - r * kRowChunks;
        goff[j] = (r * kRowBytes + ((c ^ lds_swizzle(r)) << 4)) | r;
    }
    auto issue_chunk = [&](const Cur& c, auto sc) {
        const int phys = ld_const(a.block_table, (size_t)c.b * a.max_blocks + c.n);
        const int valid = seqlen(c.b) - c.n * kPageRows - c.h * CROWS;  // rows of this chunk in use
        const uint8_t* page = reinterpret_cast<const uint8_t*>(a.kv) + (size_t)phys * kPageBytes;
        const uint8_t* src = page + c.h * CBYTES + wave * 9216;
        uint8_t* dst = ring(sc) + wave * 9216;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int off = goff[j];
            const int r = wave * 8 + (off & 7);
            const uint8_t* gp = r < valid ? src + (off & ~15) : page + lane * 16;
            load_lds16(gp, dst + j * 1024);
        }
    };

    bf16x8 qf[KS];
    f32x4 o[NDT];
    float m_run = -INFINITY, l_run = 0.f;
    int L = 0, seg_lo = cur.n;

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    // Step j refills slot j%4 with chunk j and consumes chunk j-3 from slot
    // (j+1)%4 (nothing during the first three steps). Every step issues
    // exactly one chunk's loads, so a slot's loads are always followed by two
    // steps' worth of loads before the slot is read, and all direct-to-LDS
    // loads come from the loop body itself: the compiler then proves the
    // slot read is covered by the step's wait and adds none of its own. Past
    // the partition's last chunk the refill re-reads the first chunk (an L2
    // hit) into the free slot.
    const Cur first = cur;
    Cur held[NSLOT] = {first, first, first, first};   // chunk in each slot
    bool real[NSLOT] = {false, false, false, false};  // slot holds an unconsumed chunk
    Cur last = first;
    bool more = true, started = false;
    bool seg_start = true;
    auto step = [&](auto sc) -> bool {
        constexpr int S = decltype(sc)::value;   // slot refilled this step
        constexpr int C = (S + 1) % NSLOT;       // slot consumed this step
        constexpr int N = (S + 2) % NSLOT;       // slot of the chunk after it
        Cur nxt = first;
        bool nreal = false;
        if (more) {
            const Cur c = started ? advance(last) : first;
            started = true;
            if (exists(c)) {
                nxt = c;
                nreal = true;
                last = c;
            } else {
                more = false;
            }
        }
        const bool consume = real[C];
        const Cur cur = held[C];

        if (consume && seg_start) {
            const uint16_t* qp = a.q + ((size_t)cur.b * a.M + (row_ok ? row : 0)) * kHeadDim + g * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
                qf[ks] = row_ok ? v : bf16x8{};
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run = -INFINITY;
            l_run = 0.f;
            seg_lo = cur.n;
            const int nseq = seqlen(cur.b);
            L = a.causal ? min(max(nseq - a.s_q + tok + 1, 0), nseq) : nseq;
            // the query loads were issued after the chunks in flight: drain all
            ring_barrier<0>();
        } else {
            // chunk j-3 landed once at most the two later chunks' loads are pending
            ring_barrier<2 * LOADS>();
        }
        // every wave is past its reads of chunk j-4, whose slot is refilled now
        issue_chunk(nxt, sc);
        held[S] = nxt;
        real[S] = nreal;
        if (!consume) return true;   // pipeline warm-up
        real[C] = false;

        const uint8_t* pg = ring(std::integral_constant<int, C>{});

        // ---- S^T[key][row] = K[key] . Q[row], 2 tiles of 16 keys. LDS reads
        // run KD k-steps ahead of the MFMAs that use them (a ring of operand
        // registers); the scheduling fence after each k-step keeps that order.
        f32x4 s[2];
        s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int koff0 = i16 * kRowBytes;
        const int koff1 = (16 + i16) * kRowBytes;
        const int ksw = lds_swizzle(i16);   // row 16+i16 has the same low 3 bits
        auto k_off = [&](int ks) {
            const int c = ks * 4 + g;
            return (((c & 7) ^ ksw) << 4) | ((c >> 3) << 7);
        };
        bf16x8 kf[KD][2];
#pragma unroll
        for (int d = 0; d < KD; ++d) {
            kf[d][0] = lds_read16(pg + (koff0 + k_off(d)));
            kf[d][1] = lds_read16(pg + (koff1 + k_off(d)));
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[0] = mfma16(kf[ks % KD][0], qf[ks], s[0]);
            s[1] = mfma16(kf[ks % KD][1], qf[ks], s[1]);
            if (ks + KD < KS) {
                kf[ks % KD][0] = lds_read16(pg + (koff0 + k_off(ks + KD)));
                kf[ks % KD][1] = lds_read16(pg + (koff1 + k_off(ks + KD)));
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- mask and online softmax (log2 domain). Lane holds row i16 and
        // keys kt*16 + 4g + j of this chunk.
        const int key0 = cur.n * kPageRows + cur.h * CROWS + 4 * g;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = (key0 + kt * 16 + j < L) ? s[kt][j] * a.scale_log2 : -INFINITY;
                s[kt][j] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = fmaxf(mx, wave_xor(mx, 16));
        mx = fmaxf(mx, wave_xor(mx, 32));
        // Lazy rescale: the reference max m_run only moves (and O, l are only
        // rescaled) when a row's max exceeds it by more than 2^8 in ratio, so
        // every weight exp2(s - m_run) stays <= 2^8. O and l always share the
        // same reference, so O / l is unchanged: an exact rewrite.
        const bool grow = mx > m_run + kRescaleLog2;   // true on a row's first visible key
        if (__ballot(grow) != 0) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                o[dt][0] *= alpha; o[dt][1] *= alpha; o[dt][2] *= alpha; o[dt][3] *= alpha;
            }
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = __builtin_amdgcn_exp2f(s[kt][j] - m_use);
                s[kt][j] = e;
                psum += e;
            }
        }
        l_run += psum;

        // P^T operand: k-slot 8g+j <-> key 4g+j, 8g+4+j <-> key 16+4g+j of the
        // chunk. Exactly the lane's own score registers.
        const bf16x8 pf = pack_bf16x8(s[0], s[1]);

        // ---- O^T[dim][row] += V^T[dim][key] P^T[key][row]
        // The V^T operand for k-slots 8g..8g+7 needs keys 4g+0..3 and
        // 16+4g+0..3 of one dim; two transposing reads deliver them.
        const int vr = 4 * g + (i16 >> 2);          // key row
        const int vsw = lds_swizzle(vr);            // same for vr+16
        const int vbase = vr * kRowBytes + ((i16 & 1) << 3);
        // byte offset in the chunk of dim tile dt, key half kh (keys +16*kh);
        // each read is formed as one base + offset so the compiler keeps
        // track of which LDS array it reads
        auto v_off = [&](int dt, int kh) {
            const int c = ((cg * DCOLS + dt * 16) >> 3) + ((i16 & 3) >> 1);
            return vbase + kh * 16 * kRowBytes + ((((c & 7) ^ vsw) << 4) | ((c >> 3) << 7));
        };
        // V operands run VD tiles ahead of the MFMAs that use them.
        constexpr int VDD = NDT < VD ? NDT : VD;
        bf16x4 vf[VDD][2];
#pragma unroll
        for (int d = 0; d < VDD; ++d) {
            vf[d][0] = lds_read_tr(pg + v_off(d, 0));
            vf[d][1] = lds_read_tr(pg + v_off(d, 1));
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            o[dt] = mfma16(cat_bf16x4(vf[dt % VDD][0], vf[dt % VDD][1]), pf, o[dt]);
            if (dt + VDD < NDT) {
                vf[dt % VDD][0] = lds_read_tr(pg + v_off(dt + VDD, 0));
                vf[dt % VDD][1] = lds_read_tr(pg + v_off(dt + VDD, 1));
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        const bool seg_end = !real[N] || held[N].b != cur.b;
        if (seg_end) {
            float lsum = l_run;
            lsum += wave_xor(lsum, 16);
            lsum += wave_xor(lsum, 32);
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            const float lse_v = lsum > 0.f ? (m_run + __log2f(lsum)) * kLn2 : -INFINITY;
            const bool full = (seg_lo == 0) && (cur.n + 1 == pages_of(seqlen(cur.b)));
            if (full) {
                if (row_ok) {
                    uint16_t* op = a.out + ((size_t)cur.b * a.M + row) * kHeadDimV + cg * DCOLS + 4 * g;
                    bf16x4 v[NDT];
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        v[dt][0] = (__bf16)(o[dt][0] * inv); v[dt][1] = (__bf16)(o[dt][1] * inv);
                        v[dt][2] = (__bf16)(o[dt][2] * inv); v[dt][3] = (__bf16)(o[dt][3] * inv);
                    }
                    TileStores<NDT>::out(op, v);
                    if (cg == 0 && g == 0) a.lse[(size_t)cur.b * a.M + row] = lse_v;
                }
            } else {
                const int slot = ld_const(seqinfo, 4 * cur.b + 0) + (p - ld_const(seqinfo, 4 * cur.b + 1));
                if (row_ok) {
                    float* pp = a.part_o + ((size_t)slot * a.M + row) * kHeadDimV + cg * DCOLS + 4 * g;
                    f32x4 v[NDT];
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
                        v[dt] = f32x4{o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
                    TileStores<NDT>::part(pp, v);
                    if (cg == 0 && g == 0) a.part_lse[(size_t)row * a.lse_stride + slot] = lse_v;
                }
            }
        }
        seg_start = seg_end;
        // continue while an issued chunk is still unconsumed
        return real[N] || real[(S + 3) % NSLOT] || real[S];
    };
    while (step(S0{}) && step(S1{}) && step(S2{}) && step(S3{})) {
    }
    // no direct-to-LDS load may land after the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(7 << 4);
}

hipError_t launch_decode(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    switch (plan.kernel) {
        case DecodeKernel::Rows16: return launch_decode_rows16(plan, args, stream);
        case DecodeKernel::Wide: return launch_decode_rows64(plan, args, stream);
        case DecodeKernel::WaveSplit: return launch_decode_ws(plan, args, stream);
        case DecodeKernel::Ring: break;
    }
    if (plan.nw == 4 && plan.nc == 2) {
        hipLaunchKernelGGL((mla_decode_kernel<4, 2>), dim3(plan.P * plan.R), dim3(256), 0, stream, args);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace mla
