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
// block of query rows. Per page:
//   1. gather: the page named by the block table streams HBM -> LDS with
//      16-byte direct loads, double-buffered so the next page is in flight
//      while this one is used; rows are XOR-swizzled against bank conflicts;
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

namespace mla {

// Wave layout: NW waves; wave w owns query rows 16*(w / NC) .. +15 of the
// workgroup's row block and value columns (w % NC) * 512/NC .. +512/NC.
// Each wave computes the scores of its 16 rows for the whole page (waves that
// share rows repeat that product) and the output of its own columns.
template <int NW, int NC>
__global__ __launch_bounds__(NW * 64) void mla_decode_kernel(DecodeArgs a) {
    constexpr int RG = NW / NC;           // row groups per workgroup
    constexpr int TM = 16 * RG;           // query rows per workgroup
    constexpr int DCOLS = kHeadDimV / NC; // value columns per wave
    constexpr int NDT = DCOLS / 16;       // 16-column output tiles per wave
    constexpr int WLW = (kPageBytes / 1024) / NW;  // 1 KB wave loads per wave per page
    constexpr int KS = kHeadDim / 32;     // 18 k-steps of the score product
    static_assert((kPageBytes / 1024) % NW == 0 && WLW % 9 == 0, "page split across waves");
    constexpr float kRescaleLog2 = 8.f;   // lazy rescale threshold (p <= 2^8)

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kPageBytes];

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

    const int32_t* part = a.meta + kMetaHeader + 4 * p;
    int b = part[0];
    int n = part[1];
    const int b_end = part[2];
    const int n_end = part[3];
    const int32_t* seqinfo = a.meta + kMetaHeader + 4 * a.P;

    auto inside = [&](int bb, int nn) { return bb < b_end || (bb == b_end && nn < n_end); };
    auto seg_hi = [&](int bb) { return bb == b_end ? n_end : pages_of(a.seqlens[bb]); };

    while (inside(b, n) && n >= seg_hi(b)) { ++b; n = 0; }
    if (!inside(b, n)) return;

    const int row = rb * TM + rg * 16 + i16;   // query row within the sequence
    const bool row_ok = row < a.M;
    const int tok = row_ok ? row / a.h_q : 0;  // which new token the row belongs to

    // Page gather. Chunk k (16 B) of a page's LDS image holds row k/72,
    // chunk slot k%72 = that row's logical chunk slot^swz(row). Nine 1 KB
    // wave loads cover exactly eight rows, so a lane's nine (row, offset)
    // pairs repeat every eight rows; they are computed once. Row-in-group
    // (0..7) rides in the low bits of the 16-byte-aligned offset.
    int goff[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) {
        const int k = j * 64 + lane;
        const int r = k / kRowChunks;
        const int c = k - r * kRowChunks;
        goff[j] = (r * kRowBytes + ((c ^ lds_swizzle(r)) << 4)) | r;
    }
    // Rows at or past the sequence end are not loaded; their LDS chunks are
    // zero-filled, so tails never inject NaN/Inf (a zero key row scores 0 and
    // is masked, a zero value row adds nothing).
    auto issue_page = [&](int bb, int nn, int buf) {
        const int phys = a.block_table[(size_t)bb * a.max_blocks + nn];
        const int valid = min(kPageRows, a.seqlens[bb] - nn * kPageRows);
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv) + (size_t)phys * kPageBytes;
        uint8_t* dst = lds + buf * kPageBytes;
#pragma unroll
        for (int i = 0; i < WLW; ++i) {
            const int wl = wave * WLW + i;
            const int grp = wave * (WLW / 9) + i / 9;   // wl / 9
            const int off = goff[i % 9];                // wl % 9 (compile-time index)
            const int r = grp * 8 + (off & 7);
            if (r < valid) {
                load_lds16(src + grp * 9216 + (off & ~15), dst + wl * 1024);
            } else {
                *reinterpret_cast<uint4*>(dst + wl * 1024 + lane * 16) = uint4{0u, 0u, 0u, 0u};
            }
        }
    };

    bf16x8 qf[KS];
    f32x4 o[NDT];
    float m_run = -INFINITY, l_run = 0.f;
    int L = 0, seg_lo = n;

    int buf = 0;
    issue_page(b, n, 0);
    bool seg_start = true;
    while (true) {
        int nb = b, nn = n + 1;
        while (inside(nb, nn) && nn >= seg_hi(nb)) { ++nb; nn = 0; }
        const bool has_next = inside(nb, nn);

        if (seg_start) {
            const uint16_t* qp = a.q + ((size_t)b * a.M + (row_ok ? row : 0)) * kHeadDim + g * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
                qf[ks] = row_ok ? v : bf16x8{};
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run = -INFINITY;
            l_run = 0.f;
            seg_lo = n;
            const int nseq = a.seqlens[b];
            L = a.causal ? min(max(nseq - a.s_q + tok + 1, 0), nseq) : nseq;
        }

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (has_next) issue_page(nb, nn, buf ^ 1);

        const uint8_t* pg = lds + buf * kPageBytes;

        // ---- S^T[key][row] = K[key] . Q[row], 4 tiles of 16 keys. The LDS
        // reads of k-step ks+1 are issued before the MFMAs of k-step ks; the
        // scheduling fence keeps the compiler from hoisting further reads,
        // which bounds the live operand registers to two k-steps.
        f32x4 s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        int koff[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) koff[kt] = (kt * 16 + i16) * kRowBytes;
        const int ksw = lds_swizzle(i16);   // row kt*16+i16 has the same low 3 bits
        bf16x8 kfa[4], kfb[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kfa[kt] = lds_read16(pg + koff[kt] + ((g ^ ksw) << 4));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8* cur = (ks & 1) ? kfb : kfa;
            bf16x8* nxt = (ks & 1) ? kfa : kfb;
            if (ks + 1 < KS) {
                const int c = (ks + 1) * 4 + g;
                const int co = ((c & 7) ^ ksw) << 4 | (c >> 3) << 7;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) nxt[kt] = lds_read16(pg + koff[kt] + co);
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) s[kt] = mfma16(cur[kt], qf[ks], s[kt]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- mask and online softmax (log2 domain). Lane holds row i16 and
        // keys kt*16 + 4g + j of this page.
        const int key0 = n * kPageRows + 4 * g;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
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
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = __builtin_amdgcn_exp2f(s[kt][j] - m_use);
                s[kt][j] = e;
                psum += e;
            }
        }
        l_run += psum;

        // P^T operand for keys 32u..32u+31: k-slot 8g+j <-> key 32u+4g+j,
        // 8g+4+j <-> key 32u+16+4g+j. Exactly the lane's own score registers.
        const bf16x8 pf0 = pack_bf16x8(s[0], s[1]);
        const bf16x8 pf1 = pack_bf16x8(s[2], s[3]);

        // ---- O^T[dim][row] += V^T[dim][key] P^T[key][row]
        // The V^T operand for k-slots 8g..8g+7 needs keys 32u+4g+0..3 and
        // 32u+16+4g+0..3 of one dim; two transposing reads deliver them.
        const int vr = 4 * g + (i16 >> 2);          // key row for u = 0
        const int vsw = lds_swizzle(vr);            // same for vr+16, vr+32, vr+48
        const int vhalf = (i16 & 1) << 3;
        const int vbase = vr * kRowBytes + vhalf;
        auto v_addr = [&](int dt) {
            const int c = ((cg * DCOLS + dt * 16) >> 3) + ((i16 & 3) >> 1);
            return pg + vbase + ((((c & 7) ^ vsw) << 4) | ((c >> 3) << 7));
        };
        bf16x4 va[4], vb[4];
        {
            const uint8_t* vp = v_addr(0);
            va[0] = lds_read_tr(vp);
            va[1] = lds_read_tr(vp + 16 * kRowBytes);
            va[2] = lds_read_tr(vp + 32 * kRowBytes);
            va[3] = lds_read_tr(vp + 48 * kRowBytes);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            bf16x4* cur = (dt & 1) ? vb : va;
            bf16x4* nxt = (dt & 1) ? va : vb;
            if (dt + 1 < NDT) {
                const uint8_t* vp = v_addr(dt + 1);
                nxt[0] = lds_read_tr(vp);
                nxt[1] = lds_read_tr(vp + 16 * kRowBytes);
                nxt[2] = lds_read_tr(vp + 32 * kRowBytes);
                nxt[3] = lds_read_tr(vp + 48 * kRowBytes);
            }
            o[dt] = mfma16(cat_bf16x4(cur[0], cur[1]), pf0, o[dt]);
            o[dt] = mfma16(cat_bf16x4(cur[2], cur[3]), pf1, o[dt]);
            __builtin_amdgcn_sched_barrier(0);
        }

        const bool seg_end = !has_next || nb != b;
        if (seg_end) {
            float lsum = l_run;
            lsum += wave_xor(lsum, 16);
            lsum += wave_xor(lsum, 32);
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            const float lse_v = lsum > 0.f ? (m_run + __log2f(lsum)) * kLn2 : -INFINITY;
            const bool full = (seg_lo == 0) && (n + 1 == pages_of(a.seqlens[b]));
            if (full) {
                if (row_ok) {
                    uint16_t* op = a.out + ((size_t)b * a.M + row) * kHeadDimV + cg * DCOLS + 4 * g;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        bf16x4 v;
                        v[0] = (__bf16)(o[dt][0] * inv); v[1] = (__bf16)(o[dt][1] * inv);
                        v[2] = (__bf16)(o[dt][2] * inv); v[3] = (__bf16)(o[dt][3] * inv);
                        *reinterpret_cast<bf16x4*>(op + dt * 16) = v;
                    }
                    if (cg == 0 && g == 0) a.lse[(size_t)b * a.M + row] = lse_v;
                }
            } else {
                const int slot = seqinfo[4 * b + 0] + (p - seqinfo[4 * b + 1]);
                if (row_ok) {
                    float* pp = a.part_o + ((size_t)slot * a.M + row) * kHeadDimV + cg * DCOLS + 4 * g;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        f32x4 v = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
                        *reinterpret_cast<f32x4*>(pp + dt * 16) = v;
                    }
                    if (cg == 0 && g == 0) a.part_lse[(size_t)slot * a.M + row] = lse_v;
                }
            }
        }
        if (!has_next) break;
        seg_start = nb != b;
        b = nb;
        n = nn;
        buf ^= 1;
    }
}

hipError_t launch_decode(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    const dim3 grid(plan.P * plan.R);
    if (plan.nw == 4 && plan.nc == 4) {
        hipLaunchKernelGGL((mla_decode_kernel<4, 4>), grid, dim3(256), 0, stream, args);
    } else if (plan.nw == 4 && plan.nc == 2) {
        hipLaunchKernelGGL((mla_decode_kernel<4, 2>), grid, dim3(256), 0, stream, args);
    } else if (plan.nw == 4 && plan.nc == 1) {
        hipLaunchKernelGGL((mla_decode_kernel<4, 1>), grid, dim3(256), 0, stream, args);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mla
