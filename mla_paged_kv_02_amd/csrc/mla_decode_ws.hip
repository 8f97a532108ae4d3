// mla_decode_ws.hip - split-KV MLA decode for blocks of 16, 32 or 64 query
// rows with separate score and value waves.
//
// Method as in the other decode kernels (page "MLA 和 MHA 的 Kernel 区别",
// section "MLA 的 FlashAttention": stream latent-cache tiles through on-chip
// memory, score the query block against them, one-pass softmax; absorbed
// form). This organisation is for query blocks wide enough that the two
// products and the LDS traffic that feeds them are the work:
//
//  * score waves own key tiles (16 keys of a 32-key half page). For 64-row
//    blocks there are four, two per key tile, each holding the query of two
//    row tiles in registers, so each K fragment read from LDS feeds two row
//    tiles; for 16- and 32-row blocks two, one per key tile, each holding
//    all the block's rows. They compute S^T = K Q^T, the mask and the
//    softmax weights of their keys. Four value waves own output columns
//    128v..128v+127 of all the block's rows (O^T accumulators) and compute
//    O^T += V^T P^T. P crosses over through LDS in exactly the MFMA operand
//    layout, so each V^T fragment (two transposing LDS reads) feeds every
//    row tile. While a score wave waits on LDS or runs its exps, the value
//    wave on the same SIMD keeps the matrix core busy;
//  * the cache streams through a ring of four half-page slots (32 keys,
//    36 KB): the value waves load them with 16-byte direct loads, two half
//    pages ahead. Step c scores half page c and accumulates half page c-1;
//    one workgroup barrier per step publishes half page c, the weights of
//    half page c-1 and the overflow flags, and frees the slot the value
//    waves finished. The stream is the partition's whole page list: the
//    last steps of a segment load the first two half pages of the
//    partition's next segment, which therefore starts without a fill (its
//    half pages sit two slots further on, so a segment's slots are offset
//    by 0 or 2);
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
//
// FP8 latent cache (64-row blocks; page layout of mla_decode_fp8.h: four
// 16-token groups, each its E4M3 latent rows, BF16 rotary rows and FP32
// per-token scales; latent coordinate d of token t is e4m3 * scale[t]). The
// pipeline, the roles and the barriers are the BF16 ones; what differs is
// what a ring slot holds and how the products read it:
//
//  * a slot holds the half page as it is in memory, still E4M3 (21 KB
//    instead of 36 KB): the value waves fill it with the same untracked
//    16-byte direct loads, two half pages ahead, placing latent rows at a
//    528-byte stride (a row's 16-byte gap holds four rows' scales) and
//    permuting rotary chunks, so that both products read without bank
//    conflicts and with constant offsets;
//  * score waves read 8 latent bytes per k-step and widen them to BF16 in
//    registers (exact: every E4M3 value is a BF16 value); they keep the
//    latent and rotary parts of a score apart and combine them as
//    scale * latent + rotary;
//  * value waves read V^T with the byte-transposing LDS read (8 keys of one
//    dimension per lane) and widen it the same way; P crosses over with its
//    keys in the read's byte order, and holds p_t * scale_t (the
//    normaliser sums p_t).
// So HBM, LDS writes and the LDS reads of both products carry half the
// bytes of the BF16 path, and nothing is converted twice.
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

// block of 16 kRT rows: score waves, threads, row tiles of a score wave
template <int kRT>
struct WsShape {
    static constexpr int kScoreWaves = kRT == 4 ? 4 : 2;
    static constexpr int kThreads = 64 * (kScoreWaves + 4);
    static constexpr int kRows = 16 * kRT;
    static constexpr int NR = kRT == 1 ? 1 : 2;
};
constexpr int kCRows = 32;                      // keys per ring slot (half page)
constexpr int kCBytes = kCRows * kRowBytes;     // 36864
constexpr int kWLoads = 9;                      // a value wave's wave-loads per slot (8 rows)
constexpr int kKS = kHeadDim / 32;              // 18 k-steps of the score product
constexpr int kVTiles = 8;                      // value tiles (16 columns) per value wave
constexpr float kRefMargin = 32.f;
constexpr float kHeadroom = 64.f;

// FP8 page: four groups of 16 tokens, each 16 E4M3 latent rows (512 B), 16
// BF16 rotary rows (128 B) and 16 FP32 scales; a half page is two whole
// groups, 20608 contiguous bytes
constexpr int kF8Group = 16 * 512 + 16 * 128 + 16 * 4;   // 10304
constexpr int kF8PageBytes = 4 * kF8Group;                 // 41216
constexpr int kF8HalfBytes = 2 * kF8Group;                 // 20608
constexpr int kF8RopeOff = 16 * 512;
constexpr int kF8ScaleOff = 16 * 512 + 16 * 128;
// FP8 ring slot: a half page as loaded, still E4M3. Latent rows of 512 B at
// a stride of 528 B (16 rows at the same column fall on 16 different 16-byte
// bank groups), the 16-byte gap after latent row k < 8 holding the scales of
// rows 4k..4k+3; then the 32 rotary rows of 128 B, chunk c of row r at chunk
// slot c ^ ((r >> 1) & 7). 21 wave-loads of 1 KB fill it (the end of the
// last one is padding).
constexpr int kF8LatStride = 528;
constexpr int kF8LdsRope = kCRows * kF8LatStride;   // 16896
constexpr int kF8SlotLoads = 21;
constexpr int kF8Slot = kF8SlotLoads * 1024;        // 21504
constexpr int kF8Mine = (kF8SlotLoads + 3) / 4;     // 6: value wave v issues loads v, v+4, ..
static_assert(kF8LdsRope + kCRows * 128 <= kF8Slot, "FP8 slot layout");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 8 E4M3 values (byte k = element k) -> 8 BF16 values, exact (every E4M3
// value is a BF16 value)
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(const u32x2& w) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ u32x2 lds_read8(const uint8_t* p) { return *(const MLA_AS3 u32x2*)(p); }

// Transposing LDS read of bytes: in each group of 16 lanes, lane 2k + h
// addresses bytes 8h..8h+7 of row k of an 8 x 16 block of bytes, and lane n
// receives column n of the block (byte k from row k).
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_AS3 i32x2*)(p)));
}

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

template <int kRT, bool kFp8>
__global__ __launch_bounds__(WsShape<kRT>::kThreads) void mla_decode_ws_kernel(DecodeArgs a) {
    using Sh = WsShape<kRT>;
    constexpr int kPB = kFp8 ? kF8PageBytes : kPageBytes;
    constexpr int kRows = Sh::kRows;
    constexpr int kSW = Sh::kScoreWaves;
    constexpr int kPBytes = kRT * 1024;
    constexpr int kSlot = kFp8 ? kF8Slot : kCBytes;
    // ring slots, and how many half pages ahead of the one being scored the
    // value waves load (over the FP8 cache six slots, loading four ahead,
    // measured no faster: 190 vs 192 us at 128 heads, 4096 tokens)
    constexpr int kNS = 4;
    constexpr int kDist = kNS - 2;
    // 64-row blocks: the first segment's query block is staged from slot 2
    // on (rows of 1152 B, chunks placed as in a BF16 slot) before the ring
    // reaches those slots
    constexpr bool kQStage = kRT == 4;
    constexpr int kQOff = 2 * kSlot;
    constexpr int kRingBytes = kQStage && kQOff + kRows * kRowBytes > kNS * kSlot ? kQOff + kRows * kRowBytes
                                                                                : kNS * kSlot;

    __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
    // weights of a half page for the value waves: row tile rt at 1 KB * rt,
    // lane l at 16 l (the B operand of O^T += V^T P^T); two buffers by parity
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][kPBytes];
    // per row of the block: softmax reference, and the sums of the two key
    // tiles, for the epilogue
    __shared__ float row_m[kRows];
    __shared__ float row_l[2][kRows];
    // overflow flags by step parity: set during step c in flag[c & 1], read
    // by every wave after the next barrier
    __shared__ int restart_flag[2];
    __shared__ int last_flag;   // this workgroup merges a split sequence

    if (!plan_matches_or_poison<Sh::kThreads>(a)) return;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool scorer = wid < kSW;
    // score wave sw: key tile sw & 1 (of row pair sw >> 1 for 64-row
    // blocks); value wave sw: column block sw (and rows 8 sw..8 sw+7 of
    // every half page it loads)
    const int sw = scorer ? wid : wid - kSW;
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
    const uint32_t ring_lds = lds_addr_of(ring);

    // The partition's segments: (sequence, page range) in order, each
    // holding at least one page; b < 0 past the partition's end.
    struct Seg {
        int b, lo, hi, nseq;
    };
    auto find_seg = [&](int b, int n) {
        while (b < b_end || (b == b_end && n < n_end)) {
            const int nseq = b == b0 ? len0 : ld_const_ws(a.seqlens, b);
            const int hi = (b == b_end) ? n_end : pages_of(nseq);
            if (n < hi) return Seg{b, n, hi, nseq};
            ++b;
            n = 0;
        }
        return Seg{-1, 0, 0, 0};
    };

    // ---- value waves: the fetch stream, the partition's half pages in
    // order. fseg/fc name the next half page to take; fpage is its page.
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
    Seg fseg = find_seg(b0, n0);
    int fc = 0;
    auto fpage_of = [&]() {
        const int32_t* bt_row = a.block_table + (size_t)fseg.b * a.max_blocks;
        return reinterpret_cast<const uint8_t*>(a.kv) + (size_t)ld_const_ws(bt_row, fseg.lo + fc / 2) * kPB;
    };
    const uint8_t* fpage = nullptr;
    // the half page taken for issue: its page, which half, and the rows of
    // the page that hold tokens
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
    // the sequence end read the page's first kilobyte (row 0, always
    // valid): finite data whose softmax weight is zero.
    auto issue_bf16 = [&](uint32_t dst, int j) {
        const int base = t_half * kCBytes + sw * 9216;
        const int r = t_half * kCRows + sw * 8 + (j * 64 + lane) / kRowChunks;
        const uint32_t off = r < t_rows ? (uint32_t)(base + goff[j]) : (uint32_t)(lane * 16);
        load_lds16_untracked(t_src, off, dst + sw * 9216 + j * 1024);
    };

    // FP8: this wave's loads of a slot are numbers sw + 4 i (i < 6 for value
    // wave 0, i < 5 for the others; 21 in all), lane l of load j filling
    // chunk position 64 j + l of the slot. f8_src[i]: that chunk's source
    // offset in the half page. f8_alt[i]: 64 * (source offset in the page of
    // the same chunk of the page's row 0) + 1 + (the chunk's row of the half
    // page), or 0 for a chunk read as it is (scales, padding). Rows at or
    // past the sequence end read row 0 of the page (a written token: finite);
    // their scales are read as they are and never used.
    int f8_src[kF8Mine], f8_alt[kF8Mine];
    if constexpr (kFp8) {
#pragma unroll
        for (int i = 0; i < kF8Mine; ++i) {
            const int pos = (sw + 4 * i) * 64 + lane;
            int src = 0, alt = 0;
            if (pos < kF8LdsRope / 16) {
                const int r = pos / (kF8LatStride / 16);
                const int q = pos - r * (kF8LatStride / 16);
                if (q < 32) {
                    src = (r >> 4) * kF8Group + (r & 15) * 512 + 16 * q;
                    alt = ((16 * q) << 6) + 1 + r;
                } else if (r < 8) {
                    // scales of rows 4r..4r+3 (one group)
                    src = (r >> 2) * kF8Group + kF8ScaleOff + 16 * (r & 3);
                }
            } else if (pos < (kF8LdsRope + kCRows * 128) / 16) {
                const int pp = pos - kF8LdsRope / 16;
                const int r = pp >> 3;
                const int c = (pp & 7) ^ ((r >> 1) & 7);
                src = (r >> 4) * kF8Group + kF8RopeOff + (r & 15) * 128 + 16 * c;
                alt = ((kF8RopeOff + 16 * c) << 6) + 1 + r;
            }
            f8_src[i] = src;
            f8_alt[i] = alt;
        }
    }
    auto issue_fp8 = [&](uint32_t dst, int i) {
        const int r = (f8_alt[i] & 63) - 1;
        const uint32_t off = (r < 0 || t_half * kCRows + r < t_rows) ? (uint32_t)(t_half * kF8HalfBytes + f8_src[i])
                                                                     : (uint32_t)(f8_alt[i] >> 6);
        load_lds16_untracked(t_src, off, dst + (sw + 4 * i) * 1024);
    };
    // this wave's i-th load of the taken half page into the slot at `dst`
    auto issue_one = [&](uint32_t dst, int i) {
        if constexpr (kFp8) issue_fp8(dst, i);
        else issue_bf16(dst, i);
    };
    auto issue_all = [&](uint32_t dst) {
        if constexpr (kFp8) {
#pragma unroll
            for (int i = 0; i < kF8Mine - 1; ++i) issue_fp8(dst, i);
            if (sw == 0) issue_fp8(dst, kF8Mine - 1);
        } else {
#pragma unroll
            for (int j = 0; j < kWLoads; ++j) issue_bf16(dst, j);
        }
    };
    // wait for the oldest slot in flight, `younger` slots' loads having been
    // issued after it
    auto wait_oldest = [&](int younger) {
        static_assert(kDist == 2, "waits for up to one younger slot");
        if (younger <= 0) wait_then_fence<kWaitAll>();
        else if constexpr (kFp8) {
            if (sw == 0) wait_then_fence<wait_vm_lgkm0(kF8Mine)>();
            else wait_then_fence<wait_vm_lgkm0(kF8Mine - 1)>();
        } else {
            wait_then_fence<kWaitSlot>();
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
        // score wave: key tile kt, block rows lrow[r] = 16 (rt0 + r) + i16
        constexpr int NR = kScorer ? Sh::NR : 1;
        const int kt = sw & 1;
        const int rt0 = kRT == 4 ? 2 * (sw >> 1) : 0;
        int lrow[NR], stok[NR];
        bool srow_ok[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lrow[r] = 16 * (rt0 + r) + i16;
            srow_ok[r] = rb * kRows + lrow[r] < a.M;
            stok[r] = srow_ok[r] ? (rb * kRows + lrow[r]) / a.h_q : 0;
        }
        bf16x8 qf[NR][kScorer ? kKS : 1];
        f32x4 o[kScorer ? 1 : kRT][kScorer ? 1 : kVTiles];

        // value waves: the stream's first two half pages
        // value waves: half pages of the stream issued and not yet scored
        int nq = 0;
        // fill slots soff, soff+1, .. with the stream's next kDist half pages
        auto prime = [&](int soff0) {
            nq = 0;
            for (int k = 0; k < kDist; ++k) {
                if (!take()) break;
                issue_all(ring_lds + ((soff0 + k) % kNS) * kSlot);
                ++nq;
            }
        };
        // The first segment's query block (64-row blocks): wave w brings rows
        // 8w..8w+7 into the staging area with direct loads (each byte of the
        // block crosses the memory pipeline once; rows past M read row 0 of
        // the block), ahead of the ring's first half pages.
        const bool q_staged = kQStage && fseg.b >= 0;
        if (q_staged) {
            const uint16_t* q_blk = a.q + ((size_t)fseg.b * a.M + rb * kRows) * kHeadDim;
#pragma unroll
            for (int j = 0; j < kWLoads; ++j) {
                const int rl = (j * 64 + lane) / kRowChunks;
                const int row = 8 * wid + rl;
                const int srow = rb * kRows + row < a.M ? row : 0;
                load_lds16_untracked(q_blk, (uint32_t)(srow * kRowBytes + goff[j] - rl * kRowBytes),
                                     ring_lds + kQOff + wid * 9216 + j * 1024);
            }
        }
        if constexpr (!kScorer) {
            if (fseg.b >= 0) fpage = fpage_of();
            prime(0);
        }
        if (q_staged) {
            // every wave's query loads have landed (a value wave's are older
            // than the nq slots of the prime) before the barrier publishes them
            if constexpr (kScorer) {
                wait_then_fence<kWaitAll>();
            } else if (nq <= 0) {
                wait_then_fence<kWaitAll>();
            } else if (nq == 1) {
                wait_oldest(1);
            } else {
                static_assert(kDist == 2, "the prime fills at most two slots");
                if constexpr (kFp8) {
                    if (sw == 0) wait_then_fence<wait_vm_lgkm0(2 * kF8Mine)>();
                    else wait_then_fence<wait_vm_lgkm0(2 * (kF8Mine - 1))>();
                } else {
                    wait_then_fence<wait_vm_lgkm0(2 * kWLoads)>();
                }
            }
            block_barrier();
        }
        bool q_in_lds = q_staged;
        int soff = 0;   // ring slot of the segment's first half page

        Seg seg = find_seg(b0, n0);
        while (seg.b >= 0) {
            const int b = seg.b, lo = seg.lo, hi = seg.hi, nseq = seg.nseq;
            const int npages = pages_of(nseq);
            const int nch = 2 * (hi - lo);   // half pages of the segment

            int L[NR];
            float m_ref[NR], l_run[NR];
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
                if (kQStage && q_in_lds) {
                    // from the staging area: row lrow[r] (its low three bits are
                    // those of i16, so the chunk placement is that of kofs)
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const uint8_t* qr = ring + kQOff + (lrow[r] - i16) * kRowBytes;
#pragma unroll
                        for (int ks = 0; ks < kKS; ++ks) qf[r][ks] = lds_read16(qr + kofs[ks & 1] + (ks >> 1) * 128);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const uint16_t* qp = a.q +
                            ((size_t)b * a.M + (srow_ok[r] ? rb * kRows + lrow[r] : rb * kRows)) * kHeadDim + g * 8;
#pragma unroll
                        for (int ks = 0; ks < kKS; ++ks) qf[r][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
                    }
                }
            }
            q_in_lds = false;

            bool restart = false;
            do {
                if constexpr (!kScorer) {
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt)
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

                // Step c: the value waves take the stream's next half page (this
                // segment's half page c+kDist, or one of the next segments')
                // into slot (soff+c+kDist) % kNS (its previous contents, half
                // page c-2, were accumulated in step c-1) and accumulate half
                // page c-1 from slot (soff+c-1) % kNS, while the score waves
                // turn half page c (slot (soff+c) % kNS) into weights. The last
                // step, c = nch, only accumulates.
                int c = 0;
                auto step = [&](auto sc) -> bool {
                    constexpr int S = decltype(sc)::value;
                    const unsigned rpos = (unsigned)(soff + c);
                    const uint8_t* slot_cur = ring + (rpos % kNS) * kSlot;
                    if constexpr (!kScorer) {
                        // my part of half page c (the loads of the nq - 1 half
                        // pages after it are younger)
                        if (c < nch) wait_oldest(nq - 1);
                    }
                    block_barrier();   // publishes the weights and flags of step c-1
                    if (restart_flag[(S + 1) & 1] != 0) return false;   // raised in step c-1
                    bool issue_now = false;
                    uint32_t dst = 0;
                    if constexpr (!kScorer) {
                        issue_now = c < nch && take();
                        dst = ring_lds + ((rpos + kDist) % kNS) * kSlot;
                        if (c == 0 && issue_now) issue_all(dst);
                    } else if (c < nch) {
                        // FP8: the per-token scales of this wave's keys (folded into P)
                        f32x4 my_scale = {1.f, 1.f, 1.f, 1.f};
                        // ---- S^T = K Q^T for key tile `tile` of half page c,
                        // every row tile of this wave; one K fragment feeds them
                        // all. Lane holds keys key0 + j (j < 4) of rows lrow[r],
                        // -inf where masked; lm[r] = the lane's maximum of them.
                        auto score_tile = [&](int tile, f32x4 (&sv)[NR], float (&lm)[NR]) {
                            f32x4 sp[NR][2];
                            f32x4 slat[NR];   // FP8: the latent part, scaled below
#pragma unroll
                            for (int r = 0; r < NR; ++r)
#pragma unroll
                                for (int pp = 0; pp < 2; ++pp) sp[r][pp] = f32x4{0.f, 0.f, 0.f, 0.f};
                            constexpr int KD = 4;
                            if constexpr (kFp8) {
                                // latent k-step ks: bytes 32 ks + 8 g .. +7 of key row
                                // 16 tile + i16, widened to BF16 in registers
                                const uint8_t* kl = slot_cur + (tile * 16 + i16) * kF8LatStride + 8 * g;
                                u32x2 kw[KD];
#pragma unroll
                                for (int d = 0; d < KD; ++d) kw[d] = lds_read8(kl + 32 * d);
                                // rotary k-steps: chunk 4 j + g of rotary row 16 tile + i16
                                const uint8_t* kr = slot_cur + kF8LdsRope + (tile * 16 + i16) * 128;
                                const int rsw = (i16 >> 1) & 7;
                                bf16x8 krf[2];
#pragma unroll
                                for (int ks = 0; ks < kHeadDimV / 32; ++ks) {
                                    const bf16x8 kf = e4m3x8_to_bf16(kw[ks % KD]);
                                    if (ks + KD < kHeadDimV / 32) kw[ks % KD] = lds_read8(kl + 32 * (ks + KD));
                                    if (ks == kHeadDimV / 32 - KD) {
                                        krf[0] = lds_read16(kr + ((g ^ rsw) << 4));
                                        krf[1] = lds_read16(kr + (((4 + g) ^ rsw) << 4));
                                    }
#pragma unroll
                                    for (int r = 0; r < NR; ++r) sp[r][ks & 1] = mfma16(kf, qf[r][ks], sp[r][ks & 1]);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                                // keep the latent part, accumulate the rotary part apart
#pragma unroll
                                for (int r = 0; r < NR; ++r) {
                                    slat[r] = sp[r][0] + sp[r][1];
                                    sp[r][0] = mfma16(krf[0], qf[r][kHeadDimV / 32], f32x4{0.f, 0.f, 0.f, 0.f});
                                    sp[r][1] = mfma16(krf[1], qf[r][kHeadDimV / 32 + 1], f32x4{0.f, 0.f, 0.f, 0.f});
                                }
                            } else {
                                const uint8_t* kb = slot_cur + tile * 16 * kRowBytes;
                                auto k_off = [&](int ks) { return kofs[ks & 1] + (ks >> 1) * 128; };
                                bf16x8 kf[KD];
#pragma unroll
                                for (int d = 0; d < KD; ++d) kf[d] = lds_read16(kb + k_off(d));
#pragma unroll
                                for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
                                    for (int r = 0; r < NR; ++r)
                                        sp[r][ks & 1] = mfma16(kf[ks % KD], qf[r][ks], sp[r][ks & 1]);
                                    if (ks + KD < kKS) kf[ks % KD] = lds_read16(kb + k_off(ks + KD));
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                            }
                            const int key0 = (lo + c / 2) * kPageRows + (c & 1) * kCRows + tile * 16 + 4 * g;
                            f32x4 sck = {0.f, 0.f, 0.f, 0.f};
                            if constexpr (kFp8) {
                                // scales of keys 16 tile + 4 g + j: chunk 4 tile + g of the
                                // scale chunks; those of rows past the sequence end are
                                // whatever the page holds there, replaced by 0
                                sck = *reinterpret_cast<const f32x4*>(slot_cur + (4 * tile + g) * kF8LatStride + 512);
#pragma unroll
                                for (int j = 0; j < 4; ++j) sck[j] = key0 + j < nseq ? sck[j] : 0.f;
                            }
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                float m = -INFINITY;
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const float raw = kFp8 ? fmaf(slat[r][j], sck[j], sp[r][0][j] + sp[r][1][j])
                                                           : sp[r][0][j] + sp[r][1][j];
                                    const float v = (key0 + j < L[r]) ? raw : -INFINITY;
                                    sv[r][j] = v;
                                    m = fmaxf(m, v);
                                }
                                lm[r] = m;
                            }
                            if (kFp8 && tile == kt) my_scale = sck;
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
                        // overflow: a scaled score above the reference plus
                        // the headroom. The lane's maximum times the scale is
                        // the maximum of its scaled scores (scale > 0, and
                        // rounding is monotonic), and the row maximum is at
                        // least the lane's, so a lane that reports overflow
                        // always raises its row's reference: every restart
                        // strictly raises some reference to a score of the
                        // segment plus the margin, and the restarts end.
                        bool over = false;
#pragma unroll
                        for (int r = 0; r < NR; ++r) over = over || (lm[r] * a.scale_log2 > m_ref[r] + kHeadroom);
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
                                // B = P^T of row tile rt0 + r. BF16: k-slot 4 kt + j of lane
                                // group g <-> key 16 kt + 4 g + j. FP8: k-slot k of lane group
                                // g' <-> key 8 g' + k (the byte order of the transposing
                                // read), and the value product sees p_t * scale_t, the
                                // sum p_t alone.
                                if constexpr (kFp8) {
                                    pw *= my_scale;
                                    *reinterpret_cast<bf16x4*>(
                                        &pbuf[S & 1][(rt0 + r) * 1024 + ((2 * kt + (g >> 1)) * 16 + i16) * 16 + 8 * (g & 1)]) =
                                        pack_bf16x4(pw);
                                } else {
                                    *reinterpret_cast<bf16x4*>(&pbuf[S & 1][(rt0 + r) * 1024 + lane * 16 + kt * 8]) =
                                        pack_bf16x4(pw);
                                }
                            }
                        }
                    }
                    if (!kScorer && c >= 1) {
                        // ---- O^T += V^T P^T for half page c-1: the row tiles
                        // share each V^T fragment
                        const uint8_t* cur = ring + ((rpos + kNS - 1) % kNS) * kSlot;
                        const uint8_t* pb = &pbuf[(S + 1) & 1][lane * 16];
                        bf16x8 pf[kRT];
#pragma unroll
                        for (int rt = 0; rt < kRT; ++rt) pf[rt] = lds_read16(pb + rt * 1024);
                        if constexpr (kFp8) {
                            // V^T fragment of value tile dt: one transposing byte read,
                            // lane (i16, g) receiving dims 16 dt + i16 of key rows
                            // 8 g .. 8 g + 7, widened to BF16 in registers
                            const uint8_t* vb =
                                cur + (8 * g + (i16 >> 1)) * kF8LatStride + 8 * (i16 & 1) + 16 * kVTiles * sw;
                            constexpr int VD = 4;
                            u32x2 vw[VD];
#pragma unroll
                            for (int d = 0; d < VD; ++d) vw[d] = lds_read_tr8(vb + 16 * d);
#pragma unroll
                            for (int t = 0; t < kVTiles; ++t) {
                                const bf16x8 vf = e4m3x8_to_bf16(vw[t % VD]);
                                if (t + VD < kVTiles) vw[t % VD] = lds_read_tr8(vb + 16 * (t + VD));
#pragma unroll
                                for (int rt = 0; rt < kRT; ++rt) o[rt][t] = mfma16(vf, pf[rt], o[rt][t]);
                                if (issue_now && t < kF8Mine - 1) issue_one(dst, t);
                                if (issue_now && t == kF8Mine - 1 && sw == 0) issue_one(dst, t);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        } else {
                            // two transposing reads per V^T fragment
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
                                for (int rt = 0; rt < kRT; ++rt) o[rt][t] = mfma16(vf[t % VD], pf[rt], o[rt][t]);
                                if (t + VD < kVTiles) vf[t % VD] = v_frag(t + VD);
                                if (issue_now) issue_one(dst, t);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                            static_assert(kVTiles + 1 == kWLoads, "one load per value tile and one after");
                            if (issue_now) issue_one(dst, kVTiles);
                        }
                    }
                    if constexpr (!kScorer) {
                        if (c < nch) nq += issue_now ? 0 : -1;
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
                // after the barrier every wave sees an overflow raised in the
                // last step too (the next segment's first half pages stay in
                // flight)
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
                    if constexpr (!kScorer) {
                        // drain the ring and refill it from this segment's start
                        wait_then_fence<kWaitAll>();
                        fseg = seg;
                        fc = 0;
                        fpage = fpage_of();
                        prime(soff);
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
                for (int rt = 0; rt < kRT; ++rt) {
                    const int row = rb * kRows + rt * 16 + i16;
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
            if (!full && a.counters)
                count_partial_and_combine<Sh::kThreads, kRows, (kRT == 4 ? 512 : 256)>(a, b, rb, &last_flag);
            soff = (soff + nch) % kNS;
            seg = find_seg(b + 1, 0);
        }
        if (a.counters) write_empty_sequences<Sh::kThreads>(a);
    };
    if (scorer) run(std::true_type{});
    else run(std::false_type{});
}

template <int kRT, bool kFp8 = false>
static hipError_t launch_ws(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL((mla_decode_ws_kernel<kRT, kFp8>), dim3(plan.P * plan.R), dim3(WsShape<kRT>::kThreads), 0,
                       stream, args);
    return hipGetLastError();
}

hipError_t launch_decode_ws(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    switch (plan.tm) {
        case 16: return launch_ws<1>(plan, args, stream);
        case 32: return launch_ws<2>(plan, args, stream);
        case 64: return launch_ws<4>(plan, args, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_ws_fp8(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    switch (plan.tm) {
        case 16: return launch_ws<1, true>(plan, args, stream);
        case 32: return launch_ws<2, true>(plan, args, stream);
        case 64: return launch_ws<4, true>(plan, args, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mla
