// mla_absorb.hip - the absorption products around decode (include/mla_absorb.h).
//
// Both are per-head products with the contraction dimension contiguous in
// both operands (page "MLA 和 MHA 的 Kernel 区别": K_h = c_KV W_UK_h,
// V_h = c_KV W_UV_h; folding them into the query and the output):
//
//   out[n][m] = sum_k W[m][k] * X[n][k]      per head
//
//   absorb_q: W = W_UK_h   (m: 512 latent columns, k: d_nope), X = q_nope
//   absorb_o: W = W_UV_h^T (m: d_v outputs,        k: 512),    X = o_lat
//
// computed as D = W * X^T on 16x16x32 BF16 MFMA tiles. In that orientation a
// lane's four accumulator values are four consecutive m of one token n, so
// each lane stores 8 contiguous bytes of a token's output row. Operand
// fragments are read straight from global memory (16 bytes per lane, the
// contraction dimension contiguous); the weights are the only large operand
// and each 64-row weight tile is read by the workgroups of every 64-token
// block, which are placed on the same XCD so that the re-reads hit its L2.
#include "../../include/mla_absorb.h"

#include <hip/hip_runtime.h>

#include "mla_common.h"

namespace mla {
namespace {

constexpr int kAbsThreads = 256;   // 4 waves; workgroup tile 64 m x 64 n, wave tile 32 x 32
constexpr int kAbsTile = 64;

struct AbsorbArgs {
    const uint16_t* w;     // weights, head h at w + h * w_head, row m at + m * K
    const uint16_t* x;     // activations, token n head h at x + n * x_row + h * K
    uint16_t* out;         // output, token n head h at out + n * o_row + h * o_head
    const uint16_t* rope;  // absorb_q only: q_rope [tokens][h][64], copied to out[..][512..575]
    long long w_head;
    int x_row, o_row, o_head;
    int M, K, N, H;        // rows of W per head, contraction, tokens, heads
    int mblocks, nblocks;
    int xcd_map;           // 1: XCD-aware placement of the workgroups (see each kernel)
};

struct Frag {
    bf16x8 a[2], b[2];
};

template <int kPf>
__global__ __launch_bounds__(kAbsThreads) void mla_absorb_kernel(AbsorbArgs a) {
    // workgroup -> (weight tile, token block): the token blocks of one weight
    // tile get ids 8 apart, so the same XCD (ids go round-robin over 8 XCDs)
    const int bid = blockIdx.x;
    int wt, nb;
    if (a.xcd_map) {
        const int q = bid >> 3;
        nb = q % a.nblocks;
        wt = (bid & 7) + 8 * (q / a.nblocks);
    } else {
        wt = bid / a.nblocks;
        nb = bid % a.nblocks;
    }
    const int h = wt / a.mblocks;
    const int mb = wt - h * a.mblocks;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;

    if (a.rope && mb == 0) {
        // the rotary part passes through: 64 tokens x 8 chunks of 16 bytes
        for (int c = threadIdx.x; c < kAbsTile * 8; c += kAbsThreads) {
            const int n = nb * kAbsTile + (c >> 3);
            if (n < a.N) {
                const uint4 v = *reinterpret_cast<const uint4*>(a.rope + ((size_t)n * a.H + h) * 64 + (c & 7) * 8);
                *reinterpret_cast<uint4*>(a.out + (size_t)n * a.o_row + (size_t)h * a.o_head + 512 + (c & 7) * 8) = v;
            }
        }
    }

    const int m0 = mb * kAbsTile + 32 * (wave & 1);
    const int n0 = nb * kAbsTile + 32 * (wave >> 1);
    if (m0 >= a.M) return;   // M is a multiple of 32: this wave's rows are past the end

    // operand rows of this lane: W rows m0 + 16 i + li, X rows n0 + 16 j + li
    // (token rows past the end are clamped to the last one and not stored)
    const uint16_t* wp[2];
    const uint16_t* xp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        wp[i] = a.w + (size_t)h * a.w_head + (size_t)(m0 + 16 * i + li) * a.K + 8 * lg;
        const int n = min(n0 + 16 * i + li, a.N - 1);
        xp[i] = a.x + (size_t)n * a.x_row + (size_t)h * a.K + 8 * lg;
    }
    auto load = [&](Frag& f, int s) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f.a[i] = *reinterpret_cast<const bf16x8*>(wp[i] + 32 * s);
            f.b[i] = *reinterpret_cast<const bf16x8*>(xp[i] + 32 * s);
        }
    };

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // kPf contraction steps of 32 in flight: step s + kPf is loaded into the
    // registers step s has just used (the step count is a multiple of kPf)
    const int steps = a.K / 32;
    auto mma = [&](const Frag& g) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma16(g.a[i], g.b[j], acc[i][j]);
    };
    Frag f[kPf];
#pragma unroll
    for (int p = 0; p < kPf; ++p) load(f[p], p);
    for (int s0 = kPf; s0 < steps; s0 += kPf) {   // branch-free body
#pragma unroll
        for (int p = 0; p < kPf; ++p) {
            mma(f[p]);
            load(f[p], s0 + p);
        }
    }
#pragma unroll
    for (int p = 0; p < kPf; ++p) mma(f[p]);

    // lane holds D[m0 + 16 i + 4 lg + r][n0 + 16 j + li], r = 0..3
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + 16 * j + li;
        if (n >= a.N) continue;
        uint16_t* op = a.out + (size_t)n * a.o_row + (size_t)h * a.o_head + m0 + 4 * lg;
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<bf16x4*>(op + 16 * i) = pack_bf16x4(acc[i][j]);
    }
}

// ---- LDS-staged kernel (K a multiple of 128, M a multiple of kMT) -----------
//
// Fragments read straight from global memory put 16 different rows in every
// 16 lanes, so each quarter-wave of a load touches four cache lines and the
// vector L1 becomes the bottleneck. Here operand tiles are brought into LDS
// with direct global->LDS loads instead, each lane fetching 16 contiguous
// bytes of a row (a wave instruction fills four 256-byte rows), and the MFMA
// fragments are read from LDS. A tile row holds one 128-wide chunk of the
// contraction (256 bytes, exactly one LDS bank period), so the 16-byte chunk
// c of row r is stored at chunk c ^ (r & 15): the 16 rows a fragment read
// touches then fall on 16 different bank groups. The swizzle is applied by
// choosing each lane's source chunk, since a lane's LDS destination is fixed.

constexpr int kChunkElems = 128;   // contraction elements per stage
constexpr int kChunkBytes = 256;   // bytes of one tile row per stage

// Wave-uniform copy of a pointer (scalar registers), for the base operand of
// the direct global->LDS load.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

template <int kMT, int kNT, int kBufs>
__global__ __launch_bounds__(kAbsThreads, 2) void mla_absorb_lds_kernel(AbsorbArgs a) {
    constexpr int kRows = kMT + kNT;              // W rows, then X rows
    constexpr int kStageBytes = kRows * kChunkBytes;
    constexpr int kInstr = kRows / 16;            // 4-row loads per wave per stage
    constexpr int kTM = kMT / 32, kTN = kNT / 32; // 16 x 16 tiles per wave in m and n
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kBufs][kStageBytes];

    // workgroup -> (head, weight tile, token block), head-major per XCD: all
    // workgroups of a head share its weights or its activations, so they get
    // ids 8 apart and run on one XCD (ids go round-robin over the 8 XCDs),
    // where the second reader of a tile finds it in that XCD's L2
    const int bid = blockIdx.x;
    const int per_head = a.mblocks * a.nblocks;
    int h, local;
    if (a.xcd_map) {
        const int q = bid >> 3;
        h = (bid & 7) + 8 * (q / per_head);
        local = q % per_head;
    } else {
        h = bid / per_head;
        local = bid % per_head;
    }
    const int mb = local / a.nblocks;
    const int nb = local - mb * a.nblocks;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int m_base = mb * kMT, n_base = nb * kNT;

    if (a.rope && mb == 0) {
        for (int c = threadIdx.x; c < kNT * 8; c += kAbsThreads) {
            const int n = n_base + (c >> 3);
            if (n < a.N) {
                const uint4 v = *reinterpret_cast<const uint4*>(a.rope + ((size_t)n * a.H + h) * 64 + (c & 7) * 8);
                *reinterpret_cast<uint4*>(a.out + (size_t)n * a.o_row + (size_t)h * a.o_head + 512 + (c & 7) * 8) = v;
            }
        }
    }

    // Load plan: instruction q of this wave fills stage rows 4 I .. 4 I + 3,
    // I = wave * kInstr + q; the lane takes row 4 I + lg, LDS chunk li, and
    // fetches logical chunk li ^ (row & 15) of that row's 256-byte stage slice.
    // X rows past the last token repeat the last token (never stored).
    const uint16_t* w_head = a.w + (size_t)h * a.w_head;
    const uint16_t* x_head = a.x + (size_t)h * a.K;
    uint32_t voff[kInstr];
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
        const int r = 4 * (wave * kInstr + q) + lg;
        const uint32_t chunk = (uint32_t)(li ^ (r & 15)) * 16u;
        if (r < kMT) {
            voff[q] = (uint32_t)(m_base + r) * (uint32_t)a.K * 2u + chunk;
        } else {
            const int n = min(n_base + r - kMT, a.N - 1);
            voff[q] = (uint32_t)n * (uint32_t)a.x_row * 2u + chunk;
        }
    }
    auto issue = [&](int stage, int buf) {
#pragma unroll
        for (int q = 0; q < kInstr; ++q) {
            const int I = wave * kInstr + q;
            const void* base = uniform_ptr((4 * I < kMT) ? static_cast<const void*>(w_head)
                                                         : static_cast<const void*>(x_head));
            load_lds16_untracked(base, voff[q] + (uint32_t)stage * kChunkBytes,
                                 lds_addr_of(&lds[buf][I * 1024]));
        }
    };

    const int wm = wave & 1, wn = wave >> 1;
    f32x4 acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int stages = a.K / kChunkElems;
    issue(0, 0);
    for (int s = 0; s < stages; ++s) {
        if (kBufs > 1 && s + 1 < stages) {
            issue(s + 1, (s + 1) % kBufs);
            __builtin_amdgcn_s_waitcnt((kInstr & 15) | ((kInstr >> 4) << 14) | (7 << 4));  // stage s landed
        } else {
            __builtin_amdgcn_s_waitcnt((7 << 4));                                         // vmcnt(0)
        }
        __syncthreads();
        const uint8_t* buf = lds[s % kBufs];
#pragma unroll
        for (int t = 0; t < kChunkElems / 32; ++t) {
            const int c = 4 * t + lg;
            bf16x8 fa[kTM], fb[kTN];
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                fa[i] = lds_read16(buf + (wm * (kMT / 2) + 16 * i + li) * kChunkBytes + 16 * (c ^ li));
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                fb[j] = lds_read16(buf + (kMT + wn * (kNT / 2) + 16 * j + li) * kChunkBytes + 16 * (c ^ li));
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
        }
        if (kBufs == 1 && s + 1 < stages) {   // single buffer: refill after everyone read it
            __syncthreads();
            issue(s + 1, 0);
        } else if (kBufs > 1) {
            __syncthreads();                  // buffer s % kBufs is refilled next iteration
        }
    }

    // lane holds D[m][n] for m = m0 + 16 i + 4 lg + 0..3, n = n0 + 16 j + li
    const int m0 = m_base + wm * (kMT / 2) + 4 * lg;
    const int n0 = n_base + wn * (kNT / 2) + li;
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        const int n = n0 + 16 * j;
        if (n >= a.N) continue;
        uint16_t* op = a.out + (size_t)n * a.o_row + (size_t)h * a.o_head + m0;
#pragma unroll
        for (int i = 0; i < kTM; ++i) *reinterpret_cast<bf16x4*>(op + 16 * i) = pack_bf16x4(acc[i][j]);
    }
}

bool aligned_to(const void* p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

template <int kMT, int kNT, int kBufs>
hipError_t launch_staged(AbsorbArgs a, hipStream_t stream) {
    a.mblocks = a.M / kMT;
    a.nblocks = (a.N + kNT - 1) / kNT;
    const long long tiles = (long long)a.H * a.mblocks;
    a.xcd_map = a.H % 8 == 0;   // head-major placement (see the kernel)
    const long long grid = tiles * a.nblocks;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mla_absorb_lds_kernel<kMT, kNT, kBufs>), dim3((unsigned)grid), dim3(kAbsThreads), 0,
                       stream, a);
    return hipGetLastError();
}

// Direct-fragment kernel for the shapes the staged one does not cover.
hipError_t launch_direct(AbsorbArgs a, hipStream_t stream) {
    a.mblocks = (a.M + kAbsTile - 1) / kAbsTile;
    a.nblocks = (a.N + kAbsTile - 1) / kAbsTile;
    const long long tiles = (long long)a.H * a.mblocks;
    a.xcd_map = tiles % 8 == 0;
    const long long grid = tiles * a.nblocks;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const int steps = a.K / 32;
    if (steps % 4 == 0)
        hipLaunchKernelGGL(mla_absorb_kernel<4>, dim3((unsigned)grid), dim3(kAbsThreads), 0, stream, a);
    else if (steps % 2 == 0)
        hipLaunchKernelGGL(mla_absorb_kernel<2>, dim3((unsigned)grid), dim3(kAbsThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(mla_absorb_kernel<1>, dim3((unsigned)grid), dim3(kAbsThreads), 0, stream, a);
    return hipGetLastError();
}

// Tiles: with a one-stage contraction (absorb_q, d_nope = 128), 128 weight
// rows x 128 tokens (64 KB of LDS, two workgroups per CU) up to 128 tokens,
// and 128 x 64 (48 KB, three per CU) beyond, where more, smaller workgroups
// let one round's stores overlap the next round's loads (measured on the
// 128- and 264-token query projections: 14.0 vs 15.3 us and 28.2 vs 24.3 us).
// Longer contractions use 128 x 64 double-buffered (96 KB), so a 128-token
// step still spreads over 256 workgroups.
hipError_t launch_absorb(AbsorbArgs a, hipStream_t stream) {
    if (a.K % kChunkElems == 0 && a.M % 128 == 0) {
        if (a.K == kChunkElems)
            return a.N <= 128 ? launch_staged<128, 128, 1>(a, stream) : launch_staged<128, 64, 1>(a, stream);
        return launch_staged<128, 64, 2>(a, stream);
    }
    return launch_direct(a, stream);
}

}  // namespace
}  // namespace mla

extern "C" mla_status mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int h,
                                   int d_nope, void* q_abs, void* stream) {
    using namespace mla;
    if (!q_nope || !q_rope || !w_uk || !q_abs) return MLA_ERR_INVALID_ARG;
    if (tokens < 1 || h < 1 || d_nope < 32 || d_nope > 512 || d_nope % 32) return MLA_ERR_INVALID_ARG;
    if ((long long)tokens * h * kHeadDim >= (1LL << 31) || (long long)tokens * h * d_nope >= (1LL << 31) ||
        (long long)h * kHeadDimV * d_nope >= (1LL << 31))
        return MLA_ERR_UNSUPPORTED;
    if (!aligned_to(q_nope, 16) || !aligned_to(q_rope, 16) || !aligned_to(w_uk, 16) || !aligned_to(q_abs, 16))
        return MLA_ERR_MISALIGNED;
    AbsorbArgs a{};
    a.w = static_cast<const uint16_t*>(w_uk);
    a.x = static_cast<const uint16_t*>(q_nope);
    a.out = static_cast<uint16_t*>(q_abs);
    a.rope = static_cast<const uint16_t*>(q_rope);
    a.w_head = (long long)kHeadDimV * d_nope;
    a.x_row = h * d_nope;
    a.o_row = h * kHeadDim;
    a.o_head = kHeadDim;
    a.M = kHeadDimV;
    a.K = d_nope;
    a.N = tokens;
    a.H = h;
    return launch_absorb(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" mla_status mla_absorb_o(const void* o_lat, const void* w_uv_t, int tokens, int h, int d_v, void* out,
                                   void* stream) {
    using namespace mla;
    if (!o_lat || !w_uv_t || !out) return MLA_ERR_INVALID_ARG;
    if (tokens < 1 || h < 1 || d_v < 32 || d_v > 512 || d_v % 32) return MLA_ERR_INVALID_ARG;
    if ((long long)tokens * h * kHeadDimV >= (1LL << 31) || (long long)tokens * h * d_v >= (1LL << 31) ||
        (long long)h * kHeadDimV * d_v >= (1LL << 31))
        return MLA_ERR_UNSUPPORTED;
    if (!aligned_to(o_lat, 16) || !aligned_to(w_uv_t, 16) || !aligned_to(out, 8)) return MLA_ERR_MISALIGNED;
    AbsorbArgs a{};
    a.w = static_cast<const uint16_t*>(w_uv_t);
    a.x = static_cast<const uint16_t*>(o_lat);
    a.out = static_cast<uint16_t*>(out);
    a.rope = nullptr;
    a.w_head = (long long)d_v * kHeadDimV;
    a.x_row = h * kHeadDimV;
    a.o_row = h * d_v;
    a.o_head = d_v;
    a.M = d_v;
    a.K = kHeadDimV;
    a.N = tokens;
    a.H = h;
    return launch_absorb(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
