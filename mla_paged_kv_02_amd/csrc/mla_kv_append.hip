// mla_kv_append.hip - paged latent-cache append (include/mla_kv_append.h).
//
// A pure scatter: every new token's 1152-byte row is copied into its page
// slot, p = N_b - s_new + i (FlashMLA overview page: 64-token pages behind a
// block table; the new tokens are the last s_new of the sequence, as the
// decode call's causal mask reads them). The work is one 16-byte chunk per
// thread step, numbered token-major so that a wave's loads read consecutive
// source bytes and its stores fill consecutive bytes of a page row (rows of
// consecutive positions in one page are adjacent too). No LDS, no MFMA: the
// kernel is bound by HBM and, for one decode step's few rows, by launch
// latency.
#include "../../include/mla_kv_append.h"
#include "../../include/mla_decode_fp8.h"

#include <hip/hip_runtime.h>

#include "mla_common.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr int kAppendUnroll = 4;   // chunks per thread, kAppendThreads apart
constexpr int kAppendChunksPerBlock = kAppendThreads * kAppendUnroll;

struct AppendArgs {
    const u32x4* src;        // new rows, 72 chunks each
    u32x4* kv;               // cache, 72 chunks per row
    const int32_t* seqlens;
    const int32_t* block_table;
    int32_t* skipped;        // may be null
    int batch, s_new, max_blocks, num_pages;
    int total_chunks;        // batch * s_new * 72
};

__global__ __launch_bounds__(kAppendThreads) void mla_kv_append_kernel(AppendArgs a) {
    const int g0 = blockIdx.x * kAppendChunksPerBlock + threadIdx.x;
    const int last = a.total_chunks - 1;
    // Three rounds over the thread's chunks: row loads, then the lengths,
    // then the table entries, each round's loads all in flight together, so
    // a wave waits for two memory latencies before its stores, not three per
    // chunk. Every index is clamped into its buffer (a clamped chunk's result
    // is discarded), so no load sits behind a branch.
    u32x4 v[kAppendUnroll];
    int g[kAppendUnroll], b[kAppendUnroll], p[kAppendUnroll], c[kAppendUnroll];
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        g[u] = min(g0 + u * kAppendThreads, last);
        v[u] = __builtin_nontemporal_load(a.src + g[u]);
    }
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        const int row = g[u] / kRowChunks;
        c[u] = g[u] - row * kRowChunks;
        b[u] = row / a.s_new;
        p[u] = a.seqlens[b[u]] - a.s_new + (row - b[u] * a.s_new);   // position of the token
    }
    int blk[kAppendUnroll], page[kAppendUnroll];
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        blk[u] = max(p[u], 0) >> 6;
        page[u] = a.block_table[(size_t)b[u] * a.max_blocks + min(blk[u], a.max_blocks - 1)];
    }
    // Pin the row data in registers here, before the stores' branches: left
    // alone, the compiler moves each row load down into the branch of its
    // store, where it is waited for on its own.
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) asm volatile("" : "+v"(v[u]));
    int missing = 0;   // tokens of this thread with a position but no page
#pragma unroll
    for (int u = 0; u < kAppendUnroll; ++u) {
        if (g0 + u * kAppendThreads > last) break;
        const bool placed = p[u] >= 0;
        const bool ok = placed & (blk[u] < a.max_blocks) & ((unsigned)page[u] < (unsigned)a.num_pages);
        if (ok) a.kv[((long long)page[u] * kPageRows + (p[u] & (kPageRows - 1))) * kRowChunks + c[u]] = v[u];
        missing += (placed & !ok & (c[u] == 0)) ? 1 : 0;
    }
    if (missing && a.skipped) atomicAdd(a.skipped, missing);
}

// ---- appending into the FP8 page layout --------------------------------------
//
// One wave per new token: lane l holds latent values 8l..8l+7 (16 bytes of
// the BF16 row), lanes 0..7 also its rotary chunk l. The row's largest
// magnitude comes from a wave reduction and scale = amax / 448 is an FP32
// division (correctly rounded: the stored scale is the FP32 number nearest
// amax / 448). Each code is the E4M3 value nearest the exact quotient
// |x| / scale, ties to the even mantissa: y = |x| * fl32(1 / scale), within
// a relative 2^-23 of the quotient, is rounded to E4M3 in integer arithmetic
// (magnitudes at or past 448 saturate to 448; below 2^-6 the code is the
// rounding of y * 2^9, subnormal steps of 2^-9; above, y * 2^(3 - e) lies in
// [8, 16) for e = floor(log2 y) and its rounding gives the mantissa, a carry
// to 16 moving to the next binade by itself: code = 8 (e + 7) + r - 8). A y
// whose grid position is within 2^-18 of a midpoint may sit on the other
// side of it than the exact quotient; there the sign of the exact residual
// at the midpoint decides (round_grid). Where y crosses a binade edge
// instead, both sides give the same code. The sign bit is x's.
constexpr int kAppendF8Threads = 256;   // four tokens per workgroup

struct AppendF8Args {
    const uint16_t* src;     // [batch][s_new][576] BF16
    uint8_t* pages;          // [num_pages][MLA_FP8_PAGE_BYTES]
    const int32_t* seqlens;
    const int32_t* block_table;
    int32_t* skipped;
    int batch, s_new, max_blocks, num_pages, tokens;
};

// Round t = q / step (q = |x| / scale in grid-step units: the mantissa
// position, or q * 2^9 below 2^-6) to the nearest integer, where tq is t
// computed from a = |x| * fl32(1 / scale), within a relative 2^-23 of t
// (two roundings of 2^-24), so |tq - t| <= 16 * 2^-23 = 2^-19. A tq more
// than 2^-18 from the midpoint fl + 1/2 of its unit interval is on the same
// side of it as t, and rint decides. Closer, the sign of the exact residual
// |x| - (fl + 1/2) * step * scale decides (one FMA: the midpoint has at most
// five significant bits, so the product is exact and the single rounding
// keeps the sign; zero is an exact tie, to the even integer). `up` scales
// both operands by 2^64 for |x| < 2^-60, so the residual never underflows.
__device__ __forceinline__ float round_grid(float tq, float step, float ax, float scale, float up) {
    const float fl = floorf(tq);
    const float d = tq - fl - 0.5f;   // exact wherever |d| is small
    if (fabsf(d) > 0x1p-18f) return rintf(tq);
    const float mid = (fl + 0.5f) * step;   // exact
    const float resid = fmaf(-(mid * up), scale, ax * up);
    if (resid > 0.f) return fl + 1.f;
    if (resid < 0.f) return fl;
    return ((int)fl & 1) == 0 ? fl : fl + 1.f;
}

// Maximum over the 64 lanes, in every lane: DPP within each row of 16 (quad
// swaps, then the half-row and row mirrors pair lanes i and 7 - i, i and
// 15 - i), then across rows with the lane-swap VALU ops; no LDS round trip.
__device__ __forceinline__ float dpp_max(float v, int ctrl_sel) {
    int m;
    switch (ctrl_sel) {
        case 0: m = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false); break;   // quad [1,0,3,2]
        case 1: m = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false); break;   // quad [2,3,0,1]
        case 2: m = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false); break;  // row_half_mirror
        default: m = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return fmaxf(v, __int_as_float(m));
}
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max(v, 0);
    v = dpp_max(v, 1);
    v = dpp_max(v, 2);
    v = dpp_max(v, 3);
    return max_over_kgroups(v);
}

// E4M3 code of x, the value nearest the exact quotient |x| / scale (ties to
// the even mantissa); rinv = fl32(1 / (scale * up_s)), where up_s = 2^64 for
// a scale below 2^-64 (whose reciprocal would overflow) and 1 otherwise.
__device__ __forceinline__ uint32_t e4m3_code(float x, float scale, float rinv, float up_s) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float ax = fabsf(x);
    const float a = (ax * up_s) * rinv;   // the scaling by up_s is exact
    const float up = ax < 0x1p-60f ? 0x1p64f : 1.f;
    uint32_t mag;
    if (!(a < 448.f)) {
        mag = 0x7Eu;   // at or past the largest code (and NaN)
    } else if (a < 0x1p-6f) {
        mag = (uint32_t)round_grid(a * 0x1p9f, 0x1p-9f, ax, scale, up);
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;    // -6 .. 8
        const float r = round_grid(ldexpf(a, 3 - e), ldexpf(1.f, e - 3), ax, scale, up);   // 8 .. 16
        mag = (uint32_t)(8 * (e + 7) + (int)r - 8);
        mag = mag > 0x7Eu ? 0x7Eu : mag;
    }
    return sign | mag;
}

__global__ __launch_bounds__(kAppendF8Threads) void mla_kv_append_fp8_kernel(AppendF8Args a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (kAppendF8Threads / 64) + (threadIdx.x >> 6);   // token of this wave
    if (t >= a.tokens) return;
    // The row's loads go out first, with the sequence length beside them; the
    // table entry's load, which needs the length, then flies while the wave
    // quantises the row. So a wave waits two memory latencies before its
    // stores, not three (length, entry, row) plus the arithmetic. Indices are
    // clamped into their buffers and checked only before the stores.
    const uint16_t* row = a.src + (size_t)t * kHeadDim;
    const u32x4 lat = *reinterpret_cast<const u32x4*>(row + 8 * lane);
    u32x4 rope = {0u, 0u, 0u, 0u};
    if (lane < 8) rope = *reinterpret_cast<const u32x4*>(row + 512 + 8 * lane);
    const int b = t / a.s_new;
    const int i = t - b * a.s_new;
    const int len = a.seqlens[b];
    // (the scheduler would otherwise start on the row, and so wait for it,
    // before these loads are issued)
    __builtin_amdgcn_sched_barrier(0);
    const int p = len - a.s_new + i;
    const int blk = max(p, 0) >> 6;
    const int page = a.block_table[(size_t)b * a.max_blocks + min(blk, a.max_blocks - 1)];
    __builtin_amdgcn_sched_barrier(0);
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(lat[k] << 16);
        x[2 * k + 1] = __uint_as_float(lat[k] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    const float up_s = scale < 0x1p-64f ? 0x1p64f : 1.f;
    const float rinv = 1.f / (scale * up_s);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) lo |= e4m3_code(x[k], scale, rinv, up_s) << (8 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) hi |= e4m3_code(x[4 + k], scale, rinv, up_s) << (8 * k);
    if (p < 0) return;
    if (blk >= a.max_blocks || page < 0 || page >= a.num_pages) {
        if (lane == 0 && a.skipped) atomicAdd(a.skipped, 1);
        return;
    }
    const int slot = p & (kPageRows - 1);
    uint8_t* grp = a.pages + (size_t)page * MLA_FP8_PAGE_BYTES + (slot >> 4) * (MLA_FP8_PAGE_BYTES / 4);
    const int r = slot & 15;
    *reinterpret_cast<uint2*>(grp + r * 512 + 8 * lane) = uint2{lo, hi};
    if (lane < 8) *reinterpret_cast<u32x4*>(grp + 8192 + r * 128 + 16 * lane) = rope;
    if (lane == 0) *reinterpret_cast<float*>(grp + 10240 + 4 * r) = scale;
}

bool aligned_to(const void* p, size_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace
}  // namespace mla

extern "C" mla_status mla_kv_append(const void* new_rows, int batch, int s_new, const int32_t* seqlens,
                                    const int32_t* block_table, int max_blocks_per_seq, void* kv_cache,
                                    int num_pages, int32_t* skipped_rows, void* stream) {
    using namespace mla;
    if (!new_rows || !seqlens || !block_table || !kv_cache) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || s_new < 1 || max_blocks_per_seq < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
    const long long chunks = (long long)batch * s_new * kRowChunks;
    if (chunks >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * batch > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
    if (!aligned_to(new_rows, 16) || !aligned_to(kv_cache, 16)) return MLA_ERR_MISALIGNED;
    if (!aligned_to(seqlens, 4) || !aligned_to(block_table, 4) || (skipped_rows && !aligned_to(skipped_rows, 4)))
        return MLA_ERR_MISALIGNED;
    AppendArgs a{};
    a.src = static_cast<const u32x4*>(new_rows);
    a.kv = static_cast<u32x4*>(kv_cache);
    a.seqlens = seqlens;
    a.block_table = block_table;
    a.skipped = skipped_rows;
    a.batch = batch;
    a.s_new = s_new;
    a.max_blocks = max_blocks_per_seq;
    a.num_pages = num_pages;
    a.total_chunks = (int)chunks;
    const unsigned grid = (unsigned)((chunks + kAppendChunksPerBlock - 1) / kAppendChunksPerBlock);
    hipLaunchKernelGGL(mla_kv_append_kernel, dim3(grid), dim3(kAppendThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" mla_status mla_kv_append_fp8(const void* new_rows, int batch, int s_new, const int32_t* seqlens,
                                        const int32_t* block_table, int max_blocks_per_seq, void* kv_pages,
                                        int num_pages, int32_t* skipped_rows, void* stream) {
    using namespace mla;
    if (!new_rows || !seqlens || !block_table || !kv_pages) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || s_new < 1 || max_blocks_per_seq < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
    const long long tokens = (long long)batch * s_new;
    if (tokens * kRowChunks >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * batch > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
    if (!aligned_to(new_rows, 16) || !aligned_to(kv_pages, 16)) return MLA_ERR_MISALIGNED;
    if (!aligned_to(seqlens, 4) || !aligned_to(block_table, 4) || (skipped_rows && !aligned_to(skipped_rows, 4)))
        return MLA_ERR_MISALIGNED;
    AppendF8Args a{};
    a.src = static_cast<const uint16_t*>(new_rows);
    a.pages = static_cast<uint8_t*>(kv_pages);
    a.seqlens = seqlens;
    a.block_table = block_table;
    a.skipped = skipped_rows;
    a.batch = batch;
    a.s_new = s_new;
    a.max_blocks = max_blocks_per_seq;
    a.num_pages = num_pages;
    a.tokens = (int)tokens;
    const int per_block = kAppendF8Threads / 64;
    const unsigned grid = (unsigned)((tokens + per_block - 1) / per_block);
    hipLaunchKernelGGL(mla_kv_append_fp8_kernel, dim3(grid), dim3(kAppendF8Threads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
