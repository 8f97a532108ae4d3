// mla_common.h - gfx950 device helpers shared by the decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

#define MLA_AS1 __attribute__((address_space(1)))
#define MLA_AS3 __attribute__((address_space(3)))

constexpr int kHeadDim = 576;
constexpr int kHeadDimV = 512;
constexpr int kRowBytes = kHeadDim * 2;          // 1152 B per cache row
constexpr int kPageRows = 64;
constexpr int kPageBytes = kPageRows * kRowBytes;  // 73728 B per page
constexpr int kRowChunks = kRowBytes / 16;       // 72 16-byte chunks per row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS placement of a page row. A row is 1152 B, a multiple of the bank
// period, so the same column of consecutive rows would hit the same banks.
// Chunk c (16 B) of row r is stored at chunk slot c ^ swz(r); the XOR only
// touches the low three bits, so a slot stays inside its aligned group of 8
// and inside the 72-chunk row.
__device__ __forceinline__ int lds_swizzle(int row) { return row & 7; }


// One 16-row x 16-column x 32-deep BF16 product, FP32 accumulate.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS accessors take generic pointers into __shared__ arrays and convert them
// with address-space casts (not through integers), so the compiler can still
// tell which LDS array an access touches.
// One 16x16x16 BF16 product (K = 16), FP32 accumulate.
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                       __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read16(const uint8_t* p) {
    return *(const MLA_AS3 bf16x8*)(p);
}

// Transposing LDS read: in each group of 16 lanes, lane i addresses row i/4,
// elements 4*(i%4)..+3 of a 4 x 16 block of 16-bit values and receives column
// i of that block (its 4 rows).
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_AS3 bf16x4*)(p));
}

// 16-byte direct load from global memory into LDS, issued so that the
// compiler does not track it. Every lane supplies its own source (`base` is
// wave-uniform, `voff` the lane's byte offset from it); the wave's 64 chunks
// land contiguously from LDS byte address `lds_addr` (lane k at 16 k). The
// caller owns every wait for it (s_waitcnt vmcnt before reading the
// destination, and before reusing it): the compiler's own tracking of such
// loads cannot tell two LDS buffers apart and would drain every load in
// flight before each LDS read. M0 is named as clobbered: the kernels using
// this helper have no other use of M0, so nothing the compiler keeps there
// is lost.
__device__ __forceinline__ void load_lds16_untracked(const void* base, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_addr), "v"(voff), "s"(base)
        : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)(const MLA_AS3 void*)(p);
}

__device__ __forceinline__ float wave_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over the four lanes i, i^16, i^32, i^48 (the k-groups of one
// MFMA column) with the lane-swap VALU ops, which stay out of the LDS queue.
// permlane16_swap(x, x) leaves x[l & ~16] and x[l | 16] in its two results,
// permlane32_swap(x, x) leaves x[l & ~32] and x[l | 32].
__device__ __forceinline__ float max_over_kgroups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_kgroups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


__device__ __forceinline__ bf16x4 pack_bf16x4(f32x4 v) {
    bf16x4 r;
    r[0] = (__bf16)v[0]; r[1] = (__bf16)v[1]; r[2] = (__bf16)v[2]; r[3] = (__bf16)v[3];
    return r;
}

__device__ __forceinline__ bf16x8 cat_bf16x4(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

}  // namespace mla
