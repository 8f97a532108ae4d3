// tile_probe.hip - test-only kernels that run the decode kernels' building
// blocks (mla_common.h) one at a time, so that tests can check each against
// its plain definition: the 16x16x32 BF16 MFMA and its lane layout, the
// transposing LDS read, the max/sum over a row's four lane groups and the
// BF16 rounding of the output. Built into tests/tile_probe/libtile_probe.so;
// nothing in the library uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_common.h"

using namespace mla;

namespace {

// one wave: A, B given as the MFMA operands' lane layout the kernels assume
// (lane l holds A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16]);
// C[4 (l / 16) + j][l % 16] comes back in lane l, element j
__global__ void k_mfma16(const uint16_t* a, const uint16_t* b, float* c) {
    const int l = threadIdx.x;
    bf16x8 fa, fb;
    for (int k = 0; k < 8; ++k) {
        fa[k] = __builtin_bit_cast(__bf16, a[(l % 16) * 32 + 8 * (l / 16) + k]);
        fb[k] = __builtin_bit_cast(__bf16, b[(8 * (l / 16) + k) * 16 + (l % 16)]);
    }
    const f32x4 r = mfma16(fa, fb, f32x4{0.f, 0.f, 0.f, 0.f});
    for (int j = 0; j < 4; ++j) c[(4 * (l / 16) + j) * 16 + (l % 16)] = r[j];
}

// one wave: a 16 x 16 block of 16-bit values staged row-major in LDS (row
// pitch 32 B); each lane reads with lds_read_tr at the address the kernels
// give it (row i/4, elements 4 (i % 4) .. +3 of its group's 4 x 16 block,
// groups g = lane / 16 stacked four rows apart) and returns what it got
__global__ void k_read_tr(const uint16_t* src, uint16_t* dst) {
    __shared__ __attribute__((aligned(16))) uint16_t blk[16 * 16];
    const int l = threadIdx.x;
    for (int i = l; i < 256; i += 64) blk[i] = src[i];
    __syncthreads();
    const int g = l / 16, i = l % 16;
    const uint8_t* p = reinterpret_cast<const uint8_t*>(blk) + (4 * g + i / 4) * 32 + 8 * (i % 4);
    // stored as one 64-bit word (the four elements in register order)
    *reinterpret_cast<uint2*>(dst + l * 4) = __builtin_bit_cast(uint2, lds_read_tr(p));
}

// one wave: max and sum over lanes i, i^16, i^32, i^48
__global__ void k_kgroups(const float* x, float* mx, float* sm) {
    const int l = threadIdx.x;
    mx[l] = max_over_kgroups(x[l]);
    sm[l] = sum_over_kgroups(x[l]);
}

// n values (n a multiple of 4) to BF16 with pack_bf16x4
__global__ void k_pack(const float* x, uint16_t* y, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (4 * t + 3 >= n) return;
    const f32x4 v = {x[4 * t], x[4 * t + 1], x[4 * t + 2], x[4 * t + 3]};
    *reinterpret_cast<uint2*>(y + 4 * t) = __builtin_bit_cast(uint2, pack_bf16x4(v));
}

int done() { return hipGetLastError() == hipSuccess ? 0 : 1; }

}  // namespace

extern "C" {
// a [16][32], b [32][16] BF16 bits; c [16][16] FP32 (device pointers)
int probe_mfma16(const void* a, const void* b, void* c) {
    hipLaunchKernelGGL(k_mfma16, dim3(1), dim3(64), 0, 0, (const uint16_t*)a, (const uint16_t*)b, (float*)c);
    return done();
}
// src [16][16] 16-bit values; dst [64][4]
int probe_read_tr(const void* src, void* dst) {
    hipLaunchKernelGGL(k_read_tr, dim3(1), dim3(64), 0, 0, (const uint16_t*)src, (uint16_t*)dst);
    return done();
}
// x, mx, sm [64] FP32
int probe_kgroups(const void* x, void* mx, void* sm) {
    hipLaunchKernelGGL(k_kgroups, dim3(1), dim3(64), 0, 0, (const float*)x, (float*)mx, (float*)sm);
    return done();
}
// x [n] FP32, y [n] BF16 bits, n a multiple of 4
int probe_pack(const void* x, void* y, int n) {
    if (n <= 0 || n % 4) return 2;
    hipLaunchKernelGGL(k_pack, dim3((n / 4 + 255) / 256), dim3(256), 0, 0, (const float*)x, (uint16_t*)y, n);
    return done();
}
}
