// mla_store_asm.h - epilogue stores of one wave's output row tiles.
//
// The stores are written as one inline-asm block so that the compiler does
// not track them: it counts store-data registers on the same counter as the
// direct-to-LDS loads, and a store-data register later reused as the target
// of a transposing LDS read made it wait for every load in flight before each
// such read. Nothing waits for the stores to complete: the data registers are
// read when a store issues (the closing s_nop covers the one wait state a
// VALU write to the data of a 16-byte store needs), and a vmcnt wait issued
// later for younger loads stays exact, because loads complete in order, so
// older stores can only make it wait longer.
//
// out tiles: tile t stores 4 BF16 values at p + 32*t bytes.
// partial tiles: tile t stores 4 FP32 values at p + 64*t bytes. When a
// workgroup on another XCD merges the partials in the same kernel they are
// written through to the device-coherent level (sc1), so that it reads them
// after an acquire with no write-back of this XCD's L2; when a later kernel
// merges them, ordinary write-back stores suffice (the kernel boundary makes
// them visible) and leave the workgroup sooner.
#pragma once

#include "mla_common.h"

namespace mla {

template <int N>
struct TileStores;

template <>
struct TileStores<8> {
    __device__ __forceinline__ static void out(uint16_t* p, const bf16x4 (&v)[8]) {
        asm volatile("global_store_dwordx2 %0, %1, off offset:0\n\t"
                     "global_store_dwordx2 %0, %2, off offset:32\n\t"
                     "global_store_dwordx2 %0, %3, off offset:64\n\t"
                     "global_store_dwordx2 %0, %4, off offset:96\n\t"
                     "global_store_dwordx2 %0, %5, off offset:128\n\t"
                     "global_store_dwordx2 %0, %6, off offset:160\n\t"
                     "global_store_dwordx2 %0, %7, off offset:192\n\t"
                     "global_store_dwordx2 %0, %8, off offset:224\n\t"
                     "s_nop 1"
                     :
                     : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7])
                     : "memory");
    }
    __device__ __forceinline__ static void part(float* p, const f32x4 (&v)[8], bool coherent) {
        if (coherent) {
            asm volatile("global_store_dwordx4 %0, %1, off offset:0 sc1\n\t"
                         "global_store_dwordx4 %0, %2, off offset:64 sc1\n\t"
                         "global_store_dwordx4 %0, %3, off offset:128 sc1\n\t"
                         "global_store_dwordx4 %0, %4, off offset:192 sc1\n\t"
                         "global_store_dwordx4 %0, %5, off offset:256 sc1\n\t"
                         "global_store_dwordx4 %0, %6, off offset:320 sc1\n\t"
                         "global_store_dwordx4 %0, %7, off offset:384 sc1\n\t"
                         "global_store_dwordx4 %0, %8, off offset:448 sc1\n\t"
                         "s_nop 1"
                         :
                         : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7])
                         : "memory");
        } else {
            asm volatile("global_store_dwordx4 %0, %1, off offset:0\n\t"
                         "global_store_dwordx4 %0, %2, off offset:64\n\t"
                         "global_store_dwordx4 %0, %3, off offset:128\n\t"
                         "global_store_dwordx4 %0, %4, off offset:192\n\t"
                         "global_store_dwordx4 %0, %5, off offset:256\n\t"
                         "global_store_dwordx4 %0, %6, off offset:320\n\t"
                         "global_store_dwordx4 %0, %7, off offset:384\n\t"
                         "global_store_dwordx4 %0, %8, off offset:448\n\t"
                         "s_nop 1"
                         :
                         : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7])
                         : "memory");
        }
    }
};

}  // namespace mla
