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
// partial tiles: tile t stores 4 FP32 values at p + 64*t bytes.
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
    __device__ __forceinline__ static void part(float* p, const f32x4 (&v)[8]) {
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
};

template <>
struct TileStores<16> {
    __device__ __forceinline__ static void out(uint16_t* p, const bf16x4 (&v)[16]) {
        asm volatile("global_store_dwordx2 %0, %1, off offset:0\n\t"
                     "global_store_dwordx2 %0, %2, off offset:32\n\t"
                     "global_store_dwordx2 %0, %3, off offset:64\n\t"
                     "global_store_dwordx2 %0, %4, off offset:96\n\t"
                     "global_store_dwordx2 %0, %5, off offset:128\n\t"
                     "global_store_dwordx2 %0, %6, off offset:160\n\t"
                     "global_store_dwordx2 %0, %7, off offset:192\n\t"
                     "global_store_dwordx2 %0, %8, off offset:224\n\t"
                     "global_store_dwordx2 %0, %9, off offset:256\n\t"
                     "global_store_dwordx2 %0, %10, off offset:288\n\t"
                     "global_store_dwordx2 %0, %11, off offset:320\n\t"
                     "global_store_dwordx2 %0, %12, off offset:352\n\t"
                     "global_store_dwordx2 %0, %13, off offset:384\n\t"
                     "global_store_dwordx2 %0, %14, off offset:416\n\t"
                     "global_store_dwordx2 %0, %15, off offset:448\n\t"
                     "global_store_dwordx2 %0, %16, off offset:480\n\t"
                     "s_nop 1"
                     :
                     : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15])
                     : "memory");
    }
    __device__ __forceinline__ static void part(float* p, const f32x4 (&v)[16]) {
        asm volatile("global_store_dwordx4 %0, %1, off offset:0\n\t"
                     "global_store_dwordx4 %0, %2, off offset:64\n\t"
                     "global_store_dwordx4 %0, %3, off offset:128\n\t"
                     "global_store_dwordx4 %0, %4, off offset:192\n\t"
                     "global_store_dwordx4 %0, %5, off offset:256\n\t"
                     "global_store_dwordx4 %0, %6, off offset:320\n\t"
                     "global_store_dwordx4 %0, %7, off offset:384\n\t"
                     "global_store_dwordx4 %0, %8, off offset:448\n\t"
                     "global_store_dwordx4 %0, %9, off offset:512\n\t"
                     "global_store_dwordx4 %0, %10, off offset:576\n\t"
                     "global_store_dwordx4 %0, %11, off offset:640\n\t"
                     "global_store_dwordx4 %0, %12, off offset:704\n\t"
                     "global_store_dwordx4 %0, %13, off offset:768\n\t"
                     "global_store_dwordx4 %0, %14, off offset:832\n\t"
                     "global_store_dwordx4 %0, %15, off offset:896\n\t"
                     "global_store_dwordx4 %0, %16, off offset:960\n\t"
                     "s_nop 1"
                     :
                     : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15])
                     : "memory");
    }
};

template <>
struct TileStores<32> {
    __device__ __forceinline__ static void out(uint16_t* p, const bf16x4 (&v)[32]) {
        asm volatile("global_store_dwordx2 %0, %1, off offset:0\n\t"
                     "global_store_dwordx2 %0, %2, off offset:32\n\t"
                     "global_store_dwordx2 %0, %3, off offset:64\n\t"
                     "global_store_dwordx2 %0, %4, off offset:96\n\t"
                     "global_store_dwordx2 %0, %5, off offset:128\n\t"
                     "global_store_dwordx2 %0, %6, off offset:160\n\t"
                     "global_store_dwordx2 %0, %7, off offset:192\n\t"
                     "global_store_dwordx2 %0, %8, off offset:224\n\t"
                     "global_store_dwordx2 %0, %9, off offset:256\n\t"
                     "global_store_dwordx2 %0, %10, off offset:288\n\t"
                     "global_store_dwordx2 %0, %11, off offset:320\n\t"
                     "global_store_dwordx2 %0, %12, off offset:352\n\t"
                     "global_store_dwordx2 %0, %13, off offset:384\n\t"
                     "global_store_dwordx2 %0, %14, off offset:416\n\t"
                     "global_store_dwordx2 %0, %15, off offset:448\n\t"
                     "global_store_dwordx2 %0, %16, off offset:480\n\t"
                     "global_store_dwordx2 %0, %17, off offset:512\n\t"
                     "global_store_dwordx2 %0, %18, off offset:544\n\t"
                     "global_store_dwordx2 %0, %19, off offset:576\n\t"
                     "global_store_dwordx2 %0, %20, off offset:608\n\t"
                     "global_store_dwordx2 %0, %21, off offset:640\n\t"
                     "global_store_dwordx2 %0, %22, off offset:672\n\t"
                     "global_store_dwordx2 %0, %23, off offset:704\n\t"
                     "global_store_dwordx2 %0, %24, off offset:736\n\t"
                     "global_store_dwordx2 %0, %25, off offset:768\n\t"
                     "global_store_dwordx2 %0, %26, off offset:800\n\t"
                     "global_store_dwordx2 %0, %27, off offset:832\n\t"
                     "global_store_dwordx2 %0, %28, off offset:864\n\t"
                     "global_store_dwordx2 %0, %29, off offset:896\n\t"
                     "global_store_dwordx2 %0, %30, off offset:928\n\t"
                     "global_store_dwordx2 %0, %31, off offset:960\n\t"
                     "global_store_dwordx2 %0, %32, off offset:992\n\t"
                     "s_nop 1"
                     :
                     : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]), "v"(v[16]), "v"(v[17]), "v"(v[18]), "v"(v[19]), "v"(v[20]), "v"(v[21]), "v"(v[22]), "v"(v[23]), "v"(v[24]), "v"(v[25]), "v"(v[26]), "v"(v[27]), "v"(v[28]), "v"(v[29]), "v"(v[30]), "v"(v[31])
                     : "memory");
    }
    __device__ __forceinline__ static void part(float* p, const f32x4 (&v)[32]) {
        asm volatile("global_store_dwordx4 %0, %1, off offset:0\n\t"
                     "global_store_dwordx4 %0, %2, off offset:64\n\t"
                     "global_store_dwordx4 %0, %3, off offset:128\n\t"
                     "global_store_dwordx4 %0, %4, off offset:192\n\t"
                     "global_store_dwordx4 %0, %5, off offset:256\n\t"
                     "global_store_dwordx4 %0, %6, off offset:320\n\t"
                     "global_store_dwordx4 %0, %7, off offset:384\n\t"
                     "global_store_dwordx4 %0, %8, off offset:448\n\t"
                     "global_store_dwordx4 %0, %9, off offset:512\n\t"
                     "global_store_dwordx4 %0, %10, off offset:576\n\t"
                     "global_store_dwordx4 %0, %11, off offset:640\n\t"
                     "global_store_dwordx4 %0, %12, off offset:704\n\t"
                     "global_store_dwordx4 %0, %13, off offset:768\n\t"
                     "global_store_dwordx4 %0, %14, off offset:832\n\t"
                     "global_store_dwordx4 %0, %15, off offset:896\n\t"
                     "global_store_dwordx4 %0, %16, off offset:960\n\t"
                     "global_store_dwordx4 %0, %17, off offset:1024\n\t"
                     "global_store_dwordx4 %0, %18, off offset:1088\n\t"
                     "global_store_dwordx4 %0, %19, off offset:1152\n\t"
                     "global_store_dwordx4 %0, %20, off offset:1216\n\t"
                     "global_store_dwordx4 %0, %21, off offset:1280\n\t"
                     "global_store_dwordx4 %0, %22, off offset:1344\n\t"
                     "global_store_dwordx4 %0, %23, off offset:1408\n\t"
                     "global_store_dwordx4 %0, %24, off offset:1472\n\t"
                     "global_store_dwordx4 %0, %25, off offset:1536\n\t"
                     "global_store_dwordx4 %0, %26, off offset:1600\n\t"
                     "global_store_dwordx4 %0, %27, off offset:1664\n\t"
                     "global_store_dwordx4 %0, %28, off offset:1728\n\t"
                     "global_store_dwordx4 %0, %29, off offset:1792\n\t"
                     "global_store_dwordx4 %0, %30, off offset:1856\n\t"
                     "global_store_dwordx4 %0, %31, off offset:1920\n\t"
                     "global_store_dwordx4 %0, %32, off offset:1984\n\t"
                     "s_nop 1"
                     :
                     : "v"(p), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]), "v"(v[16]), "v"(v[17]), "v"(v[18]), "v"(v[19]), "v"(v[20]), "v"(v[21]), "v"(v[22]), "v"(v[23]), "v"(v[24]), "v"(v[25]), "v"(v[26]), "v"(v[27]), "v"(v[28]), "v"(v[29]), "v"(v[30]), "v"(v[31])
                     : "memory");
    }
};

}  // namespace mla
