// kda_device.hpp -- device-side helpers shared by the prefill kernels (kda_prefill.hip,
// kda_carry.hip): vector types, MFMA wrappers, swizzled LDS tile indexing, bf16
// conversions, and the layout of one chunk record of the chunk-parallel prefill.  The
// decode kernels use its vector types, barrier and sigmoid (through
// kda_decode_common.hpp).
// Not part of the public ABI.
#pragma once

#include "kda_internal.hpp"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 [rows][64] and [rows][128] tiles, 16-byte chunks XOR-swizzled by row, so that
// 16 lanes reading one 16-byte chunk from each of 16 consecutive rows hit distinct banks
__device__ __forceinline__ int sw64(int row, int col) {
    return row * 64 + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}
__device__ __forceinline__ int sw128(int row, int col) {
    return row * 128 + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}
// The same tiles for A operands read with the accumulator row interleave (lane l reads
// row 32p + 8(l/4) + 4x + l%4): the chunk index is XORed with a row function that is
// distinct over the rows 8 consecutive lanes read (row & 7 repeats after 4 of them,
// which costs a 2-way bank conflict on every read).
__device__ __forceinline__ int swi64(int row, int col) {
    const int f = (row & 3) | ((row >> 1) & 4);
    return row * 64 + (((col >> 3) ^ f) << 3) + (col & 7);
}
__device__ __forceinline__ int swi128(int row, int col) {
    const int f = (row & 3) | ((row >> 1) & 12);
    return row * 128 + (((col >> 3) ^ f) << 3) + (col & 7);
}

// D += A B on one 16x16 tile.  bf16, K = 32: lane l holds A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16] (j < 8) and receives D[4(l/16)+i][l%16] (i < 4).
__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32, K = 4: lane l holds A[l%16][l/16] and B[l/16][l%16]
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS traffic.  __syncthreads() also waits for all of the wave's
// outstanding global loads and stores (this GPU counts both on one counter), which would
// expose the latency of prefetches and output stores meant to run across it; this one
// waits for the wave's LDS operations only.  Use it where every cross-wave dependency
// goes through LDS.  The memory clobber keeps the compiler from moving any memory
// access across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
// sigmoid with the hardware reciprocal (about 1 ulp) instead of an IEEE division
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// x = hi + lo with hi, lo bf16 (hi = RNE(x)); hi*hi' + lo*hi' + hi*lo' then carries about
// 16 significant bits of each operand through a bf16 MFMA
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = (__bf16)x[j];
        hi[j] = h;
        lo[j] = (__bf16)(x[j] - (float)h);
    }
}
__device__ __forceinline__ bf16x8 to_bf8(const float *x) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
    return r;
}
__device__ __forceinline__ void unpack8(const u32x4 &u, float *x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void lds_read8(const float *p, float *x) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void lds_write8(float *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// ---- one chunk record of the chunk-parallel prefill (bytes) ----
// Everything a chunk contributes that does not depend on the state entering it: the
// first five entries are the LDS images (swizzled as above) of the MFMA A operands of
// the state-side products, U' is stored in the register order of the consumer (value
// column group cg of 16, token pair tp, interleave x, lane: 16 bytes each, the
// accumulator rows of token 32tp + 8(l/16) + 4x + i, column 16cg + l%16).
constexpr int REC_W = 0;           // W = T (beta k e^G)        bf16 swi128 [64 tok][128 key]
constexpr int REC_Q = 16384;       // Q~ = q e^G                 bf16 sw128 [64 tok][128 key]
constexpr int REC_PH = 32768;      // P, hi part                 bf16 sw64  [64 tok][64 tok]
constexpr int REC_PL = 40960;      // P, lo part
constexpr int REC_KH = 49152;      // K_end^T = (k e^{G_end-G})^T, hi   bf16 swi64 [128 key][64 tok]
constexpr int REC_KL = 65536;      // K_end^T, lo part
constexpr int REC_IMG = 81920;     // bytes of the five operand images
constexpr int REC_U = 81920;       // U' = T (beta v)            fp32 [8 cg][2 tp][2 x][64 lanes][4]
constexpr int REC_E = 114688;      // e^{G_end}                  fp32 [128 key]
static_assert(REC_U + 8 * 2 * 2 * 64 * 16 == REC_E && REC_E + 512 == kRecBytes, "record layout");

}  // namespace kda
