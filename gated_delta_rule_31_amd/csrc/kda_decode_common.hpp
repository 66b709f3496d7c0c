// kda_decode_common.hpp -- the per-token arithmetic of the decode kernels (kda_decode.hip:
// one token; kda_decode_multi.hip: the conv, gate and norm steps of several tokens per
// launch).  Not part of the public ABI.
//
// Floating-point contraction is off from here to the end of the including file, and every
// fused multiply-add is written out (fmaf): left to the compiler, the choice of which
// product of a*b + c*d to fuse depends on the surrounding code and on register pressure,
// and so could differ between kernels that share these steps.
#pragma once

#include "kda_device.hpp"

#pragma clang fp contract(off)

namespace kda {

// Workgroups are dealt to the 8 XCDs round-robin in id order.  This maps hardware id i
// (XCD i % 8, its (i / 8)-th workgroup) to a logical id so that each XCD walks one
// contiguous eighth of the (sequence, head) range in order: its L2, address translation
// and DRAM pages then see one streaming region instead of every eighth 64 KiB state.
// A bijection for any n, so the result does not depend on the dispatch order.
__device__ __forceinline__ int xcd_contiguous(int i, int n) {
    const int q = n >> 3, r = n & 7, x = i & 7;
    return x * q + min(x, r) + (i >> 3);
}

// x + x of the lane that the DPP control ctrl names (the source lane always active)
template <int kCtrl>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// Sum over groups of W consecutive lanes (W a power of two <= 64), the same bits on every
// lane of a group: a butterfly over lane distances 1, 2, 4, ..., W/2, smallest first.
// Distances 1 and 2 pair lanes l and l ^ d (DPP quad permutes); after them each quad
// holds one value, so distances 4 and 8 may pair whole quads and octets by reversing
// half-rows and rows (DPP mirrors) instead of by l ^ d; 16 and 32 take the permlane
// swaps.  Each stage adds two equal-length partial sums, and both lanes of a pair add
// the same two numbers.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 2) x = add_dpp<0xb1>(x);   // quad_perm [1, 0, 3, 2]
    if constexpr (W >= 4) x = add_dpp<0x4e>(x);   // quad_perm [2, 3, 0, 1]
    if constexpr (W >= 8) x = add_dpp<0x141>(x);  // row_half_mirror
    if constexpr (W >= 16) x = add_dpp<0x140>(x); // row_mirror
    if constexpr (W >= 32) x = add_xor16(x);
    if constexpr (W >= 64) x = add_xor32(x);
    return x;
}

// ShortConv4 of one channel: taps w against the carried window (w0 oldest) and the new
// input x
__device__ __forceinline__ float conv4(const float4 &w, float w0, float w1, float w2, float x) {
    return fmaf(w.w, x, fmaf(w.z, w2, fmaf(w.y, w1, w.x * w0)));
}

__device__ __forceinline__ float silu(float y) { return y * sigm(y); }

// the decay of one key channel, alpha = exp(lower * sigmoid(rate (z + dt_bias)))
__device__ __forceinline__ float decay(float lower, float rate, float z, float dtb) {
    return __expf(lower * sigm(rate * (z + dtb)));
}

// 1 / sqrt(x) from the hardware reciprocal square root (about 1 ulp), for the L2 and RMS
// norms
__device__ __forceinline__ float inv_sqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// One lane's share of the state: rows rg + 8j (j < 16) of value columns 4cg .. 4cg+3.

// pa += S^T (alpha k^), pc += S^T (alpha q^) over the lane's 16 rows; akq[r] holds
// (alpha k^, alpha q^) of key row r
__device__ __forceinline__ void key_dots(const f32x4 (&s)[16], const float2 *akq, int rg, float (&pa)[4],
                                         float (&pc)[4]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float2 f = akq[rg + 8 * j];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pa[c] = fmaf(s[j][c], f.x, pa[c]);
            pc[c] = fmaf(s[j][c], f.y, pc[c]);
        }
    }
}

// u = beta (v - a) and o = c + (k^ . q^) u on the lane's 4 columns, from the four waves'
// partial dot products part[wave][0: a, 1: c][column]
__device__ __forceinline__ void delta_and_readout(const float (*part)[2][kD], const float *v, float beta, float kappa,
                                                  int cg, float (&u)[4], float (&o)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int col = 4 * cg + c;
        const float av = part[0][0][col] + part[1][0][col] + part[2][0][col] + part[3][0][col];
        const float cv = part[0][1][col] + part[1][1][col] + part[2][1][col] + part[3][1][col];
        u[c] = beta * (v[col] - av);
        o[c] = fmaf(kappa, u[c], cv);
    }
}

// one row of S' = Diag(alpha) S + k^ u^T; alk = (alpha, k^) of the row
__device__ __forceinline__ f32x4 update_row(const f32x4 &s, float2 alk, const float (&u)[4]) {
    f32x4 n;
#pragma unroll
    for (int c = 0; c < 4; ++c) n[c] = fmaf(alk.y, u[c], alk.x * s[c]);
    return n;
}

// 1 / RMS over the 128 columns held by lanes 0..31 (4 each) of one wave
__device__ __forceinline__ float rms_inv(const float (&o)[4], float eps) {
    const float ss = group_sum<32>(fmaf(o[3], o[3], fmaf(o[2], o[2], fmaf(o[1], o[1], o[0] * o[0]))));
    return inv_sqrt(fmaf(ss, 1.0f / kD, eps));
}

}  // namespace kda
