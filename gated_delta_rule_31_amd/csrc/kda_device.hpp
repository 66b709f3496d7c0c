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

// x[l] + x[l ^ 32] on every lane l of the wave.  v_permlane32_swap with both operands x
// returns x of lane l & 31 in its first result and of lane l | 32 in its second, so one
// instruction replaces the LDS permute (and its lane-index arithmetic) of a shuffle.  The
// sum has the same two terms as x + shuffle_xor(x, 32), in the same order on lanes
// 0..31 and swapped on lanes 32..63, which fp32 addition does not see: same bits.
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x[l] + x[l ^ 16], likewise with v_permlane16_swap (first result: lane l & ~16, second:
// lane l | 16)
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// The lo part x - hi of x = hi + lo, rounded to bf16.  The subtraction stays a plain
// subtraction: fast contraction could otherwise fuse it with the multiply that produced x
// or not, depending on how the inlining kernel happens to be scheduled, and the lo bits
// would then differ between kernels that must agree bit for bit.
__device__ __forceinline__ __bf16 bf16_lo(float x, __bf16 hi) {
#pragma clang fp contract(off)
    return (__bf16)(x - (float)hi);
}
// x = hi + lo with hi, lo bf16 (hi = RNE(x)); hi*hi' + lo*hi' + hi*lo' then carries about
// 16 significant bits of each operand through a bf16 MFMA
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = (__bf16)x[j];
        hi[j] = h;
        lo[j] = bf16_lo(x[j], h);
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

// The cache-policy operand of the load builtins for a device-scope (sc1) access: it does
// not return a copy that one XCD's caches hold, so it sees what another workgroup of the
// same launch made visible at device scope.
constexpr int kCpolSc1 = 16;
// Word 3 of a raw buffer resource (stride 0, byte-addressed, range-checked against its
// size) on gfx9-family chips such as gfx950.
constexpr int kBufferRsrcWord3 = 0x00020000;
// The s_waitcnt operand (gfx9 encoding) of vmcnt(0) alone: expcnt 7 and lgkmcnt 15 wait
// for nothing.
constexpr int kWaitVmcnt0 = 0x0F70;

// ---- workgroup order of the per-(sequence, head) prefill kernels ----
// Workgroups start in id order as compute units free up, so in a batch of unequal
// sequences the last long ones would run alone at the end.  For batches of up to
// kOrderMaxSeqs sequences the fused kernel and the carry give workgroup r*H + h the
// r-th longest sequence (ties by index), longest first; larger batches keep index order.
// Every workgroup ranks the lengths itself (at most kOrderMaxSeqs comparisons per lane),
// so no table is needed.  order: kOrderMaxSeqs ints of LDS, free until the barrier.
constexpr int kOrderMaxSeqs = 64;
__device__ __forceinline__ int seq_longest_first(const int32_t *cu_seqlens, int B, int N, int r, int *order) {
    if (B > kOrderMaxSeqs) return r;  // (uniform)
    const int tid = (int)threadIdx.x;
    auto len = [&](int s) {
        const int t0 = min(max(cu_seqlens[s], 0), N);
        return min(max(cu_seqlens[s + 1], t0), N) - t0;
    };
    if (tid < B) {
        const int ls = len(tid);
        int rank = 0;
        for (int s = 0; s < B; ++s) {
            const int l = len(s);
            rank += (l > ls || (l == ls && s < tid)) ? 1 : 0;
        }
        order[rank] = tid;  // the ranks are a permutation of 0 .. B-1
    }
    __syncthreads();
    const int seq = order[r];
    __syncthreads();  // the caller reuses the space
    return seq;
}

// ---- one chunk record of the chunk-parallel prefill ----
// Everything a chunk contributes that does not depend on the state entering it.  The
// first Rec::kPieces pieces of 1 KB are the MFMA operands of the carry's products in the
// order the carry reads them: piece p holds at byte 16l the 16 bytes (8 bf16) that lane
// l = 16lg + lr of every carry wave reads for that MFMA.  The carry copies the pieces into
// LDS as they are (one direct-to-LDS load of 1 KB each) and reads each operand with one
// linear, conflict-free 16-byte LDS read.
//   W   16 pieces (tp, x, P):       W[32tp + 8(lr/4) + 4x + lr%4][32P + 8lg .. +7]
//   Q~  16 pieces (tt, P):          Q~[16tt + lr][32P + 8lg .. +7]
//   P   12 pieces (slab s, hi/lo):  P[16tt + lr][32tp + 8lg .. +7] for the slabs
//                                   s = (tt, tp) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
//                                   (the others are zero: P is lower triangular)
//   K   32 pieces (P, x, tp, hi/lo): K_end^T[32P + 8(lr/4) + 4x + lr%4][32tp + 8lg .. +7]
//   E    1 piece:                   e^{G_end} fp32 [128 keys], then 512 zero bytes
// with W = T (beta k e^G), Q~ = q e^G, K_end = k e^{G_end - G}, P and K_end split into
// bf16 hi + lo.  The high-precision record (kPrecise) also carries the lo parts of W and
// Q~ (16 pieces each, right after their hi parts), so that the carry's W S0 and Q~ S0 take
// both operands split.  After the pieces, U' = T (beta v) in fp32, in the register order of
// the consumer: [8 waves][2 tp][2 x][64 lanes][4] (the accumulator rows of token
// 32tp + 8lg + 4x + i, value column 16w + lr).
constexpr int REC_PIECE = 1024;
template <bool kPrecise>
struct Rec {
    static constexpr int kW = 0;                       // piece indices
    static constexpr int kWL = 16;                     // (kPrecise only)
    static constexpr int kQ = kPrecise ? 32 : 16;
    static constexpr int kQL = 48;                     // (kPrecise only)
    static constexpr int kP = kPrecise ? 64 : 32;
    static constexpr int kK = kPrecise ? 76 : 44;
    static constexpr int kE = kPrecise ? 108 : 76;
    static constexpr int kPieces = kE + 1;
    static constexpr int kU = kPieces * REC_PIECE;     // byte offset of U'
    static constexpr int kBytes = kU + 8 * 2 * 2 * 64 * 16;
    // hl: 0 = hi, 1 = lo (the lo parts of W and Q~ exist in the precise record only)
    __device__ static __forceinline__ int w(int tp, int x, int P, int hl = 0) {
        return (hl ? kWL : kW) + (tp * 2 + x) * 4 + P;
    }
    __device__ static __forceinline__ int q(int tt, int P, int hl = 0) { return (hl ? kQL : kQ) + tt * 4 + P; }
    __device__ static __forceinline__ int p(int tt, int tp, int hl) { return kP + 2 * (tt < 2 ? tt : 2 * tt - 2 + tp) + hl; }
    __device__ static __forceinline__ int k(int P, int x, int tp, int hl) { return kK + ((P * 2 + x) * 2 + tp) * 2 + hl; }
};
static_assert(Rec<false>::kBytes == kRecBytes, "record layout");
static_assert(Rec<true>::kBytes == kRecBytesPrecise, "record layout");

// ---- the state-side readout and its epilogue, shared by the fused and chunked plans ----
// O is computed transposed, O^T = S0^T Q~^T + U^T P^T, so that lane (lr, lg) of wave w
// holds o[tt][i] = O[token 16tt + lr][value 16w + 4lg + i]: four consecutive values of one
// output row, stored with one 16-byte (fp32) or 8-byte (bf16) store.  Both plans run the
// same MFMAs in the same order and the same reductions below, so they give the same bits.

// The wave's partial sums of squares of each token's 16 values, into part[token][wave]
// ([64][8] fp32).
__device__ __forceinline__ void rms_partials(const f32x4 (&o)[4], float *part, int w, int lr, int lg) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        float s = o[tt][0] * o[tt][0];
        s = __builtin_fmaf(o[tt][1], o[tt][1], s);
        s = __builtin_fmaf(o[tt][2], o[tt][2], s);
        s = __builtin_fmaf(o[tt][3], o[tt][3], s);
        s = add_xor16(s);
        s = add_xor32(s);
        if (lg == 0) part[(16 * tt + lr) * 8 + w] = s;
    }
}

// This lane's part of the element index of its epilogue values in a [tokens][H*128] row
// block: row lr of a 16-row group, value columns 16w + 4lg .. +3.  The chunk's first
// row, the head and the 16-row group are wave-uniform and added per use, so a chunk's
// gate loads and output stores need one 64-bit multiply per lane instead of one per
// 16-row group (the opaque copy keeps the compiler from expanding it back).  The fused
// kernel's epilogue takes this form (its 1x8192 and 16-sequence prefills ran 1.7% and
// 1.4% faster); the carry keeps the per-row form, which the compiler schedules among its
// record loads better (the offset form was 0.5-1.3% slower there).
__device__ __forceinline__ size_t epi_lane_offset(size_t HD, int w, int lr, int lg) {
    size_t off = (size_t)lr * HD + (size_t)(16 * w + 4 * lg);
    asm volatile("" : "+v"(off));
    return off;
}

// The output-gate logits of this lane's values (4 bf16 of each of its 4 tokens; rows
// past the sequence's end are clamped to its last row and never stored), per row.
__device__ __forceinline__ void load_gate4(uint2 (&g4)[4], const uint16_t *g, size_t HD, int h, int tok0, int L,
                                           int w, int lr, int lg) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok = min(16 * tt + lr, L - 1);
        g4[tt] = *reinterpret_cast<const uint2 *>(g + (size_t)(tok0 + tok) * HD + (size_t)h * kD + 16 * w + 4 * lg);
    }
}
// The same loads with the lane's offset (epi_lane_offset) for a whole chunk, and the
// per-row clamp only for a partial one.
__device__ __forceinline__ void load_gate4_off(uint2 (&g4)[4], const uint16_t *g, size_t HD, int h, int tok0, int L,
                                               size_t lane_off, int w, int lr, int lg) {
    if (L == kChunk) {
        const uint16_t *g0 = g + (size_t)tok0 * HD + (size_t)h * kD;  // the chunk's first row (uniform)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            g4[tt] = *reinterpret_cast<const uint2 *>(g0 + (size_t)(16 * tt) * HD + lane_off);
    } else {
        load_gate4(g4, g, HD, h, tok0, L, w, lr, lg);
    }
}

// out = sigmoid(g) * RMSNorm(O) for tokens 16tt + lr < L of a chunk whose first token is
// packed row tok0, once every wave's partial sums are in part.  nw: the RMSNorm weight of
// this lane's 4 value columns.  kBf16: the output buffer holds bf16 (round to nearest
// even), else fp32.  The norm's reciprocal square root is the hardware one (about 1 ulp).
// Branch-free when L is the full chunk, so that the compiler can interleave it with
// independent MFMAs.  kLaneOff: output addresses from lane_off (epi_lane_offset), else per
// row from w, lr and lg.
template <bool kBf16, bool kLaneOff>
__device__ __forceinline__ void gated_rms_store(const f32x4 (&o)[4], const uint2 (&g4)[4], const float *part,
                                                const float (&nw)[4], float rms_eps, void *out, size_t HD, int h,
                                                int tok0, int L, size_t lane_off, int w, int lr, int lg) {
    const size_t row0 = (size_t)tok0 * HD + (size_t)h * kD;  // the chunk's first row (uniform)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok = 16 * tt + lr;
        const float2 pp = *reinterpret_cast<const float2 *>(part + tok * 8 + 2 * lg);
        float s = pp.x + pp.y;
        s = add_xor16(s);
        s = add_xor32(s);
        const float rinv = __builtin_amdgcn_rsqf(s * (1.0f / kD) + rms_eps);
        const float gg[4] = {__uint_as_float(g4[tt].x << 16), __uint_as_float(g4[tt].x & 0xffff0000u),
                             __uint_as_float(g4[tt].y << 16), __uint_as_float(g4[tt].y & 0xffff0000u)};
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = sigm(gg[i]) * (o[tt][i] * rinv * nw[i]);
        const size_t idx = kLaneOff ? row0 + (size_t)(16 * tt) * HD + lane_off
                                    : (size_t)(tok0 + tok) * HD + (size_t)h * kD + 16 * w + 4 * lg;
        if (tok < L) store_out4(out, idx, y[0], y[1], y[2], y[3], kBf16);
    }
}

}  // namespace kda
