// kda_prefill.hip -- chunked varlen KDA prefill on gfx950 (bf16 MFMA, fp32 state).
//
// One workgroup (4 waves) per (sequence, head) walks the sequence in chunks of 64 tokens
// and carries the 128x128 fp32 state in MFMA accumulator registers.  Every step of the
// header comment "KDA per-head recurrence" (page "colibri/c/kimi_k3.c") is fused: conv
// with the carried window, SiLU, L2 norms, gates, the chunked state update and readout,
// the gated RMSNorm and the final state / conv window write.
//
// Chunk algebra (exact rewrite of the token recurrence; G_t = sum_{s<=t} gk_s per key
// channel, chunk-local):
//   A_ts = beta_t sum_i k_ti k_si e^{G_ti - G_si}  (s < t)      T = (I + A)^-1
//   P_ts = sum_i q_ti k_si e^{G_ti - G_si}         (s <= t)
//   W = T (beta k e^G),  U' = T (beta v),  U = U' - W S0
//   O = (q e^G) S0 + P U,        S_end = Diag(e^{G_end}) S0 + (k e^{G_end - G})^T U
// e^{G_t - G_s} is never formed from e^{G_t} and e^{-G_s}, which overflow fp32 after ~18
// tokens of strong decay: each 16-token sub-chunk I has a reference r_I = G at the token
// before it, and a block (I, J) of A or P uses e^{G_t - r_I} (<= 1) times
// e^{r_I - G_s} = e^{r_I - r_J} e^{r_J - G_s} (<= e^80 on the diagonal block, since
// |gk| < 5), so no factor leaves the fp32 / bf16 exponent range.
//
// Precision: bf16 MFMA operands with fp32 accumulation; T is computed in fp32.  The
// products whose operands were measured to decide the error of the fp32 state and of
// the normalised output use a hi+lo bf16 split of those operands (3 MFMAs instead of
// 1): P (both operands), beta*v in U', U in P.U and K_end^T U, and K_end.
//
// Layout tricks.  Wave w owns value columns 32w..32w+31 of the state for all 128 keys:
// 16 accumulator tiles.  Inside each 32-key block the two 16-row tiles interleave their
// rows (tile x, row m -> key 32P + 8(m/4) + 4x + m%4), so that a lane's 8 accumulator
// values of one column are 8 consecutive keys: exactly the B-operand layout of a
// K = 32 MFMA.  The state therefore feeds W S0 and (q e^G) S0 straight from registers.
// U uses the same interleave over tokens, so it feeds P U and K_end^T U the same way.
//
// In the prologue, lane (wave w, lane l) owns token 16w + l%16 and the 32 channels
// 32(l/16) .. 32(l/16)+31: these are also the A-operand rows/K-slices of block row w of
// A and P, which wave w therefore computes from its own registers.

#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// ---- LDS map (bytes).  Regions are reused once their first tenant is dead. ----
constexpr int OFF_R1 = 0;        // sCB fp32 [64][132]          -> sKe hi/lo bf16 [128][64] x2
constexpr int OFF_R2 = 33792;    // sVt hi/lo bf16 [128][64] x2 (beta*v, transposed)
constexpr int OFF_R3 = 66560;    // sWr bf16 [128][64]          (beta k e^G, transposed)
constexpr int OFF_R4 = 82944;    // sA fp32 [64][68]            -> sW bf16 [64][128]
constexpr int OFF_R5 = 100352;   // sP fp32 [64][68]
constexpr int OFF_R6 = 117760;   // sT fp32 [64][68]            -> sQe bf16 [64][128]
constexpr int OFF_R7 = 135168;   // sTb bf16 [64][64]
constexpr int OFF_TAB = 143360;  // small fp32 tables
constexpr int kTabFloats = 512 + 640 + 768 + 512 + 512 + 128 + 64;
constexpr int OFF_CW = OFF_TAB + kTabFloats * 4;  // conv taps of this head, fp32 [3][128][4]
constexpr int kLdsBytes = OFF_CW + 3 * 128 * 4 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

constexpr int CB_LD = 132;  // fp32 row pitch of sCB
constexpr int F_LD = 68;    // fp32 row pitch of sA, sP, sT

// bf16 [rows][64] and [rows][128] tiles, 16-byte chunks XOR-swizzled by row
__device__ __forceinline__ int sw64(int row, int col) {
    return row * 64 + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}
__device__ __forceinline__ int sw128(int row, int col) {
    return row * 128 + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
// sigmoid with the hardware reciprocal (about 1 ulp) instead of an IEEE division
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

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
__device__ __forceinline__ void load8_bf16(const uint16_t *p, float *x) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
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
// inclusive prefix sum over the 16 lanes of a DPP row (lanes 16g .. 16g+15)
// (DPP row_shr:n moves lane i-n of the same 16-lane row into lane i; lanes without a
//  source receive 0)
__device__ __forceinline__ float row_scan16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
    return v;
}
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }  // J < I

// Lane coordinates, re-derived at the start of every phase from an opaque copy of the
// thread id.  Without this the compiler hoists every lane-dependent LDS address of the
// chunk loop out of the loop and keeps (or spills) hundreds of them across it.
#define KDA_LANE_IDS()                                         \
    int tid_ = (int)threadIdx.x;                               \
    asm volatile("" : "+v"(tid_));                             \
    const int w = __builtin_amdgcn_readfirstlane(tid_ >> 6);   \
    const int lr = tid_ & 15;                                  \
    const int lg = (tid_ >> 4) & 3;                            \
    const int t = 16 * w + lr;                                 \
    (void)w;                                                   \
    (void)lr;                                                  \
    (void)lg;                                                  \
    (void)t

__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sCB = reinterpret_cast<float *>(smem + OFF_R1);              // [64][132] k e^{r - G}
    float *sUq = sCB;                                                    // [64][132] q before norm
    float *sUk = reinterpret_cast<float *>(smem + OFF_R4);              // [64][132] k before norm
    __bf16 *sKeHi = reinterpret_cast<__bf16 *>(smem + OFF_R1);          // [128][64] K_end^T
    __bf16 *sKeLo = sKeHi + 128 * 64;
    __bf16 *sVtHi = reinterpret_cast<__bf16 *>(smem + OFF_R2);          // [128][64] (beta v)^T
    __bf16 *sVtLo = sVtHi + 128 * 64;
    float *sO = reinterpret_cast<float *>(smem + OFF_R2);               // [64][128] readout
    __bf16 *sWr = reinterpret_cast<__bf16 *>(smem + OFF_R3);            // [128][64] (beta k e^G)^T
    float *sA = reinterpret_cast<float *>(smem + OFF_R4);               // [64][68]
    __bf16 *sW = reinterpret_cast<__bf16 *>(smem + OFF_R4);             // [64][128]
    float *sP = reinterpret_cast<float *>(smem + OFF_R5);               // [64][68]
    float *sT = reinterpret_cast<float *>(smem + OFF_R6);               // [64][68]
    __bf16 *sQe = reinterpret_cast<__bf16 *>(smem + OFF_R6);            // [64][128] q e^G
    __bf16 *sTb = reinterpret_cast<__bf16 *>(smem + OFF_R7);            // [64][64]
    float *sTot = reinterpret_cast<float *>(smem + OFF_TAB);  // [4][128] per-wave gk sums
    float *sRef = sTot + 512;                                  // [5][128] r_0..r_3, G_end
    float *sPair = sRef + 640;                                 // [6][128] e^{r_I - r_J}, J < I
    float *sExpRef = sPair + 768;                              // [4][128] e^{r_I}
    float *sEndRef = sExpRef + 512;                            // [4][128] e^{G_end - r_I}
    float *sExpEnd = sEndRef + 512;                            // [128]    e^{G_end}
    float *sBeta = sExpEnd + 128;                              // [64]
    float *sConvW = reinterpret_cast<float *>(smem + OFF_CW);  // [3][128][4] taps, oldest first

    const int H = a.c.H;
    const int N = a.N;
    const int seq = blockIdx.x / H;
    const int h = blockIdx.x - seq * H;
    const size_t HD = (size_t)H * kD;
    int t0 = a.cu_seqlens[seq];
    int t1 = a.cu_seqlens[seq + 1];
    t0 = min(max(t0, 0), N);
    t1 = min(max(t1, t0), N);
    const int T = t1 - t0;

    const float gmin = a.c.gate_lower_bound;
    const float rate = __expf(a.A_log[h]);
    const float qscale = a.c.q_scale;
    const float l2eps = a.c.l2_eps;
    const size_t conv_seq = (size_t)seq * 3 * HD * 3;  // this sequence's conv windows
    const uint16_t *X[3] = {a.q, a.k, a.v};

    // ---- the state: S[P][x][nt][i] = S[key 32P + 8lg + 4x + i][value 32w + 16nt + lr] ----
    f32x4 S[4][2][2];
    {
        KDA_LANE_IDS();
        const float *S0 = a.initial_state ? a.initial_state + ((size_t)seq * H + h) * kD * kD : nullptr;
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = 32 * P + 8 * lg + 4 * x + i;
                        const int val = 32 * w + 16 * nt + lr;
                        S[P][x][nt][i] = S0 ? S0[key * kD + val] : 0.0f;
                    }
    }

    // the conv taps of this head's 384 channels, and its initial conv windows (zeros if
    // none): these sit in sPair/sExpRef, which the first chunk's tables step overwrites
    // only after the last read of the windows (phase 1 of chunk 0)
    float *sWin0 = sPair;  // [3*128][3]
    for (int i = threadIdx.x; i < 3 * kD; i += kThreads) {
        const int blk = i >> 7, c = i & 127;
        const size_t ch = (size_t)blk * HD + (size_t)h * kD + c;
        *reinterpret_cast<float4 *>(sConvW + i * 4) = *reinterpret_cast<const float4 *>(a.conv_w + ch * 4);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            sWin0[i * 3 + j] = a.initial_conv_state ? a.initial_conv_state[conv_seq + ch * 3 + j] : 0.f;
    }
    __syncthreads();

    for (int c0 = 0; c0 < T; c0 += kChunk) {
        const int L = min(kChunk, T - c0);

        // ================= phase 1: conv, SiLU, norms, gates =================
        // lane: token t = 16w + lr of the chunk, channels 32lg .. 32lg+31
        float qr[32], kr[32], cbk[32];  // q e^{G-r_w}, k e^{G-r_w}, k e^{r_w-G} (normalised q, k)
        {
            KDA_LANE_IDS();
            const bool valid = t < L;
            const int tau = t0 + c0 + t;  // packed row of the token
            // All raw loads first, branch-free so that they are all in flight together: rows
            // tau-3 .. tau of this lane's 32 channels of q, k, v and its z row.  Rows are
            // clamped into the sequence so every address is valid; rows before the sequence
            // start are replaced by the carried window below, padding tokens are zeroed.
            const int tauc = valid ? tau : t0 + c0;  // a padding lane reads the chunk's first row
            // uniform base of the rows this chunk may touch; lane offsets stay 32-bit
            const int rbase = max(t0 + c0 - 3, t0);
            const size_t ebase = (size_t)rbase * HD + (size_t)h * kD;
            uint4 raw[3][4][4];  // [block q,k,v][piece][row tau-3+r]
            uint4 zraw[4];
#pragma unroll
            for (int blk = 0; blk < 3; ++blk) {
                const uint16_t *base = X[blk] + ebase;
#pragma unroll
                for (int pc = 0; pc < 4; ++pc)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t tok = (uint32_t)(max(tauc - 3 + r, t0) - rbase);
                        raw[blk][pc][r] =
                            *reinterpret_cast<const uint4 *>(base + (tok * (uint32_t)HD + 32u * lg + 8u * pc));
                    }
            }
            {
                const uint16_t *base = a.z + ebase;
                const uint32_t tok = (uint32_t)(tauc - rbase);
#pragma unroll
                for (int pc = 0; pc < 4; ++pc)
                    zraw[pc] = *reinterpret_cast<const uint4 *>(base + (tok * (uint32_t)HD + 32u * lg + 8u * pc));
            }
            const float braw = bf2f(a.b[(size_t)tauc * H + h]);
            const float beta = valid ? sigm(braw) : 0.0f;
            const bool head_of_seq = c0 == 0 && t < 3;  // rows before the sequence start
            // SiLU(ShortConv4(x)) of the 8 channels 32lg + 8pc .. +7 of block blk (0 q, 1 k, 2 v)
            auto conv_piece = [&](const int blk, const int pc, float *u) {
                const int cb0 = 32 * lg + 8 * pc;
                float xr[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t wv[4] = {raw[blk][pc][r].x, raw[blk][pc][r].y, raw[blk][pc][r].z,
                                            raw[blk][pc][r].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xr[r][2 * j] = __uint_as_float(wv[j] << 16);
                        xr[r][2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
                    }
                }
                if (head_of_seq) {
#pragma unroll
                    for (int r = 0; r < 3; ++r) {
                        const int tok = tau - 3 + r;
                        if (tok < t0) {
                            const int p = tok - t0 + 3;  // slot of the carried window, 0..2
#pragma unroll
                            for (int j = 0; j < 8; ++j) xr[r][j] = sWin0[(blk * kD + cb0 + j) * 3 + p];
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float4 cw = *reinterpret_cast<const float4 *>(sConvW + (blk * kD + cb0 + j) * 4);
                    const float y = cw.x * xr[0][j] + cw.y * xr[1][j] + cw.z * xr[2][j] + cw.w * xr[3][j];
                    u[j] = valid ? y * sigm(y) : 0.f;
                }
            };
            // v: beta * v, hi/lo, transposed into sVt
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                float u[8];
                conv_piece(2, pc, u);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float bv = beta * u[j];
                    const __bf16 hi = (__bf16)bv;
                    sVtHi[sw64(32 * lg + 8 * pc + j, t)] = hi;
                    sVtLo[sw64(32 * lg + 8 * pc + j, t)] = (__bf16)(bv - (float)hi);
                }
            }
            // q, k parked in LDS until their norms are known (each lane reads back only what
            // it wrote), and their sums of squares
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                float u[8];
                float *dq = sUq + t * CB_LD + 32 * lg + 8 * pc;
                float *dk = sUk + t * CB_LD + 32 * lg + 8 * pc;
                conv_piece(0, pc, u);
#pragma unroll
                for (int j = 0; j < 8; ++j) ssq += u[j] * u[j];
                *reinterpret_cast<float4 *>(dq) = make_float4(u[0], u[1], u[2], u[3]);
                *reinterpret_cast<float4 *>(dq + 4) = make_float4(u[4], u[5], u[6], u[7]);
                conv_piece(1, pc, u);
#pragma unroll
                for (int j = 0; j < 8; ++j) ssk += u[j] * u[j];
                *reinterpret_cast<float4 *>(dk) = make_float4(u[0], u[1], u[2], u[3]);
                *reinterpret_cast<float4 *>(dk + 4) = make_float4(u[4], u[5], u[6], u[7]);
            }
            // L2 norms over the 4 lanes that hold this token's 128 channels
            ssq += __shfl_xor(ssq, 16, 64);
            ssq += __shfl_xor(ssq, 32, 64);
            ssk += __shfl_xor(ssk, 16, 64);
            ssk += __shfl_xor(ssk, 32, 64);
            const float inv_q = qscale / sqrtf(ssq + l2eps);
            const float inv_k = 1.0f / sqrtf(ssk + l2eps);
            // decay gate gk = gmin * sigmoid(exp(A_log) * (z + dt_bias)) and its cumulative sum
            // over the wave's 16 tokens (G_t - r_w); the operand rows built from it
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                const int cb0 = 32 * lg + 8 * pc;
                const uint32_t zw[4] = {zraw[pc].x, zraw[pc].y, zraw[pc].z, zraw[pc].w};
                float zz[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    zz[2 * j] = __uint_as_float(zw[j] << 16);
                    zz[2 * j + 1] = __uint_as_float(zw[j] & 0xffff0000u);
                }
                float cbv[8], uq8[8], uk8[8];
                lds_read8(sUq + t * CB_LD + cb0, uq8);
                lds_read8(sUk + t * CB_LD + cb0, uk8);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float g = valid ? gmin * sigm(rate * (zz[j] + a.dt_bias[(size_t)h * kD + cb0 + j])) : 0.f;
                    g = row_scan16(g);
                    if (lr == 15) sTot[w * 128 + cb0 + j] = g;
                    const float rf = __expf(g);
                    const float cf = __expf(-g);
                    const float kh = uk8[j] * inv_k;
                    qr[8 * pc + j] = uq8[j] * inv_q * rf;
                    kr[8 * pc + j] = kh * rf;
                    cbv[j] = kh * cf;
                    cbk[8 * pc + j] = cbv[j];
                }
                float *dst = sCB + t * CB_LD + cb0;  // overwrites this lane's own q slot
                *reinterpret_cast<float4 *>(dst) = make_float4(cbv[0], cbv[1], cbv[2], cbv[3]);
                *reinterpret_cast<float4 *>(dst + 4) = make_float4(cbv[4], cbv[5], cbv[6], cbv[7]);
            }
            if (lg == 0) sBeta[t] = beta;
        }
        __syncthreads();

        // ---- per-chunk channel tables: sub-chunk references and their exponentials ----
        {
            const int tid = threadIdx.x;
            const int c = tid & 127;
            float r[5];
            r[0] = 0.f;
            r[1] = sTot[c];
            r[2] = r[1] + sTot[128 + c];
            r[3] = r[2] + sTot[256 + c];
            r[4] = r[3] + sTot[384 + c];
            if (tid < 128) {
#pragma unroll
                for (int I = 0; I < 5; ++I) sRef[I * 128 + c] = r[I];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    sExpRef[I * 128 + c] = __expf(r[I]);
                    sEndRef[I * 128 + c] = __expf(r[4] - r[I]);
                }
                sExpEnd[c] = __expf(r[4]);
            } else {
#pragma unroll
                for (int I = 1; I < 4; ++I)
#pragma unroll
                    for (int J = 0; J < I; ++J) sPair[pair_index(I, J) * 128 + c] = __expf(r[I] - r[J]);
            }
        }
        __syncthreads();

        // ---- rows that need the tables; MFMA operands of block row w ----
        bf16x8 ak[4], aqh[4], aql[4], qe8[4];  // k e^{G-r}, q e^{G-r} (hi/lo), q e^G
        float ke[32];                            // K_end = k e^{G_end - G}
        {
            KDA_LANE_IDS();
            const float beta = sBeta[t];
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                const int cb0 = 32 * lg + 8 * pc;
                float qe[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float er = sExpRef[w * 128 + cb0 + j];
                    sWr[sw64(cb0 + j, t)] = (__bf16)(beta * kr[8 * pc + j] * er);
                    qe[j] = qr[8 * pc + j] * er;
                    ke[8 * pc + j] = cbk[8 * pc + j] * sEndRef[w * 128 + cb0 + j];
                }
                qe8[pc] = to_bf8(qe);
                ak[pc] = to_bf8(kr + 8 * pc);
                split8(qr + 8 * pc, aqh[pc], aql[pc]);
            }
        }

        // ================= phase 2: blocks (w, J <= w) of A and P =================
        {
            KDA_LANE_IDS();
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
                if (J <= w) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int cb0 = 32 * lg + 8 * ks;
                        float col[8];
                        lds_read8(sCB + (16 * J + lr) * CB_LD + cb0, col);
                        if (J < w) {
                            float pf[8];
                            lds_read8(sPair + pair_index(w, J) * 128 + cb0, pf);
#pragma unroll
                            for (int j = 0; j < 8; ++j) col[j] *= pf[j];
                        }
                        bf16x8 ch, cl;
                        split8(col, ch, cl);
                        accA = mma(ak[ks], ch, accA);
                        accP = mma(aqh[ks], ch, accP);
                        accP = mma(aql[ks], ch, accP);
                        accP = mma(aqh[ks], cl, accP);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tr = 4 * lg + i;  // row inside the 16x16 block
                    const int trow = 16 * w + tr;
                    float va = accA[i] * sBeta[trow];
                    float vp = accP[i];
                    if (J == w) {
                        if (lr >= tr) va = 0.f;
                        if (lr > tr) vp = 0.f;
                    }
                    sA[trow * F_LD + 16 * J + lr] = va;
                    sP[trow * F_LD + 16 * J + lr] = vp;
                }
            }
        }
        __syncthreads();

        // sCB is dead: K_end^T, hi/lo, into region 1
        {
            KDA_LANE_IDS();
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int c = 32 * lg + j;
                const __bf16 hi = (__bf16)ke[j];
                sKeHi[sw64(c, t)] = hi;
                sKeLo[sw64(c, t)] = (__bf16)(ke[j] - (float)hi);
            }
        }

        // ================= phase 3: T = (I + A)^-1 in fp32 =================
        // diagonal 16x16 blocks by forward substitution: wave w, lanes 0..15 own columns
        {
            KDA_LANE_IDS();
            if (lg == 0) {
                float xcol[16];
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) {
                    float acc = (tt == lr) ? 1.0f : 0.0f;
#pragma unroll
                    for (int j = 0; j < tt; ++j) acc -= sA[(16 * w + tt) * F_LD + 16 * w + j] * xcol[j];
                    xcol[tt] = acc;
                }
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) sT[(16 * w + tt) * F_LD + 16 * w + lr] = xcol[tt];
            }
        }
        __syncthreads();
        // off-diagonal blocks, by distance d = I - J:  T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
        // (fp32 MFMA; the sum M is parked in the unused upper block (J, I) of sT)
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            {
                KDA_LANE_IDS();
                if (w < 4 - d) {
                    const int J = w, I = w + d;
                    f32x4 M = {0.f, 0.f, 0.f, 0.f};
                    for (int K = J; K < I; ++K)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            M = mma_f32(sA[(16 * I + lr) * F_LD + 16 * K + 4 * kk + lg],
                                        sT[(16 * K + 4 * kk + lg) * F_LD + 16 * J + lr], M);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sT[(16 * J + 4 * lg + i) * F_LD + 16 * I + lr] = M[i];
                }
            }
            __syncthreads();
            {
                KDA_LANE_IDS();
                if (w < 4 - d) {
                    const int J = w, I = w + d;
                    f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        R = mma_f32(-sT[(16 * I + lr) * F_LD + 16 * I + 4 * kk + lg],
                                    sT[(16 * J + 4 * kk + lg) * F_LD + 16 * I + lr], R);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sT[(16 * I + 4 * lg + i) * F_LD + 16 * J + lr] = R[i];
                }
            }
            __syncthreads();
        }
        // T -> bf16 (upper blocks, which held scratch, become zero)
        {
            int tid_ = (int)threadIdx.x;
            asm volatile("" : "+v"(tid_));
            const int r = tid_ >> 2;
#pragma unroll
            for (int cc = 0; cc < 16; ++cc) {
                const int c = 16 * (tid_ & 3) + cc;
                const float v = ((c >> 4) <= (r >> 4)) ? sT[r * F_LD + c] : 0.0f;
                sTb[sw64(r, c)] = (__bf16)v;
            }
        }
        __syncthreads();
        // sT is dead: Q~ = q e^G into region 6
        {
            KDA_LANE_IDS();
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) *reinterpret_cast<bf16x8 *>(sQe + sw128(t, 32 * lg + 8 * pc)) = qe8[pc];
        }

        // ================= phase 4: W = T (beta k e^G) -> LDS;  U' = T (beta v) -> regs ====
        f32x4 U[2][2][2];  // [tp][x][nt]: U[token 32tp + 8lg + 4x + i][value 32w + 16nt + lr]
        {
            KDA_LANE_IDS();
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (ks == 1 && tt < 2) continue;  // T is lower triangular
                        const bf16x8 A8 =
                            *reinterpret_cast<const bf16x8 *>(sTb + sw64(16 * tt + lr, 32 * ks + 8 * lg));
                        const bf16x8 B8 =
                            *reinterpret_cast<const bf16x8 *>(sWr + sw64(32 * w + 16 * nt + lr, 32 * ks + 8 * lg));
                        acc = mma(A8, B8, acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sW[sw128(16 * tt + 4 * lg + i, 32 * w + 16 * nt + lr)] = (__bf16)acc[i];
                }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                        const int trow = 32 * tp + 8 * (lr >> 2) + 4 * x + (lr & 3);
                        const int vrow = 32 * w + 16 * nt + lr;
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            if (ks > tp) continue;
                            const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sTb + sw64(trow, 32 * ks + 8 * lg));
                            const bf16x8 Bh = *reinterpret_cast<const bf16x8 *>(sVtHi + sw64(vrow, 32 * ks + 8 * lg));
                            const bf16x8 Bl = *reinterpret_cast<const bf16x8 *>(sVtLo + sw64(vrow, 32 * ks + 8 * lg));
                            acc = mma(A8, Bh, acc);
                            acc = mma(A8, Bl, acc);
                        }
                        U[tp][x][nt] = acc;
                    }
        }
        __syncthreads();

        // ================= phase 5: state side =================
        // (the epilogue's output-gate logits are loaded now, to arrive during the MFMAs)
        uint4 graw[4];
        {
            int tid_ = (int)threadIdx.x;
            asm volatile("" : "+v"(tid_));
            const int tok = min(tid_ >> 2, L - 1);
            const uint16_t *gp = a.g + (size_t)(t0 + c0 + tok) * HD + (size_t)h * kD + 32 * (tid_ & 3);
#pragma unroll
            for (int j = 0; j < 4; ++j) graw[j] = *reinterpret_cast<const uint4 *>(gp + 8 * j);
        }
        {
            KDA_LANE_IDS();
            bf16x8 Sh[4][2];  // S0 as the B operand of key contractions (hi part)
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float v8[8] = {S[P][0][nt][0], S[P][0][nt][1], S[P][0][nt][2], S[P][0][nt][3],
                                   S[P][1][nt][0], S[P][1][nt][1], S[P][1][nt][2], S[P][1][nt][3]};
                    Sh[P][nt] = to_bf8(v8);
                }
            // U = U' - W S0
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int trow = 32 * tp + 8 * (lr >> 2) + 4 * x + (lr & 3);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int P = 0; P < 4; ++P) {
                            const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sW + sw128(trow, 32 * P + 8 * lg));
                            ws = mma(A8, Sh[P][nt], ws);
                        }
                        U[tp][x][nt] -= ws;
                    }
                }
            bf16x8 Uh[2][2], Ul[2][2];  // [tp][nt]
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    float v8[8] = {U[tp][0][nt][0], U[tp][0][nt][1], U[tp][0][nt][2], U[tp][0][nt][3],
                                   U[tp][1][nt][0], U[tp][1][nt][1], U[tp][1][nt][2], U[tp][1][nt][3]};
                    split8(v8, Uh[tp][nt], Ul[tp][nt]);
                }
            // O = Q~ S0 + P U   (rows: token 16tt + 4lg + i), parked in region 2 (beta v is dead)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x8 Ph[2], Pl[2];
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    if (tp > (tt >> 1)) continue;
                    float p8[8];
                    lds_read8(sP + (16 * tt + lr) * F_LD + 32 * tp + 8 * lg, p8);
                    split8(p8, Ph[tp], Pl[tp]);
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int P = 0; P < 4; ++P) {
                        const bf16x8 A8 =
                            *reinterpret_cast<const bf16x8 *>(sQe + sw128(16 * tt + lr, 32 * P + 8 * lg));
                        acc = mma(A8, Sh[P][nt], acc);
                    }
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp) {
                        if (tp > (tt >> 1)) continue;  // P is lower triangular
                        acc = mma(Ph[tp], Uh[tp][nt], acc);
                        acc = mma(Pl[tp], Uh[tp][nt], acc);
                        acc = mma(Ph[tp], Ul[tp][nt], acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) sO[(16 * tt + 4 * lg + i) * kD + 32 * w + 16 * nt + lr] = acc[i];
                }
            }
            // S = Diag(e^{G_end}) S0 + K_end^T U
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int krow = 32 * P + 8 * (lr >> 2) + 4 * x + (lr & 3);
                    float dec[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) dec[i] = sExpEnd[32 * P + 8 * lg + 4 * x + i];
                    bf16x8 Kh[2], Kl[2];
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp) {
                        Kh[tp] = *reinterpret_cast<const bf16x8 *>(sKeHi + sw64(krow, 32 * tp + 8 * lg));
                        Kl[tp] = *reinterpret_cast<const bf16x8 *>(sKeLo + sw64(krow, 32 * tp + 8 * lg));
                    }
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        f32x4 acc = S[P][x][nt];
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= dec[i];
#pragma unroll
                        for (int tp = 0; tp < 2; ++tp) {
                            acc = mma(Kh[tp], Uh[tp][nt], acc);
                            acc = mma(Kl[tp], Uh[tp][nt], acc);
                            acc = mma(Kh[tp], Ul[tp][nt], acc);
                        }
                        S[P][x][nt] = acc;
                    }
                }
        }
        __syncthreads();

        // ================= epilogue: out = sigmoid(g) * RMSNorm(o) =================
        // four adjacent lanes own one token row: 32 values each, 16-byte loads and stores
        {
            int tid_ = (int)threadIdx.x;
            asm volatile("" : "+v"(tid_));
            const int tok = tid_ >> 2;
            const int v0 = 32 * (tid_ & 3);
            float o[32];
#pragma unroll
            for (int j = 0; j < 32; j += 8) lds_read8(sO + tok * kD + v0 + j, o + j);
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) ss += o[j] * o[j];
            ss += __shfl_xor(ss, 1, 64);
            ss += __shfl_xor(ss, 2, 64);
            if (tok < L) {
                const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + a.c.rms_eps);
                const size_t row = (size_t)(t0 + c0 + tok) * HD + (size_t)h * kD + v0;
#pragma unroll
                for (int j = 0; j < 32; j += 8) {
                    float g8[8];
                    const uint32_t gw[4] = {graw[j / 8].x, graw[j / 8].y, graw[j / 8].z, graw[j / 8].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        g8[2 * e] = __uint_as_float(gw[e] << 16);
                        g8[2 * e + 1] = __uint_as_float(gw[e] & 0xffff0000u);
                    }
                    const float4 w0 = *reinterpret_cast<const float4 *>(a.norm_w + v0 + j);
                    const float4 w1 = *reinterpret_cast<const float4 *>(a.norm_w + v0 + j + 4);
                    float4 y0, y1;
                    y0.x = sigm(g8[0]) * (o[j + 0] * rinv * w0.x);
                    y0.y = sigm(g8[1]) * (o[j + 1] * rinv * w0.y);
                    y0.z = sigm(g8[2]) * (o[j + 2] * rinv * w0.z);
                    y0.w = sigm(g8[3]) * (o[j + 3] * rinv * w0.w);
                    y1.x = sigm(g8[4]) * (o[j + 4] * rinv * w1.x);
                    y1.y = sigm(g8[5]) * (o[j + 5] * rinv * w1.y);
                    y1.z = sigm(g8[6]) * (o[j + 6] * rinv * w1.z);
                    y1.w = sigm(g8[7]) * (o[j + 7] * rinv * w1.w);
                    *reinterpret_cast<float4 *>(a.out + row + j) = y0;
                    *reinterpret_cast<float4 *>(a.out + row + j + 4) = y1;
                }
            }
        }
        __syncthreads();  // LDS is rewritten by the next chunk
    }

    // ---- final state ----
    {
        KDA_LANE_IDS();
        float *Sf = a.final_state + ((size_t)seq * H + h) * kD * kD;
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = 32 * P + 8 * lg + 4 * x + i;
                        const int val = 32 * w + 16 * nt + lr;
                        Sf[key * kD + val] = S[P][x][nt][i];
                    }
    }
    // ---- final conv windows: the last 3 pre-conv inputs (from the initial window if T < 3) ----
    for (int q = threadIdx.x; q < 3 * kD; q += kThreads) {
        const int blk = q >> 7, cc = q & 127;
        const size_t ch = (size_t)blk * HD + (size_t)h * kD + cc;
        float win[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int tok = t1 - 3 + j;
            if (tok >= t0)
                win[j] = bf2f(X[blk][(size_t)tok * HD + (size_t)h * kD + cc]);
            else
                win[j] = a.initial_conv_state ? a.initial_conv_state[conv_seq + ch * 3 + (tok - t0 + 3)] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) a.final_conv_state[conv_seq + ch * 3 + j] = win[j];
    }
}

#undef KDA_LANE_IDS

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (attr != hipSuccess) return attr;
    dim3 grid((unsigned)((size_t)a.B * a.c.H)), block(kThreads);
    void *args[] = {const_cast<PrefillArgs *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_kernel), grid, block, args, kLdsBytes, stream);
}

}  // namespace kda
