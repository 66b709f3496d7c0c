// kda_decode_multi.hip -- several known tokens per sequence in one launch (gfx950).
//
// The recurrence of the header comment "KDA per-head recurrence" (page
// "colibri/c/kimi_k3.c"), S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
// and o_t = S_t^T q_t, over up to T tokens of each sequence: the 64 KiB head state is
// read once, carried in registers through the tokens, and written once (to state_out,
// which may be state_in); the conv windows likewise stay in registers.  One workgroup of
// four waves per (sequence, head).
//
// Tokens go in blocks of eight in the chunk form of the same recurrence (the WY form the
// prefill uses, without sub-chunk reference points: over eight tokens the cumulative log
// decay G_t = sum_{s<=t} log alpha_s stays above -40, so e^{+-G} is a normal fp32):
//   K~_t = k_t e^{G_t},  Q~_t = q_t e^{G_t},  K^_s = k_s e^{-G_s},  K_end_s = k_s e^{G_8 - G_s}
//   A_ts = K~_t . K^_s (s < t),  P_ts = Q~_t . K^_s (s <= t)
//   u_t = beta_t (v_t - (K~ S)_t - sum_{s<t} A_ts u_s),   o_t = (Q~ S)_t + sum_{s<=t} P_ts u_s
//   S' = Diag(e^{G_8}) S + K_end^T U
// which is the token-by-token recurrence reordered (the same terms, summed in another
// order), so results agree with that many one-token calls to fp32 rounding.  The state
// products K~ S, Q~ S, [K~; Q~] K^^T and K_end^T U are fp32 MFMAs (16x16x4): the state
// lives in registers as the accumulator tiles of K_end^T U (rows: keys, columns: values),
// and each tile element is also the B operand of K~ S and Q~ S for one contraction step.
// Only per-token vectors and 8x8 matrices go through LDS.
//
// State tiles.  Wave w owns values 32w .. 32w+31 (two 16-value tiles vt) for all 128 keys
// (eight 16-key tiles kt).  The state is loaded with 16-byte loads (lane l: key rows
// l/8 + 8j, values 32w + 4(l%8) .. +3, whole 128-byte lines) and one exchange of lane bit
// 3 with a register bit turns this into tiles: lane (n = l%16, g = l/16) holds, in quad i
// of tile (kt, vt), key K(kt, g, i) = 16kt + 8(i/2) + 4(g/2) + 2(g%2) + i%2 of value
// V(vt, n) = 32w + vt + 2(n/8) + 4(n%8).  Per-key tables in LDS are kept in the tile
// order pos(K(kt, g, i)) = 16kt + 4g + i, so that a lane reads its four keys of a tile
// with one 16-byte read.

#include <type_traits>

#include "kda_decode_common.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kBlk = 8;  // tokens per block

// table position of key k (see the header)
__device__ __forceinline__ int key_pos(int k) {
    return (k & ~15) | (((k >> 1) & 3) << 2) | (k & 1) | (((k >> 3) & 1) << 1);
}
// value of column n of value tile vt of wave w
__device__ __forceinline__ int tile_value(int w, int vt, int n) { return 32 * w + vt + 2 * (n >> 3) + 4 * (n & 7); }

// The exchange of lane bit 3 with register bit c1 for one register pair (a = c1 0,
// b = c1 1): lanes with bit 3 clear keep a and take the partner's a as b; lanes with it
// set take the partner's b as a and keep b.  Its own inverse.
// (DPP row_ror:8 pairs lanes l and l ^ 8.)  Applied to elements (c0, c0 + 2) of s.
__device__ __forceinline__ void swap_bit3(f32x4 &s, int c0, bool hi) {
    const float x = s[c0], y = s[c0 + 2];
    const float send = hi ? x : y;
    const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0x128, 0xf, 0xf, false));
    s[c0] = hi ? recv : x;
    s[c0 + 2] = hi ? y : recv;
}

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store_out1(void *out, size_t i, float y, bool bf16) {
    if (bf16)
        static_cast<__bf16 *>(out)[i] = (__bf16)y;
    else
        static_cast<float *>(out)[i] = y;
}

// kSlots: batch row bs reads and writes pool entry a.slots[bs] of the state and window
// pools instead of entry bs; a row whose slot lies outside [0, a.pool) is skipped.
// The first block's token inputs are loaded with the state, so that a workgroup waits for
// memory once per call for up to eight tokens (later blocks' inputs are loaded at the end
// of the block before); the per-column steps read their LDS operands with 16-byte reads
// from column-major tables.
template <bool kSlots>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_multi_kernel(
    DecodeMultiArgs a) {
    const int H = a.c.H;
    const int T = a.T;
    const int bh = xcd_contiguous(blockIdx.x, gridDim.x);  // batch row * H + head
    const int bs = bh / H;
    const int h = bh - bs * H;
    int slot = bs;
    if (kSlots) {
        slot = a.slots[bs];                       // uniform over the workgroup
        if (slot < 0 || slot >= a.pool) return;   // before any barrier
    }
    const size_t sofs = (size_t)slot * H + h;     // this head's state in the buffers
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lgq = lane >> 4;  // tile column / row group of the lane
    const bool hi8 = (lane & 8) != 0;
    const size_t HD = (size_t)H * kD;
    const int n = a.n_tokens ? min(max(a.n_tokens[bs], 0), T) : T;

    __shared__ __align__(16) float sh_y[16][kD];      // K~_t (rows 0..7), Q~_t (rows 8..15), key order pos
    __shared__ __align__(16) float sh_kh[kBlk][kD];   // K^_s, key order pos
    __shared__ __align__(16) float sh_ke[kBlk][kD];   // K_end_s, key order pos
    __shared__ __align__(16) float sh_gam[kD];        // e^{G_8}, key order pos
    __shared__ __align__(16) float sh_gT[kD][kBlk];   // G_t of key channel i: [i][t]
    __shared__ __align__(16) float sh_vT[kD][kBlk];   // v_t of value column c (0 past n): [c][t]
    __shared__ __align__(16) float sh_gateT[kD][kBlk];  // sigmoid of the output-gate logits: [c][t]
    __shared__ __align__(16) float sh_beta[kBlk];
    __shared__ __align__(16) float sh_nrm[kBlk][4];   // sums of squares of q (waves 0, 1), then of k
    __shared__ __align__(16) float sh_xT[kD][16];     // [value][K~ S rows 0..7, Q~ S rows 8..15]
    __shared__ __align__(16) float sh_ap[4][16][16];  // per-wave parts of [K~; Q~] K^^T
    __shared__ __align__(16) float sh_apf[64];        // their sum: A_ts (s < t) at t(t-1)/2 + s, then
                                                      // P_ts (s <= t) at 28 + t(t+1)/2 + s
    __shared__ float sh_u[kBlk][kD];                  // U, natural values
    __shared__ __align__(16) float sh_rms[kBlk][4];   // per-wave sums of squares of o_t

    // ---- loads: parameters and windows, the first block's token inputs, then the state
    //      (16-byte loads, whole lines), which is not needed before the first block's
    //      products, so that its latency overlaps the first prologue ----
    // this lane's channels: their taps and carried windows (A: q or v, B: k)
    const size_t conv_seq = (size_t)slot * 3 * HD * 3;
    const bool qk = tid < kD;  // waves 0-1: q and k of channel i; waves 2-3: v, z, g of channel i
    const int i = qk ? tid : tid - kD;
    const size_t chA = (qk ? 0 : 2 * HD) + (size_t)h * kD + i;
    const size_t chB = HD + (size_t)h * kD + i;
    const float4 wA = *reinterpret_cast<const float4 *>(a.conv_w + chA * 4);
    const float4 wB = *reinterpret_cast<const float4 *>(a.conv_w + chB * 4);
    float winA[3], winB[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        winA[j] = a.conv_in[conv_seq + chA * 3 + j];
        winB[j] = qk ? a.conv_in[conv_seq + chB * 3 + j] : 0.f;
    }
    const float dtb = a.dt_bias[h * kD + i];
    const float alog = a.A_log[h];
    const int col = 32 * w + (lane & 31);  // the value column of lanes 0..31 in the per-column steps
    const float nwc = a.norm_w[col];
    const float *srcA = qk ? a.q : a.v;
    const float *srcB = qk ? a.k : a.z;
    const size_t ldB = qk ? a.qkv_ld : HD;
    float xa[kBlk], xb[kBlk], xg[kBlk], xbeta[kBlk];
    auto load_block = [&](int t0) {
#pragma unroll
        for (int t = 0; t < kBlk; ++t) {
            const size_t row = (size_t)bs * T + min(t0 + t, max(n - 1, 0));
            xa[t] = srcA[row * a.qkv_ld + (size_t)h * kD + i];
            xb[t] = srcB[row * ldB + (size_t)h * kD + i];
            xg[t] = qk ? 0.f : a.g[row * HD + (size_t)h * kD + i];
            xbeta[t] = a.b[row * H + h];
        }
    };
    if (n > 0) load_block(0);
    f32x4 s[16];
    {
        const float *Sin = a.state_in + sofs * kD * kD;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            s[j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(Sin + ((lane >> 3) + 8 * j) * kD + 32 * w + 4 * (lane & 7)));
    }
    const float rate = expf(alog);

    // ---- the state, as tiles ----
    f32x4 Sd[8][2];
    auto to_tiles = [&]() {
        // (the empty asm pins the state's first use here: without it the compiler hoists
        //  the exchange above the prologue and waits there for the state loads)
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(s[j]));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            swap_bit3(s[j], 0, hi8);
            swap_bit3(s[j], 1, hi8);
        }
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
                Sd[kt][vt] = f32x4{s[2 * kt][vt], s[2 * kt][vt + 2], s[2 * kt + 1][vt], s[2 * kt + 1][vt + 2]};
    };

    // One block of tokens t0 .. t0+7; the first (a straight-line copy, so that the waits for
    // its inputs need not wait for the state) turns the loaded state into tiles before the
    // first products.
    auto run_block = [&](int t0, auto first_c) {
        constexpr bool kFirst = decltype(first_c)::value;
        // ================= prologue: conv, SiLU, gates of the block's tokens =================
        float uq[kBlk], uk[kBlk];
        if (qk) {
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                const bool valid = t0 + t < n;
                uq[t] = silu(conv4(wA, winA[0], winA[1], winA[2], xa[t]));
                uk[t] = silu(conv4(wB, winB[0], winB[1], winB[2], xb[t]));
                if (valid) {
                    winA[0] = winA[1]; winA[1] = winA[2]; winA[2] = xa[t];
                    winB[0] = winB[1]; winB[1] = winB[2]; winB[2] = xb[t];
                }
                const float sqq = group_sum<64>(uq[t] * uq[t]);
                const float skk = group_sum<64>(uk[t] * uk[t]);
                if (lane == 0) {
                    sh_nrm[t][w] = sqq;
                    sh_nrm[t][2 + w] = skk;
                }
            }
        } else {
            float G = 0.f;
            float gv[kBlk], vv[kBlk], gt[kBlk];
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                const bool valid = t0 + t < n;
                const float v = silu(conv4(wA, winA[0], winA[1], winA[2], xa[t]));
                if (valid) {
                    winA[0] = winA[1]; winA[1] = winA[2]; winA[2] = xa[t];
                }
                vv[t] = valid ? v : 0.f;
                G += valid ? a.c.gate_lower_bound * sigm(rate * (xb[t] + dtb)) : 0.f;
                gv[t] = G;
                gt[t] = sigm(xg[t]);
                if (i == 0) sh_beta[t] = valid ? sigm(xbeta[t]) : 0.f;
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                *reinterpret_cast<f32x4 *>(&sh_gT[i][4 * q]) = f32x4{gv[4 * q], gv[4 * q + 1], gv[4 * q + 2], gv[4 * q + 3]};
                *reinterpret_cast<f32x4 *>(&sh_vT[i][4 * q]) = f32x4{vv[4 * q], vv[4 * q + 1], vv[4 * q + 2], vv[4 * q + 3]};
                *reinterpret_cast<f32x4 *>(&sh_gateT[i][4 * q]) = f32x4{gt[4 * q], gt[4 * q + 1], gt[4 * q + 2], gt[4 * q + 3]};
            }
        }
        lds_barrier();

        // ================= the per-key tables of the block =================
        if (qk) {
            const int p = key_pos(i);
            const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&sh_gT[i][0]);
            const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&sh_gT[i][4]);
            const float G[kBlk] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            const float G8 = G[kBlk - 1];
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                const bool valid = t0 + t < n;
                const f32x4 nr = *reinterpret_cast<const f32x4 *>(&sh_nrm[t][0]);
                const float inv_q = a.c.q_scale * inv_sqrt(nr[0] + nr[1] + a.c.l2_eps);
                const float inv_k = inv_sqrt(nr[2] + nr[3] + a.c.l2_eps);
                const float kh = valid ? uk[t] * inv_k : 0.f;
                const float qh = valid ? uq[t] * inv_q : 0.f;
                const float eg = __expf(G[t]);
                sh_y[t][p] = kh * eg;
                sh_y[kBlk + t][p] = qh * eg;
                sh_kh[t][p] = kh * __expf(-G[t]);
                sh_ke[t][p] = kh * __expf(G8 - G[t]);
            }
            sh_gam[p] = __expf(G8);
        }
        lds_barrier();

        if constexpr (kFirst) to_tiles();
        // ================= K~ S, Q~ S and [K~; Q~] K^^T =================
        {
            f32x4 y4[8];  // A operand: row ln of [K~; Q~], the lane's four keys of tile kt
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) y4[kt] = *reinterpret_cast<const f32x4 *>(&sh_y[ln][16 * kt + 4 * lgq]);
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = mma4(y4[kt][q], Sd[kt][vt][q], acc);
                // rows 4lgq .. +3 of value column tile_value(w, vt, ln)
                *reinterpret_cast<f32x4 *>(&sh_xT[tile_value(w, vt, ln)][4 * lgq]) = acc;
            }
            // this wave's key tiles 2w, 2w+1 of [K~; Q~] K^^T (columns s < 8; 8..15 zero)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int kt = 2 * w + kk;
                const f32x4 yk = *reinterpret_cast<const f32x4 *>(&sh_y[ln][16 * kt + 4 * lgq]);
                const f32x4 kb = ln < kBlk ? *reinterpret_cast<const f32x4 *>(&sh_kh[ln & (kBlk - 1)][16 * kt + 4 * lgq])
                                           : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = mma4(yk[q], kb[q], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sh_ap[w][4 * lgq + r][ln] = acc[r];
        }
        lds_barrier();
        {
            // the entries of A (rows 0..7, s < t) and P (rows 8..15, s <= t) that are used
            const int r = tid >> 4, c = tid & 15;
            const int t = r & 7;
            const bool isA = r < kBlk;
            if (c < kBlk && (isA ? c < t : c <= t)) {
                const float x = ((sh_ap[0][r][c] + sh_ap[1][r][c]) + sh_ap[2][r][c]) + sh_ap[3][r][c];
                sh_apf[isA ? t * (t - 1) / 2 + c : 28 + t * (t + 1) / 2 + c] = x;
            }
        }
        lds_barrier();

        // ================= U, O and the outputs (lanes 0..31 of each wave: one value column) ====
        float o[kBlk];
        if (lane < 32) {
            f32x4 xr[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) xr[q] = *reinterpret_cast<const f32x4 *>(&sh_xT[col][4 * q]);
            auto X = [&](int m) { return xr[m >> 2][m & 3]; };
            float u[kBlk];
            {
                f32x4 vr[2];  // v of the tokens
#pragma unroll
                for (int q = 0; q < 2; ++q) vr[q] = *reinterpret_cast<const f32x4 *>(&sh_vT[col][4 * q]);
#pragma unroll
                for (int t = 0; t < kBlk; ++t) {
                    float acc = vr[t >> 2][t & 3] - X(t);
#pragma unroll
                    for (int s2 = 0; s2 < t; ++s2) acc = fmaf(-sh_apf[t * (t - 1) / 2 + s2], u[s2], acc);
                    u[t] = sh_beta[t] * acc;
                    sh_u[t][col] = u[t];
                }
            }
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                float acc = X(kBlk + t);
#pragma unroll
                for (int s2 = 0; s2 <= t; ++s2) acc = fmaf(sh_apf[28 + t * (t + 1) / 2 + s2], u[s2], acc);
                o[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                const float ss = group_sum<32>(o[t] * o[t]);
                if (lane == 0) sh_rms[t][w] = ss;
            }
        }
        lds_barrier();
        if (lane < 32) {
            f32x4 gr[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) gr[q] = *reinterpret_cast<const f32x4 *>(&sh_gateT[col][4 * q]);
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                if (t0 + t >= n) break;
                const f32x4 rr = *reinterpret_cast<const f32x4 *>(&sh_rms[t][0]);
                const float ss = ((rr[0] + rr[1]) + rr[2]) + rr[3];
                const float rinv = inv_sqrt(fmaf(ss, 1.0f / kD, a.c.rms_eps));
                const size_t row = (size_t)bs * T + t0 + t;
                store_out1(a.out, row * HD + (size_t)h * kD + col, gr[t >> 2][t & 3] * (o[t] * rinv * nwc),
                           a.c.out_bf16);
            }
        }

        // ================= S' = Diag(e^{G_8}) S + K_end^T U =================
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(&sh_gam[16 * kt + 4 * lgq]);
            const float ke0 = sh_ke[lgq][16 * kt + ln];      // A: token 4ks + lgq, key row ln of tile kt
            const float ke1 = sh_ke[4 + lgq][16 * kt + ln];
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                const int v = tile_value(w, vt, ln);
                f32x4 acc = Sd[kt][vt] * gam;
                acc = mma4(ke0, sh_u[lgq][v], acc);
                acc = mma4(ke1, sh_u[4 + lgq][v], acc);
                Sd[kt][vt] = acc;
            }
        }
        // the next block's inputs (issued here, where few registers are live)
        if (t0 + kBlk < n) load_block(t0 + kBlk);
        lds_barrier();  // the tables are rewritten by the next block
    };
    if (n > 0) {
        run_block(0, std::true_type{});
        for (int t0 = kBlk; t0 < n; t0 += kBlk) run_block(t0, std::false_type{});
    } else {
        to_tiles();
    }

    // ---- the state and windows out ----
    {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                s[2 * kt][vt] = Sd[kt][vt][0];
                s[2 * kt][vt + 2] = Sd[kt][vt][1];
                s[2 * kt + 1][vt] = Sd[kt][vt][2];
                s[2 * kt + 1][vt + 2] = Sd[kt][vt][3];
            }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            swap_bit3(s[j], 0, hi8);
            swap_bit3(s[j], 1, hi8);
        }
        float *Sout = a.state_out + sofs * kD * kD;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            __builtin_nontemporal_store(
                s[j], reinterpret_cast<f32x4 *>(Sout + ((lane >> 3) + 8 * j) * kD + 32 * w + 4 * (lane & 7)));
    }
    float *cwA = a.conv_out + conv_seq + chA * 3;
    float *cwB = a.conv_out + conv_seq + chB * 3;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        cwA[j] = winA[j];
        if (qk) cwB[j] = winB[j];
    }
}

}  // namespace

hipError_t launch_decode_multi(const DecodeMultiArgs &a, hipStream_t stream) {
    dim3 grid((unsigned)((size_t)a.B * a.c.H)), block(kThreads);
    void *args[] = {const_cast<DecodeMultiArgs *>(&a)};
    const void *fn = a.slots ? reinterpret_cast<const void *>(&decode_multi_kernel<true>)
                             : reinterpret_cast<const void *>(&decode_multi_kernel<false>);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace kda
