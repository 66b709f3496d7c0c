// kda_decode.hip -- one-token KDA decode against resident fp32 states (gfx950).
//
// One workgroup of 256 lanes owns one (sequence, head).  The kernel fuses the whole
// per-token path of the header comment "KDA per-head recurrence" (page
// "colibri/c/kimi_k3.c"): ShortConv4 with the carried window, SiLU, the q/k L2 norm and
// q scale, the decay and beta gates, the state update, the readout and the gated
// RMSNorm.
//
// Single pass over the state.  Writing D_a = Diag(alpha), the update
//     S' = (I - beta k k^T) D_a S + beta k v^T,   o = S'^T q
// is evaluated as
//     a = S^T (alpha*k),  c = S^T (alpha*q),  u = beta (v - a),
//     S' = D_a S + k u^T,  o = c + (k.q) u,
// which needs only two reductions over the key index of the *old* state before any
// element of S' is written.  The 64 KiB head state therefore stays in registers between
// its read and its write: lane (rg, cg) holds rows rg + 8j (j < 16) of columns
// 4cg..4cg+3, read and written with 16-byte accesses, each wave covering two adjacent
// 512-byte rows per instruction.  The key-index reduction runs over the 16 rows in a
// lane, then across the two row groups of a wave (lane ^ 32), then across the four
// waves through 4 KiB of LDS.
//
// The state loads are issued first so that the conv/norm/gate prologue runs while they
// are in flight.  The kernel is bound by HBM: 128 KiB of state traffic per (sequence,
// head) against ~98 KFLOP.

#include "kda_decode_common.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;

// kSlots: batch row bs updates pool entry a.slots[bs] of the state and conv-window
// pools instead of entry bs; a row whose slot lies outside [0, a.pool) is skipped.
template <bool kSlots>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    const int H = a.c.H;
    const int bh = xcd_contiguous(blockIdx.x, gridDim.x);  // batch row * H + head
    const int bs = bh / H;
    const int h = bh - bs * H;
    int slot = bs;
    if (kSlots) {
        slot = a.slots[bs];                               // uniform over the workgroup
        if (slot < 0 || slot >= a.pool) return;           // before any barrier
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = tid & 31;  // column group: value columns 4cg .. 4cg+3
    const int rg = tid >> 5;  // row group: key rows rg + 8j
    const size_t HD = (size_t)H * kD;

    // ---- 1. issue the state reads (64 floats per lane) ----
    // (nontemporal: the state is streamed once per step and must not evict the small,
    //  reused per-head parameters from the caches)
    float *S = a.state + ((size_t)slot * H + h) * kD * kD;
    f32x4 s[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (rg + 8 * j) * kD + 4 * cg));

    __shared__ float2 sh_akq[kD];   // (alpha k^, alpha q^) of a key row (q^ scaled)
    __shared__ float2 sh_alk[kD];   // (alpha, k^) of a key row
    __shared__ float sh_alpha[kD];  // decay
    __shared__ float sh_v[kD];      // SiLU(conv(v))
    __shared__ float sh_gate[kD];   // sigmoid(g)
    __shared__ float sh_red[2][3];  // per-wave sums of q.q, k.k, q.k (waves 0, 1)
    __shared__ float sh_beta;
    __shared__ float sh_part[4][2][kD];  // per-wave partial S^T(alpha k), S^T(alpha q)

    // ---- 2. prologue: conv + SiLU (+ sums for the L2 norms), gates ----
    const size_t tok = (size_t)bs * HD + (size_t)h * kD;        // this head's channels of the token row
    const size_t tokx = (size_t)bs * a.qkv_ld + (size_t)h * kD;  // the same in the q, k, v rows
    float *cstate = a.conv_state + (size_t)slot * 3 * HD * 3;
    float uq = 0.f, uk = 0.f;
    if (tid < kD) {
        const int i = tid;
        const size_t chq = (size_t)h * kD + i;
        const size_t chk = HD + chq;
        const float4 wq = *reinterpret_cast<const float4 *>(a.conv_w + chq * 4);
        const float4 wk = *reinterpret_cast<const float4 *>(a.conv_w + chk * 4);
        float *wnq = cstate + chq * 3;
        float *wnk = cstate + chk * 3;
        const float q0 = wnq[0], q1 = wnq[1], q2 = wnq[2], xq = a.q[tokx + i];
        const float k0 = wnk[0], k1 = wnk[1], k2 = wnk[2], xk = a.k[tokx + i];
        wnq[0] = q1; wnq[1] = q2; wnq[2] = xq;
        wnk[0] = k1; wnk[1] = k2; wnk[2] = xk;
        uq = silu(conv4(wq, q0, q1, q2, xq));
        uk = silu(conv4(wk, k0, k1, k2, xk));
        const float sqq = group_sum<64>(uq * uq);
        const float skk = group_sum<64>(uk * uk);
        const float sqk = group_sum<64>(uq * uk);
        if (lane == 0) {
            sh_red[wave][0] = sqq;
            sh_red[wave][1] = skk;
            sh_red[wave][2] = sqk;
        }
    } else {
        const int i = tid - kD;
        const size_t chv = 2 * HD + (size_t)h * kD + i;
        const float4 wv = *reinterpret_cast<const float4 *>(a.conv_w + chv * 4);
        float *wnv = cstate + chv * 3;
        const float v0 = wnv[0], v1 = wnv[1], v2 = wnv[2], xv = a.v[tokx + i];
        wnv[0] = v1; wnv[1] = v2; wnv[2] = xv;
        sh_v[i] = silu(conv4(wv, v0, v1, v2, xv));
        const float rate = expf(a.A_log[h]);
        sh_alpha[i] = decay(a.c.gate_lower_bound, rate, a.z[tok + i], a.dt_bias[h * kD + i]);
        sh_gate[i] = sigm(a.g[tok + i]);
        if (i == 0) sh_beta = sigm(a.b[(size_t)bs * H + h]);
    }
    __syncthreads();

    const float ssq = sh_red[0][0] + sh_red[1][0];
    const float ssk = sh_red[0][1] + sh_red[1][1];
    const float sqk = sh_red[0][2] + sh_red[1][2];
    const float inv_q = a.c.q_scale * inv_sqrt(ssq + a.c.l2_eps);
    const float inv_k = inv_sqrt(ssk + a.c.l2_eps);
    const float kappa = sqk * inv_q * inv_k;  // k^ . q^
    const float beta = sh_beta;
    if (tid < kD) {
        const float qh = uq * inv_q, kh = uk * inv_k, al = sh_alpha[tid];
        sh_alk[tid] = make_float2(al, kh);
        sh_akq[tid] = make_float2(al * kh, al * qh);
    }
    __syncthreads();

    // ---- 3. a = S^T(alpha k), c = S^T(alpha q) over this lane's 16 rows ----
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
    key_dots(s, sh_akq, rg, pa, pc);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        pa[c] = add_xor32(pa[c]);
        pc[c] = add_xor32(pc[c]);
    }
    if (lane < 32) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sh_part[wave][0][4 * cg + c] = pa[c];
            sh_part[wave][1][4 * cg + c] = pc[c];
        }
    }
    __syncthreads();

    // ---- 4. u = beta (v - a), o = c + kappa u, S' = D_a S + k u^T ----
    float u[4], o[4];
    delta_and_readout(sh_part, sh_v, beta, kappa, cg, u, o);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = rg + 8 * j;
        __builtin_nontemporal_store(update_row(s[j], sh_alk[r], u), reinterpret_cast<f32x4 *>(S + r * kD + 4 * cg));
    }

    // ---- 5. out = sigmoid(g) * RMSNorm(o) (lanes 0..31 of wave 0 hold all 128 columns) ----
    if (tid < 32) {
        const float rinv = rms_inv(o, a.c.rms_eps);
        const float4 w = *reinterpret_cast<const float4 *>(a.norm_w + 4 * cg);
        store_out4(a.out, tok + 4 * cg, sh_gate[4 * cg + 0] * (o[0] * rinv * w.x),
                   sh_gate[4 * cg + 1] * (o[1] * rinv * w.y), sh_gate[4 * cg + 2] * (o[2] * rinv * w.z),
                   sh_gate[4 * cg + 3] * (o[3] * rinv * w.w), a.c.out_bf16);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    // One workgroup per (batch row, head), ids remapped by xcd_contiguous.
    dim3 grid((unsigned)((size_t)a.B * a.c.H)), block(kThreads);
    void *args[] = {const_cast<DecodeArgs *>(&a)};
    const void *fn = a.slots ? reinterpret_cast<const void *>(&decode_kernel<true>)
                             : reinterpret_cast<const void *>(&decode_kernel<false>);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace kda
