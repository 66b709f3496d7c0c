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

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// Workgroups are dealt to the 8 XCDs round-robin in id order.  This maps hardware id i
// (XCD i % 8, its (i / 8)-th workgroup) to a logical id so that each XCD walks one
// contiguous eighth of the (sequence, head) range in order: its L2, address translation
// and DRAM pages then see one streaming region instead of every eighth 64 KiB state.
// A bijection for any n, so the result does not depend on the dispatch order.
__device__ __forceinline__ int xcd_contiguous(int i, int n) {
    const int q = n >> 3, r = n & 7, x = i & 7;
    return x * q + min(x, r) + (i >> 3);
}

// sum over groups of W consecutive lanes (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

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

    __shared__ float sh_kh[kD];     // normalised k
    __shared__ float sh_ak[kD];     // alpha * k
    __shared__ float sh_aq[kD];     // alpha * q (scaled)
    __shared__ float sh_alpha[kD];  // decay
    __shared__ float sh_v[kD];      // SiLU(conv(v))
    __shared__ float sh_gate[kD];   // sigmoid(g)
    __shared__ float sh_red[2][3];  // per-wave sums of q.q, k.k, q.k (waves 0, 1)
    __shared__ float sh_beta;
    __shared__ float sh_part[4][2][kD];  // per-wave partial S^T(alpha k), S^T(alpha q)

    // ---- 2. prologue: conv + SiLU (+ sums for the L2 norms), gates ----
    const size_t tok = (size_t)bs * HD + (size_t)h * kD;  // this head's channels of the token row
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
        const float q0 = wnq[0], q1 = wnq[1], q2 = wnq[2], xq = a.q[tok + i];
        const float k0 = wnk[0], k1 = wnk[1], k2 = wnk[2], xk = a.k[tok + i];
        const float yq = wq.x * q0 + wq.y * q1 + wq.z * q2 + wq.w * xq;
        const float yk = wk.x * k0 + wk.y * k1 + wk.z * k2 + wk.w * xk;
        wnq[0] = q1; wnq[1] = q2; wnq[2] = xq;
        wnk[0] = k1; wnk[1] = k2; wnk[2] = xk;
        uq = yq * sigmoid_f(yq);
        uk = yk * sigmoid_f(yk);
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
        const float v0 = wnv[0], v1 = wnv[1], v2 = wnv[2], xv = a.v[tok + i];
        const float yv = wv.x * v0 + wv.y * v1 + wv.z * v2 + wv.w * xv;
        wnv[0] = v1; wnv[1] = v2; wnv[2] = xv;
        sh_v[i] = yv * sigmoid_f(yv);
        const float rate = expf(a.A_log[h]);
        const float gk = a.c.gate_lower_bound * sigmoid_f(rate * (a.z[tok + i] + a.dt_bias[h * kD + i]));
        sh_alpha[i] = expf(gk);
        sh_gate[i] = sigmoid_f(a.g[tok + i]);
        if (i == 0) sh_beta = sigmoid_f(a.b[(size_t)bs * H + h]);
    }
    __syncthreads();

    const float ssq = sh_red[0][0] + sh_red[1][0];
    const float ssk = sh_red[0][1] + sh_red[1][1];
    const float sqk = sh_red[0][2] + sh_red[1][2];
    const float inv_q = a.c.q_scale / sqrtf(ssq + a.c.l2_eps);
    const float inv_k = 1.0f / sqrtf(ssk + a.c.l2_eps);
    const float kappa = sqk * inv_q * inv_k;  // k^ . q^
    const float beta = sh_beta;
    if (tid < kD) {
        const float qh = uq * inv_q, kh = uk * inv_k, al = sh_alpha[tid];
        sh_kh[tid] = kh;
        sh_ak[tid] = al * kh;
        sh_aq[tid] = al * qh;
    }
    __syncthreads();

    // ---- 3. a = S^T(alpha k), c = S^T(alpha q) over this lane's 16 rows ----
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = rg + 8 * j;
        const float fk = sh_ak[r], fq = sh_aq[r];
        pa[0] += s[j].x * fk; pa[1] += s[j].y * fk; pa[2] += s[j].z * fk; pa[3] += s[j].w * fk;
        pc[0] += s[j].x * fq; pc[1] += s[j].y * fq; pc[2] += s[j].z * fq; pc[3] += s[j].w * fq;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        pa[c] += __shfl_xor(pa[c], 32, 64);
        pc[c] += __shfl_xor(pc[c], 32, 64);
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
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int col = 4 * cg + c;
        const float av = sh_part[0][0][col] + sh_part[1][0][col] + sh_part[2][0][col] + sh_part[3][0][col];
        const float cv = sh_part[0][1][col] + sh_part[1][1][col] + sh_part[2][1][col] + sh_part[3][1][col];
        u[c] = beta * (sh_v[col] - av);
        o[c] = cv + kappa * u[c];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = rg + 8 * j;
        const float al = sh_alpha[r], kr = sh_kh[r];
        f32x4 n;
        n.x = al * s[j].x + kr * u[0];
        n.y = al * s[j].y + kr * u[1];
        n.z = al * s[j].z + kr * u[2];
        n.w = al * s[j].w + kr * u[3];
        __builtin_nontemporal_store(n, reinterpret_cast<f32x4 *>(S + r * kD + 4 * cg));
    }

    // ---- 5. out = sigmoid(g) * RMSNorm(o) (lanes 0..31 of wave 0 hold all 128 columns) ----
    if (tid < 32) {
        const float ss = group_sum<32>(o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3]);
        const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + a.c.rms_eps);
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
