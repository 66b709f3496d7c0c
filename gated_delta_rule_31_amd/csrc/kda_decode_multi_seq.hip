// kda_decode_multi_seq.hip -- several known tokens per sequence in one launch, token by
// token (gfx950): the form of kda_decode_multi that gives the bits of n one-token calls
// (kda_config.decode_multi_form = KDA_MULTI_SEQUENTIAL).
//
// The one-token decode of kda_decode.hip, applied to up to T tokens of each sequence:
// the 64 KiB head state is read once, carried in registers through the tokens, and
// written once (to state_out, which may be state_in); the conv windows likewise stay in
// registers.  Each token follows the header comment "KDA per-head recurrence" (page
// "colibri/c/kimi_k3.c") with decode_kernel's arithmetic (the helpers of
// kda_decode_common.hpp, in the same order), so n tokens here give the bits of n calls
// of decode_kernel.  Lanes < 128 own the q and k
// channel of their index, lanes >= 128 the v channel; the state layout (lane (rg, cg):
// rows rg + 8j of columns 4cg..4cg+3) and the two key reductions are decode_kernel's.
// Outputs of tokens t >= n_tokens[b] are not written.

#include "kda_decode_common.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;

// kSlots: batch row bs reads and writes pool entry a.slots[bs] of the state and window
// pools instead of entry bs; a row whose slot lies outside [0, a.pool) is skipped.
// Three workgroups' waves per SIMD: the register budget (at most 168 VGPRs) leaves room
// for three 4-wave workgroups per compute unit, which hide each other's per-token chain of
// barriers and LDS round trips (measured with 64 sequences x 96 heads: 4 tokens 211 ->
// 193 us, 8 tokens 312 -> 280 us against two per SIMD at 176 VGPRs).
template <bool kSlots>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void decode_multi_seq_kernel(
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
    const int wave = tid >> 6;
    const int cg = tid & 31;
    const int rg = tid >> 5;
    const size_t HD = (size_t)H * kD;
    const int n = a.n_tokens ? min(max(a.n_tokens[bs], 0), T) : T;

    f32x4 s[16];
    const float *Sin = a.state_in + sofs * kD * kD;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sin + (rg + 8 * j) * kD + 4 * cg));

    // Three barriers per token.  The arrays a token's prologue writes and that its
    // predecessor's update and epilogue still read (v, output gate) alternate between two
    // copies by token parity; every other array is rewritten only behind a barrier that
    // all reads of its previous contents precede.
    __shared__ float2 sh_akq[kD];  // (alpha k^, alpha q^) of a key row
    __shared__ float2 sh_alk[kD];  // (alpha, k^) of a key row
    __shared__ float sh_alpha[kD];
    __shared__ float sh_v[2][kD];
    __shared__ float sh_gate[2][kD];
    __shared__ float sh_red[2][3];
    __shared__ float sh_beta;
    __shared__ float sh_part[4][2][kD];

    // this lane's channels: their taps and carried windows (A: q or v, B: k)
    const size_t conv_seq = (size_t)slot * 3 * HD * 3;
    const int i = tid < kD ? tid : tid - kD;
    const size_t chA = (tid < kD ? 0 : 2 * HD) + (size_t)h * kD + i;
    const size_t chB = HD + (size_t)h * kD + i;
    const float4 wA = *reinterpret_cast<const float4 *>(a.conv_w + chA * 4);
    const float4 wB = *reinterpret_cast<const float4 *>(a.conv_w + chB * 4);
    float winA[3], winB[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        winA[j] = a.conv_in[conv_seq + chA * 3 + j];
        winB[j] = tid < kD ? a.conv_in[conv_seq + chB * 3 + j] : 0.f;
    }
    const float dtb = a.dt_bias[h * kD + i];
    const float rate = expf(a.A_log[h]);
    // the RMSNorm weight of this lane's 4 output columns (lanes 0..31 write the outputs)
    const float4 wn = *reinterpret_cast<const float4 *>(a.norm_w + 4 * cg);

    // This lane's inputs of a token (A: q or v, B: k or z, G: g, beta logit), loaded one
    // token ahead: requested once the current token's inputs are consumed (so that no wait
    // for them also waits for these), and the loop's barriers wait for LDS traffic only,
    // so they stay in flight across them.  Addresses are a wave-uniform pointer to the
    // head's first channel in the token's row plus the lane's channel (a 32-bit offset),
    // so that no 64-bit per-lane address lives across the loop.
    const bool qk_wave = __builtin_amdgcn_readfirstlane(tid) < kD;  // waves 0-1: q and k; 2-3: v and z
    const float *srcA = qk_wave ? a.q : a.v;
    const float *srcB = qk_wave ? a.k : a.z;
    const size_t ldB = qk_wave ? a.qkv_ld : HD;  // k rows or z rows (uniform)
    struct TokenLoads {
        float A, B, G, b;
    };
    auto load_token = [&](int t) {
        const size_t row = (size_t)bs * T + t;
        const size_t head0 = row * HD + (size_t)h * kD;
        TokenLoads r;
        r.A = srcA[row * a.qkv_ld + (size_t)h * kD + (unsigned)i];
        r.B = srcB[row * ldB + (size_t)h * kD + (unsigned)i];
        r.G = a.g[head0 + (unsigned)i];
        r.b = a.b[row * H + h];
        return r;
    };
    TokenLoads cur = {0.f, 0.f, 0.f, 0.f};
    if (n > 0) cur = load_token(0);
    // Wait once, here, for everything loaded so far.  The compiler cannot count memory
    // operations across the loop's back edge; with loads from before the loop still
    // possibly in flight it makes the loop wait for all of them, and so for the next
    // token's loads and this token's output store too, on every token.
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(s[j]));
    asm volatile("" ::"v"(wA.x), "v"(wA.y), "v"(wA.z), "v"(wA.w), "v"(wB.x), "v"(wB.y), "v"(wB.z), "v"(wB.w));
    asm volatile("" ::"v"(winA[0]), "v"(winA[1]), "v"(winA[2]), "v"(winB[0]), "v"(winB[1]), "v"(winB[2]));
    asm volatile("" ::"v"(dtb), "v"(rate), "v"(wn.x), "v"(wn.y), "v"(wn.z), "v"(wn.w));
    asm volatile("" ::"v"(cur.A), "v"(cur.B), "v"(cur.G), "v"(cur.b));

    for (int t = 0; t < n; ++t) {
        const size_t row = (size_t)bs * T + t;
        const size_t tok = row * HD + (size_t)h * kD;
        const TokenLoads x = cur;
        const int p = t & 1;
        // ---- prologue of token t ----
        float uq = 0.f, uk = 0.f;
        if (tid < kD) {
            const float xq = x.A, xk = x.B;
            uq = silu(conv4(wA, winA[0], winA[1], winA[2], xq));
            uk = silu(conv4(wB, winB[0], winB[1], winB[2], xk));
            winA[0] = winA[1]; winA[1] = winA[2]; winA[2] = xq;
            winB[0] = winB[1]; winB[1] = winB[2]; winB[2] = xk;
            const float sqq = group_sum<64>(uq * uq);
            const float skk = group_sum<64>(uk * uk);
            const float sqk = group_sum<64>(uq * uk);
            if (lane == 0) {
                sh_red[wave][0] = sqq;
                sh_red[wave][1] = skk;
                sh_red[wave][2] = sqk;
            }
        } else {
            const float xv = x.A;
            sh_v[p][i] = silu(conv4(wA, winA[0], winA[1], winA[2], xv));
            winA[0] = winA[1]; winA[1] = winA[2]; winA[2] = xv;
            sh_alpha[i] = decay(a.c.gate_lower_bound, rate, x.B, dtb);
            sh_gate[p][i] = sigm(x.G);
            if (i == 0) sh_beta = sigm(x.b);
        }
        if (t + 1 < n) cur = load_token(t + 1);
        lds_barrier();

        const float ssq = sh_red[0][0] + sh_red[1][0];
        const float ssk = sh_red[0][1] + sh_red[1][1];
        const float sqk = sh_red[0][2] + sh_red[1][2];
        const float inv_q = a.c.q_scale * inv_sqrt(ssq + a.c.l2_eps);
        const float inv_k = inv_sqrt(ssk + a.c.l2_eps);
        const float kappa = sqk * inv_q * inv_k;
        const float beta = sh_beta;
        if (tid < kD) {
            const float qh = uq * inv_q, kh = uk * inv_k, al = sh_alpha[tid];
            sh_alk[tid] = make_float2(al, kh);
            sh_akq[tid] = make_float2(al * kh, al * qh);
        }
        lds_barrier();

        // ---- a = S^T(alpha k), c = S^T(alpha q) ----
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
        lds_barrier();

        // ---- u = beta (v - a), o = c + kappa u, S' = D_a S + k u^T ----
        float u[4], o[4];
        delta_and_readout(sh_part, sh_v[p], beta, kappa, cg, u, o);
#pragma unroll
        for (int j = 0; j < 16; ++j) s[j] = update_row(s[j], sh_alk[rg + 8 * j], u);

        // ---- out = sigmoid(g) * RMSNorm(o) ----
        if (tid < 32) {
            const float rinv = rms_inv(o, a.c.rms_eps);
            const float *gt = sh_gate[p] + 4 * cg;
            void *orow = static_cast<char *>(a.out) + tok * (a.c.out_bf16 ? 2 : 4);  // uniform
            store_out4(orow, (unsigned)(4 * cg), gt[0] * (o[0] * rinv * wn.x), gt[1] * (o[1] * rinv * wn.y),
                       gt[2] * (o[2] * rinv * wn.z), gt[3] * (o[3] * rinv * wn.w), a.c.out_bf16);
        }
    }

    // (lane offsets re-derived from an opaque copy of the lane id: shared with the loads
    //  before the loop, they would stay live, 64-bit, across it)
    int tid_ = tid;
    asm volatile("" : "+v"(tid_));
    const int i_ = tid_ < kD ? tid_ : tid_ - kD;
    float *Sout = a.state_out + sofs * kD * kD;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        __builtin_nontemporal_store(
            s[j], reinterpret_cast<f32x4 *>(Sout + (unsigned)(((tid_ >> 5) + 8 * j) * kD + 4 * (tid_ & 31))));
    float *cwA = a.conv_out + conv_seq + ((qk_wave ? 0 : 2 * HD) + (size_t)h * kD) * 3;  // uniform
    float *cwB = a.conv_out + conv_seq + (HD + (size_t)h * kD) * 3;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        cwA[(unsigned)(i_ * 3 + j)] = winA[j];
        if (qk_wave) cwB[(unsigned)(i_ * 3 + j)] = winB[j];
    }
}

}  // namespace

hipError_t launch_decode_multi_seq(const DecodeMultiArgs &a, hipStream_t stream) {
    dim3 grid((unsigned)((size_t)a.B * a.c.H)), block(kThreads);
    void *args[] = {const_cast<DecodeMultiArgs *>(&a)};
    const void *fn = a.slots ? reinterpret_cast<const void *>(&decode_multi_seq_kernel<true>)
                             : reinterpret_cast<const void *>(&decode_multi_seq_kernel<false>);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace kda
