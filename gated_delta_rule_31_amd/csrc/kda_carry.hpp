// kda_carry.hpp -- the one-workgroup carry's body and the helpers the carry forms share.
// Included by kda_carry.hip (the carry kernels) and by kda_prefill.hip, whose pipelined
// chunked plan runs the chunk workgroups and the carries in one launch.  The design of the
// carry is described at the top of kda_carry.hip.
#pragma once

#include <type_traits>

#include "kda_device.hpp"

namespace kda {
namespace {

constexpr int kCarryThreads = 512;
using RecS = Rec<false>;
using RecP = Rec<true>;
constexpr int kLoPieces = RecS::kP;                    // W and Q~: pieces 0 .. 31
constexpr int kHiPieces = RecS::kPieces - RecS::kP;    // P, K_end, E: pieces 32 .. 76
constexpr int kPiecesPerWave = (RecS::kPieces + 7) / 8;  // 10 (the last ones repeat piece 76)
constexpr int kPiecesPerWaveP = (RecP::kPieces + 7) / 8;  // 14 (the last ones repeat piece 108)

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier after every global load (direct-to-LDS ones included), store and LDS
// access of each wave has completed: s_waitcnt vmcnt(0) lgkmcnt(0), as a builtin so that
// the compiler's own wait insertion knows the loads are done, then s_barrier.  The empty
// statements with a memory clobber keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_all_mem() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
}

// The final state (from the carry's registers) and the final conv windows (the last 3
// pre-conv inputs of the sequence, from the initial window if it has fewer than 3 tokens).
// Wave w holds value columns 16 (col_wave0 + w) .. +15; the workgroup's `threads` lanes
// write windows q0 .. q1 - 1 of the head's 384 (q, k, v channels).
__device__ __forceinline__ void carry_finish(const PrefillArgs &a, const f32x4 (&S)[4][2], int seq, int h, int t0,
                                             int t1, int col_wave0 = 0, int threads = kCarryThreads, int q0 = 0,
                                             int q1 = 3 * kD) {
    const int H = a.c.H;
    const size_t HD = (size_t)H * kD;
    const int tid = (int)threadIdx.x;
    const int w = col_wave0 + __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = tid & 15;
    const int lg = (tid >> 4) & 3;
    // ---- final state ----
    {
        float *Sf = a.final_state + ((size_t)seq * H + h) * kD * kD;
        // (the initial state may alias the final one: each element is read and written by
        //  the same lane)
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 32 * P + 8 * lg + 4 * x + i;
                    Sf[key * kD + 16 * w + lr] = S[P][x][i];
                }
    }
    // ---- final conv windows: the last 3 pre-conv inputs (from the initial window if T < 3) ----
    const size_t conv_seq = (size_t)seq * 3 * HD * 3;
    for (int q = q0 + tid; q < q1; q += threads) {
        const int blk = q >> 7, cc = q & 127;
        const size_t ch = (size_t)blk * HD + (size_t)h * kD + cc;
        float win[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int tok = t1 - 3 + j;
            const uint16_t *src = blk == 0 ? a.q : (blk == 1 ? a.k : a.v);
            if (tok >= t0)
                win[j] = bf2f(src[(size_t)tok * a.qkv_ld + (size_t)h * kD + cc]);
            else
                win[j] = a.initial_conv_state ? a.initial_conv_state[conv_seq + ch * 3 + (tok - t0 + 3)] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) a.final_conv_state[conv_seq + ch * 3 + j] = win[j];
    }
}

// ---- the standard carry's epilogue, one token per 32 lanes ----
// Wave w normalises and stores tokens 8w .. 8w+7 of a chunk, two per step s (0..3), from
// the chunk's O staged in LDS as [64 tokens][128 values] fp32 (16-byte unit u of token r
// at unit u ^ (r & 31), so that the O^T tiles' writes and the token reads are spread over
// the banks).  Lane bits 0, 1, 4, 5 and 2 are bits 0..4 of the lane's unit j (values 4j ..
// 4j+3) and lane bit 3 picks the step's token, so that each gate load and output store of
// the wave covers two whole rows.  The RMS sum of a token is then a butterfly over j in bit
// order: (j, j^1) and (j, j^2) by DPP, j^4 and j^8 by the permlane swaps, j^16 by a
// swizzle.  That is the tree of the fused kernel's epilogue (the per-wave sums over
// 4-value units j^1, j^2, then across waves j^4, j^8, j^16), so the layouts agree bit for
// bit.
__device__ __forceinline__ int epi_unit(int lane) {
    return (lane & 3) | (((lane >> 4) & 3) << 2) | (((lane >> 2) & 1) << 4);
}
__device__ __forceinline__ int epi_token(int w, int s, int lane) { return 8 * w + 2 * s + ((lane >> 3) & 1); }

// x[l] + x[l ^ m] for DPP control kCtrl: quad_perm 1,0,3,2 (m = 1) or 2,3,0,1 (m = 2)
template <int kCtrl>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float token_sum(float s) {
    s = add_dpp<0xB1>(s);
    s = add_dpp<0x4E>(s);
    s = add_xor16(s);
    s = add_xor32(s);
    // x[l] + x[l ^ 4] inside each 32-lane half: swizzle with and-mask 31, xor-mask 4
    return s + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(s), 0x101F));
}

// The output-gate logits of the lane's 4 values of its tokens (rows past the sequence's
// end clamped to its last row, never stored)
__device__ __forceinline__ void load_gate_rows(uint2 (&g4)[4], const uint16_t *g, size_t HD, int h, int tok0, int L,
                                               int w, int lane) {
    const int j = epi_unit(lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = min(epi_token(w, s, lane), L - 1);
        g4[s] = *reinterpret_cast<const uint2 *>(g + (size_t)(tok0 + r) * HD + (size_t)h * kD + 4 * j);
    }
}

// this wave's O^T tiles (values 16w + 4lg .. +3 of tokens 16tt + lr) into the staging area
__device__ __forceinline__ void stage_o(const unsigned char *stage, const f32x4 (&o)[4], int w, int lr, int lg) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int r = 16 * tt + lr, u = 4 * w + lg;
        *reinterpret_cast<f32x4 *>(const_cast<unsigned char *>(stage) + r * 512 + ((u ^ (r & 31)) << 4)) = o[tt];
    }
}

// out = sigmoid(g) * RMSNorm(O) for the wave's tokens r < L of the staged chunk
template <bool kBf16>
__device__ __forceinline__ void epilogue_rows(const unsigned char *stage, const uint2 (&g4)[4], const float (&nw)[4],
                                              float rms_eps, void *out, size_t HD, int h, int tok0, int L, int w,
                                              int lane) {
    const int j = epi_unit(lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = epi_token(w, s, lane);
        const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + r * 512 + ((j ^ (r & 31)) << 4));
        float q = v[0] * v[0];
        q = __builtin_fmaf(v[1], v[1], q);
        q = __builtin_fmaf(v[2], v[2], q);
        q = __builtin_fmaf(v[3], v[3], q);
        q = token_sum(q);
        const float rinv = __builtin_amdgcn_rsqf(q * (1.0f / kD) + rms_eps);
        const float gg[4] = {__uint_as_float(g4[s].x << 16), __uint_as_float(g4[s].x & 0xffff0000u),
                             __uint_as_float(g4[s].y << 16), __uint_as_float(g4[s].y & 0xffff0000u)};
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = sigm(gg[i]) * (v[i] * rinv * nw[i]);
        if (r < L) store_out4(out, (size_t)(tok0 + r) * HD + (size_t)h * kD + 4 * j, y[0], y[1], y[2], y[3], kBf16);
    }
}

// 16 bytes of a record that another workgroup of the same launch wrote: two device-scope
// (sc1) loads, which do not take a copy that this compute unit's caches may hold
__device__ __forceinline__ f32x4 load_f32x4_agent(const void *p) {
    const unsigned long long *q = reinterpret_cast<const unsigned long long *>(p);
    const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)), __uint_as_float((uint32_t)hi),
                 __uint_as_float((uint32_t)(hi >> 32))};
}

// The one-workgroup carry of (sequence seq, head h).  The record pieces are double-
// buffered in four distinct LDS ranges: lo0/hi0 for even chunks, lo1/hi1 for odd ones
// (pieces 0 .. 31 and 32 .. 76).  They are passed as restrict pointers, so the compiler
// can tell the range being read from the one being filled and does not wait for the
// loads in flight.  kBf16: the output buffer holds bf16 (round to nearest even), else
// fp32.
// kFollow (the pipelined plan: the carries run in the chunk kernel's launch, beside the
// workgroups that write the records): record c is read only after its ready word
// a.ready[row][h] is set, and every read of a record is a device-scope (sc1) load.  The
// ready word of the record after next is loaded at each chunk's start and checked at the
// next one, where the opening barrier has waited for it, so a record that is already
// written costs no wait.  The wait is bounded (kReadyMaxPolls polls, a few seconds): a wave
// that times out sets its columns of the state to NaN (so every later output and its part
// of the final state are NaN) and stops waiting.
template <bool kBf16, bool kFollow>
__device__ __forceinline__ void carry_body(const PrefillArgs &a, int seq, int h, unsigned char *__restrict__ lo0,
                                           unsigned char *__restrict__ hi0, unsigned char *__restrict__ lo1,
                                           unsigned char *__restrict__ hi1) {
    const int H = a.c.H;
    const int N = a.N;
    const size_t HD = (size_t)H * kD;
    int t0 = a.cu_seqlens[seq];
    int t1 = a.cu_seqlens[seq + 1];
    t0 = min(max(t0, 0), N);
    t1 = min(max(t1, t0), N);
    const int T = t1 - t0;
    const int r0 = a.chunk_start[seq];
    const int nrec = a.chunk_start[seq + 1] - r0;  // ceil(T / 64) for a valid batch
    const size_t rec_stride = (size_t)H * RecS::kBytes;
    const unsigned char *rec0 = a.records + ((size_t)r0 * H + h) * RecS::kBytes;

    const int tid = (int)threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = tid & 15;
    const int lg = (tid >> 4) & 3;

    // ---- the state: S[P][x][i] = S[key 32P + 8lg + 4x + i][value 16w + lr] ----
    f32x4 S[4][2];
    {
        const float *S0 = a.initial_state ? a.initial_state + ((size_t)seq * H + h) * kD * kD : nullptr;
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 32 * P + 8 * lg + 4 * x + i;
                    S[P][x][i] = S0 ? S0[key * kD + 16 * w + lr] : 0.0f;
                }
    }
    float nw[4];  // the RMSNorm weight of this lane's epilogue values 4j .. 4j+3
#pragma unroll
    for (int i = 0; i < 4; ++i) nw[i] = a.norm_w[4 * epi_unit(lane) + i];

    // Part `part` (0..3) of record c: operand pieces 8j + w for the part's j into an LDS
    // buffer, and one of the wave's four U' tiles into registers.  c is clamped to the last
    // record, so the request past it is a harmless reload, and every wave issues the same
    // number of loads on every path.  Parts 0 and 1 hold pieces 32 .. 76 (P, K_end, E),
    // parts 2 and 3 pieces 0 .. 31 (W, Q~), whose place holds the staged O of the previous
    // chunk until its epilogue has read it.
    auto request = [&](auto part_c, auto parity, int c, f32x4 (&Un)[2][2]) {
        constexpr int part = decltype(part_c)::value;
        constexpr int BP = decltype(parity)::value;  // the buffer filled
        constexpr int j0 = part == 0 ? 4 : (part == 1 ? 7 : (part == 2 ? 0 : 2));
        constexpr int j1 = part == 0 ? 7 : (part == 1 ? kPiecesPerWave : (part == 2 ? 2 : 4));
        const unsigned char *rec = rec0 + (size_t)min(c, nrec - 1) * rec_stride;
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int piece = min(8 * j + w, RecS::kPieces - 1);
            unsigned char *dst = part >= 2 ? (BP ? lo1 : lo0) + piece * REC_PIECE
                                           : (BP ? hi1 : hi0) + (piece - kLoPieces) * REC_PIECE;
            __builtin_amdgcn_global_load_lds(rec + piece * REC_PIECE + lane * 16, (lds_void *)dst, 16, 0,
                                             kFollow ? kCpolSc1 : 0);
        }
        constexpr int tp = part >> 1, x = part & 1;
        const unsigned char *u = rec + RecS::kU + (((w * 2 + tp) * 2 + x) * 64 + lane) * 16;
        if constexpr (kFollow)
            Un[tp][x] = load_f32x4_agent(u);
        else
            Un[tp][x] = *reinterpret_cast<const f32x4 *>(u);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;

    f32x4 Unext[2][2] = {};
    uint2 gprev[4] = {};  // the previous chunk's output-gate logits

    // kFollow: the ready word of record c (clamped like the requests), a wait for it, and
    // the word of the record after next, loaded one chunk ahead
    const unsigned *ready = kFollow ? a.ready + (size_t)r0 * H + h : nullptr;
    [[maybe_unused]] const int max_polls = a.ready_max_polls > 0 ? a.ready_max_polls : kReadyMaxPolls;
    [[maybe_unused]] bool dead = false;  // this wave timed out (wave-uniform)
    [[maybe_unused]] unsigned ready_ahead = 0;  // the ready word of the next chunk's record after next
    [[maybe_unused]] auto ready_word = [&](int c) {
        return __hip_atomic_load(ready + (size_t)min(c, nrec - 1) * H, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    [[maybe_unused]] auto await_record = [&](int c, unsigned seen) {
        if constexpr (kFollow) {
            if (dead || seen != 0u) return;
            for (int n = 0; ready_word(c) == 0u; ++n) {
                if (n >= max_polls) {
                    dead = true;
                    const float nan = __builtin_nanf("");
#pragma unroll
                    for (int P = 0; P < 4; ++P)
#pragma unroll
                        for (int x = 0; x < 2; ++x) S[P][x] = f32x4{nan, nan, nan, nan};
                    return;
                }
                // short sleeps while the record is likely close, then long ones: the bound
                // is then several seconds, not one
                if (n < kReadyShortPolls)
                    __builtin_amdgcn_s_sleep(4);
                else
                    __builtin_amdgcn_s_sleep(127);
            }
        }
    };

    // one chunk; the buffer parity B is a compile-time constant.  Chunk c's O is staged in
    // pieces 0 .. 31 of its own buffer (W and Q~ are dead once every wave has its O) and
    // normalised and stored early in chunk c + 1, whose stores then have a whole chunk to
    // drain before the next barrier waits for them.
    auto chunk = [&](auto parity, int c) {
        constexpr int B = decltype(parity)::value;
        using Nxt = std::integral_constant<int, B ^ 1>;
        const unsigned char *cur_lo = B ? lo1 : lo0;
        const unsigned char *cur_hi = B ? hi1 : hi0;
        const unsigned char *prv_lo = B ? lo0 : lo1;  // chunk c - 1's staged O
        const int c0 = c * kChunk;
        const int L = min(kChunk, T - c0);

        // this chunk's pieces (every wave's) are in `cur`; nobody reads `prv` but the
        // epilogue; the previous chunk's O is staged in it
        barrier_all_mem();

        f32x4 U[2][2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int x = 0; x < 2; ++x) U[tp][x] = Unext[tp][x];
        if constexpr (kFollow) {
            await_record(c + 1, ready_ahead);
            ready_ahead = ready_word(c + 2);
        }
        request(P0{}, Nxt{}, c + 1, Unext);

        // the previous chunk's epilogue (a full chunk: only the last can be partial)
        if (c > 0)
            epilogue_rows<kBf16>(prv_lo, gprev, nw, a.c.rms_eps, a.out, HD, h, t0 + c0 - kChunk, kChunk, w, lane);
        uint2 g4[4];
        load_gate_rows(g4, a.g, HD, h, t0 + c0, L, w, lane);
        request(P1{}, Nxt{}, c + 1, Unext);

        auto opnd = [&](int piece) {
            const unsigned char *p = piece < kLoPieces ? cur_lo + piece * REC_PIECE
                                                       : cur_hi + (piece - kLoPieces) * REC_PIECE;
            return *reinterpret_cast<const bf16x8 *>(p + lane * 16);
        };

        bf16x8 Sh[4];  // S0 as the B operand of key contractions
#pragma unroll
        for (int P = 0; P < 4; ++P) {
            const float v8[8] = {S[P][0][0], S[P][0][1], S[P][0][2], S[P][0][3],
                                 S[P][1][0], S[P][1][1], S[P][1][2], S[P][1][3]};
            Sh[P] = to_bf8(v8);
        }
        // U = U' - W S0.  The products issue their MFMAs round-robin over independent
        // accumulators (each still takes its terms in the same order: the same bits), so
        // that no MFMA waits for the one before it on the same accumulator.
        {
            f32x4 ws[4] = {};  // [tp][x]
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int i = 0; i < 4; ++i) ws[i] = mma(opnd(RecS::w(i >> 1, i & 1, P)), Sh[P], ws[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) U[i >> 1][i & 1] -= ws[i];
        }
        // every wave's epilogue has read the staged O: pieces 0 .. 31 of `prv` may be loaded
        lds_barrier();
        request(P2{}, Nxt{}, c + 1, Unext);
        bf16x8 Uh[2], Ul[2];  // U as the B operand of token contractions, hi/lo [tp]
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            const float v8[8] = {U[tp][0][0], U[tp][0][1], U[tp][0][2], U[tp][0][3],
                                 U[tp][1][0], U[tp][1][1], U[tp][1][2], U[tp][1][3]};
            split8(v8, Uh[tp], Ul[tp]);
        }
        // O^T = S0^T Q~^T + U^T P^T
        f32x4 o[4] = {};
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) o[tt] = mma(Sh[P], opnd(RecS::q(tt, P)), o[tt]);
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {  // P is lower triangular: tt >= 2 tp
            bf16x8 Ph[4], Pl[4];
#pragma unroll
            for (int tt = 2 * tp; tt < 4; ++tt) {
                Ph[tt] = opnd(RecS::p(tt, tp, 0));
                Pl[tt] = opnd(RecS::p(tt, tp, 1));
            }
#pragma unroll
            for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Uh[tp], Ph[tt], o[tt]);
#pragma unroll
            for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Uh[tp], Pl[tt], o[tt]);
#pragma unroll
            for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Ul[tp], Ph[tt], o[tt]);
        }
        request(P3{}, Nxt{}, c + 1, Unext);
        // every wave is done with W and Q~: O goes into their place
        lds_barrier();
        stage_o(cur_lo, o, w, lr, lg);
        // S = Diag(e^{G_end}) S0 + K_end^T U
        const float *sE = reinterpret_cast<const float *>(cur_hi + (RecS::kE - kLoPieces) * REC_PIECE);
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x) S[P][x] = S[P][x] * *reinterpret_cast<const f32x4 *>(sE + 32 * P + 8 * lg + 4 * x);
        // (two groups of four accumulators (P, x) = (2g + n / 2, n % 2))
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                bf16x8 Kh[4], Kl[4];
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    Kh[n] = opnd(RecS::k(2 * g + (n >> 1), n & 1, tp, 0));
                    Kl[n] = opnd(RecS::k(2 * g + (n >> 1), n & 1, tp, 1));
                }
#pragma unroll
                for (int n = 0; n < 4; ++n) S[2 * g + (n >> 1)][n & 1] = mma(Kh[n], Uh[tp], S[2 * g + (n >> 1)][n & 1]);
#pragma unroll
                for (int n = 0; n < 4; ++n) S[2 * g + (n >> 1)][n & 1] = mma(Kl[n], Uh[tp], S[2 * g + (n >> 1)][n & 1]);
#pragma unroll
                for (int n = 0; n < 4; ++n) S[2 * g + (n >> 1)][n & 1] = mma(Kh[n], Ul[tp], S[2 * g + (n >> 1)][n & 1]);
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) gprev[s] = g4[s];
    };

    if (nrec > 0) {
        using B0 = std::integral_constant<int, 0>;
        if constexpr (kFollow) {
            await_record(0, 0u);
            ready_ahead = ready_word(1);
        }
        request(P0{}, B0{}, 0, Unext);
        request(P1{}, B0{}, 0, Unext);
        request(P2{}, B0{}, 0, Unext);
        request(P3{}, B0{}, 0, Unext);
        for (int c = 0; c < nrec; c += 2) {
            chunk(std::integral_constant<int, 0>{}, c);
            if (c + 1 < nrec) chunk(std::integral_constant<int, 1>{}, c + 1);
        }
        // the last chunk's epilogue; the wait also drains the reload requested past the
        // last record (into the other buffer) and publishes the staged O
        barrier_all_mem();
        const int cl = nrec - 1;
        epilogue_rows<kBf16>((cl & 1) ? lo1 : lo0, gprev, nw, a.c.rms_eps, a.out, HD, h,
                             t0 + cl * kChunk, min(kChunk, T - cl * kChunk), w, lane);
    }

    carry_finish(a, S, seq, h, t0, t1);
}

// The high-precision carry (records of the precise chunk kernel) of (sequence seq, head h):
// the same products with every operand split into bf16 hi + lo, W S0 and Q~ S0 included.
// Its 109-piece record does not fit twice in the LDS, so one buffer holds the current
// chunk's pieces and the next chunk's are requested once every wave is done with them;
// their latency overlaps the chunk's epilogue only.  pbuf (the record's 109 KB) and ppart
// (RMS partial sums, [64 tokens][8 waves]) are two distinct LDS ranges, passed as restrict
// pointers.  kFollow: as in carry_body, for the pipelined plan.
template <bool kBf16, bool kFollow>
__device__ __forceinline__ void carry_body_precise(const PrefillArgs &a, int seq, int h, unsigned char *__restrict__ pbuf,
                                                   float *__restrict__ ppart) {
    const int H = a.c.H;
    const int N = a.N;
    const size_t HD = (size_t)H * kD;
    int t0 = a.cu_seqlens[seq];
    int t1 = a.cu_seqlens[seq + 1];
    t0 = min(max(t0, 0), N);
    t1 = min(max(t1, t0), N);
    const int T = t1 - t0;
    const int r0 = a.chunk_start[seq];
    const int nrec = a.chunk_start[seq + 1] - r0;  // ceil(T / 64) for a valid batch
    const size_t rec_stride = (size_t)H * RecP::kBytes;
    const unsigned char *rec0 = a.records + ((size_t)r0 * H + h) * RecP::kBytes;

    const int tid = (int)threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = tid & 15;
    const int lg = (tid >> 4) & 3;

    f32x4 S[4][2];  // S[P][x][i] = S[key 32P + 8lg + 4x + i][value 16w + lr]
    {
        const float *S0 = a.initial_state ? a.initial_state + ((size_t)seq * H + h) * kD * kD : nullptr;
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 32 * P + 8 * lg + 4 * x + i;
                    S[P][x][i] = S0 ? S0[key * kD + 16 * w + lr] : 0.0f;
                }
    }
    float nw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) nw[i] = a.norm_w[16 * w + 4 * lg + i];

    auto request = [&](int c, f32x4 (&Un)[2][2]) {
        const unsigned char *rec = rec0 + (size_t)c * rec_stride;
#pragma unroll
        for (int j = 0; j < kPiecesPerWaveP; ++j) {
            const int piece = min(8 * j + w, RecP::kPieces - 1);
            __builtin_amdgcn_global_load_lds(rec + piece * REC_PIECE + lane * 16,
                                             (lds_void *)(pbuf + piece * REC_PIECE), 16, 0, kFollow ? kCpolSc1 : 0);
        }
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const unsigned char *u = rec + RecP::kU + (((w * 2 + tp) * 2 + x) * 64 + lane) * 16;
                if constexpr (kFollow)
                    Un[tp][x] = load_f32x4_agent(u);
                else
                    Un[tp][x] = *reinterpret_cast<const f32x4 *>(u);
            }
    };
    auto opnd = [&](int piece) {
        return *reinterpret_cast<const bf16x8 *>(pbuf + piece * REC_PIECE + lane * 16);
    };

    // kFollow: record c is requested only once its ready word is set; the word of the next
    // record is loaded at each chunk's start and checked before its request at the end
    const unsigned *ready = kFollow ? a.ready + (size_t)r0 * H + h : nullptr;
    [[maybe_unused]] const int max_polls = a.ready_max_polls > 0 ? a.ready_max_polls : kReadyMaxPolls;
    [[maybe_unused]] bool dead = false;  // this wave timed out (wave-uniform)
    [[maybe_unused]] unsigned ready_next = 0;
    [[maybe_unused]] auto ready_word = [&](int c) {
        return __hip_atomic_load(ready + (size_t)c * H, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    [[maybe_unused]] auto await_record = [&](int c, unsigned seen) {
        if constexpr (kFollow) {
            if (dead || seen != 0u) return;
            for (int n = 0; ready_word(c) == 0u; ++n) {
                if (n >= max_polls) {
                    dead = true;
                    const float nan = __builtin_nanf("");
#pragma unroll
                    for (int P = 0; P < 4; ++P)
#pragma unroll
                        for (int x = 0; x < 2; ++x) S[P][x] = f32x4{nan, nan, nan, nan};
                    return;
                }
                if (n < kReadyShortPolls)
                    __builtin_amdgcn_s_sleep(4);
                else
                    __builtin_amdgcn_s_sleep(127);
            }
        }
    };

    f32x4 Unext[2][2] = {};
    if (nrec > 0) {
        await_record(0, 0u);
        request(0, Unext);
    }
    for (int c = 0; c < nrec; ++c) {
        const int c0 = c * kChunk;
        const int L = min(kChunk, T - c0);
        barrier_all_mem();  // chunk c's pieces are in the buffer; the last epilogue is done
        if constexpr (kFollow)
            if (c + 1 < nrec) ready_next = ready_word(c + 1);
        f32x4 U[2][2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int x = 0; x < 2; ++x) U[tp][x] = Unext[tp][x];
        uint2 g4[4];
        load_gate4(g4, a.g, HD, h, t0 + c0, L, w, lr, lg);

        bf16x8 Sh[4], Sl[4];
#pragma unroll
        for (int P = 0; P < 4; ++P) {
            const float v8[8] = {S[P][0][0], S[P][0][1], S[P][0][2], S[P][0][3],
                                 S[P][1][0], S[P][1][1], S[P][1][2], S[P][1][3]};
            split8(v8, Sh[P], Sl[P]);
        }
        // U = U' - W S0
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int P = 0; P < 4; ++P) {
                    const bf16x8 Wh = opnd(RecP::w(tp, x, P, 0));
                    const bf16x8 Wl = opnd(RecP::w(tp, x, P, 1));
                    ws = mma(Wh, Sh[P], ws);
                    ws = mma(Wh, Sl[P], ws);
                    ws = mma(Wl, Sh[P], ws);
                }
                U[tp][x] -= ws;
            }
        bf16x8 Uh[2], Ul[2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            const float v8[8] = {U[tp][0][0], U[tp][0][1], U[tp][0][2], U[tp][0][3],
                                 U[tp][1][0], U[tp][1][1], U[tp][1][2], U[tp][1][3]};
            split8(v8, Uh[tp], Ul[tp]);
        }
        // O^T = S0^T Q~^T + U^T P^T
        f32x4 o[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int P = 0; P < 4; ++P) {
                const bf16x8 Qh = opnd(RecP::q(tt, P, 0));
                const bf16x8 Ql = opnd(RecP::q(tt, P, 1));
                acc = mma(Sh[P], Qh, acc);
                acc = mma(Sh[P], Ql, acc);
                acc = mma(Sl[P], Qh, acc);
            }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                if (tp > (tt >> 1)) continue;  // P is lower triangular
                const bf16x8 Ph = opnd(RecP::p(tt, tp, 0));
                const bf16x8 Pl = opnd(RecP::p(tt, tp, 1));
                acc = mma(Uh[tp], Ph, acc);
                acc = mma(Uh[tp], Pl, acc);
                acc = mma(Ul[tp], Ph, acc);
            }
            o[tt] = acc;
        }
        rms_partials(o, ppart, w, lr, lg);
        // S = Diag(e^{G_end}) S0 + K_end^T U
        const float *sE = reinterpret_cast<const float *>(pbuf + RecP::kE * REC_PIECE);
#pragma unroll
        for (int P = 0; P < 4; ++P)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                f32x4 acc = S[P][x] * *reinterpret_cast<const f32x4 *>(sE + 32 * P + 8 * lg + 4 * x);
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    const bf16x8 Kh = opnd(RecP::k(P, x, tp, 0));
                    const bf16x8 Kl = opnd(RecP::k(P, x, tp, 1));
                    acc = mma(Kh, Uh[tp], acc);
                    acc = mma(Kl, Uh[tp], acc);
                    acc = mma(Kh, Ul[tp], acc);
                }
                S[P][x] = acc;
            }
        lds_barrier();  // every wave is done with the buffer and has published its sums
        if (c + 1 < nrec) {
            await_record(c + 1, ready_next);
            request(c + 1, Unext);
        }
        gated_rms_store<kBf16, false>(o, g4, ppart, nw, a.c.rms_eps, a.out, HD, h, t0 + c0, L, 0, w, lr, lg);
    }
    barrier_all_mem();  // the last epilogue's reads of the sums are done before the LDS is released
    carry_finish(a, S, seq, h, t0, t1);
}


}  // namespace
}  // namespace kda
