// kda_carry.hip -- the sequential half of the chunked prefill plan (gfx950).
//
// The carry walks each (sequence, head)'s chunk records, which the chunk kernel
// (kda_prefill.hip) wrote, and carries the 128x128 fp32 state in MFMA accumulator
// registers.  Three forms: carry_kernel (one 8-wave workgroup per pair, described first
// below), carry_split_kernel (two 4-wave workgroups per pair, each owning half the value
// columns, for batches with B*H <= 128; described before it) and carry_kernel_precise
// (the high-precision records).  Per chunk, in the notation of the chunk algebra there,
//   U = U' - W S0,   O = Q~ S0 + P U,   S_end = Diag(e^{G_end}) S0 + K_end^T U,
// followed by out = sigmoid(g) * RMSNorm(O) (header comment "KDA per-head recurrence",
// page "colibri/c/kimi_k3.c").  These are the state-side products of the fused kernel
// with the same operand precisions, in the same order: S0 enters W S0 and Q~ S0 as bf16,
// U enters P U and K_end^T U split into bf16 hi + lo, P and K_end are stored split.
//
// Eight waves, two per SIMD so that each hides the other's LDS and MFMA latencies: wave w
// owns value columns 16w .. 16w+15 for all 128 keys.  Inside each 32-key block the rows
// of the two 16-row accumulator tiles interleave (tile x, row m -> key 32P + 8(m/4) + 4x
// + m%4), so a lane's 8 accumulator values of one column are 8 consecutive keys, the
// B-operand layout of a K = 32 MFMA; U interleaves its tokens the same way.
//
// Streaming.  A record's operand pieces (77 KB, in the order the MFMAs read them) go
// straight from global memory into LDS with direct-to-LDS loads, double-buffered: the
// next chunk's pieces are requested in four parts spread over the current chunk (after
// its opening barrier, after the previous epilogue, after W S0 and after O) and arrive
// while it computes, without occupying registers or issue slots for LDS writes.  Each
// chunk-parity buffer is its own LDS array and the loop body is instantiated once per
// parity, so the compiler can tell the buffer being read from the one being filled and
// does not wait for the loads in flight.  U' (this wave's 4 KB) is
// prefetched into registers one chunk ahead.  O is computed transposed, staged in LDS as
// token rows in the place of W and Q~ (dead by then), and normalised and stored a token per
// 32 lanes early in the next chunk, so that every gate load and output store covers whole
// rows.

#include <type_traits>

#include "kda_carry.hpp"

namespace kda {
namespace {

// The two chunk-parity buffers of operand pieces, each as two arrays (pieces 0 .. 31, which
// later hold the staged O, and pieces 32 .. 76), so that the compiler can tell the part
// being read from a part being filled and does not wait for the loads in flight.
__shared__ __align__(16) unsigned char carry_lo0[kLoPieces * REC_PIECE];
__shared__ __align__(16) unsigned char carry_hi0[kHiPieces * REC_PIECE];
__shared__ __align__(16) unsigned char carry_lo1[kLoPieces * REC_PIECE];
__shared__ __align__(16) unsigned char carry_hi1[kHiPieces * REC_PIECE];
__shared__ int carry_order[kOrderMaxSeqs];  // longest-first workgroup order
// the high-precision carry's single buffer of record pieces (109 KB: two would not fit)
// and its RMS partial sums [64 tokens][8 waves]
__shared__ __align__(16) unsigned char carry_pbuf[RecP::kPieces * REC_PIECE];
__shared__ __align__(16) float carry_ppart[kChunk * 8];

// kBf16: the output buffer holds bf16 (round to nearest even), else fp32
template <bool kBf16>
__global__ __launch_bounds__(kCarryThreads, 1) void carry_kernel(PrefillArgs a) {
    const int H = a.c.H;
    const int seq = seq_longest_first(a.cu_seqlens, a.B, a.N, blockIdx.x / H, carry_order);
    carry_body<kBf16, false>(a, seq, blockIdx.x % H, carry_lo0, carry_hi0, carry_lo1, carry_hi1);
}

// ---- the split carry: two 4-wave workgroups per (sequence, head) ----
// The state recurrence is separable over value columns: U, O and S_end of a column need
// only that column of S0 and U'.  So for batches with B*H <= 128 each (sequence, head) is
// carried by two workgroups of 4 waves, half hf owning value columns 64hf .. 64hf+63
// (wave w: 16(4hf + w) .. +15), on twice the compute units and with one wave per SIMD.
// Both halves stream the whole record (every operand piece is needed for every column)
// but only their own U' tiles.  The only cross-column step is the RMS norm of each output
// row: each half sums the squares of its 64 values with the first four butterfly steps of
// the one-workgroup carry (units j^1, j^2, j^4, j^8 of the 32 four-value units of a row),
// publishes the per-token sums and adds the other half's, which is the last step (j^16):
// the bits of the one-workgroup carry and of the fused kernel.
//
// Exchange: a per-call area of the workspace, zeroed by the chunk table kernel, holds for
// each (pair, half, slot c % 4, token) a 64-bit word {sum, c + 1}; sum and tag are written
// and read as one agent-scope atomic, so no fence orders them.  Chunk c's sums are
// published at the start of chunk c + 1; the other half's are loaded at the end of chunk
// c + 1 (the next opening barrier waits for them together with the record loads, so that
// their check waits for nothing) and used in chunk c + 2.  A half rewrites slot c % 4
// (with chunk c + 4) only after it has seen the other half's sums of chunk c + 2, which the
// other half published after it had read chunk c's: no slot is overwritten before it is
// read.  The wait is bounded (2^20 polls, about a second): a wave that times out writes
// NaN for that chunk's outputs and for every later one, without waiting again, so a
// missing partner costs one bounded wait, not one per chunk.  Both workgroups of a pair
// must be resident together: the
// host launches this form only when every workgroup of the grid has its own compute unit,
// and the workgroup ids of a pair (16q + x and 16q + 8 + x) fall on the same XCD, so the
// second read of each record is an L2 hit.
constexpr int kSplitThreads = 256;
constexpr int kSplitPiecesPerWave = (RecS::kPieces + 3) / 4;  // 20 (the last ones repeat piece 76)
constexpr int kSplitSlots = 4;
constexpr int kSplitMaxPolls = 1 << 20;
static_assert(kSplitXchgBytes == 2 * kSplitSlots * kChunk * 8, "exchange area");

// Epilogue lanes: unit u (values 4u .. 4u+3 of the half) from lane bits 0, 1, 4, 5 (so the
// butterfly is two DPP steps and the two permlane swaps) and the step's token from lane
// bits 2 and 3; wave w stores tokens 16w .. 16w+15, four per step, each store covering
// four whole 256-byte rows.
__device__ __forceinline__ int split_unit(int lane) { return (lane & 3) | (((lane >> 4) & 3) << 2); }
__device__ __forceinline__ int split_token(int w, int s, int lane) { return 16 * w + 4 * s + ((lane >> 2) & 3); }

// this wave's O^T tiles (values 16w + 4lg .. +3 of the half, tokens 16tt + lr) into the
// staging area [64 tokens][16 units] fp32, unit u of token r at u ^ (r & 15)
__device__ __forceinline__ void stage_o_split(const unsigned char *stage, const f32x4 (&o)[4], int w, int lr, int lg) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int r = 16 * tt + lr, u = 4 * w + lg;
        *reinterpret_cast<f32x4 *>(const_cast<unsigned char *>(stage) + r * 256 + ((u ^ (r & 15)) << 4)) = o[tt];
    }
}

// One chunk's epilogue state of a lane: its staged values of its four tokens, the half's
// sums of squares of those tokens and their output-gate logits.
struct SplitEpi {
    f32x4 v[4];
    float part[4];
    uint2 g[4];
};

// The other half's words of chunk cp for this lane's tokens (issued only; checked by
// split_epi_store)
__device__ __forceinline__ void split_poll(unsigned long long (&x)[4], const unsigned long long *other, int cp, int w,
                                           int lane) {
    const unsigned long long *slot = other + (cp % kSplitSlots) * kChunk;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        x[s] = __hip_atomic_load(slot + split_token(w, s, lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The first half of the epilogue of chunk cp: the staged values and the half's sums of
// squares, published for the other half.
__device__ __forceinline__ void split_epi_sums(const unsigned char *stage, SplitEpi &e, unsigned long long *mine,
                                               int cp, int w, int lane, bool publish) {
    const int u = split_unit(lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = split_token(w, s, lane);
        e.v[s] = *reinterpret_cast<const f32x4 *>(stage + r * 256 + ((u ^ (r & 15)) << 4));
        float q = e.v[s][0] * e.v[s][0];
        q = __builtin_fmaf(e.v[s][1], e.v[s][1], q);
        q = __builtin_fmaf(e.v[s][2], e.v[s][2], q);
        q = __builtin_fmaf(e.v[s][3], e.v[s][3], q);
        q = add_dpp<0xB1>(q);
        q = add_dpp<0x4E>(q);
        q = add_xor16(q);
        e.part[s] = add_xor32(q);
    }
    if (u == 0 && publish) {
        const unsigned long long tag = (unsigned long long)(unsigned)(cp + 1) << 32;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            __hip_atomic_store(mine + (cp % kSplitSlots) * kChunk + split_token(w, s, lane),
                               tag | __float_as_uint(e.part[s]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The second half: the other half's sums of chunk cp (x from split_poll; polled again,
// bounded, if not there yet), then out = sigmoid(g) * RMSNorm(O) for the wave's tokens r < L.
// dead: this wave has timed out before (wave-uniform); it then takes NaN at once.
template <bool kBf16>
__device__ __forceinline__ void split_epi_store(const SplitEpi &e, unsigned long long (&x)[4], const float (&nw)[4],
                                                const unsigned long long *other, int cp, float rms_eps, void *out,
                                                size_t col0, size_t HD, int tok0, int L, int w, int lane,
                                                int max_polls, bool &dead) {
    const unsigned tag = (unsigned)(cp + 1);
    auto arrived = [&]() {
        bool ok = true;
#pragma unroll
        for (int s = 0; s < 4; ++s) ok = ok && (unsigned)(x[s] >> 32) == tag;
        return __builtin_amdgcn_ballot_w64(!ok) == 0;
    };
    // (the first check stays out of the retry loop, whose reloads would make it wait for
    //  every load in flight)
    if (!arrived()) {
        for (int tries = 0; !dead; ++tries) {
            if (tries >= max_polls) {
                dead = true;  // the other half never published
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            split_poll(x, other, cp, w, lane);
            if (arrived()) break;
        }
        if (dead) {
#pragma unroll
            for (int s = 0; s < 4; ++s) x[s] = ((unsigned long long)tag << 32) | 0x7fc00000u;
        }
    }
    const int u = split_unit(lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = split_token(w, s, lane);
        const float q = e.part[s] + __uint_as_float((unsigned)x[s]);
        const float rinv = __builtin_amdgcn_rsqf(q * (1.0f / kD) + rms_eps);
        const float gg[4] = {__uint_as_float(e.g[s].x << 16), __uint_as_float(e.g[s].x & 0xffff0000u),
                             __uint_as_float(e.g[s].y << 16), __uint_as_float(e.g[s].y & 0xffff0000u)};
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = sigm(gg[i]) * (e.v[s][i] * rinv * nw[i]);
        if (r < L) store_out4(out, (size_t)(tok0 + r) * HD + col0 + 4 * u, y[0], y[1], y[2], y[3], kBf16);
    }
}

template <bool kBf16>
__global__ __launch_bounds__(kSplitThreads, 1) void carry_split_kernel(PrefillArgs a) {
    const int H = a.c.H;
    const int N = a.N;
    // pair p = 8 (b / 16) + b % 8 and half (b / 8) % 2: both halves of a pair on one XCD
    const int b = (int)blockIdx.x;
    const int pair = 8 * (b >> 4) + (b & 7);
    const int hf = (b >> 3) & 1;
    if (pair >= a.B * H) return;  // (uniform; both halves of a pair agree)
    const int h = pair % H;
    const int seq = seq_longest_first(a.cu_seqlens, a.B, N, pair / H, carry_order);
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
    unsigned long long *mine = a.xchg + ((size_t)pair * 2 + hf) * kSplitSlots * kChunk;
    const unsigned long long *other = a.xchg + ((size_t)pair * 2 + (hf ^ 1)) * kSplitSlots * kChunk;
    const size_t col0 = (size_t)h * kD + 64 * hf;  // this half's first value column in a row

    const int tid = (int)threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..3
    const int gw = 4 * hf + w;                                 // the wave's value columns 16gw ..
    const int lane = tid & 63;
    const int lr = tid & 15;
    const int lg = (tid >> 4) & 3;

    // ---- the state: S[P][x][i] = S[key 32P + 8lg + 4x + i][value 16gw + lr] ----
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
                    S[P][x][i] = S0 ? S0[key * kD + 16 * gw + lr] : 0.0f;
                }
    }
    float nw[4];  // the RMSNorm weight of this lane's epilogue values
#pragma unroll
    for (int i = 0; i < 4; ++i) nw[i] = a.norm_w[64 * hf + 4 * split_unit(lane) + i];

    // Part `part` (0..3) of record c: operand pieces 4j + w for the part's j into an LDS
    // buffer, and one of the wave's four U' tiles into registers (c clamped to the last
    // record, as in the one-workgroup carry).  Parts 0 and 1 hold pieces 32 .. 76, parts 2
    // and 3 pieces 0 .. 31, whose place holds the staged O of the previous chunk until its
    // epilogue has read it.  (Eight smaller parts spread over the chunk measured the same.)
    auto request = [&](auto part_c, auto parity, int c, f32x4 (&Un)[2][2]) {
        constexpr int part = decltype(part_c)::value;
        constexpr int BP = decltype(parity)::value;
        constexpr int j0 = part == 0 ? 8 : (part == 1 ? 14 : (part == 2 ? 0 : 4));
        constexpr int j1 = part == 0 ? 14 : (part == 1 ? kSplitPiecesPerWave : (part == 2 ? 4 : 8));
        const unsigned char *rec = rec0 + (size_t)min(c, nrec - 1) * rec_stride;
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int piece = min(4 * j + w, RecS::kPieces - 1);
            unsigned char *dst = part >= 2 ? (BP ? carry_lo1 : carry_lo0) + piece * REC_PIECE
                                           : (BP ? carry_hi1 : carry_hi0) + (piece - kLoPieces) * REC_PIECE;
            __builtin_amdgcn_global_load_lds(rec + piece * REC_PIECE + lane * 16, (lds_void *)dst, 16, 0, 0);
        }
        constexpr int tp = part >> 1, x = part & 1;
        Un[tp][x] = *reinterpret_cast<const f32x4 *>(rec + RecS::kU + (((gw * 2 + tp) * 2 + x) * 64 + lane) * 16);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;

    f32x4 Unext[2][2] = {};
    uint2 gprev[4] = {};  // the previous chunk's output-gate logits of this lane's values
    SplitEpi pend = {};   // the epilogue of the chunk before that, awaiting the other half's sums
    unsigned long long px[4] = {};  // the other half's words for `pend`, loaded at the previous chunk's end
    bool dead = false;              // this wave timed out waiting for the other half (wave-uniform)
    const bool publish = a.xchg_publish != 0;
    const int max_polls = a.xchg_max_polls > 0 ? a.xchg_max_polls : kSplitMaxPolls;

    auto chunk = [&](auto parity, int c) {
        constexpr int B = decltype(parity)::value;
        using Nxt = std::integral_constant<int, B ^ 1>;
        const unsigned char *cur_lo = B ? carry_lo1 : carry_lo0;
        const unsigned char *cur_hi = B ? carry_hi1 : carry_hi0;
        const unsigned char *prv_lo = B ? carry_lo0 : carry_lo1;  // chunk c - 1's staged O
        const int c0 = c * kChunk;
        const int L = min(kChunk, T - c0);

        barrier_all_mem();
        f32x4 U[2][2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int x = 0; x < 2; ++x) U[tp][x] = Unext[tp][x];
        request(P0{}, Nxt{}, c + 1, Unext);
        // chunk c - 1's sums of squares, published for the other half
        SplitEpi cur;
        if (c > 0) {
            split_epi_sums(prv_lo, cur, mine, c - 1, w, lane, publish);
#pragma unroll
            for (int s = 0; s < 4; ++s) cur.g[s] = gprev[s];
        }
        uint2 g4[4];
        {
            const int u = split_unit(lane);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = min(split_token(w, s, lane), L - 1);
                g4[s] = *reinterpret_cast<const uint2 *>(a.g + (size_t)(t0 + c0 + r) * HD + col0 + 4 * u);
            }
        }
        request(P1{}, Nxt{}, c + 1, Unext);

        auto opnd = [&](int piece) {
            const unsigned char *p = piece < kLoPieces ? cur_lo + piece * REC_PIECE
                                                       : cur_hi + (piece - kLoPieces) * REC_PIECE;
            return *reinterpret_cast<const bf16x8 *>(p + lane * 16);
        };

        bf16x8 Sh[4];
#pragma unroll
        for (int P = 0; P < 4; ++P) {
            const float v8[8] = {S[P][0][0], S[P][0][1], S[P][0][2], S[P][0][3],
                                 S[P][1][0], S[P][1][1], S[P][1][2], S[P][1][3]};
            Sh[P] = to_bf8(v8);
        }
        // U = U' - W S0.  Every product of this chunk takes its operands from LDS into
        // registers first and issues its MFMAs round-robin over the independent
        // accumulators (each accumulator still sees its terms in the order of the
        // one-workgroup carry, so the bits are the same): with one wave per SIMD nothing
        // else would hide an MFMA's wait for the one before it on the same accumulator.
        {
            bf16x8 Wop[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) Wop[i] = opnd(RecS::w(i >> 3, (i >> 2) & 1, i & 3));
            f32x4 ws[4] = {};
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int i = 0; i < 4; ++i) ws[i] = mma(Wop[4 * i + P], Sh[P], ws[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) U[i >> 1][i & 1] -= ws[i];
        }
        // chunk c - 2's outputs (a full chunk: only the last can be partial)
        if (c > 1)
            split_epi_store<kBf16>(pend, px, nw, other, c - 2, a.c.rms_eps, a.out, col0, HD, t0 + c0 - 2 * kChunk,
                                   kChunk, w, lane, max_polls, dead);
        if (c > 0) pend = cur;
        // every wave has read the staged O: pieces 0 .. 31 of `prv` may be loaded
        lds_barrier();
        request(P2{}, Nxt{}, c + 1, Unext);
        bf16x8 Uh[2], Ul[2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            const float v8[8] = {U[tp][0][0], U[tp][0][1], U[tp][0][2], U[tp][0][3],
                                 U[tp][1][0], U[tp][1][1], U[tp][1][2], U[tp][1][3]};
            split8(v8, Uh[tp], Ul[tp]);
        }
        // O^T = S0^T Q~^T + U^T P^T
        f32x4 o[4] = {};
        {
            bf16x8 Qop[16], Pop[12];
#pragma unroll
            for (int i = 0; i < 16; ++i) Qop[i] = opnd(RecS::q(i >> 2, i & 3));
#pragma unroll
            for (int i = 0; i < 12; ++i) Pop[i] = opnd(RecS::kP + i);  // slab i / 2, hi / lo
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) o[tt] = mma(Sh[P], Qop[4 * tt + P], o[tt]);
            // slab of (tt, tp): P is lower triangular, tt >= 2 tp
#define KDA_SLAB(tt, tp) ((tt) < 2 ? (tt) : 2 * (tt) - 2 + (tp))
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Uh[tp], Pop[2 * KDA_SLAB(tt, tp)], o[tt]);
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Uh[tp], Pop[2 * KDA_SLAB(tt, tp) + 1], o[tt]);
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Ul[tp], Pop[2 * KDA_SLAB(tt, tp)], o[tt]);
            }
#undef KDA_SLAB
        }
        request(P3{}, Nxt{}, c + 1, Unext);
        // every wave is done with W and Q~: O goes into their place
        lds_barrier();
        stage_o_split(cur_lo, o, w, lr, lg);
        // S = Diag(e^{G_end}) S0 + K_end^T U
        {
            const float *sE = reinterpret_cast<const float *>(cur_hi + (RecS::kE - kLoPieces) * REC_PIECE);
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int x = 0; x < 2; ++x) S[P][x] = S[P][x] * *reinterpret_cast<const f32x4 *>(sE + 32 * P + 8 * lg + 4 * x);
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                bf16x8 Kop[16];  // [P][x][hi/lo]
#pragma unroll
                for (int i = 0; i < 16; ++i) Kop[i] = opnd(RecS::k(i >> 2, (i >> 1) & 1, tp, i & 1));
#pragma unroll
                for (int i = 0; i < 8; ++i) S[i >> 1][i & 1] = mma(Kop[2 * i], Uh[tp], S[i >> 1][i & 1]);
#pragma unroll
                for (int i = 0; i < 8; ++i) S[i >> 1][i & 1] = mma(Kop[2 * i + 1], Uh[tp], S[i >> 1][i & 1]);
#pragma unroll
                for (int i = 0; i < 8; ++i) S[i >> 1][i & 1] = mma(Kop[2 * i], Ul[tp], S[i >> 1][i & 1]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) gprev[s] = g4[s];
        // the other half's sums of chunk c - 1, for chunk c + 1: loaded now, so that the
        // next opening barrier (which waits for the record loads anyway) also covers them
        // and their check waits for nothing
        split_poll(px, other, max(c - 1, 0), w, lane);
    };

    if (nrec > 0) {
        using B0 = std::integral_constant<int, 0>;
        request(P0{}, B0{}, 0, Unext);
        request(P1{}, B0{}, 0, Unext);
        request(P2{}, B0{}, 0, Unext);
        request(P3{}, B0{}, 0, Unext);
        for (int c = 0; c < nrec; c += 2) {
            chunk(std::integral_constant<int, 0>{}, c);
            if (c + 1 < nrec) chunk(std::integral_constant<int, 1>{}, c + 1);
        }
        // the last two chunks' epilogues
        barrier_all_mem();
        const int cl = nrec - 1;
        SplitEpi last;
        split_epi_sums((cl & 1) ? carry_lo1 : carry_lo0, last, mine, cl, w, lane, publish);
#pragma unroll
        for (int s = 0; s < 4; ++s) last.g[s] = gprev[s];
        if (cl > 0)
            split_epi_store<kBf16>(pend, px, nw, other, cl - 1, a.c.rms_eps, a.out, col0, HD,
                                   t0 + (cl - 1) * kChunk, kChunk, w, lane, max_polls, dead);
        split_poll(px, other, cl, w, lane);
        split_epi_store<kBf16>(last, px, nw, other, cl, a.c.rms_eps, a.out, col0, HD, t0 + cl * kChunk,
                               min(kChunk, T - cl * kChunk), w, lane, max_polls, dead);
    }

    // half hf writes the conv windows of 192 of the head's 384 channels
    carry_finish(a, S, seq, h, t0, t1, 4 * hf, kSplitThreads, 192 * hf, 192 * hf + 192);
}

// kBf16: the output buffer holds bf16 (round to nearest even), else fp32
template <bool kBf16>
__global__ __launch_bounds__(kCarryThreads, 1) void carry_kernel_precise(PrefillArgs a) {
    const int H = a.c.H;
    const int seq = seq_longest_first(a.cu_seqlens, a.B, a.N, blockIdx.x / H, carry_order);
    carry_body_precise<kBf16, false>(a, seq, blockIdx.x % H, carry_pbuf, carry_ppart);
}

}  // namespace

hipError_t launch_carry(const PrefillArgs &a, hipStream_t stream) {
    void *args[] = {const_cast<PrefillArgs *>(&a)};
    if (a.xchg && !a.c.precise) {
        // pairs 8q .. 8q+7 take workgroups 16q .. 16q+15 (see carry_split_kernel)
        const size_t pairs = (size_t)a.B * a.c.H;
        const void *sfn = a.c.out_bf16 ? reinterpret_cast<const void *>(&carry_split_kernel<true>)
                                       : reinterpret_cast<const void *>(&carry_split_kernel<false>);
        return hipLaunchKernel(sfn, dim3((unsigned)(16 * ((pairs + 7) / 8))), dim3(kSplitThreads), args, 0, stream);
    }
    const void *fn = a.c.precise ? (a.c.out_bf16 ? reinterpret_cast<const void *>(&carry_kernel_precise<true>)
                                                  : reinterpret_cast<const void *>(&carry_kernel_precise<false>))
                                 : (a.c.out_bf16 ? reinterpret_cast<const void *>(&carry_kernel<true>)
                                                 : reinterpret_cast<const void *>(&carry_kernel<false>));
    dim3 grid((unsigned)((size_t)a.B * a.c.H)), block(kCarryThreads);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace kda
