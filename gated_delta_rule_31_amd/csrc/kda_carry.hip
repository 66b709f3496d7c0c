// kda_carry.hip -- the sequential half of the chunked prefill plan (gfx950).
//
// One workgroup of 8 waves per (sequence, head) walks the sequence's chunk records, which
// the chunk kernel (kda_prefill.hip) wrote, and carries the 128x128 fp32 state in MFMA
// accumulator registers.  Per chunk, in the notation of the chunk algebra there,
//   U = U' - W S0,   O = Q~ S0 + P U,   S_end = Diag(e^{G_end}) S0 + K_end^T U,
// followed by out = sigmoid(g) * RMSNorm(O) (header comment "KDA per-head recurrence",
// page "colibri/c/kimi_k3.c").  These are the state-side products of the fused kernel,
// with the same operand precisions: S0 enters W S0 and Q~ S0 as bf16, U enters P U and
// K_end^T U split into bf16 hi + lo, P and K_end are stored split.
//
// Eight waves, two per SIMD so that each hides the other's LDS and MFMA latencies: wave w
// owns value columns 16w .. 16w+15 for all 128 keys.  Inside each 32-key block the rows
// of the two 16-row accumulator tiles interleave (tile x, row m -> key 32P + 8(m/4) + 4x
// + m%4), so a lane's 8 accumulator values of one column are 8 consecutive keys, the
// B-operand layout of a K = 32 MFMA; U interleaves its tokens the same way.
//
// Overlap: the next chunk's record is loaded into registers in three parts, issued
// between the phases of the current chunk (a record is 115 KB per workgroup, about 2K
// cycles of the compute unit's load path, so issuing it at once would stall every wave
// behind it), and a chunk's epilogue runs after the next chunk's first barrier, beside
// that chunk's MFMAs, from a second O tile.

#include "kda_device.hpp"

namespace kda {
namespace {

constexpr int kCarryThreads = 512;

// ---- LDS map (bytes) ----
constexpr int C_E = REC_IMG;                         // e^{G_end} fp32 [128]
constexpr int C_NW = C_E + 512;                      // norm_w fp32 [128]
constexpr int C_O = C_NW + 512;                      // O fp32 [2 tiles][64][CO_LD]
constexpr int CO_LD = 132;                           // padded row pitch of O
constexpr int kOTile = kChunk * CO_LD;               // floats of one O tile
constexpr int kCarryLds = C_O + 2 * kOTile * 4;      // the operand images sit at 0
static_assert(kCarryLds <= 160 * 1024, "LDS budget");
static_assert(REC_IMG % (16 * kCarryThreads) == 0, "image pieces split evenly over the lanes");
constexpr int kImgPieces = REC_IMG / 16 / kCarryThreads;  // 10

// One record as this lane loads it: its pieces of the operand images (copied to LDS
// as they are), a piece of e^{G_end} (lanes < 32) and its U' values.
struct RecordLoads {
    u32x4 img[kImgPieces];
    u32x4 e;
    f32x4 u[2][2];  // [tp][x]
};

// image pieces J0 .. J1-1 of a record
template <int J0, int J1>
__device__ __forceinline__ void load_images(RecordLoads &r, const unsigned char *rec, int tid) {
#pragma unroll
    for (int j = J0; j < J1; ++j) r.img[j] = *reinterpret_cast<const u32x4 *>(rec + (tid + kCarryThreads * j) * 16);
}
// e^{G_end} and U' of a record
__device__ __forceinline__ void load_tail(RecordLoads &r, const unsigned char *rec, int tid) {
    const int w = tid >> 6, lane = tid & 63;
    r.e = *reinterpret_cast<const u32x4 *>(rec + REC_E + min(tid, 31) * 16);
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int x = 0; x < 2; ++x)
            r.u[tp][x] = *reinterpret_cast<const f32x4 *>(rec + REC_U + (((w * 2 + tp) * 2 + x) * 64 + lane) * 16);
}

// Lane coordinates.  (Unlike the chunk kernel, this one has the registers to keep its
// lane-dependent LDS addresses across the chunk loop, so the compiler may hoist them: that
// halves the loop's VALU work.)
#define CARRY_LANE_IDS()                                       \
    int tid_ = (int)threadIdx.x;                               \
    const int w = __builtin_amdgcn_readfirstlane(tid_ >> 6);   \
    const int lr = tid_ & 15;                                  \
    const int lg = (tid_ >> 4) & 3;                            \
    (void)w;                                                   \
    (void)lr;                                                  \
    (void)lg

__global__ __launch_bounds__(kCarryThreads, 1) void carry_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const __bf16 *sW = reinterpret_cast<const __bf16 *>(smem + REC_W);
    const __bf16 *sQ = reinterpret_cast<const __bf16 *>(smem + REC_Q);
    const __bf16 *sPh = reinterpret_cast<const __bf16 *>(smem + REC_PH);
    const __bf16 *sPl = reinterpret_cast<const __bf16 *>(smem + REC_PL);
    const __bf16 *sKh = reinterpret_cast<const __bf16 *>(smem + REC_KH);
    const __bf16 *sKl = reinterpret_cast<const __bf16 *>(smem + REC_KL);
    const float *sE = reinterpret_cast<const float *>(smem + C_E);
    float *sNw = reinterpret_cast<float *>(smem + C_NW);
    float *sO = reinterpret_cast<float *>(smem + C_O);

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
    const int r0 = a.chunk_start[seq];
    const int nrec = a.chunk_start[seq + 1] - r0;  // ceil(T / 64) for a valid batch
    const size_t rec_stride = (size_t)H * kRecBytes;
    const unsigned char *rec0 = a.records + ((size_t)r0 * H + h) * kRecBytes;

    // ---- the state: S[P][x][i] = S[key 32P + 8lg + 4x + i][value 16w + lr] ----
    f32x4 S[4][2];
    {
        CARRY_LANE_IDS();
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
        if (tid_ < kD) sNw[tid_] = a.norm_w[tid_];
    }

    // out = sigmoid(g) * RMSNorm(O) for the L tokens from c0 of an O tile: eight adjacent
    // lanes own one token row (16 values each), 16-byte loads and stores
    auto epilogue = [&](const float *tile, const u32x4 *graw, int c0, int L) {
        const int tid_ = (int)threadIdx.x;
        const int tok = tid_ >> 3;
        const int v0 = 16 * (tid_ & 7);
        float o[16];
        lds_read8(tile + tok * CO_LD + v0, o);
        lds_read8(tile + tok * CO_LD + v0 + 8, o + 8);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) ss += o[j] * o[j];
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        ss += __shfl_xor(ss, 4, 64);
        if (tok < L) {
            const float rinv = 1.0f / sqrtf(ss * (1.0f / kD) + a.c.rms_eps);
            const size_t orow = (size_t)(t0 + c0 + tok) * HD + (size_t)h * kD + v0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float g8[8], nw[8], y[8];
                unpack8(graw[j], g8);
                lds_read8(sNw + v0 + 8 * j, nw);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = sigm(g8[e]) * (o[8 * j + e] * rinv * nw[e]);
                store_out4(a.out, orow + 8 * j, y[0], y[1], y[2], y[3], a.c.out_bf16);
                store_out4(a.out, orow + 8 * j + 4, y[4], y[5], y[6], y[7], a.c.out_bf16);
            }
        }
    };

    RecordLoads ld = {};
    if (nrec > 0) {
        const int tid_ = (int)threadIdx.x;
        load_images<0, kImgPieces>(ld, rec0, tid_);
        load_tail(ld, rec0, tid_);
    }
    u32x4 gprev[2] = {};  // output-gate logits of the previous chunk

    for (int c = 0; c < nrec; ++c) {
        const int c0 = c * kChunk;
        const int L = min(kChunk, T - c0);
        const bool more = c + 1 < nrec;
        const unsigned char *next = rec0 + (size_t)(c + 1) * rec_stride;
        float *tile = sO + (c & 1) * kOTile;

        // ---- this chunk's operand images and e^{G_end} into LDS; U' into registers ----
        f32x4 U[2][2];
        {
            const int tid_ = (int)threadIdx.x;
#pragma unroll
            for (int j = 0; j < kImgPieces; ++j)
                *reinterpret_cast<u32x4 *>(smem + (tid_ + kCarryThreads * j) * 16) = ld.img[j];
            if (tid_ < 32) *reinterpret_cast<u32x4 *>(smem + C_E + tid_ * 16) = ld.e;
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int x = 0; x < 2; ++x) U[tp][x] = ld.u[tp][x];
        }
        lds_barrier();

        // the previous chunk's epilogue (a full chunk: only the last can be partial)
        if (c > 0) epilogue(sO + ((c - 1) & 1) * kOTile, gprev, c0 - kChunk, kChunk);
        // this chunk's output-gate logits, used by its epilogue one chunk later
        u32x4 gcur[2];
        {
            const int tid_ = (int)threadIdx.x;
            const int tok = min(tid_ >> 3, L - 1);
            const uint16_t *gp = a.g + (size_t)(t0 + c0 + tok) * HD + (size_t)h * kD + 16 * (tid_ & 7);
#pragma unroll
            for (int j = 0; j < 2; ++j) gcur[j] = *reinterpret_cast<const u32x4 *>(gp + 8 * j);
            if (more) load_images<0, 4>(ld, next, tid_);
        }

        bf16x8 Sh[4];  // S0 as the B operand of key contractions
        bf16x8 Uh[2], Ul[2];  // U as the B operand of token contractions, hi/lo [tp]
        {
            CARRY_LANE_IDS();
#pragma unroll
            for (int P = 0; P < 4; ++P) {
                const float v8[8] = {S[P][0][0], S[P][0][1], S[P][0][2], S[P][0][3],
                                     S[P][1][0], S[P][1][1], S[P][1][2], S[P][1][3]};
                Sh[P] = to_bf8(v8);
            }
            // U = U' - W S0
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int trow = 32 * tp + 8 * (lr >> 2) + 4 * x + (lr & 3);
                    f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int P = 0; P < 4; ++P) {
                        const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sW + swi128(trow, 32 * P + 8 * lg));
                        ws = mma(A8, Sh[P], ws);
                    }
                    U[tp][x] -= ws;
                }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                const float v8[8] = {U[tp][0][0], U[tp][0][1], U[tp][0][2], U[tp][0][3],
                                     U[tp][1][0], U[tp][1][1], U[tp][1][2], U[tp][1][3]};
                split8(v8, Uh[tp], Ul[tp]);
            }
        }
        {
            const int tid_ = (int)threadIdx.x;
            if (more) load_images<4, 7>(ld, next, tid_);
        }
        {
            CARRY_LANE_IDS();
            // O = Q~ S0 + P U   (rows: token 16tt + 4lg + i)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int P = 0; P < 4; ++P) {
                    const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sQ + sw128(16 * tt + lr, 32 * P + 8 * lg));
                    acc = mma(A8, Sh[P], acc);
                }
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    if (tp > (tt >> 1)) continue;  // P is lower triangular
                    const bf16x8 Ph = *reinterpret_cast<const bf16x8 *>(sPh + sw64(16 * tt + lr, 32 * tp + 8 * lg));
                    const bf16x8 Pl = *reinterpret_cast<const bf16x8 *>(sPl + sw64(16 * tt + lr, 32 * tp + 8 * lg));
                    acc = mma(Ph, Uh[tp], acc);
                    acc = mma(Pl, Uh[tp], acc);
                    acc = mma(Ph, Ul[tp], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) tile[(16 * tt + 4 * lg + i) * CO_LD + 16 * w + lr] = acc[i];
            }
        }
        {
            const int tid_ = (int)threadIdx.x;
            if (more) {
                load_images<7, kImgPieces>(ld, next, tid_);
                load_tail(ld, next, tid_);
            }
        }
        {
            CARRY_LANE_IDS();
            // S = Diag(e^{G_end}) S0 + K_end^T U
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int krow = 32 * P + 8 * (lr >> 2) + 4 * x + (lr & 3);
                    f32x4 acc = S[P][x] * *reinterpret_cast<const f32x4 *>(sE + 32 * P + 8 * lg + 4 * x);
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp) {
                        const bf16x8 Kh = *reinterpret_cast<const bf16x8 *>(sKh + swi64(krow, 32 * tp + 8 * lg));
                        const bf16x8 Kl = *reinterpret_cast<const bf16x8 *>(sKl + swi64(krow, 32 * tp + 8 * lg));
                        acc = mma(Kh, Uh[tp], acc);
                        acc = mma(Kl, Uh[tp], acc);
                        acc = mma(Kh, Ul[tp], acc);
                    }
                    S[P][x] = acc;
                }
        }
        gprev[0] = gcur[0];
        gprev[1] = gcur[1];
        lds_barrier();  // the operand images are rewritten by the next chunk
    }
    if (nrec > 0)
        epilogue(sO + ((nrec - 1) & 1) * kOTile, gprev, (nrec - 1) * kChunk, min(kChunk, T - (nrec - 1) * kChunk));

    // ---- final state ----
    {
        CARRY_LANE_IDS();
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
    for (int q = threadIdx.x; q < 3 * kD; q += kCarryThreads) {
        const int blk = q >> 7, cc = q & 127;
        const size_t ch = (size_t)blk * HD + (size_t)h * kD + cc;
        float win[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int tok = t1 - 3 + j;
            const uint16_t *src = blk == 0 ? a.q : (blk == 1 ? a.k : a.v);
            if (tok >= t0)
                win[j] = bf2f(src[(size_t)tok * HD + (size_t)h * kD + cc]);
            else
                win[j] = a.initial_conv_state ? a.initial_conv_state[conv_seq + ch * 3 + (tok - t0 + 3)] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) a.final_conv_state[conv_seq + ch * 3 + j] = win[j];
    }
}

#undef CARRY_LANE_IDS

}  // namespace

hipError_t launch_carry(const PrefillArgs &a, hipStream_t stream) {
    const void *fn = reinterpret_cast<const void *>(&carry_kernel);
    static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kCarryLds);
    if (attr != hipSuccess) return attr;
    dim3 grid((unsigned)((size_t)a.B * a.c.H)), block(kCarryThreads);
    void *args[] = {const_cast<PrefillArgs *>(&a)};
    return hipLaunchKernel(fn, grid, block, args, kCarryLds, stream);
}

}  // namespace kda
