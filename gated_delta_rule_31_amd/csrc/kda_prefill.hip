// kda_prefill.hip -- chunked varlen KDA prefill on gfx950 (bf16 MFMA, fp32 state).
//
// One workgroup (8 waves, two per SIMD) per (sequence, head) walks the sequence in
// chunks of 64 tokens and carries the 128x128 fp32 state in MFMA accumulator registers.
// Every step of the header comment "KDA per-head recurrence" (page "colibri/c/kimi_k3.c")
// is fused: conv with the carried window, SiLU, L2 norms, gates, the chunked state update
// and readout, the gated RMSNorm (written fp32 or bf16) and the final state / conv window
// write.  Instantiated with kChunked, the same kernel instead stops each chunk after its
// state-independent products and stores them as a record for the carry kernel
// (kda_carry.hip), one workgroup per segment of 4, 8 or 16 chunks (the host's choice for
// the batch's size) and head.
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
// products whose operands decide the error of the fp32 state and of the normalised
// output use a hi+lo bf16 split of those operands (3 MFMAs instead of 1): P (both
// operands), beta*v in U', U in P.U and K_end^T U, and K_end.
//
// Work split.  Wave w (0..7) owns value columns 16w..16w+15 of the state for all 128
// keys (8 accumulator tiles).  Inside each 32-key block the two 16-row tiles interleave
// their rows (tile x, row m -> key 32P + 8(m/4) + 4x + m%4), so that a lane's 8
// accumulator values of one column are 8 consecutive keys: the B-operand layout of a
// K = 32 MFMA.  The state therefore feeds W S0 and (q e^G) S0 straight from registers.
// U uses the same interleave over tokens, so it feeds P U and K_end^T U the same way.
//
// In the prologue wave w handles channel half w / 4 of sub-chunk I (tokens 16I..16I+15),
// I = w % 4 for half 0 and 3 - w % 4 for half 1; lane l owns token 16I + l%16 and 16
// channels 64(w/4) + 16(l/16) + 0..15.  Those are also the operand rows and K-slices of
// block row I of A and P over that channel half, so each wave computes its half of block
// row I from its own registers; the two halves are added through LDS.  Block row I has
// I + 1 blocks, and waves w and w + 4 share a SIMD: pairing sub-chunks I and 3 - I there
// gives every SIMD the same 5 blocks.

#include <type_traits>

#include "kda_carry.hpp"
#include "kda_device.hpp"

namespace kda {
namespace {

constexpr int kThreads = 512;

// ---- LDS map (bytes).  Regions are reused once their first tenant is dead. ----
constexpr int OFF_R1 = 0;        // sCB fp32 [64][132]          -> sKe hi/lo bf16 64 x 128 x2
constexpr int OFF_R2 = 33792;    // sVt hi/lo bf16 [64][128] x2 -> RMS partial sums fp32 [64][8]
constexpr int OFF_R3 = 66560;    // sWr bf16 [64][128]          (beta k e^G)
constexpr int OFF_R4 = 82944;    // sA fp32 [64][68]            -> sW bf16 [64][128]
constexpr int OFF_R5 = 100352;   // sPh, sPl bf16 [64][64] (P split hi/lo)
constexpr int OFF_R6 = 117760;   // sT fp32 [64][68]            -> sQe bf16 [64][128]
constexpr int OFF_R7 = 135168;   // sTb bf16 [64][64]
constexpr int OFF_TAB = 143360;  // small fp32 tables
constexpr int kTabFloats = 512 + 640 + 768 + 512 + 512 + 128 + 256;
constexpr int OFF_CW = OFF_TAB + kTabFloats * 4;  // conv taps of this head, fp32 [3][128][4]
constexpr int OFF_DTB = OFF_CW + 3 * 128 * 4 * 4;  // dt_bias of this head, fp32 [128]
constexpr int OFF_NW = OFF_DTB + 128 * 4;  // RMSNorm weight, fp32 [128] (fused layout's epilogue)
constexpr int kLdsBytes = OFF_NW + 128 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// raw q, k, v rows of a chunk, staged once per chunk in regions 4-7 (free until phase 2):
// [3 blocks][67 rows = the chunk's 64 tokens and the 3 before][136 bf16], the row pitch
// padded by 16 bytes so that 16 lanes reading 16 consecutive rows hit different banks
constexpr int STG_ROWS = kChunk + 3;
constexpr int STG_LD = 136;
static_assert(OFF_R4 + 3 * STG_ROWS * STG_LD * 2 <= OFF_TAB, "staging fits regions 4-7");

// Where each tile lives, per precision mode (byte offsets into the LDS).  The
// high-precision mode keeps the lo halves of beta k e^G, T, W and Q~ as well; K_end^T and
// Q~ stay in registers until W and U' are done, so that their tiles can take the space
// of beta v and beta k e^G:
//   [0, 32768)        sVt hi/lo (phase 1 .. 4)                 -> sKe hi/lo (after 4)
//   [32768, 65536)    staging (.. phase 1), sWr hi/lo (rows .. 4) -> sQe hi/lo (after 4)
//   [65536, 99328)    sCB (tables .. phase 2) -> sA [65536, 82944) (combine .. 3) and
//                     sPh/sPl [82944, 99328) (combine .. 5); sW hi [65536, 81920) (4 .. 5)
//   [99328, 119808)   sPart (phase 2 .. combine) -> sT [99328, 116736) (3)
//                     -> sW lo [99328, 115712) (4 .. 5)
//   [116736, 133120)  sTb hi/lo (3 .. 4) -> RMS partial sums (5 .. epilogue)
// wfb: the head's rows of the decay projection's second factor [128][128] bf16 (gate
// projection only), staged at the chunk start and read in phase 1, where the region is
// free in either map (standard: sCB's, written after phase 1; precise: above the staging).
struct LdsMap {
    int vt, wr, stg, cb, part, a, ph, t, tb, w, wl, ke, qe, rms, wfb;
};
constexpr LdsMap kMapStd = {OFF_R2, OFF_R3, OFF_R4, OFF_R1, OFF_R6, OFF_R4, OFF_R5,
                            OFF_R6, OFF_R7, OFF_R4, -1,     OFF_R1, OFF_R6, OFF_R2, OFF_R1};
constexpr LdsMap kMapPrecise = {0,     32768, 32768, 65536, 99328, 65536, 82944, 99328,
                                116736, 65536, 99328, 0, 32768, 116736, 98304};
static_assert(kMapStd.wfb + kD * kRank * 2 <= OFF_R2, "W_fb block fits region 1");
static_assert(kMapPrecise.wfb >= kMapPrecise.stg + 3 * STG_ROWS * STG_LD * 2 &&
                  kMapPrecise.wfb + kD * kRank * 2 <= OFF_TAB,
              "W_fb block clear of the staging");
static_assert(kMapPrecise.stg + 3 * STG_ROWS * STG_LD * 2 <= OFF_TAB, "staging fits");
static_assert(kMapPrecise.tb + 2 * 64 * 64 * 2 <= OFF_TAB, "precise map fits");

// One chunk's raw inputs as this lane loads them: the chunk's 64 rows of q, k, v as 16-byte
// pieces (lane l loads piece l%16 of rows l/16 and l/16 + 32 of each block), one piece of
// the 3 rows before the chunk (lanes < 144), and the lane's own z row and beta logit.
// (With the gate projection the lane's f row is loaded in phase 1 instead of z.)
struct ChunkLoads {
    u32x4 row[3][2];
    u32x4 hist;
    u32x4 z[2];
    float b;
};

// The 16-byte chunk swizzle of the staged W_fb block [128 rows][16 chunks]: distinct over
// the 16 rows one MFMA's lanes read (rows 64h + 16(l/4) + 4m + l%4 of lanes l < 16).
__device__ __forceinline__ int wfb_swz(int row) { return (row & 3) | (((row >> 4) & 3) << 2); }

constexpr int CB_LD = 132;  // fp32 row pitch of sCB
constexpr int F_LD = 68;    // fp32 row pitch of sA, sT

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
// the prologue sub-chunk of wave w (see the header)
__device__ __forceinline__ int wave_sub(int w) { return (w >> 2) ? 3 - (w & 3) : (w & 3); }
// 4 consecutive bf16 of one row of a swizzled tile (8 bytes, one LDS store)
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---- token-major operand tiles, read transposed ----
// beta v, beta k e^G and K_end^T are kept token-major, [64 tokens][128 channels] bf16 in the
// sw128 layout, so that a lane holding 8 channels of one token writes them with one 16-byte
// store.  Their MFMAs take them channel-major (8 consecutive tokens of one channel per
// lane), which ds_read_b64_tr_b16 (gfx950) gives: within each group of 16 lanes, lane 4k + a
// supplies the address of channels col(a) .. col(a)+3 of token t0 + k, and lane 4a + b
// receives channel col(a) + b of tokens t0 .. t0+3 (the lane layout measured on the
// device).  col_a is this lane's col(lane % 4), a multiple of 4; t0 is uniform over the
// 16-lane group.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr4(const __bf16 *tile, int t0, int col_a) {
    const int t = t0 + (((int)threadIdx.x >> 2) & 3);
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(const_cast<__bf16 *>(tile) + sw128(t, col_a)));
    return __builtin_bit_cast(bf16x4, r);
}
// the 8 tokens t0 .. t0+7 of the lane's channel: two transposed reads
__device__ __forceinline__ bf16x8 lds_tr8(const __bf16 *tile, int t0, int col_a) {
    const bf16x4 x = lds_tr4(tile, t0, col_a), y = lds_tr4(tile, t0 + 4, col_a);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane coordinates, re-derived at the start of every phase from an opaque copy of the
// thread id.  Without this the compiler hoists every lane-dependent LDS address of the
// chunk loop out of the loop and keeps (or spills) hundreds of them across it.
//   w: wave (uniform), lr: lane % 16, lg: lane / 16, sub: sub-chunk of the wave's
//   prologue tokens, half: its channel half, t: its prologue token.
#define KDA_LANE_IDS()                                         \
    int tid_ = (int)threadIdx.x;                               \
    asm volatile("" : "+v"(tid_));                             \
    const int w = __builtin_amdgcn_readfirstlane(tid_ >> 6);   \
    const int lr = tid_ & 15;                                  \
    const int lg = (tid_ >> 4) & 3;                            \
    const int sub = wave_sub(w);                               \
    const int half = w >> 2;                                   \
    const int t = 16 * sub + lr;                               \
    (void)w;                                                   \
    (void)lr;                                                  \
    (void)lg;                                                  \
    (void)sub;                                                 \
    (void)half;                                                \
    (void)t

// Rows are clamped into the sequence [t0, t1): rows before its start are replaced by the
// carried window later, rows past its end belong to padding tokens and are never used.
// The base row is uniform, so lane offsets stay 32-bit.  The loads come in two parts,
// issued in different phases so that no wave stalls behind a full memory pipe at a
// barrier: part 0 the q rows, the lane's z row and beta logit; part 1 the k and v rows
// and the 3 rows before the chunk.
template <int kPart, bool kGateProj>
__device__ __forceinline__ void load_chunk(ChunkLoads &r, const PrefillArgs &a, int tid, int h, int t0, int t1,
                                           int c0) {
    const size_t HD = (size_t)a.c.H * kD;
    const uint32_t LDX = (uint32_t)a.qkv_ld;  // q, k, v row stride (<= 2^24, so 67 rows fit 32 bits)
    // every row below lies in [rbase, t1 - 1] (t1 > t0), also when c0 is past the end
    const int rbase = min(max(t0 + c0 - 3, t0), t1 - 1);
    const size_t ebase = (size_t)rbase * HD + (size_t)h * kD;        // z rows
    const size_t xbase = (size_t)rbase * a.qkv_ld + (size_t)h * kD;  // q, k, v rows
    const uint16_t *X[3] = {a.q, a.k, a.v};
    const uint32_t piece = 8u * (uint32_t)(tid & 15);
#pragma unroll
    for (int blk = (kPart == 0 ? 0 : 1); blk < (kPart == 0 ? 1 : 3); ++blk)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int row = (tid >> 4) + 32 * k;  // chunk row 0..63
            const uint32_t tok = (uint32_t)(min(max(t0 + c0 + row, t0), t1 - 1) - rbase);
            r.row[blk][k] = *reinterpret_cast<const u32x4 *>(X[blk] + xbase + (tok * LDX + piece));
        }
    if constexpr (kPart == 1) {
        const int i = min(tid, 143);  // 3 blocks x 3 rows x 16 pieces
        const int blk = i / 48, row = (i % 48) >> 4;  // history row 0..2 = token c0 - 3 + row
        const uint16_t *src = blk == 0 ? a.q : (blk == 1 ? a.k : a.v);
        const uint32_t tok = (uint32_t)(min(max(t0 + c0 - 3 + row, t0), t1 - 1) - rbase);
        r.hist = *reinterpret_cast<const u32x4 *>(src + xbase + (tok * LDX + piece));
    } else {
        const int lane_t = 16 * wave_sub(tid >> 6) + (tid & 15);    // the prologue token of this lane
        const int cbase = 64 * (tid >> 8) + 16 * ((tid >> 4) & 3);  // and its 16 channels
        const int tauc = min(max(t0 + c0 + lane_t, t0), t1 - 1);
        const uint32_t ztok = (uint32_t)(tauc - rbase);
        if constexpr (!kGateProj) {
#pragma unroll
            for (int pc = 0; pc < 2; ++pc)
                r.z[pc] = *reinterpret_cast<const u32x4 *>(a.z + ebase + (ztok * (uint32_t)HD + (uint32_t)(cbase + 8 * pc)));
        }
        r.b = bf2f(a.b[(size_t)tauc * a.c.H + h]);
    }
}

// kChunked = false: the fused plan, one workgroup per (sequence, head) over all chunks.
// kChunked = true: one workgroup per (segment, head) computes up to a.seg_chunks
// consecutive chunks of one sequence up to U' and stores each chunk's record instead of
// carrying the state.
// kPrecise: every MFMA operand of the chunk algebra is split into bf16 hi + lo (A's two
// operands, T and beta k e^G in W, T in U', W and S0 in W S0, Q~ and S0 in Q~ S0, besides
// the splits of the standard mode), so that no product rounds an operand to 8 bits.
// kGateProj: the decay logits are z = W_fb f (a.f, a.w_fb) instead of a.z: each chunk
// stages the head's 128 rows of W_fb in LDS and phase 1 forms its 64 x 128 logits with
// MFMAs, laid out as the gate computation wants them (see phase 1).
// kPipe (with the chunked forms only): the pipelined plan, whose carries run in the same
// launch; each chunk's record is announced in a.ready once every wave's
// stores of it have completed.  bid: the workgroup's segment-major index (sg * H + h),
// or (sequence order) * H + h in the fused plan.
template <bool kChunked, bool kPrecise, bool kGateProj, bool kPipe = false>
__device__ __forceinline__ void prefill_body(const PrefillArgs a, const int bid) {
    static_assert(!kPipe || kChunked, "the pipelined plan's form");
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr LdsMap M = kPrecise ? kMapPrecise : kMapStd;
    using R = Rec<kPrecise>;
    float *sCB = reinterpret_cast<float *>(smem + M.cb);                // [64][132] k e^{r - G}
    __bf16 *sKeHi = reinterpret_cast<__bf16 *>(smem + M.ke);            // K_end (see store_ke)
    __bf16 *sKeLo = sKeHi + 128 * 64;
    __bf16 *sVtHi = reinterpret_cast<__bf16 *>(smem + M.vt);            // [64][128] beta v, read transposed
    __bf16 *sVtLo = sVtHi + 128 * 64;
    __bf16 *sWr = reinterpret_cast<__bf16 *>(smem + M.wr);              // [64][128] beta k e^G, read transposed
    __bf16 *sWrLo = sWr + 128 * 64;                                     // (kPrecise) its lo part
    float *sA = reinterpret_cast<float *>(smem + M.a);                  // [64][68]
    __bf16 *sW = reinterpret_cast<__bf16 *>(smem + M.w);                // [64][128]
    __bf16 *sWLo = reinterpret_cast<__bf16 *>(smem + (kPrecise ? M.wl : 0));  // (kPrecise) [64][128]
    __bf16 *sPh = reinterpret_cast<__bf16 *>(smem + M.ph);              // [64][64] P, hi part
    __bf16 *sPl = sPh + 64 * 64;                                        // [64][64] P, lo part
    float *sT = reinterpret_cast<float *>(smem + M.t);                  // [64][68]
    __bf16 *sQe = reinterpret_cast<__bf16 *>(smem + M.qe);              // [64][128] q e^G
    __bf16 *sQeLo = sQe + 64 * 128;                                     // (kPrecise) its lo part
    __bf16 *sTb = reinterpret_cast<__bf16 *>(smem + M.tb);              // [64][64]
    __bf16 *sTbLo = sTb + 64 * 64;                                      // (kPrecise) its lo part
    // K_end (hi/lo) of token t, channels cb .. cb+15.  The chunked plan keeps it token-major
    // (16-byte stores; its record copy reads it transposed, once); the fused plan, whose
    // state update reads it 32 times a chunk, keeps K_end^T channel-major (swi64: 16-byte
    // operand reads, 2-byte stores).
    auto store_ke = [&](const float *ke16, int t, int cb) {
        if constexpr (kChunked) {
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                bf16x8 kh, kl;
                split8(ke16 + 8 * pc, kh, kl);
                *reinterpret_cast<bf16x8 *>(sKeHi + sw128(t, cb + 8 * pc)) = kh;
                *reinterpret_cast<bf16x8 *>(sKeLo + sw128(t, cb + 8 * pc)) = kl;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const __bf16 hi = (__bf16)ke16[j];
                sKeHi[swi64(cb + j, t)] = hi;
                sKeLo[swi64(cb + j, t)] = bf16_lo(ke16[j], hi);
            }
        }
    };
    // (decay sums in log2 units: G below is the natural-log decay times log2(e))
    float *sTot = reinterpret_cast<float *>(smem + OFF_TAB);  // [4][128] per-sub-chunk gk sums
    float *sPair = sTot + 512 + 640;                           // [6][128] e^{r_I - r_J}, J < I
    float *sExpRef = sPair + 768;                              // [4][128] e^{r_I}
    float *sEndRef = sExpRef + 512;                            // [4][128] e^{G_end - r_I}
    float *sExpEnd = sEndRef + 512;                            // [128]    e^{G_end}
    float *sNorm = sExpEnd + 128;                              // [2 halves][q,k][64] sums of squares
    float *sConvW = reinterpret_cast<float *>(smem + OFF_CW);  // [3][128][4] taps, oldest first
    float *sDtb = reinterpret_cast<float *>(smem + OFF_DTB);   // [128] -exp(A_log) log2(e) dt_bias
    float *sNw = reinterpret_cast<float *>(smem + OFF_NW);     // [128] RMSNorm weight

    const int H = a.c.H;
    const int N = a.N;
    // cbeg, cend: token offsets (in the sequence) of the chunks this workgroup walks;
    // rec0: record row of the sequence's first chunk (chunked plan)
    int seq, h, cbeg, nrec = 0, rec0 = 0;
    if constexpr (kChunked) {
        int sg = bid / H;
        h = bid - sg * H;
        if (sg >= a.seg_start[a.B]) return;  // past the batch's last segment (uniform)
        if constexpr (kPipe)
            if (a.item_sg) sg = a.item_sg[sg];  // several sequences: row-major order
        // the sequence owning segment sg: seg_start[lo] <= sg < seg_start[hi]
        int lo = 0, hi = a.B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.seg_start[mid] <= sg) lo = mid; else hi = mid;
        }
        seq = lo;
        rec0 = a.chunk_start[seq];
        nrec = a.chunk_start[seq + 1] - rec0;  // ceil(T / 64) for a valid batch
        cbeg = (sg - a.seg_start[seq]) * a.seg_chunks * kChunk;
    } else {
        const int r = bid / H;
        h = bid - r * H;
        // (region 1 is free until the first chunk's operand rows)
        seq = seq_longest_first(a.cu_seqlens, a.B, N, r, reinterpret_cast<int *>(smem + OFF_R1));
        cbeg = 0;
    }
    const size_t HD = (size_t)H * kD;
    int t0 = a.cu_seqlens[seq];
    int t1 = a.cu_seqlens[seq + 1];
    t0 = min(max(t0, 0), N);
    t1 = min(max(t1, t0), N);
    const int T = t1 - t0;

    // The decay gate gk = gmin sigmoid(exp(A_log) (z + dt_bias)) is formed in log2 units:
    // 1 / (1 + 2^(z zr + dtb')) with zr = -exp(A_log) log2(e) and dtb' = zr dt_bias (one FMA),
    // scaled by gmin log2(e), so that every e^x of the chunk algebra below is one exp2.
    constexpr float kLog2e = 1.4426950408889634f;
    const float gmin2 = a.c.gate_lower_bound * kLog2e;
    const float zr = -__expf(a.A_log[h]) * kLog2e;
    // SiLU in the same units: the conv taps are staged times -log2(e), so that a conv output
    // y' = -log2(e) y gives sigmoid(y) = 1 / (1 + 2^y') and u' = y' sigmoid(y) =
    // -log2(e) SiLU(y) with no multiply.  The L2 norms of q and k absorb the factor (the
    // eps scaled by log2(e)^2, the sign by negated scales); v's is folded into beta.
    constexpr float kLn2 = 0.6931471805599453f;
    const float qscale = -a.c.q_scale;
    const float l2eps = a.c.l2_eps * (kLog2e * kLog2e);
    const size_t conv_seq = (size_t)seq * 3 * HD * 3;  // this sequence's conv windows

    // ---- the state: S[P][x][i] = S[key 32P + 8lg + 4x + i][value 16w + lr] ----
    f32x4 S[4][2];
    if constexpr (!kChunked) {
        KDA_LANE_IDS();
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

    // the conv taps of this head's 384 channels, and its initial conv windows (zeros if
    // none; read only by the sequence's first chunk): these sit in sPair/sExpRef, which
    // the first chunk's tables step overwrites only after the last read of the windows
    // (phase 1 of chunk 0)
    float *sWin0 = sPair;  // [3*128][3]
    for (int i = threadIdx.x; i < 3 * kD; i += kThreads) {
        const int blk = i >> 7, c = i & 127;
        const size_t ch = (size_t)blk * HD + (size_t)h * kD + c;
        *reinterpret_cast<float4 *>(sConvW + i * 4) = *reinterpret_cast<const float4 *>(a.conv_w + ch * 4) * -kLog2e;
        if (i < kD) {
            sDtb[i] = zr * a.dt_bias[(size_t)h * kD + i];
            if (!kChunked) sNw[i] = a.norm_w[i];
        }
        if (cbeg == 0) {
#pragma unroll
            for (int j = 0; j < 3; ++j)
                sWin0[i * 3 + j] = a.initial_conv_state ? a.initial_conv_state[conv_seq + ch * 3 + j] : 0.f;
        }
    }
    __syncthreads();

    // Raw inputs of a chunk are loaded one chunk ahead (issued before the previous chunk's
    // state-side MFMAs, so that their latency is hidden) and the q, k, v rows are staged
    // in LDS at the chunk's start, each 16-byte piece once.
    uint16_t *sStage = reinterpret_cast<uint16_t *>(smem + M.stg);
    ChunkLoads ld = {};
    if (T > 0) {
        int tid_ = (int)threadIdx.x;
        asm volatile("" : "+v"(tid_));
        load_chunk<0, kGateProj>(ld, a, tid_, h, t0, t1, cbeg);
        load_chunk<1, kGateProj>(ld, a, tid_, h, t0, t1, cbeg);
    }
    // (the prefetched z and b are marked consumed where no store is in flight: once here,
    //  and in every chunk before its stores; without that the compiler cannot count the
    //  stores issued after them across the loop's back edge and makes phase 1 wait for
    //  every memory operation in flight, stores included)
    if constexpr (kGateProj)
        asm volatile("" ::"v"(ld.b));
    else
        asm volatile("" ::"v"(ld.z[0]), "v"(ld.z[1]), "v"(ld.b));

    // chunked plan: the LDS byte offset (/16, two per register) of the 16 bytes this lane
    // copies into each record piece it writes (pieces 8j + w); see the record layout in
    // kda_device.hpp
    constexpr int kPPW = (R::kPieces + 7) / 8;  // record pieces each wave copies
    uint32_t rec_src[(kPPW + 1) / 2] = {};
    if constexpr (kChunked) {
        const int tid = (int)threadIdx.x;
        const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int j = 0; j < kPPW; ++j) {
            const int piece = 8 * j + w;
            int off = 0;  // bytes from smem
            if (piece < R::kQ) {
                const int pw = piece - R::kW, hl = kPrecise ? pw >> 4 : 0, pp = pw & 15;
                const int tp = pp >> 3, x = (pp >> 2) & 1, P = pp & 3;
                const int trow = 32 * tp + 8 * (lr >> 2) + 4 * x + (lr & 3);
                off = (hl ? M.wl : M.w) + 2 * swi128(trow, 32 * P + 8 * lg);  // W (hi / lo)
            } else if (piece < R::kP) {
                const int pq = piece - R::kQ, hl = kPrecise ? pq >> 4 : 0, pp = pq & 15;
                const int tt = pp >> 2, P = pp & 3;
                off = M.qe + hl * 64 * 128 * 2 + 2 * sw128(16 * tt + lr, 32 * P + 8 * lg);  // Q~ (hi / lo)
            } else if (piece < R::kK) {
                const int sl = (piece - R::kP) >> 1, hl = (piece - R::kP) & 1;
                const int tt = sl < 2 ? sl : (sl + 2) >> 1, tp = sl < 2 ? 0 : (sl & 1);
                off = M.ph + hl * 64 * 64 * 2 + 2 * sw64(16 * tt + lr, 32 * tp + 8 * lg);  // P hi / lo
            } else if (piece < R::kE) {
                off = 0;  // K_end^T: read transposed in the copy loop
            } else if (piece == R::kE) {
                off = OFF_TAB + (512 + 640 + 768 + 512 + 512) * 4 + 16 * min(lane, 31);  // e^{G_end}
            }
            rec_src[j >> 1] |= (uint32_t)(off >> 4) << (16 * (j & 1));
        }
#pragma unroll
        for (int i = 0; i < (kPPW + 1) / 2; ++i) asm volatile("" : "+v"(rec_src[i]));
    }

    const int cend = kChunked ? min(min(cbeg + a.seg_chunks * kChunk, nrec * kChunk), T) : T;
    // kPipe: chunk cc's record is complete (every wave has waited for its own device-scope
    // stores of it, then a barrier): its ready word, a device-scope store
    auto publish_ready = [&](int cc) {
        if constexpr (kPipe) {
            if (threadIdx.x == 0 && a.ready_publish)
                __hip_atomic_store(a.ready + (size_t)(rec0 + cc / kChunk) * H + h, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    // (inside the chunk loop every cross-wave dependency goes through LDS, so its
    //  barriers wait for LDS traffic only: the next chunk's loads and this chunk's output
    //  stores stay in flight across them)
    for (int c0 = cbeg; c0 < cend; c0 += kChunk) {
        const int L = min(kChunk, T - c0);

        // stage this chunk's raw rows (regions 4-7 are dead since the last chunk's phase 5);
        // staging row r holds token c0 - 3 + r
        {
            int tid_ = (int)threadIdx.x;
            asm volatile("" : "+v"(tid_));
            const int piece = 8 * (tid_ & 15);
#pragma unroll
            for (int blk = 0; blk < 3; ++blk)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    *reinterpret_cast<u32x4 *>(sStage + (blk * STG_ROWS + 3 + (tid_ >> 4) + 32 * k) * STG_LD + piece) =
                        ld.row[blk][k];
            if (tid_ < 144) {
                const int blk = tid_ / 48, row = (tid_ % 48) >> 4;
                *reinterpret_cast<u32x4 *>(sStage + (blk * STG_ROWS + row) * STG_LD + piece) = ld.hist;
            }
            if constexpr (kGateProj) {
                // the head's W_fb block [128][128] bf16 into LDS (direct-to-LDS loads, 1 KB per
                // wave instruction = 4 rows; lane l writes physical chunk l%16 of its row, which
                // holds the row's logical chunk (l%16) ^ wfb_swz(row)); waited for in phase 1
                const int w = tid_ >> 6, lane = tid_ & 63;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = w + 8 * i;  // rows 4n .. 4n+3
                    const int row = 4 * n + (lane >> 4);
                    const int j = (lane & 15) ^ wfb_swz(row);
                    __builtin_amdgcn_global_load_lds(
                        a.w_fb + ((size_t)h * kD + row) * kRank + 8 * j,
                        (__attribute__((address_space(3))) void *)((__attribute__((address_space(3))) unsigned char *)
                                                                       (smem + M.wfb) + n * 1024),
                        16, 0, 0);
                }
            }
        }
        lds_barrier();

        // ================= phase 1: conv, SiLU, partial norms, gates =================
        float uq[16], uk[16], gs[16];  // q, k before the norm; G_t - r_sub of the 16 channels
        float beta;
        {
            KDA_LANE_IDS();
            const bool valid = t < L;
            const int tau = t0 + c0 + t;                // packed row of the token
            const bool head_of_seq = c0 == 0 && t < 3;  // rows before the sequence start
            const int cbase = 64 * half + 16 * lg;      // first of this lane's 16 channels
            beta = valid ? sigm(ld.b) : 0.0f;

            // -log2(e) SiLU(ShortConv4(x)) of the 8 channels cbase + 8pc .. +7 of block blk.  Tokens
            // past the sequence end (t >= L) get finite values of no effect: their beta and
            // decay gate are zero, so their rows of W, U' and U are exactly zero and their
            // rows of A are masked; only their own output rows (never stored) see them.
            auto conv_piece = [&](const int blk, const int pc, float *u) {
                const int cb0 = cbase + 8 * pc;
                float xr[4][8];  // rows tau-3 .. tau = staging rows t .. t+3
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    unpack8(*reinterpret_cast<const u32x4 *>(sStage + (blk * STG_ROWS + t + r) * STG_LD + cb0), xr[r]);
                float4 cw[8];
                float y[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    cw[j] = *reinterpret_cast<const float4 *>(sConvW + (blk * kD + cb0 + j) * 4);
                    y[j] = cw[j].x * xr[0][j] + cw[j].y * xr[1][j] + cw[j].z * xr[2][j] + cw[j].w * xr[3][j];
                }
                if (head_of_seq) {
                    // the rows before the sequence start come from the carried window: the
                    // same sum again with those rows replaced
#pragma unroll
                    for (int r = 0; r < 3; ++r) {
                        const int tok = tau - 3 + r;
                        if (tok < t0) {
                            const int p = tok - t0 + 3;  // slot of the carried window, 0..2
#pragma unroll
                            for (int j = 0; j < 8; ++j) xr[r][j] = sWin0[(blk * kD + cb0 + j) * 3 + p];
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        y[j] = cw[j].x * xr[0][j] + cw[j].y * xr[1][j] + cw[j].z * xr[2][j] + cw[j].w * xr[3][j];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) u[j] = y[j] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y[j]));
            };
            const float vscale = beta * -kLn2;  // beta v = vscale u'
            // v: beta * v, hi/lo, into the token-major sVt
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                float u[8], bv[8];
                conv_piece(2, pc, u);
#pragma unroll
                for (int j = 0; j < 8; ++j) bv[j] = vscale * u[j];
                bf16x8 hi, lo;
                split8(bv, hi, lo);
                *reinterpret_cast<bf16x8 *>(sVtHi + sw128(t, cbase + 8 * pc)) = hi;
                *reinterpret_cast<bf16x8 *>(sVtLo + sw128(t, cbase + 8 * pc)) = lo;
            }
            // q, k and their partial sums of squares over this wave's 64 channels
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                conv_piece(0, pc, uq + 8 * pc);
                conv_piece(1, pc, uk + 8 * pc);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ssq += uq[8 * pc + j] * uq[8 * pc + j];
                    ssk += uk[8 * pc + j] * uk[8 * pc + j];
                }
            }
            ssq = add_xor32(add_xor16(ssq));
            ssk = add_xor32(add_xor16(ssk));
            if (lg == 0) {
                sNorm[half * 128 + t] = ssq;
                sNorm[half * 128 + 64 + t] = ssk;
            }
            // decay logits z = W_fb f of the lane's 16 channels (gate projection): four 16 x 16
            // tiles per wave, A = W_fb rows from LDS, B = the f rows of the wave's 16 tokens.
            // Tile m gives A-operand row r the channel 64 half + 16(r/4) + 4m + r%4, so output
            // row 4lg + i is channel cbase + 4m + i and column lr the lane's token: each lane
            // receives exactly its 16 logits.
            float zf[16];
            if constexpr (kGateProj) {
                const int tauc = min(max(tau, t0), t1 - 1);
                bf16x8 fop[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    fop[ks] = *reinterpret_cast<const bf16x8 *>(a.f + (size_t)tauc * kRank + 32 * ks + 8 * lg);
                __builtin_amdgcn_s_waitcnt(0x0070);  // this wave's W_fb rows (and f rows) have landed
                asm volatile("s_barrier" ::: "memory");  // and every other wave's
                const __bf16 *sFb = reinterpret_cast<const __bf16 *>(smem + M.wfb);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int row = 64 * half + 16 * (lr >> 2) + 4 * m + (lr & 3);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const int j = (4 * ks + lg) ^ wfb_swz(row);
                        acc = mma(*reinterpret_cast<const bf16x8 *>(sFb + row * kRank + 8 * j), fop[ks], acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) zf[4 * m + i] = acc[i];
                }
            }
            // decay gate gk (log2 units, see above) and its cumulative sum over the
            // sub-chunk's 16 tokens (= G_t - r_sub)
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                float zz[8], dtb[8];
                if constexpr (kGateProj) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) zz[j] = zf[8 * pc + j];
                } else {
                    unpack8(ld.z[pc], zz);
                }
                lds_read8(sDtb + cbase + 8 * pc, dtb);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(zz[j], zr, dtb[j]));
                    const float g = valid ? gmin2 * __builtin_amdgcn_rcpf(1.0f + e) : 0.f;
                    gs[8 * pc + j] = row_scan16(g);
                }
            }
            // the sub-chunk's totals (the scan's last lane), one masked block of stores
            if (lr == 15) {
                lds_write8(sTot + sub * 128 + cbase, gs);
                lds_write8(sTot + sub * 128 + cbase + 8, gs + 8);
            }
        }
        // kPipe: the previous chunk's record stores were issued a whole phase ago, and no
        // other global access is in flight here: wait for them, so that the barrier orders
        // every wave's stores before the ready word
        if constexpr (kPipe)
            if (c0 > cbeg) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
        if (c0 > cbeg) publish_ready(c0 - kChunk);

        // ---- per-chunk channel tables (threads 0..255), and this lane's operand rows ----
        float qr[16], kr[16], cbk[16];  // q e^{G-r}, k e^{G-r}, k e^{r-G} of the normalised q, k
        {
            int tid = (int)threadIdx.x;
            asm volatile("" : "+v"(tid));
            if (tid < 256) {
                const int c = tid & 127;
                float r[5];
                r[0] = 0.f;
                r[1] = sTot[c];
                r[2] = r[1] + sTot[128 + c];
                r[3] = r[2] + sTot[256 + c];
                r[4] = r[3] + sTot[384 + c];
                if (tid < 128) {
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        sExpRef[I * 128 + c] = __builtin_amdgcn_exp2f(r[I]);
                        sEndRef[I * 128 + c] = __builtin_amdgcn_exp2f(r[4] - r[I]);
                    }
                    sExpEnd[c] = __builtin_amdgcn_exp2f(r[4]);
                } else {
#pragma unroll
                    for (int I = 1; I < 4; ++I)
#pragma unroll
                        for (int J = 0; J < I; ++J)
                            sPair[pair_index(I, J) * 128 + c] = __builtin_amdgcn_exp2f(r[I] - r[J]);
                }
            }
        }
        {
            KDA_LANE_IDS();
            const int cbase = 64 * half + 16 * lg;
            const float ssq = sNorm[t] + sNorm[128 + t];
            const float ssk = sNorm[64 + t] + sNorm[192 + t];
            const float inv_q = qscale / sqrtf(ssq + l2eps);
            const float inv_k = -1.0f / sqrtf(ssk + l2eps);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float rf = __builtin_amdgcn_exp2f(gs[j]);
                const float cf = __builtin_amdgcn_exp2f(-gs[j]);
                const float kh = uk[j] * inv_k;
                qr[j] = uq[j] * inv_q * rf;
                kr[j] = kh * rf;
                cbk[j] = kh * cf;
            }
            lds_write8(sCB + t * CB_LD + cbase, cbk);
            lds_write8(sCB + t * CB_LD + cbase + 8, cbk + 8);
        }
        lds_barrier();

        // ---- rows that need the tables; MFMA operands of block row `sub` ----
        bf16x8 ak[2], aqh[2], aql[2], qe8[2];  // k e^{G-r}, q e^{G-r} (hi/lo), q e^G
        bf16x8 akl[2], qel[2];                   // (kPrecise) lo parts of k e^{G-r} and q e^G
        float ke[16];                            // K_end = k e^{G_end - G}
        {
            KDA_LANE_IDS();
            const int cbase = 64 * half + 16 * lg;
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                float qe[8], bw[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = cbase + 8 * pc + j;
                    const float er = sExpRef[sub * 128 + c];
                    bw[j] = beta * kr[8 * pc + j] * er;
                    qe[j] = qr[8 * pc + j] * er;
                    ke[8 * pc + j] = cbk[8 * pc + j] * sEndRef[sub * 128 + c];
                }
                if constexpr (kPrecise) {
                    bf16x8 bh, bl;
                    split8(bw, bh, bl);
                    *reinterpret_cast<bf16x8 *>(sWr + sw128(t, cbase + 8 * pc)) = bh;
                    *reinterpret_cast<bf16x8 *>(sWrLo + sw128(t, cbase + 8 * pc)) = bl;
                } else {
                    *reinterpret_cast<bf16x8 *>(sWr + sw128(t, cbase + 8 * pc)) = to_bf8(bw);
                }
                if constexpr (kPrecise) {
                    split8(qe, qe8[pc], qel[pc]);
                    split8(kr + 8 * pc, ak[pc], akl[pc]);
                } else {
                    qe8[pc] = to_bf8(qe);
                    ak[pc] = to_bf8(kr + 8 * pc);
                }
                split8(qr + 8 * pc, aqh[pc], aql[pc]);
            }
        }

        // ================= phase 2: block row `sub` of A and P over this channel half =====
        // K-step ks is the lane's piece ks: channels 64 half + 16 lg + 8 ks .. +7 (both
        // operands use the same channel order, so the contraction is over the half).  The
        // channel-half-1 waves park their partial tiles in regions 6-7 (free until phase 3);
        // the half-0 waves add them after the barrier (LDS float atomics are far slower).
        float *sPart = reinterpret_cast<float *>(smem + M.part);  // [10 blocks][A,P][64 lanes][4]
        f32x4 accA[4], accP[4];
        {
            KDA_LANE_IDS();
            const int lane = tid_ & 63;
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                accP[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (J > sub) continue;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int cb0 = 64 * half + 16 * lg + 8 * ks;
                    float col[8];
                    lds_read8(sCB + (16 * J + lr) * CB_LD + cb0, col);
                    if (J < sub) {
                        float pf[8];
                        lds_read8(sPair + pair_index(sub, J) * 128 + cb0, pf);
#pragma unroll
                        for (int j = 0; j < 8; ++j) col[j] *= pf[j];
                    }
                    bf16x8 ch, cl;
                    split8(col, ch, cl);
                    // the transposed tiles: lane (lr, lg) receives the entries (t, s) of
                    // token t = 16 sub + lr and the 4 tokens s = 16J + 4lg + i
                    accA[J] = mma(ch, ak[ks], accA[J]);
                    if constexpr (kPrecise) {
                        accA[J] = mma(ch, akl[ks], accA[J]);
                        accA[J] = mma(cl, ak[ks], accA[J]);
                    }
                    accP[J] = mma(ch, aqh[ks], accP[J]);
                    accP[J] = mma(ch, aql[ks], accP[J]);
                    accP[J] = mma(cl, aqh[ks], accP[J]);
                }
                if (half == 1) {
                    const int bi = sub * (sub + 1) / 2 + J;  // block (sub, J), 0..9
                    *reinterpret_cast<f32x4 *>(sPart + ((bi * 2 + 0) * 64 + lane) * 4) = accA[J];
                    *reinterpret_cast<f32x4 *>(sPart + ((bi * 2 + 1) * 64 + lane) * 4) = accP[J];
                }
            }
        }
        lds_barrier();
        {
            KDA_LANE_IDS();
            const int lane = tid_ & 63;
            if (half == 0) {
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    f32x4 pa = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
                    if (J <= sub) {
                        const int bi = sub * (sub + 1) / 2 + J;
                        pa = accA[J] + *reinterpret_cast<const f32x4 *>(sPart + ((bi * 2 + 0) * 64 + lane) * 4);
                        pp = accP[J] + *reinterpret_cast<const f32x4 *>(sPart + ((bi * 2 + 1) * 64 + lane) * 4);
                    }
                    // row t of A (scaled by beta_t) and of P, columns 16J + 4lg .. +3
                    f32x4 va;
                    bf16x4 ph, pl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int sr = 4 * lg + i;  // column inside the 16x16 block
                        float x = pa[i] * beta;
                        float y = pp[i];
                        if (J == sub) {
                            if (sr >= lr) x = 0.f;
                            if (sr > lr) y = 0.f;
                        }
                        va[i] = x;
                        ph[i] = (__bf16)y;
                        pl[i] = bf16_lo(y, ph[i]);
                    }
                    *reinterpret_cast<f32x4 *>(sA + t * F_LD + 16 * J + 4 * lg) = va;
                    *reinterpret_cast<bf16x4 *>(sPh + sw64(t, 16 * J + 4 * lg)) = ph;
                    *reinterpret_cast<bf16x4 *>(sPl + sw64(t, 16 * J + 4 * lg)) = pl;
                }
            }
            // sCB is dead: K_end^T, hi/lo, into region 1 (channel half 1 now, half 0 in
            // phase 4; the precise mode writes both halves after phase 4)
            if (!kPrecise && half == 1) {
                store_ke(ke, t, 64 * half + 16 * lg);
            }
        }
        lds_barrier();

        // ================= phase 3: T = (I + A)^-1 in fp32 =================
        // diagonal 16x16 blocks: wave 3, lane group lg inverts block lg, lane lr its column lr,
        // by forward substitution in right-looking order (once x[k] is final it is subtracted
        // from every later row, so the updates of one step are independent).  Every block of
        // T is also written as bf16 into sTb for the MFMAs of phase 4; waves 4..7 clear sTb's
        // upper blocks meanwhile.
        {
            KDA_LANE_IDS();
            if (w == 3) {
                const int d = 16 * lg;
                // the block's strictly lower part is read up front (the same 120 values in
                // all 16 lanes of the group), so that no step waits for LDS
                float arow[16][16];
#pragma unroll
                for (int tt = 1; tt < 16; ++tt)
#pragma unroll
                    for (int j = 0; j < tt; ++j) arow[tt][j] = sA[(d + tt) * F_LD + d + j];
                float x[16];
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) x[tt] = (tt == lr) ? 1.0f : 0.0f;
#pragma unroll
                for (int k = 0; k < 15; ++k)
#pragma unroll
                    for (int tt = k + 1; tt < 16; ++tt) x[tt] -= arow[tt][k] * x[k];
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) {
                    sT[(d + tt) * F_LD + d + lr] = x[tt];
                    const __bf16 xh = (__bf16)x[tt];
                    sTb[sw64(d + tt, d + lr)] = xh;
                    if constexpr (kPrecise) sTbLo[sw64(d + tt, d + lr)] = bf16_lo(x[tt], xh);
                }
            } else if (w >= 4) {
                // upper blocks (I < J) of sTb: 6 blocks x 256 values over 256 lanes
                const int lane = tid_ & 255;
#pragma unroll
                for (int b = 0; b < 6; ++b) {
                    const int I = b < 3 ? 0 : (b < 5 ? 1 : 2);
                    const int J = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
                    sTb[sw64(16 * I + (lane >> 4), 16 * J + (lane & 15))] = (__bf16)0.0f;
                    if constexpr (kPrecise) sTbLo[sw64(16 * I + (lane >> 4), 16 * J + (lane & 15))] = (__bf16)0.0f;
                }
            }
            // The next chunk's raw inputs are requested now and in the next phase, to arrive
            // during phases 3-5 (past the last chunk this reloads clamped rows that are never
            // used).  Issuing all eight waves' loads at once held the memory pipe for about
            // 2K cycles and wave 3, issuing after its inverse, waited behind them: part 0
            // here (the other waves while wave 3 inverts), part 1 after the off-diagonal
            // blocks.
            load_chunk<0, kGateProj>(ld, a, tid_, h, t0, t1, c0 + kChunk);
        }
        lds_barrier();
        // off-diagonal blocks, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ: wave J (< 3) walks
        // column J downward (fp32 MFMA, K = 4 per step).  Step kk of a product takes lane
        // group lg's contraction index as 4lg + kk, so the B operand of that step is element
        // kk of the lane's own accumulator tile (rows 4lg + i): the wave's earlier results
        // T_KJ and the sum M feed the next products from registers, and only the rows of
        // A_IK and T_II (16-byte reads) and the diagonal block T_JJ come from LDS.
        {
            KDA_LANE_IDS();
            auto column = [&](auto jc) {
                constexpr int J = decltype(jc)::value;
                f32x4 M[4];  // M[I] = A_IJ T_JJ + sum_K A_IK T_KJ, rows 16I + 4lg + i, column 16J + lr
                float tjj[4];  // T_JJ[4lg + kk][lr]
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) tjj[kk] = sT[(16 * J + 4 * lg + kk) * F_LD + 16 * J + lr];
                // Every M[I] starts at once with its A_IJ T_JJ term, and takes A_IK T_KJ as soon as
                // T_KJ is known; each M[I] still sums its terms in the order K = J, J+1, .., so
                // the bits are those of one block at a time, with the chains of independent
                // blocks interleaved.
#pragma unroll
                for (int I = J + 1; I < 4; ++I) {
                    const f32x4 aj = *reinterpret_cast<const f32x4 *>(sA + (16 * I + lr) * F_LD + 16 * J + 4 * lg);
                    M[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) M[I] = mma_f32(aj[kk], tjj[kk], M[I]);
                }
#pragma unroll
                for (int K = J + 1; K < 4; ++K) {
                    // M[K] is complete: T_KJ = -T_KK M[K]
                    const f32x4 tkk = *reinterpret_cast<const f32x4 *>(sT + (16 * K + lr) * F_LD + 16 * K + 4 * lg);
                    f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) r = mma_f32(-tkk[kk], M[K][kk], r);
#pragma unroll
                    for (int I = K + 1; I < 4; ++I) {
                        const f32x4 ak4 = *reinterpret_cast<const f32x4 *>(sA + (16 * I + lr) * F_LD + 16 * K + 4 * lg);
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) M[I] = mma_f32(ak4[kk], r[kk], M[I]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const __bf16 rh = (__bf16)r[i];
                        sTb[sw64(16 * K + 4 * lg + i, 16 * J + lr)] = rh;
                        if constexpr (kPrecise) sTbLo[sw64(16 * K + 4 * lg + i, 16 * J + lr)] = bf16_lo(r[i], rh);
                    }
                }
            };
            if (w == 0) column(std::integral_constant<int, 0>{});
            else if (w == 1) column(std::integral_constant<int, 1>{});
            else if (w == 2) column(std::integral_constant<int, 2>{});
            load_chunk<1, kGateProj>(ld, a, tid_, h, t0, t1, c0 + kChunk);
        }
        lds_barrier();
        // sT is dead: Q~ = q e^G into region 6 (the precise mode after phase 4)
        if constexpr (!kPrecise) {
            KDA_LANE_IDS();
#pragma unroll
            for (int pc = 0; pc < 2; ++pc)
                *reinterpret_cast<bf16x8 *>(sQe + sw128(t, 64 * half + 16 * lg + 8 * pc)) = qe8[pc];
        }

        // ================= phase 4: W = T (beta k e^G) -> LDS;  U' = T (beta v) -> regs ====
        f32x4 U[2][2];  // [tp][x]: U[token 32tp + 8lg + 4x + i][value 16w + lr]
        {
            KDA_LANE_IDS();
            // K_end^T of channel half 0 (its LDS writes issue beside this phase's MFMAs)
            if (!kPrecise && half == 0) {
                store_ke(ke, t, 16 * lg);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks == 1 && tt < 2) continue;  // T is lower triangular
                    const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sTb + sw64(16 * tt + lr, 32 * ks + 8 * lg));
                    const bf16x8 B8 = lds_tr8(sWr, 32 * ks + 8 * lg, 16 * w + 4 * (lr & 3));
                    acc = mma(B8, A8, acc);  // W^T tile: keys 16w + 4lg + i of token 16tt + lr
                    if constexpr (kPrecise) {
                        const bf16x8 A8l = *reinterpret_cast<const bf16x8 *>(sTbLo + sw64(16 * tt + lr, 32 * ks + 8 * lg));
                        const bf16x8 B8l = lds_tr8(sWrLo, 32 * ks + 8 * lg, 16 * w + 4 * (lr & 3));
                        acc = mma(B8, A8l, acc);
                        acc = mma(B8l, A8, acc);
                    }
                }
                bf16x4 w4, w4l;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    w4[i] = (__bf16)acc[i];
                    if constexpr (kPrecise) w4l[i] = bf16_lo(acc[i], w4[i]);
                }
                *reinterpret_cast<bf16x4 *>(sW + swi128(16 * tt + lr, 16 * w + 4 * lg)) = w4;
                if constexpr (kPrecise) *reinterpret_cast<bf16x4 *>(sWLo + swi128(16 * tt + lr, 16 * w + 4 * lg)) = w4l;
            }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const int trow = 32 * tp + 8 * (lr >> 2) + 4 * x + (lr & 3);
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (ks > tp) continue;
                        const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sTb + sw64(trow, 32 * ks + 8 * lg));
                        const bf16x8 Bh = lds_tr8(sVtHi, 32 * ks + 8 * lg, 16 * w + 4 * (lr & 3));
                        const bf16x8 Bl = lds_tr8(sVtLo, 32 * ks + 8 * lg, 16 * w + 4 * (lr & 3));
                        acc = mma(A8, Bh, acc);
                        acc = mma(A8, Bl, acc);
                        if constexpr (kPrecise) {
                            const bf16x8 A8l = *reinterpret_cast<const bf16x8 *>(sTbLo + sw64(trow, 32 * ks + 8 * lg));
                            acc = mma(A8l, Bh, acc);
                        }
                    }
                    U[tp][x] = acc;
                }
        }
        if constexpr (kGateProj)
            asm volatile("" ::"v"(ld.b));  // (see before the loop)
        else
            asm volatile("" ::"v"(ld.z[0]), "v"(ld.z[1]), "v"(ld.b));
        lds_barrier();
        if constexpr (kPrecise) {
            // beta v and beta k e^G are dead: K_end^T hi/lo and Q~ hi/lo from registers
            KDA_LANE_IDS();
            store_ke(ke, t, 64 * half + 16 * lg);
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                *reinterpret_cast<bf16x8 *>(sQe + sw128(t, 64 * half + 16 * lg + 8 * pc)) = qe8[pc];
                *reinterpret_cast<bf16x8 *>(sQeLo + sw128(t, 64 * half + 16 * lg + 8 * pc)) = qel[pc];
            }
            lds_barrier();
        }

        if constexpr (kChunked) {
            // ================= the chunk record (layout in kda_device.hpp) =================
            KDA_LANE_IDS();
            const int lane = tid_ & 63;
            unsigned char *rec = a.records + ((size_t)(rec0 + c0 / kChunk) * H + h) * R::kBytes;
            // kPipe: device-scope (sc1) stores, written through to where the carries' device-
            // scope loads read them, on any XCD; no cache needs writing back before the ready word
            auto put = [&](int off, const u32x4 &v) {
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, __builtin_amdgcn_make_buffer_rsrc(rec, 0, R::kBytes, kBufferRsrcWord3), off, 0, kCpolSc1);
            };
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int off = R::kU + (((w * 2 + tp) * 2 + x) * 64 + lane) * 16;
                    if constexpr (kPipe)
                        put(off, __builtin_bit_cast(u32x4, U[tp][x]));
                    else
                        *reinterpret_cast<f32x4 *>(rec + off) = U[tp][x];
                }
            // the operand pieces, in the order the carry reads them: piece 8j + w is copied
            // by wave w, lane l taking the 16 bytes lane l of a carry wave reads (source
            // offsets computed once, before the chunk loop)
#pragma unroll
            for (int j = 0; j < kPPW; ++j) {
                const int piece = 8 * j + w;
                if (piece >= R::kPieces) break;  // (uniform)
                u32x4 v;
                if (piece >= R::kK && piece < R::kE) {
                    // K_end^T hi / lo: key rows 32P + 8(lr/4) + 4x + lr%4, tokens 32tp + 8lg ..
                    const int q = piece - R::kK;
                    const int hl = q & 1, tp = (q >> 1) & 1, x = (q >> 2) & 1, P = q >> 3;
                    v = __builtin_bit_cast(u32x4, lds_tr8(hl ? sKeLo : sKeHi, 32 * tp + 8 * lg,
                                                          32 * P + 4 * x + 8 * (lr & 3)));
                } else {
                    const uint32_t off = ((rec_src[j >> 1] >> (16 * (j & 1))) & 0xffffu) << 4;
                    v = *reinterpret_cast<const u32x4 *>(smem + off);
                }
                if (piece == R::kE && lane >= 32) v = u32x4{0u, 0u, 0u, 0u};
                if constexpr (kPipe)
                    put(piece * REC_PIECE + lane * 16, v);
                else
                    *reinterpret_cast<u32x4 *>(rec + piece * REC_PIECE + lane * 16) = v;
            }
            lds_barrier();  // LDS is rewritten by the next chunk
            continue;
        }

        // ================= phase 5: state side and epilogue =================
        // (the epilogue's output-gate logits are loaded now, to arrive during the MFMAs)
        uint2 g4[4];
        size_t lane_off;  // this lane's epilogue offset, for the gate loads and the output stores
        {
            KDA_LANE_IDS();
            lane_off = epi_lane_offset(HD, w, lr, lg);
            load_gate4_off(g4, a.g, HD, h, t0 + c0, L, lane_off, w, lr, lg);
        }
        float *sRms = reinterpret_cast<float *>(smem + M.rms);  // [64][8] (beta v is dead)
        f32x4 o[4];  // o[tt][i] = O[token 16tt + lr][value 16w + 4lg + i]
        {
            KDA_LANE_IDS();
            bf16x8 Sh[4], Sl[4];  // S0 as the B operand of key contractions (hi part; lo: kPrecise)
#pragma unroll
            for (int P = 0; P < 4; ++P) {
                float v8[8] = {S[P][0][0], S[P][0][1], S[P][0][2], S[P][0][3],
                               S[P][1][0], S[P][1][1], S[P][1][2], S[P][1][3]};
                if constexpr (kPrecise)
                    split8(v8, Sh[P], Sl[P]);
                else
                    Sh[P] = to_bf8(v8);
            }
            // U = U' - W S0.  The state-side products issue their MFMAs round-robin over
            // independent accumulators, so that no MFMA waits for the one before it on the
            // same accumulator; each accumulator still takes its terms in the same order.
            {
                f32x4 ws[4] = {};  // [tp][x]
#pragma unroll
                for (int P = 0; P < 4; ++P)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int trow = 32 * (i >> 1) + 8 * (lr >> 2) + 4 * (i & 1) + (lr & 3);
                        const bf16x8 A8 = *reinterpret_cast<const bf16x8 *>(sW + swi128(trow, 32 * P + 8 * lg));
                        ws[i] = mma(A8, Sh[P], ws[i]);
                        if constexpr (kPrecise) {
                            const bf16x8 A8l = *reinterpret_cast<const bf16x8 *>(sWLo + swi128(trow, 32 * P + 8 * lg));
                            ws[i] = mma(A8, Sl[P], ws[i]);
                            ws[i] = mma(A8l, Sh[P], ws[i]);
                        }
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i) U[i >> 1][i & 1] -= ws[i];
            }
            bf16x8 Uh[2], Ul[2];  // [tp]
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                float v8[8] = {U[tp][0][0], U[tp][0][1], U[tp][0][2], U[tp][0][3],
                               U[tp][1][0], U[tp][1][1], U[tp][1][2], U[tp][1][3]};
                split8(v8, Uh[tp], Ul[tp]);
            }
            // O^T = S0^T Q~^T + U^T P^T
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const bf16x8 B8 = *reinterpret_cast<const bf16x8 *>(sQe + sw128(16 * tt + lr, 32 * P + 8 * lg));
                    o[tt] = mma(Sh[P], B8, o[tt]);
                    if constexpr (kPrecise) {
                        const bf16x8 B8l = *reinterpret_cast<const bf16x8 *>(sQeLo + sw128(16 * tt + lr, 32 * P + 8 * lg));
                        o[tt] = mma(Sh[P], B8l, o[tt]);
                        o[tt] = mma(Sl[P], B8, o[tt]);
                    }
                }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {  // P is lower triangular: tt >= 2 tp
                bf16x8 Ph[4], Pl[4];
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) {
                    Ph[tt] = *reinterpret_cast<const bf16x8 *>(sPh + sw64(16 * tt + lr, 32 * tp + 8 * lg));
                    Pl[tt] = *reinterpret_cast<const bf16x8 *>(sPl + sw64(16 * tt + lr, 32 * tp + 8 * lg));
                }
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Uh[tp], Ph[tt], o[tt]);
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Uh[tp], Pl[tt], o[tt]);
#pragma unroll
                for (int tt = 2 * tp; tt < 4; ++tt) o[tt] = mma(Ul[tp], Ph[tt], o[tt]);
            }
            rms_partials(o, sRms, w, lr, lg);
            // S = Diag(e^{G_end}) S0 + K_end^T U, in two groups of four accumulators
#pragma unroll
            for (int P = 0; P < 4; ++P)
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[P][x][i] *= sExpEnd[32 * P + 8 * lg + 4 * x + i];
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    bf16x8 Kh[4], Kl[4];  // accumulators (P, x) = (2g + n / 2, n % 2)
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        const int krow = 32 * (2 * g + (n >> 1)) + 8 * (lr >> 2) + 4 * (n & 1) + (lr & 3);
                        Kh[n] = *reinterpret_cast<const bf16x8 *>(sKeHi + swi64(krow, 32 * tp + 8 * lg));
                        Kl[n] = *reinterpret_cast<const bf16x8 *>(sKeLo + swi64(krow, 32 * tp + 8 * lg));
                    }
#pragma unroll
                    for (int n = 0; n < 4; ++n) S[2 * g + (n >> 1)][n & 1] = mma(Kh[n], Uh[tp], S[2 * g + (n >> 1)][n & 1]);
#pragma unroll
                    for (int n = 0; n < 4; ++n) S[2 * g + (n >> 1)][n & 1] = mma(Kl[n], Uh[tp], S[2 * g + (n >> 1)][n & 1]);
#pragma unroll
                    for (int n = 0; n < 4; ++n) S[2 * g + (n >> 1)][n & 1] = mma(Kh[n], Ul[tp], S[2 * g + (n >> 1)][n & 1]);
                }
        }
        lds_barrier();

        // ================= epilogue: out = sigmoid(g) * RMSNorm(o) =================
        {
            KDA_LANE_IDS();
            float nw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) nw[i] = sNw[16 * w + 4 * lg + i];
            if (a.c.out_bf16)
                gated_rms_store<true, true>(o, g4, sRms, nw, a.c.rms_eps, a.out, HD, h, t0 + c0, L, lane_off, w, lr,
                                            lg);
            else
                gated_rms_store<false, true>(o, g4, sRms, nw, a.c.rms_eps, a.out, HD, h, t0 + c0, L, lane_off, w, lr,
                                             lg);
        }
        lds_barrier();  // LDS is rewritten by the next chunk
    }

    if constexpr (kChunked) {
        // the last chunk's ready word (kPipe); the carry writes the final state and windows
        if constexpr (kPipe) {
            if (cend > cbeg) {
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                lds_barrier();
                publish_ready(cbeg + (cend - cbeg - 1) / kChunk * kChunk);
            }
        }
        return;
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
                for (int i = 0; i < 4; ++i) {
                    const int key = 32 * P + 8 * lg + 4 * x + i;
                    Sf[key * kD + 16 * w + lr] = S[P][x][i];
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

#undef KDA_LANE_IDS

template <bool kChunked, bool kPrecise, bool kGateProj>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
    prefill_body<kChunked, kPrecise, kGateProj>(a, (int)blockIdx.x);
}

// ---- the pipelined chunked plan: chunk workgroups and carries in one launch ----
// Grid indices pipe_first .. pipe_first + pipe_units - 1 are the one-workgroup carries of
// pairs 0 .. B*H - 1 (kda_carry.hpp, following the ready words); the others are the chunk
// workgroups of the segment-major order, the carries' indices skipped.  Workgroups start
// in index order as compute units free up, so the carries start once the first pipe_first
// chunk workgroups are under way and never hold more compute units than the host allows;
// the chunk workgroups never wait, so every record is written whatever the carries do.
// The carry's record buffers take the first 154 KB (high precision: 111 KB) of the same
// dynamic LDS.
template <bool kBf16, bool kPrecise, bool kGateProj>
__global__ __launch_bounds__(kThreads, 1) void prefill_pipe_kernel(PrefillArgs a) {
    static_assert(kThreads == kCarryThreads, "one block size for both roles");
    static_assert(2 * (kLoPieces + kHiPieces) * REC_PIECE <= kLdsBytes, "the carry's buffers");
    static_assert(RecP::kPieces * REC_PIECE + kChunk * 8 * 4 <= kLdsBytes, "the precise carry's buffers");
    extern __shared__ __align__(16) unsigned char smem[];
    const int b = (int)blockIdx.x;
    if (b >= a.pipe_first && b < a.pipe_first + a.pipe_units) {
        const int pair = b - a.pipe_first;
        if constexpr (kPrecise)
            carry_body_precise<kBf16, true>(a, pair / a.c.H, pair % a.c.H, smem,
                                            reinterpret_cast<float *>(smem + RecP::kPieces * REC_PIECE));
        else
            carry_body<kBf16, true>(a, pair / a.c.H, pair % a.c.H, smem, smem + kLoPieces * REC_PIECE,
                                    smem + (kLoPieces + kHiPieces) * REC_PIECE,
                                    smem + (2 * kLoPieces + kHiPieces) * REC_PIECE);
        return;
    }
    prefill_body<true, kPrecise, kGateProj, true>(a, b < a.pipe_first ? b : b - a.pipe_units);
}

// ---- the chunked plan's tables ----
// Sequence s owns record rows chunk_start[s] .. chunk_start[s+1]-1, one per chunk of 64
// tokens (a partial last chunk included), in order, and chunk-kernel segments
// seg_start[s] .. seg_start[s+1]-1 of up to seg_chunks of those rows each.  The running
// record count is capped at nchunk_cap, so no record lies past the workspace even for a
// cu_seqlens that breaks its contract (such a batch then loses its trailing chunks,
// never memory safety); the segment count then stays within nseg_cap.
constexpr int kTableThreads = 256;

// inclusive prefix sum of v over the workgroup's lanes (Hillis-Steele through LDS)
__device__ long long block_scan(long long *part, long long v) {
    const int tid = threadIdx.x;
    part[tid] = v;
    __syncthreads();
    for (int off = 1; off < kTableThreads; off <<= 1) {
        const long long x = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    return part[tid];
}

__global__ __launch_bounds__(kTableThreads) void chunk_table_kernel(PrefillArgs a) {
    __shared__ long long part[kTableThreads];
    __shared__ int seq_first[kTableThreads], seq_nseg[kTableThreads];  // (item table: B <= kTableThreads)
    const int tid = threadIdx.x;
    // the split carry's exchange words start at zero (no tag matches a chunk)
    if (a.xchg) {
        const size_t n = (size_t)a.B * a.c.H * (kSplitXchgBytes / 16);
        uint4 *x = reinterpret_cast<uint4 *>(a.xchg);
        for (size_t i = tid; i < n; i += kTableThreads) x[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    // the pipelined plan's ready words start at zero
    if (a.ready) {
        const size_t n = ((size_t)a.nchunk_cap * a.c.H + 3) / 4;
        uint4 *x = reinterpret_cast<uint4 *>(a.ready);
        for (size_t i = tid; i < n; i += kTableThreads) x[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    const long long cap = a.nchunk_cap;
    long long carry_c = 0, carry_s = 0;  // records and segments of the tiles before
    for (int base = 0; base < a.B; base += kTableThreads) {
        const int s = base + tid;
        long long n = 0;
        if (s < a.B) {
            const int t0 = min(max(a.cu_seqlens[s], 0), a.N);
            const int t1 = min(max(a.cu_seqlens[s + 1], t0), a.N);
            n = (t1 - t0 + kChunk - 1) / kChunk;
        }
        const long long incl = block_scan(part, n);
        const long long tile = part[kTableThreads - 1];
        const long long lo = min(carry_c + incl - n, cap), hi = min(carry_c + incl, cap);
        const long long nseg = (hi - lo + a.seg_chunks - 1) / a.seg_chunks;
        __syncthreads();
        const long long incl_s = block_scan(part, nseg);
        const long long tile_s = part[kTableThreads - 1];
        if (s < a.B) {
            a.chunk_start[s] = (int)lo;
            a.seg_start[s] = (int)(carry_s + incl_s - nseg);
            if (base == 0) {
                seq_first[s] = (int)(carry_s + incl_s - nseg);
                seq_nseg[s] = (int)nseg;
            }
        }
        carry_c += tile;
        carry_s += tile_s;
        __syncthreads();
    }
    if (tid == 0) {
        a.chunk_start[a.B] = (int)min(carry_c, cap);
        a.seg_start[a.B] = (int)carry_s;
    }
    // The pipelined plan over several sequences takes the segments row by row: row j of
    // every sequence (in sequence order) before row j + 1, so that the sequences' records,
    // which their carries read in order, advance together.  item_sg[i] is the segment of
    // row-major position i: segment j of sequence s sits after the sum over sequences t of
    // min(n_t, j) segments of the rows before and after the sequences t < s with n_t > j.
    if (a.item_sg && a.B <= kTableThreads) {
        __syncthreads();
        const int total = (int)carry_s;
        for (int sg = tid; sg < total; sg += kTableThreads) {
            int lo = 0, hi = a.B;  // the sequence owning sg: the last with seq_first <= sg
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (seq_first[mid] <= sg) lo = mid; else hi = mid;
            }
            const int j = sg - seq_first[lo];
            int idx = 0;
            for (int t = 0; t < a.B; ++t) {
                const int n = seq_nseg[t];
                idx += min(n, j) + ((t < lo && n > j) ? 1 : 0);
            }
            a.item_sg[idx] = sg;
        }
    }
}

template <bool kChunked, bool kPrecise, bool kGateProj>
hipError_t launch_prefill_kernel_t(const PrefillArgs &a, size_t blocks, hipStream_t stream) {
    const void *fn = reinterpret_cast<const void *>(&prefill_kernel<kChunked, kPrecise, kGateProj>);
    static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (attr != hipSuccess) return attr;
    dim3 grid((unsigned)blocks), block(kThreads);
    void *args[] = {const_cast<PrefillArgs *>(&a)};
    return hipLaunchKernel(fn, grid, block, args, kLdsBytes, stream);
}

template <bool kChunked>
hipError_t launch_prefill_kernel(const PrefillArgs &a, size_t blocks, hipStream_t stream) {
    const bool gp = a.w_fb != nullptr;
    if (a.c.precise)
        return gp ? launch_prefill_kernel_t<kChunked, true, true>(a, blocks, stream)
                  : launch_prefill_kernel_t<kChunked, true, false>(a, blocks, stream);
    return gp ? launch_prefill_kernel_t<kChunked, false, true>(a, blocks, stream)
              : launch_prefill_kernel_t<kChunked, false, false>(a, blocks, stream);
}

template <bool kBf16, bool kPrecise, bool kGateProj>
hipError_t launch_pipe_t(const PrefillArgs &a, size_t blocks, hipStream_t stream) {
    const void *fn = reinterpret_cast<const void *>(&prefill_pipe_kernel<kBf16, kPrecise, kGateProj>);
    static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (attr != hipSuccess) return attr;
    void *args[] = {const_cast<PrefillArgs *>(&a)};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, kLdsBytes, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (a.path == kPathFused) return launch_prefill_kernel<false>(a, (size_t)a.B * a.c.H, stream);
    void *args[] = {const_cast<PrefillArgs *>(&a)};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&chunk_table_kernel), dim3(1), dim3(kTableThreads),
                                   args, 0, stream);
    if (e != hipSuccess) return e;
    if (a.ready) {
        const bool gp = a.w_fb != nullptr;
        const size_t blocks = (size_t)a.nseg_cap * a.c.H + (size_t)a.pipe_units;
        if (a.c.precise) {
            if (a.c.out_bf16)
                return gp ? launch_pipe_t<true, true, true>(a, blocks, stream)
                          : launch_pipe_t<true, true, false>(a, blocks, stream);
            return gp ? launch_pipe_t<false, true, true>(a, blocks, stream)
                      : launch_pipe_t<false, true, false>(a, blocks, stream);
        }
        if (a.c.out_bf16)
            return gp ? launch_pipe_t<true, false, true>(a, blocks, stream)
                      : launch_pipe_t<true, false, false>(a, blocks, stream);
        return gp ? launch_pipe_t<false, false, true>(a, blocks, stream)
                  : launch_pipe_t<false, false, false>(a, blocks, stream);
    }
    e = launch_prefill_kernel<true>(a, (size_t)a.nseg_cap * a.c.H, stream);
    if (e != hipSuccess) return e;
    return launch_carry(a, stream);
}

}  // namespace kda
