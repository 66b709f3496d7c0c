// kda_internal.hpp -- launch descriptors shared by the entry points (kda_api.hip) and
// the kernels (kda_decode.hip, kda_prefill.hip, kda_carry.hip).  Not part of the public
// ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;     // head dim (key = value = 128)
constexpr int kConv = 4;    // ShortConv taps
constexpr int kChunk = 64;  // prefill chunk length
constexpr int kRank = 128;  // rank of the low-rank decay projection (kda_prefill_gate_proj)

struct MixerConsts {
    int H;
    float gate_lower_bound;
    float l2_eps;
    float rms_eps;
    float q_scale;
    int out_bf16;  // the output buffers hold bf16 (round to nearest even), else fp32
    int precise;   // prefill: every MFMA operand of the chunk algebra split into bf16 hi + lo
    int multi_seq; // decode_multi: token by token (the bits of one-token calls), else blocks
};

// Four consecutive output values at element i (a multiple of 4) of an fp32 or bf16
// output buffer: one 16- or 8-byte store.
__device__ __forceinline__ void store_out4(void *out, size_t i, float a, float b, float c, float d, bool bf16) {
    if (bf16) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        const bf16x4_t v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
        *reinterpret_cast<bf16x4_t *>(static_cast<__bf16 *>(out) + i) = v;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + i) = make_float4(a, b, c, d);
    }
}

struct DecodeArgs {
    MixerConsts c;
    int B;
    const float *q, *k, *v, *z, *b, *g;
    size_t qkv_ld;  // elements between consecutive token rows of q, k, v (>= H*D)
    const float *conv_w, *A_log, *dt_bias, *norm_w;
    float *state, *conv_state;
    void *out;  // fp32 or bf16 (c.out_bf16)
    // NULL: row b owns state[b] and conv_state[b].  Otherwise row b owns pool entry
    // slots[b] of the `pool` entries of state / conv_state (rows outside are skipped).
    const int32_t *slots;
    int pool;
};

// Multi-token decode: up to T tokens per sequence ([B, T, ...] inputs), the state read
// from state_in and written to state_out (which may be the same buffer).
struct DecodeMultiArgs {
    MixerConsts c;
    int B, T;
    const int32_t *n_tokens;  // device [B] tokens to apply per sequence, or null (= T)
    const float *q, *k, *v, *z, *b, *g;
    size_t qkv_ld;  // elements between consecutive token rows of q, k, v (>= H*D)
    const float *conv_w, *A_log, *dt_bias, *norm_w;
    const float *state_in, *conv_in;
    float *state_out, *conv_out;
    void *out;  // fp32 or bf16 (c.out_bf16)
    // NULL: row b owns entry b of the state and window buffers.  Otherwise row b owns
    // pool entry slots[b] of the `pool` entries (rows outside are skipped).
    const int32_t *slots;
    int pool;
};

// Prefill launch plans (kda_config.prefill_path):
//   kPathFused   one workgroup per (sequence, head) walks the sequence chunk by chunk;
//                every intermediate stays on chip
//   kPathChunked a workgroup per (chunk, head) computes each chunk's state-independent
//                products into the workspace (chunk records), then one workgroup per
//                (sequence, head) carries the state across the records
enum PrefillPath { kPathAuto = 0, kPathFused = 1, kPathChunked = 2 };

// Head count and q/k/v row-stride limits: the kernels form in-chunk row offsets
// (up to 67 rows) of H*D and of the row stride in 32 bits.
constexpr int kMaxHeads = 65536;
constexpr int64_t kMaxRowStride = (int64_t)1 << 24;

// Launch-size limits: a dispatch holds fewer than 2^32 work-items per grid dimension.
constexpr int64_t kMaxPrefillUnits = (int64_t)0xFFFFFFFF / 512;  // workgroups of 512 lanes
constexpr int64_t kMaxDecodeUnits = (int64_t)0xFFFFFFFF / 256;   // workgroups of 256 lanes

// The automatic choice between the two prefill plans compares estimates of their times,
// with per-chunk costs measured on MI355X (256 compute units, one 8-wave prefill
// workgroup per compute unit):
//   fused:   rounds * chunks * 17.6 us                 (every workgroup walks its sequence)
//   chunked: records * 17.0 us / 256 + rounds * chunks * 5.9 us
//            (the records spread over all compute units, then the carry walks them)
// where rounds = ceil(B*H / 256) waves of workgroups, chunks = the mean sequence length
// in 64-token chunks and records = (floor(N/64) + B) * H.  (The host does not read
// cu_seqlens, so the lengths are taken as equal.)  The model matches the measured times
// of both plans within about 10% from 1 to 16 sequences of 1K-8K tokens.
constexpr int kComputeUnits = 256;
constexpr double kFusedChunkUs = 17.6;
constexpr double kRecordUs = 17.0;
constexpr double kCarryChunkUs = 5.9;
// the same three costs in the high-precision mode (every operand split into hi + lo;
// measured on 1 x 8192 tokens x 96 heads: fused 2.43 ms, chunk kernel 805 us, carry 1019 us)
constexpr double kFusedChunkUsPrecise = 19.0;
constexpr double kRecordUsPrecise = 18.0;
constexpr double kCarryChunkUsPrecise = 8.0;
// The split carry (kda_carry.hip) runs two 4-wave workgroups per (sequence, head), each on
// its own compute unit and resident together, so it is used for B*H <= 128; its rounds
// term is then 1 and its per-chunk cost kSplitCarryChunkUs.
constexpr int64_t kSplitCarryMaxUnits = kComputeUnits / 2;
constexpr double kSplitCarryChunkUs = 5.2;
// exchange bytes per (sequence, head) of the split carry: 2 halves x 4 slots x 64 x 8
constexpr int64_t kSplitXchgBytes = 2 * 4 * kChunk * 8;

// The pipelined chunked plan (kda_prefill.hip) puts the B*H one-workgroup carries into
// the chunk kernel's grid after its first pipe_first workgroups, so that they start once
// those finish and then follow the records as the rest are written.  It is used for
// B*H <= (compute units) / 2, so that the chunk workgroups keep at least half the compute
// units; with several sequences the chunk workgroups take the segments row by row.  The
// carries should start late enough never to wait: with p the time
// of a chunk-head on one compute unit (kRecordUs), r a carry's time per chunk
// (kPipeCarryChunkUs), I chunk-heads, R chunks per sequence, C compute units and B*H carries,
// the workgroups that start before them cover I - R (r / p) (C - B*H) chunk-heads, the
// work that C - B*H compute units finish while a carry walks its R chunks.  The plan's
// time is then that start plus R r.  Beside the chunk workgroups a carry walks a chunk in
// about 5.0-5.9 us on MI355X (4.9 alone); kPipeCarryChunkUs = 6.4 model microseconds (the
// model's chunk-head takes 17.0 for about 15.7 measured) puts the start where a sweep of
// it was fastest on 1 x 8192 x 96 with the GPU warmed up by ten earlier calls (4.9 to 7.6:
// 6.4 fastest, 5.9 2% slower, 7.2 3% slower): a carry that starts early only waits, one
// that starts late lengthens the call.  The chunk workgroups of this plan take segments of
// kPipeSegChunks chunks: a row of records is complete only when every head's segment is,
// so long segments would make the carries wait for whole rows (measured on 1 x 8192
// tokens x 96 heads: 1.14 ms with 4 or 8 chunks, 1.21 ms with 16).  A carry waits for a
// record at most kReadyMaxPolls polls: the first kReadyShortPolls about a microsecond
// apart, the rest about five (so a few seconds in all, which also covers chunk workgroups
// held off the GPU for a while by other streams' work).
constexpr double kPipeCarryChunkUs = 6.4;
// The high-precision carry walks a chunk in about 11 us beside the chunk workgroups and 8
// alone, slower than the records arrive: its start point comes out at the grid's start
// (on 1 x 8192 x 96, a start after 0, 250 and 1,000 chunk workgroups took 1.44, 1.48 and
// 1.57 ms), and after the last record it walks at kCarryChunkUsPrecise.
constexpr double kPipeCarryChunkUsPrecise = 11.0;
constexpr int kPipeSegChunks = 4;
constexpr int kReadyMaxPolls = 1 << 20;
constexpr int kReadyShortPolls = 1 << 12;
constexpr int64_t kPipeMaxUnits = kComputeUnits / 2;

// Bytes of one chunk record (the layout is in kda_device.hpp); multiples of 256.  The
// high-precision record also holds the lo parts of W and Q~.
constexpr int kRecBytes = 111616;
constexpr int kRecBytesPrecise = 144384;
inline int64_t rec_bytes(bool precise) { return precise ? kRecBytesPrecise : kRecBytes; }

// Chunk records that a batch of B sequences and N tokens can need at most:
// sum_s ceil(len_s / 64) <= floor(N / 64) + B.
inline int64_t chunk_cap(int64_t B, int64_t N) { return N / kChunk + B; }

// The chunk kernel gives each workgroup a segment of up to seg_chunks consecutive chunks
// of one sequence (it loads a chunk's inputs while it finishes the one before).  A batch
// whose sequences hold n_s records in total has at most floor(sum n_s / seg_chunks) + B
// segments.
inline int64_t seg_cap(int64_t B, int64_t nchunk_cap, int seg_chunks) { return nchunk_cap / seg_chunks + B; }

// Segment length: longer segments start fewer workgroups, and a workgroup's first chunk
// costs about a quarter chunk more than the others (nothing overlaps its input loads),
// but a last round of workgroups that fills only part of the compute units wastes the
// rest.  Of 4, 8 and 16 chunks this takes the length whose rounds * (length + 1/4) is
// least, the sequences taken at the batch's mean length (the shorter length on a tie).
// Measured on MI355X with 96 heads: 16 for one 8K sequence, 8 for five of 130-3000
// tokens, 4 for one 2K sequence, each the fastest of the three.
inline int seg_chunks_for(int64_t B, int64_t N, int64_t H) {
    if (B <= 0) return 4;
    const int64_t chunks = (N + kChunk * B - 1) / (kChunk * B);  // mean length, rounded up
    int best = 4;
    double best_t = 0.0;
    for (int s = 4; s <= 16; s *= 2) {
        const int64_t wgs = B * ((chunks + s - 1) / s) * H;
        const double t = (double)((wgs + kComputeUnits - 1) / kComputeUnits) * (s + 0.25);
        if (s == 4 || t < best_t) {
            best = s;
            best_t = t;
        }
    }
    return best;
}

struct PrefillArgs {
    MixerConsts c;
    int B, N;
    int path;            // kPathFused or kPathChunked (resolved)
    int nchunk_cap;      // chunked plan: records available in the workspace
    int nseg_cap;        // chunked plan: chunk-kernel workgroups per head
    int seg_chunks;      // chunked plan: chunks per chunk-kernel segment (4, 8 or 16)
    int32_t *chunk_start;     // chunked plan: [B+1] first record row of each sequence
    int32_t *seg_start;       // chunked plan: [B+1] first segment of each sequence
    unsigned char *records;   // chunked plan: [nchunk_cap][H] records
    // chunked plan with the split carry (two workgroups per (sequence, head), B*H <=
    // kSplitCarryMaxUnits): [B*H][2 halves][4 slots][64 tokens] exchange words of the RMS
    // sums, zeroed by the chunk table kernel; null otherwise
    unsigned long long *xchg;
    int xchg_publish;    // 1; 0 only under kda_test_split_carry (every wait then times out)
    int xchg_max_polls;  // polls per wait, 0 = the kernel's bound
    // chunked plan, pipelined: the chunk kernel's grid also holds the B*H one-workgroup
    // carries (grid indices pipe_first .. pipe_first + pipe_units - 1), which read each
    // record once its word in `ready` ([nchunk_cap][H], zeroed by the chunk table kernel)
    // is set; null and 0 otherwise
    unsigned *ready;
    int32_t *item_sg;  // pipelined, B > 1: [nseg_cap] segments in row-major order; null otherwise
    int pipe_first, pipe_units;
    int ready_publish;    // 1; 0 only under kda_test_pipeline (every wait then times out)
    int ready_max_polls;  // polls per wait, 0 = the kernel's bound
    const int32_t *cu_seqlens;
    const uint16_t *q, *k, *v, *z, *b, *g;
    size_t qkv_ld;  // elements between consecutive token rows of q, k, v (>= H*D)
    // the decay logits from the low-rank projection instead of z (z == nullptr):
    // f [N, kRank] (W_fa x, shared by the heads) and w_fb [H*D, kRank], z = W_fb f
    const uint16_t *f, *w_fb;
    const float *conv_w, *A_log, *dt_bias, *norm_w;
    const float *initial_state, *initial_conv_state;
    void *out;  // fp32 or bf16 (c.out_bf16)
    float *final_state, *final_conv_state;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeMultiArgs &a, hipStream_t stream);
// the token-by-token form (kda_decode_multi_seq.hip)
hipError_t launch_decode_multi_seq(const DecodeMultiArgs &a, hipStream_t stream);
// the whole prefill in the chosen layout (kda_prefill.hip); the chunked layout's last
// launch, the carry, is in kda_carry.hip
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_carry(const PrefillArgs &a, hipStream_t stream);

}  // namespace kda
