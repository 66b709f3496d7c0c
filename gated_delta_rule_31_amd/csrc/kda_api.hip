// kda_api.hip -- the C-ABI entry points of libkda.so: host-side argument checks, then
// the kernel launches on the caller's stream.  Declarations and contracts: include/kda.h.
//
// Every check runs before the first HIP call, so a rejected call touches neither the
// device nor the HIP runtime's error state (and the checks run on a machine without a
// GPU).

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "kda.h"
#include "kda_internal.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A byte range of a buffer the call reads or writes (null or empty: no range).
struct Span {
    const void *p;
    size_t n;
};
bool overlaps(Span a, Span b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + b.n && y < x + a.n;
}
// The byte span of `rows` rows of `width` elements, `ld` elements apart.
Span rows_span(const void *p, int64_t rows, int64_t width, int64_t ld, size_t esize) {
    if (rows <= 0) return {p, 0};
    return {p, ((size_t)(rows - 1) * (size_t)ld + (size_t)width) * esize};
}
// Every output is disjoint from every input and from the other outputs, except that
// output i may coincide exactly with its allowed alias alias[i] (same pointer, same size).
kda_status check_disjoint(const Span *outs, const Span *alias, int n_out, const Span *ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j) {
            const bool exact = alias && alias[i].p && ins[j].p == alias[i].p && outs[i].p == alias[i].p &&
                               outs[i].n == ins[j].n;
            if (!exact && overlaps(outs[i], ins[j])) return KDA_ERR_OVERLAP;
        }
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], outs[j])) return KDA_ERR_OVERLAP;
    }
    return KDA_OK;
}
// qkv_row_stride: 0 selects dense rows (H*D); otherwise >= H*D, a multiple of 8 (16-byte
// rows for bf16 and fp32) and at most kMaxRowStride.
bool resolve_stride(int64_t stride, int H, size_t *ld) {
    const int64_t HD = (int64_t)H * kda::kD;
    if (stride == 0) stride = HD;
    if (stride < HD || stride % 8 != 0 || stride > kda::kMaxRowStride) return false;
    *ld = (size_t)stride;
    return true;
}

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.0f; }

kda_status check_config(const kda_config *cfg, kda::MixerConsts *out) {
    if (!cfg) return KDA_ERR_NULL_ARG;
    if (cfg->num_heads < 1 || cfg->num_heads > kda::kMaxHeads || cfg->head_dim != kda::kD ||
        cfg->conv_size != kda::kConv)
        return KDA_ERR_BAD_CONFIG;
    if (!isfinite(cfg->gate_lower_bound) || !finite_nonneg(cfg->l2_eps) || !finite_nonneg(cfg->rms_eps) ||
        !isfinite(cfg->q_scale))
        return KDA_ERR_BAD_CONFIG;
    if (cfg->out_dtype != KDA_OUT_F32 && cfg->out_dtype != KDA_OUT_BF16) return KDA_ERR_BAD_CONFIG;
    if (cfg->precision != KDA_PRECISION_STANDARD && cfg->precision != KDA_PRECISION_HIGH) return KDA_ERR_BAD_CONFIG;
    if (cfg->decode_multi_form != KDA_MULTI_BLOCK && cfg->decode_multi_form != KDA_MULTI_SEQUENTIAL)
        return KDA_ERR_BAD_CONFIG;
    out->H = cfg->num_heads;
    out->gate_lower_bound = cfg->gate_lower_bound;
    out->l2_eps = cfg->l2_eps;
    out->rms_eps = cfg->rms_eps;
    out->q_scale = cfg->q_scale > 0.0f ? cfg->q_scale : 1.0f / sqrtf((float)kda::kD);
    out->out_bf16 = cfg->out_dtype == KDA_OUT_BF16;
    out->precise = cfg->precision == KDA_PRECISION_HIGH;
    out->multi_seq = cfg->decode_multi_form == KDA_MULTI_SEQUENTIAL;
    return KDA_OK;
}

// [B*H] units must fit the 1-D grid; [B or N, H*D] extents must fit size_t arithmetic.
bool units_fit(int64_t rows, int64_t H, int64_t max_units) { return rows >= 0 && rows * H <= max_units; }

// The prefill layout for these sizes, and the workspace it needs; false for sizes
// kda_prefill rejects.
struct PrefillPlan {
    int path;
    int64_t nchunk_cap, nseg_cap;
    int seg_chunks;
    bool carry_split;  // chunked: the two-workgroup carry (standard precision, B*H <= 128)
    bool pipe;         // chunked: the carries in the chunk kernel's launch
    size_t ready_off;  // pipe: byte offset of the ready words in the workspace
    size_t items_off;  // pipe with B > 1: byte offset of the row-major segment order
    size_t table_bytes, workspace_bytes;
};

// kda_test_pipeline's settings, read by every prefill call: mode 0 = the plan's choice,
// 1 = never pipelined, 2 = pipelined wherever it can be
std::atomic<int32_t> pipe_mode{0};
std::atomic<int32_t> pipe_publish{1};
std::atomic<int32_t> pipe_max_polls{0};

// The time model of the pipelined plan (kda_internal.hpp): its time and the number of
// chunk-heads whose workgroups start before the carries, for I chunk-heads, R chunks per
// sequence, C compute units and NC carries, in the standard or high-precision mode.
struct PipeModel {
    double us, lead_chunk_heads;
};
PipeModel pipe_model(double I, double R, double C, double NC, bool precise) {
    const double p = precise ? kda::kRecordUsPrecise : kda::kRecordUs;
    const double r = precise ? kda::kPipeCarryChunkUsPrecise : kda::kPipeCarryChunkUs;
    const double r_alone = precise ? kda::kCarryChunkUsPrecise : kda::kCarryChunkUs;
    const double lead = std::max(0.0, I - R * (r / p) * (C - NC));
    const double start = lead * p / C;
    const double rest = (I - lead) * p / (C - NC);  // chunk-heads after the carries start
    // (with lead > 0, R r = rest; with lead = 0 the carries walk rest / r chunks beside the
    // chunk workgroups and the others alone)
    const double carry = R * r <= rest ? rest : rest + (R - rest / r) * r_alone;
    return {start + carry, lead};
}
// max_workspace >= 0: the workspace is a fixed array of that many bytes; the automatic
// choice then takes the chunked layout only if its workspace fits (else fused, which
// needs none).
bool plan_prefill(const kda_config *cfg, int64_t B, int64_t N, PrefillPlan *plan, int64_t max_workspace = -1) {
    const int64_t H = cfg->num_heads;
    if (B < 0 || N < 0 || N > INT32_MAX || !units_fit(B, H, kda::kMaxPrefillUnits)) return false;
    const int64_t cap = kda::chunk_cap(B, N);
    const int seg_chunks = kda::seg_chunks_for(B, N, H);
    const int64_t segs = kda::seg_cap(B, cap, seg_chunks);
    const bool chunked_fits = cap * H <= kda::kMaxPrefillUnits && segs * H <= kda::kMaxPrefillUnits;
    const bool precise = cfg->precision == KDA_PRECISION_HIGH;
    const bool split_ok = !precise && B * H <= kda::kSplitCarryMaxUnits;
    const double rounds = (double)((B * H + kda::kComputeUnits - 1) / kda::kComputeUnits);
    const double chunks = B > 0 ? (double)((N + 64 * B - 1) / (64 * B)) : 0.0;  // mean length, rounded up
    const double records_us =
        (double)cap * (double)H * (precise ? kda::kRecordUsPrecise : kda::kRecordUs) / kda::kComputeUnits;
    const double serial_us =
        records_us + (split_ok ? chunks * kda::kSplitCarryChunkUs
                               : rounds * chunks * (precise ? kda::kCarryChunkUsPrecise : kda::kCarryChunkUs));
    // the pipelined plan: B*H <= 128 (at most half the compute units for the carries);
    // taken where its model beats the serial one (mode 0)
    const int32_t mode = pipe_mode.load();
    const int64_t pipe_segs = kda::seg_cap(B, cap, kda::kPipeSegChunks);
    bool pipe = mode != 1 && B >= 1 && B * H <= kda::kPipeMaxUnits && N > 0 && chunked_fits &&
                pipe_segs * H + B * H <= kda::kMaxPrefillUnits;
    if (pipe && mode == 0)
        pipe = pipe_model((double)cap * (double)H, chunks, kda::kComputeUnits, (double)(B * H), precise).us <
               serial_us;
    const bool split = split_ok && !pipe;
    // chunk_start and seg_start, then the RMS-sum exchange words (split carry) or the
    // records' ready words (pipelined)
    const size_t base_bytes = (size_t)((8 * (B + 1) + 255) / 256 * 256);
    const size_t ready_bytes = pipe ? (size_t)((cap * H * 4 + 255) / 256 * 256) : 0;
    const size_t items_bytes = pipe && B > 1 ? (size_t)((pipe_segs * 4 + 255) / 256 * 256) : 0;
    const size_t table_bytes =
        base_bytes + (split ? (size_t)(B * H * kda::kSplitXchgBytes) : 0) + ready_bytes + items_bytes;
    const size_t chunked_bytes = table_bytes + (size_t)cap * (size_t)H * (size_t)kda::rec_bytes(precise);
    int path = cfg->prefill_path;
    if (path == kda::kPathAuto) {
        path = kda::kPathFused;
        if (chunked_fits && B > 0) {
            const double fused = rounds * chunks * (precise ? kda::kFusedChunkUsPrecise : kda::kFusedChunkUs);
            const double chunked =
                pipe ? pipe_model((double)cap * (double)H, chunks, kda::kComputeUnits, (double)(B * H), precise).us
                     : serial_us;
            if (chunked < fused && (max_workspace < 0 || chunked_bytes <= (size_t)max_workspace))
                path = kda::kPathChunked;
        }
    }
    if (path != kda::kPathFused && path != kda::kPathChunked) return false;
    if (path == kda::kPathChunked && !chunked_fits) return false;
    plan->path = path;
    plan->nchunk_cap = cap;
    plan->nseg_cap = pipe ? pipe_segs : segs;
    plan->seg_chunks = pipe ? kda::kPipeSegChunks : seg_chunks;
    plan->carry_split = path == kda::kPathChunked && split;
    plan->pipe = path == kda::kPathChunked && pipe;
    plan->ready_off = base_bytes;
    plan->items_off = base_bytes + ready_bytes;
    plan->table_bytes = table_bytes;
    plan->workspace_bytes = path == kda::kPathFused ? 0 : chunked_bytes;
    return true;
}

// The byte spans of the fp32 per-token inputs and parameters of a decode call over `rows`
// token rows (q, k, v strided), in the order q, k, v, z, b, g, conv_w, A_log, dt_bias,
// norm_w.
void decode_input_spans(Span *sp, int64_t rows, int H, size_t ld, const float *q, const float *k, const float *v,
                        const float *z, const float *b, const float *g, const float *conv_w, const float *A_log,
                        const float *dt_bias, const float *norm_w) {
    const int64_t HD = (int64_t)H * kda::kD;
    sp[0] = rows_span(q, rows, HD, ld, 4);
    sp[1] = rows_span(k, rows, HD, ld, 4);
    sp[2] = rows_span(v, rows, HD, ld, 4);
    sp[3] = rows_span(z, rows, HD, HD, 4);
    sp[4] = rows_span(b, rows, H, H, 4);
    sp[5] = rows_span(g, rows, HD, HD, 4);
    sp[6] = {conv_w, (size_t)3 * HD * kda::kConv * 4};
    sp[7] = {A_log, (size_t)H * 4};
    sp[8] = {dt_bias, (size_t)HD * 4};
    sp[9] = {norm_w, (size_t)kda::kD * 4};
}

// kda_decode_step and (pooled) kda_decode_step_slots
kda_status decode_one(const kda_config *cfg, int32_t batch, const int32_t *slots, int32_t pool_size, bool pooled,
                      const float *q, const float *k, const float *v, int64_t qkv_row_stride, const float *z,
                      const float *b, const float *g, const float *conv_w, const float *A_log, const float *dt_bias,
                      const float *norm_w, float *state, float *conv_state, void *out, void *stream) {
    kda::DecodeArgs a;
    kda_status st = check_config(cfg, &a.c);
    if (st != KDA_OK) return st;
    if (batch < 0 || pool_size < 0 || !units_fit(batch, a.c.H, kda::kMaxDecodeUnits)) return KDA_ERR_BAD_SHAPE;
    if (!resolve_stride(qkv_row_stride, a.c.H, &a.qkv_ld)) return KDA_ERR_BAD_SHAPE;
    if (batch == 0 || (pooled && pool_size == 0)) return KDA_OK;  // nothing to do / every row skipped
    const void *ptrs[] = {q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state, conv_state, out};
    if (pooled && !slots) return KDA_ERR_NULL_ARG;
    for (const void *p : ptrs)
        if (!p) return KDA_ERR_NULL_ARG;
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_MISALIGNED;
    if (pooled && (reinterpret_cast<uintptr_t>(slots) & 3u) != 0) return KDA_ERR_MISALIGNED;
    const int64_t HD = (int64_t)a.c.H * kda::kD;
    const int64_t entries = pooled ? pool_size : batch;
    Span ins[11];
    decode_input_spans(ins, batch, a.c.H, a.qkv_ld, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w);
    ins[10] = {slots, pooled ? (size_t)batch * 4 : 0};
    const Span outs[3] = {{state, (size_t)entries * HD * kda::kD * 4},
                          {conv_state, (size_t)entries * 3 * HD * (kda::kConv - 1) * 4},
                          {out, (size_t)batch * HD * (a.c.out_bf16 ? 2 : 4)}};
    if ((st = check_disjoint(outs, nullptr, 3, ins, 11)) != KDA_OK) return st;
    a.B = batch;
    a.q = q; a.k = k; a.v = v; a.z = z; a.b = b; a.g = g;
    a.conv_w = conv_w; a.A_log = A_log; a.dt_bias = dt_bias; a.norm_w = norm_w;
    a.state = state; a.conv_state = conv_state; a.out = out;
    a.slots = pooled ? slots : nullptr;
    a.pool = pooled ? pool_size : 0;
    return kda::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {


kda_config kda_config_default(void) {
    kda_config c;
    c.num_heads = 96;
    c.head_dim = 128;
    c.conv_size = 4;
    c.gate_lower_bound = -5.0f;
    c.l2_eps = 1e-6f;
    c.rms_eps = 1e-5f;
    c.q_scale = 0.0f;
    c.prefill_path = KDA_PREFILL_AUTO;
    c.out_dtype = KDA_OUT_F32;
    c.precision = KDA_PRECISION_STANDARD;
    c.decode_multi_form = KDA_MULTI_BLOCK;
    return c;
}

kda_status kda_decode_step(const kda_config *cfg, int32_t batch, const float *q, const float *k,
                           const float *v, int64_t qkv_row_stride, const float *z, const float *b, const float *g,
                           const float *conv_w, const float *A_log, const float *dt_bias,
                           const float *norm_w, float *state, float *conv_state, void *out,
                           void *stream) {
    return decode_one(cfg, batch, nullptr, 0, false, q, k, v, qkv_row_stride, z, b, g, conv_w, A_log, dt_bias, norm_w,
                      state, conv_state, out, stream);
}

kda_status kda_decode_step_slots(const kda_config *cfg, int32_t batch, const int32_t *slots, int32_t pool_size,
                                 const float *q, const float *k, const float *v, int64_t qkv_row_stride,
                                 const float *z, const float *b, const float *g, const float *conv_w,
                                 const float *A_log, const float *dt_bias, const float *norm_w, float *state_pool,
                                 float *conv_pool, void *out, void *stream) {
    return decode_one(cfg, batch, slots, pool_size, true, q, k, v, qkv_row_stride, z, b, g, conv_w, A_log, dt_bias,
                      norm_w, state_pool, conv_pool, out, stream);
}

}  // extern "C"

namespace {

// pooled: the slot-indexed form (slots required)
kda_status decode_multi(const kda_config *cfg, int32_t batch, int32_t tokens, const int32_t *n_tokens,
                        bool pooled, const int32_t *slots, int32_t pool_size, const float *q, const float *k, const float *v,
                        int64_t qkv_row_stride, const float *z, const float *b, const float *g, const float *conv_w, const float *A_log,
                        const float *dt_bias, const float *norm_w, const float *state_in, float *state_out,
                        const float *conv_state_in, float *conv_state_out, void *out, void *stream) {
    kda::DecodeMultiArgs a;
    kda_status st = check_config(cfg, &a.c);
    if (st != KDA_OK) return st;
    if (batch < 0 || tokens < 0 || pool_size < 0 || !units_fit(batch, a.c.H, kda::kMaxDecodeUnits) ||
        !units_fit(batch, tokens, INT32_MAX))
        return KDA_ERR_BAD_SHAPE;
    if (!resolve_stride(qkv_row_stride, a.c.H, &a.qkv_ld)) return KDA_ERR_BAD_SHAPE;
    if (batch == 0) return KDA_OK;
    if (tokens == 0) return KDA_ERR_BAD_SHAPE;
    if (pooled && !slots) return KDA_ERR_NULL_ARG;
    if (pooled && pool_size == 0) return KDA_OK;  // every row would be skipped
    const void *ptrs[] = {q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w,
                          state_in, state_out, conv_state_in, conv_state_out, out};
    for (const void *p : ptrs)
        if (!p) return KDA_ERR_NULL_ARG;
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(n_tokens) & 3u) != 0 || (reinterpret_cast<uintptr_t>(slots) & 3u) != 0)
        return KDA_ERR_MISALIGNED;
    {
        const int64_t HD = (int64_t)a.c.H * kda::kD;
        const int64_t entries = pooled ? pool_size : batch;
        const size_t sbytes = (size_t)entries * HD * kda::kD * 4;
        const size_t cbytes = (size_t)entries * 3 * HD * (kda::kConv - 1) * 4;
        Span ins[14];
        decode_input_spans(ins, (int64_t)batch * tokens, a.c.H, a.qkv_ld, q, k, v, z, b, g, conv_w, A_log, dt_bias,
                           norm_w);
        ins[10] = {state_in, sbytes};
        ins[11] = {conv_state_in, cbytes};
        ins[12] = {n_tokens, n_tokens ? (size_t)batch * 4 : 0};
        ins[13] = {pooled ? slots : nullptr, pooled ? (size_t)batch * 4 : 0};
        const Span outs[3] = {{state_out, sbytes}, {conv_state_out, cbytes},
                              {out, (size_t)batch * tokens * HD * (a.c.out_bf16 ? 2 : 4)}};
        const Span alias[3] = {{state_in, sbytes}, {conv_state_in, cbytes}, {nullptr, 0}};
        if ((st = check_disjoint(outs, alias, 3, ins, 14)) != KDA_OK) return st;
    }
    a.B = batch;
    a.T = tokens;
    a.n_tokens = n_tokens;
    a.q = q; a.k = k; a.v = v; a.z = z; a.b = b; a.g = g;
    a.conv_w = conv_w; a.A_log = A_log; a.dt_bias = dt_bias; a.norm_w = norm_w;
    a.state_in = state_in; a.state_out = state_out;
    a.conv_in = conv_state_in; a.conv_out = conv_state_out;
    a.out = out;
    a.slots = pooled ? slots : nullptr;
    a.pool = pool_size;
    const hipError_t e = a.c.multi_seq ? kda::launch_decode_multi_seq(a, static_cast<hipStream_t>(stream))
                                       : kda::launch_decode_multi(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// ---- the scratch array of kda_prefill_noalloc ----
// The chunked layout's workspace (chunk table and records) for callers that cannot
// allocate: a fixed array in device memory, one per device the library runs on, held
// until the process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, looked up once per device (with that device
// current) and kept.  Every call on a device uses that device's array, and nothing in
// it has to start at any value (each call writes its table and records before reading
// them), so it is never cleared.
constexpr size_t kScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

kda_status device_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_LAUNCH;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return KDA_OK;
}

// The current device's compute units, looked up once per device.  The two-workgroup
// carry needs every workgroup pair resident together, so it runs only where the device
// has a compute unit for each of its workgroups (one per compute unit by LDS); a device
// that shows fewer (a partition of the GPU, say) takes the one-workgroup carry instead.
std::mutex cu_mu;
int cu_count[kMaxDevices] = {};

int device_compute_units() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lock(cu_mu);
    if (!cu_count[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        cu_count[dev] = n;
    }
    return cu_count[dev];
}

// kda_prefill, and (static_scratch) kda_prefill_noalloc: the workspace is then this
// device's scratch array, looked up after every argument check has passed
// kda_test_split_carry's settings, read by every prefill call
std::atomic<int32_t> split_publish{1};
std::atomic<int32_t> split_max_polls{0};

kda_status prefill_impl(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens, const int32_t *cu_seqlens,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t qkv_row_stride,
                        const uint16_t *z, const uint16_t *b, const uint16_t *g, const float *conv_w,
                        const float *A_log, const float *dt_bias, const float *norm_w, const float *initial_state,
                        const float *initial_conv_state, void *out, float *final_state, float *final_conv_state,
                        void *workspace, size_t workspace_bytes, bool static_scratch, void *stream,
                        bool gate_proj = false, const uint16_t *f = nullptr, const uint16_t *w_fb = nullptr) {
    kda::PrefillArgs a = {};
    kda_status st = check_config(cfg, &a.c);
    if (st != KDA_OK) return st;
    if (cfg->prefill_path < kda::kPathAuto || cfg->prefill_path > kda::kPathChunked) return KDA_ERR_BAD_CONFIG;
    PrefillPlan plan;
    if (!plan_prefill(cfg, num_seqs, total_tokens, &plan, static_scratch ? (int64_t)kScratchBytes : -1))
        return KDA_ERR_BAD_SHAPE;
    if (!resolve_stride(qkv_row_stride, a.c.H, &a.qkv_ld)) return KDA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return total_tokens == 0 ? KDA_OK : KDA_ERR_BAD_SHAPE;
    const void *req[] = {cu_seqlens, conv_w, A_log, dt_bias, norm_w, final_state, final_conv_state};
    for (const void *p : req)
        if (!p) return KDA_ERR_NULL_ARG;
    if (gate_proj && !w_fb) return KDA_ERR_NULL_ARG;
    if (total_tokens > 0) {
        const void *tok[] = {q, k, v, gate_proj ? f : z, b, g, out};
        for (const void *p : tok)
            if (!p) return KDA_ERR_NULL_ARG;
        for (const void *p : tok)
            if (!aligned16(p)) return KDA_ERR_MISALIGNED;
    }
    if (gate_proj && !aligned16(w_fb)) return KDA_ERR_MISALIGNED;
    const void *al[] = {conv_w, A_log, dt_bias, norm_w, final_state, final_conv_state, initial_state,
                        initial_conv_state};
    for (const void *p : al)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_MISALIGNED;
    if (static_scratch) {
        if (plan.workspace_bytes > kScratchBytes) return KDA_ERR_WORKSPACE;  // explicit chunked layout
    } else {
        if (workspace_bytes < plan.workspace_bytes || (plan.workspace_bytes > 0 && !workspace))
            return KDA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_MISALIGNED;
    }
    {
        const int64_t H = a.c.H, HD = H * kda::kD, N = total_tokens, B = num_seqs;
        const size_t sbytes = (size_t)B * HD * kda::kD * 4;
        const size_t cbytes = (size_t)B * 3 * HD * (kda::kConv - 1) * 4;
        const Span ins[14] = {{cu_seqlens, (size_t)(B + 1) * 4},
                              rows_span(q, N, HD, a.qkv_ld, 2), rows_span(k, N, HD, a.qkv_ld, 2),
                              rows_span(v, N, HD, a.qkv_ld, 2),
                              gate_proj ? rows_span(f, N, kda::kRank, kda::kRank, 2) : rows_span(z, N, HD, HD, 2),
                              rows_span(b, N, H, H, 2), rows_span(g, N, HD, HD, 2),
                              {conv_w, (size_t)3 * HD * kda::kConv * 4}, {A_log, (size_t)H * 4},
                              {dt_bias, (size_t)HD * 4}, {norm_w, (size_t)kda::kD * 4},
                              {initial_state, initial_state ? sbytes : 0},
                              {initial_conv_state, initial_conv_state ? cbytes : 0},
                              {w_fb, gate_proj ? (size_t)HD * kda::kRank * 2 : 0}};
        const Span outs[4] = {{out, (size_t)N * HD * (a.c.out_bf16 ? 2 : 4)}, {final_state, sbytes},
                              {final_conv_state, cbytes}, {workspace, plan.workspace_bytes}};
        const Span alias[4] = {{nullptr, 0}, {initial_state, sbytes}, {initial_conv_state, cbytes}, {nullptr, 0}};
        if ((st = check_disjoint(outs, alias, 4, ins, 14)) != KDA_OK) return st;
    }
    if (static_scratch && plan.workspace_bytes > 0 && (st = device_scratch(&workspace)) != KDA_OK) return st;
    a.B = num_seqs;
    a.N = total_tokens;
    a.path = plan.path;
    a.nchunk_cap = (int)plan.nchunk_cap;
    a.nseg_cap = (int)plan.nseg_cap;
    a.seg_chunks = plan.seg_chunks;
    const bool chunked = plan.path == kda::kPathChunked;
    a.chunk_start = chunked ? static_cast<int32_t *>(workspace) : nullptr;
    a.seg_start = chunked ? static_cast<int32_t *>(workspace) + (num_seqs + 1) : nullptr;
    a.records = chunked ? static_cast<unsigned char *>(workspace) + plan.table_bytes : nullptr;
    // (the workspace keeps the exchange area either way; an unused one costs nothing)
    const bool split = plan.carry_split && 2 * (int64_t)num_seqs * cfg->num_heads <= device_compute_units();
    a.xchg = split ? reinterpret_cast<unsigned long long *>(static_cast<unsigned char *>(workspace) +
                                                            (8 * (num_seqs + 1) + 255) / 256 * 256)
                   : nullptr;
    a.xchg_publish = split_publish.load();
    a.xchg_max_polls = split_max_polls.load();
    // the pipelined plan, where the device keeps at least half its compute units for the
    // chunk workgroups (else the serial one-workgroup carry on the same workspace)
    const int cus = device_compute_units();
    const int64_t pairs = (int64_t)num_seqs * cfg->num_heads;
    const bool pipe = plan.pipe && 2 * pairs <= cus;
    a.ready = pipe ? reinterpret_cast<unsigned *>(static_cast<unsigned char *>(workspace) + plan.ready_off) : nullptr;
    a.item_sg = pipe && num_seqs > 1
                    ? reinterpret_cast<int32_t *>(static_cast<unsigned char *>(workspace) + plan.items_off)
                    : nullptr;
    a.pipe_units = pipe ? (int)pairs : 0;
    a.pipe_first = 0;
    if (pipe) {
        // (the sequences taken as equal in length, as in the plan)
        const double chunks = (double)((total_tokens + kda::kChunk * num_seqs - 1) / (kda::kChunk * num_seqs));
        const double lead =
            pipe_model((double)plan.nchunk_cap * cfg->num_heads, chunks, cus, (double)pairs, cfg->precision == KDA_PRECISION_HIGH)
                .lead_chunk_heads;
        a.pipe_first = (int)std::min((double)plan.nseg_cap * cfg->num_heads, std::floor(lead / plan.seg_chunks));
    }
    a.ready_publish = pipe_publish.load();
    a.ready_max_polls = pipe_max_polls.load();
    a.cu_seqlens = cu_seqlens;
    a.q = q; a.k = k; a.v = v; a.z = gate_proj ? nullptr : z; a.b = b; a.g = g;
    a.f = gate_proj ? f : nullptr;
    a.w_fb = gate_proj ? w_fb : nullptr;
    a.conv_w = conv_w; a.A_log = A_log; a.dt_bias = dt_bias; a.norm_w = norm_w;
    a.initial_state = initial_state;
    a.initial_conv_state = initial_conv_state;
    a.out = out;
    a.final_state = final_state;
    a.final_conv_state = final_conv_state;
    return kda::launch_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status kda_decode_multi(const kda_config *cfg, int32_t batch, int32_t tokens, const int32_t *n_tokens,
                            const float *q, const float *k, const float *v, int64_t qkv_row_stride,
                            const float *z, const float *b,
                            const float *g, const float *conv_w, const float *A_log, const float *dt_bias,
                            const float *norm_w, const float *state_in, float *state_out,
                            const float *conv_state_in, float *conv_state_out, void *out, void *stream) {
    return decode_multi(cfg, batch, tokens, n_tokens, false, nullptr, 0, q, k, v, qkv_row_stride, z, b, g, conv_w, A_log,
                        dt_bias, norm_w,
                        state_in, state_out, conv_state_in, conv_state_out, out, stream);
}

kda_status kda_decode_multi_slots(const kda_config *cfg, int32_t batch, int32_t tokens, const int32_t *n_tokens,
                                  const int32_t *slots, int32_t pool_size, const float *q, const float *k,
                                  const float *v, int64_t qkv_row_stride, const float *z, const float *b,
                                  const float *g,
                                  const float *conv_w, const float *A_log, const float *dt_bias,
                                  const float *norm_w, const float *state_in, float *state_out,
                                  const float *conv_state_in, float *conv_state_out, void *out, void *stream) {
    return decode_multi(cfg, batch, tokens, n_tokens, true, slots, pool_size, q, k, v, qkv_row_stride, z, b, g, conv_w,
                        A_log, dt_bias,
                        norm_w, state_in, state_out, conv_state_in, conv_state_out, out, stream);
}

size_t kda_prefill_workspace_bytes(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens) {
    kda::MixerConsts c;
    PrefillPlan plan;
    if (check_config(cfg, &c) != KDA_OK || !plan_prefill(cfg, num_seqs, total_tokens, &plan)) return 0;
    return plan.workspace_bytes;
}

kda_status kda_prefill(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                       const int32_t *cu_seqlens, const uint16_t *q, const uint16_t *k,
                       const uint16_t *v, int64_t qkv_row_stride, const uint16_t *z, const uint16_t *b,
                       const uint16_t *g,
                       const float *conv_w, const float *A_log, const float *dt_bias, const float *norm_w,
                       const float *initial_state, const float *initial_conv_state, void *out,
                       float *final_state, float *final_conv_state, void *workspace,
                       size_t workspace_bytes, void *stream) {
    return prefill_impl(cfg, num_seqs, total_tokens, cu_seqlens, q, k, v, qkv_row_stride, z, b, g, conv_w, A_log,
                        dt_bias, norm_w, initial_state, initial_conv_state, out, final_state, final_conv_state,
                        workspace, workspace_bytes, false, stream);
}

kda_status kda_prefill_gate_proj(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                                 const int32_t *cu_seqlens, const uint16_t *q, const uint16_t *k,
                                 const uint16_t *v, int64_t qkv_row_stride, const uint16_t *f, const uint16_t *w_fb,
                                 const uint16_t *b, const uint16_t *g, const float *conv_w, const float *A_log,
                                 const float *dt_bias, const float *norm_w, const float *initial_state,
                                 const float *initial_conv_state, void *out, float *final_state,
                                 float *final_conv_state, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(cfg, num_seqs, total_tokens, cu_seqlens, q, k, v, qkv_row_stride, nullptr, b, g, conv_w,
                        A_log, dt_bias, norm_w, initial_state, initial_conv_state, out, final_state, final_conv_state,
                        workspace, workspace_bytes, false, stream, true, f, w_fb);
}

kda_status kda_prefill_noalloc(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                               const int32_t *cu_seqlens, const uint16_t *q, const uint16_t *k,
                               const uint16_t *v, int64_t qkv_row_stride, const uint16_t *z, const uint16_t *b,
                               const uint16_t *g, const float *conv_w, const float *A_log, const float *dt_bias,
                               const float *norm_w, const float *initial_state, const float *initial_conv_state,
                               void *out, float *final_state, float *final_conv_state, void *stream) {
    return prefill_impl(cfg, num_seqs, total_tokens, cu_seqlens, q, k, v, qkv_row_stride, z, b, g, conv_w, A_log,
                        dt_bias, norm_w, initial_state, initial_conv_state, out, final_state, final_conv_state,
                        nullptr, 0, true, stream);
}

kda_status kda_state_copy(const kda_config *cfg, int32_t n, const float *src_state, const float *src_conv,
                          int32_t src_entries, const int32_t *src_slots, float *dst_state, float *dst_conv,
                          int32_t dst_entries, const int32_t *dst_slots, void *stream) {
    kda::MixerConsts c;
    kda_status st = check_config(cfg, &c);
    if (st != KDA_OK) return st;
    if (n < 0 || src_entries < 0 || dst_entries < 0) return KDA_ERR_BAD_SHAPE;
    if (n == 0) return KDA_OK;
    const void *ptrs[] = {src_state, src_conv, dst_state, dst_conv};
    if (!src_slots || !dst_slots) return KDA_ERR_NULL_ARG;
    for (const void *p : ptrs)
        if (!p) return KDA_ERR_NULL_ARG;
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_MISALIGNED;
    for (int32_t i = 0; i < n; ++i)
        if (src_slots[i] < 0 || src_slots[i] >= src_entries || dst_slots[i] < 0 || dst_slots[i] >= dst_entries)
            return KDA_ERR_BAD_SHAPE;
    const size_t state_bytes = (size_t)c.H * kda::kD * kda::kD * sizeof(float);
    const size_t conv_bytes = (size_t)3 * c.H * kda::kD * (kda::kConv - 1) * sizeof(float);
    // a source buffer and the destination buffer of the same kind are the same one or
    // disjoint; a state buffer and a conv buffer are always disjoint
    auto disjoint = [](const void *s, size_t sn, const void *d, size_t dn) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(s), b = reinterpret_cast<uintptr_t>(d);
        return a + sn <= b || b + dn <= a;
    };
    const size_t ss_n = state_bytes * src_entries, sc_n = conv_bytes * src_entries;
    const size_t ds_n = state_bytes * dst_entries, dc_n = conv_bytes * dst_entries;
    if ((src_state != dst_state && !disjoint(src_state, ss_n, dst_state, ds_n)) ||
        (src_conv != dst_conv && !disjoint(src_conv, sc_n, dst_conv, dc_n)) ||
        !disjoint(src_state, ss_n, dst_conv, dc_n) || !disjoint(src_conv, sc_n, dst_state, ds_n))
        return KDA_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < n; ++i) {
        const size_t si = (size_t)src_slots[i], di = (size_t)dst_slots[i];
        const char *ss = reinterpret_cast<const char *>(src_state) + si * state_bytes;
        char *ds = reinterpret_cast<char *>(dst_state) + di * state_bytes;
        const char *sc = reinterpret_cast<const char *>(src_conv) + si * conv_bytes;
        char *dc = reinterpret_cast<char *>(dst_conv) + di * conv_bytes;
        // an entry onto itself is left as it is; the state and the conv windows are
        // decided separately (one may map onto itself while the other does not)
        if (ss != ds && hipMemcpyAsync(ds, ss, state_bytes, hipMemcpyDefault, s) != hipSuccess) return KDA_ERR_LAUNCH;
        if (sc != dc && hipMemcpyAsync(dc, sc, conv_bytes, hipMemcpyDefault, s) != hipSuccess) return KDA_ERR_LAUNCH;
    }
    return KDA_OK;
}

void kda_test_split_carry(int32_t publish, int32_t max_polls) {
    split_publish.store(publish != 0 ? 1 : 0);
    split_max_polls.store(max_polls > 0 ? max_polls : 0);
}

void kda_test_pipeline(int32_t mode, int32_t publish, int32_t max_polls) {
    pipe_mode.store(mode == 1 || mode == 2 ? mode : 0);
    pipe_publish.store(publish != 0 ? 1 : 0);
    pipe_max_polls.store(max_polls > 0 ? max_polls : 0);
}

const char *kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_ARG: return "a required pointer is NULL";
        case KDA_ERR_BAD_CONFIG: return "unsupported config (head_dim must be 128, conv_size 4, num_heads 1..65536, finite eps >= 0, prefill_path 0..2, out_dtype 0..1, precision 0..1)";
        case KDA_ERR_BAD_SHAPE: return "negative, inconsistent or too large sizes";
        case KDA_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "workspace too small";
        case KDA_ERR_LAUNCH: return "the HIP runtime refused a kernel launch or a copy";
        case KDA_ERR_OVERLAP: return "an output buffer overlaps an input or another output";
    }
    return "unknown status";
}

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
