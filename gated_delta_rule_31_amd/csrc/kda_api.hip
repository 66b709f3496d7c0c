// kda_api.hip -- the C-ABI entry points of libkda.so: host-side argument checks, then
// one kernel launch on the caller's stream.  Declarations and contracts: include/kda.h.
//
// Every check runs before the first HIP call, so a rejected call touches neither the
// device nor the HIP runtime's error state (and the checks run on a machine without a
// GPU).

#include <math.h>
#include <stdint.h>

#include "kda.h"
#include "kda_internal.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.0f; }

kda_status check_config(const kda_config *cfg, kda::MixerConsts *out) {
    if (!cfg) return KDA_ERR_NULL_ARG;
    if (cfg->num_heads < 1 || cfg->head_dim != kda::kD || cfg->conv_size != kda::kConv)
        return KDA_ERR_BAD_CONFIG;
    if (!isfinite(cfg->gate_lower_bound) || !finite_nonneg(cfg->l2_eps) || !finite_nonneg(cfg->rms_eps) ||
        !isfinite(cfg->q_scale))
        return KDA_ERR_BAD_CONFIG;
    out->H = cfg->num_heads;
    out->gate_lower_bound = cfg->gate_lower_bound;
    out->l2_eps = cfg->l2_eps;
    out->rms_eps = cfg->rms_eps;
    out->q_scale = cfg->q_scale > 0.0f ? cfg->q_scale : 1.0f / sqrtf((float)kda::kD);
    return KDA_OK;
}

// [B*H] units must fit the 1-D grid; [B or N, H*D] extents must fit size_t arithmetic.
bool units_fit(int64_t rows, int64_t H) { return rows >= 0 && rows * H <= INT32_MAX; }

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
    return c;
}

kda_status kda_decode_step(const kda_config *cfg, int32_t batch, const float *q, const float *k,
                           const float *v, const float *z, const float *b, const float *g,
                           const float *conv_w, const float *A_log, const float *dt_bias,
                           const float *norm_w, float *state, float *conv_state, float *out,
                           void *stream) {
    kda::DecodeArgs a;
    kda_status st = check_config(cfg, &a.c);
    if (st != KDA_OK) return st;
    if (batch < 0 || !units_fit(batch, a.c.H)) return KDA_ERR_BAD_SHAPE;
    if (batch == 0) return KDA_OK;
    const void *ptrs[] = {q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state, conv_state, out};
    for (const void *p : ptrs)
        if (!p) return KDA_ERR_NULL_ARG;
    for (const void *p : ptrs)
        if (!aligned16(p)) return KDA_ERR_MISALIGNED;
    a.B = batch;
    a.q = q; a.k = k; a.v = v; a.z = z; a.b = b; a.g = g;
    a.conv_w = conv_w; a.A_log = A_log; a.dt_bias = dt_bias; a.norm_w = norm_w;
    a.state = state; a.conv_state = conv_state; a.out = out;
    return kda::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t kda_prefill_workspace_bytes(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens) {
    (void)cfg;
    (void)num_seqs;
    (void)total_tokens;
    return 0;  // the fused chunk kernel keeps every intermediate on chip
}

kda_status kda_prefill(const kda_config *cfg, int32_t num_seqs, int32_t total_tokens,
                       const int32_t *cu_seqlens, const uint16_t *q, const uint16_t *k,
                       const uint16_t *v, const uint16_t *z, const uint16_t *b, const uint16_t *g,
                       const float *conv_w, const float *A_log, const float *dt_bias, const float *norm_w,
                       const float *initial_state, const float *initial_conv_state, float *out,
                       float *final_state, float *final_conv_state, void *workspace,
                       size_t workspace_bytes, void *stream) {
    kda::PrefillArgs a;
    kda_status st = check_config(cfg, &a.c);
    if (st != KDA_OK) return st;
    if (num_seqs < 0 || total_tokens < 0 || !units_fit(num_seqs, a.c.H) || !units_fit(total_tokens, 1))
        return KDA_ERR_BAD_SHAPE;
    if (workspace_bytes < kda_prefill_workspace_bytes(cfg, num_seqs, total_tokens)) return KDA_ERR_WORKSPACE;
    (void)workspace;
    if (num_seqs == 0) return total_tokens == 0 ? KDA_OK : KDA_ERR_BAD_SHAPE;
    const void *req[] = {cu_seqlens, conv_w, A_log, dt_bias, norm_w, final_state, final_conv_state};
    for (const void *p : req)
        if (!p) return KDA_ERR_NULL_ARG;
    if (total_tokens > 0) {
        const void *tok[] = {q, k, v, z, b, g, out};
        for (const void *p : tok)
            if (!p) return KDA_ERR_NULL_ARG;
        for (const void *p : tok)
            if (!aligned16(p)) return KDA_ERR_MISALIGNED;
    }
    const void *al[] = {conv_w, A_log, dt_bias, norm_w, final_state, final_conv_state, initial_state,
                        initial_conv_state};
    for (const void *p : al)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_MISALIGNED;
    a.B = num_seqs;
    a.N = total_tokens;
    a.cu_seqlens = cu_seqlens;
    a.q = q; a.k = k; a.v = v; a.z = z; a.b = b; a.g = g;
    a.conv_w = conv_w; a.A_log = A_log; a.dt_bias = dt_bias; a.norm_w = norm_w;
    a.initial_state = initial_state;
    a.initial_conv_state = initial_conv_state;
    a.out = out;
    a.final_state = final_state;
    a.final_conv_state = final_conv_state;
    return kda::launch_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

const char *kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_ARG: return "a required pointer is NULL";
        case KDA_ERR_BAD_CONFIG: return "unsupported config (head_dim must be 128, conv_size 4, num_heads >= 1, finite eps >= 0)";
        case KDA_ERR_BAD_SHAPE: return "negative, inconsistent or too large sizes";
        case KDA_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "workspace too small";
        case KDA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
