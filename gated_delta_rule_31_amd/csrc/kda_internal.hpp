// kda_internal.hpp -- launch descriptors shared by the entry points (kda_api.cpp) and
// the kernels (kda_decode.hip, kda_prefill.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;     // head dim (key = value = 128)
constexpr int kConv = 4;    // ShortConv taps
constexpr int kChunk = 64;  // prefill chunk length

struct MixerConsts {
    int H;
    float gate_lower_bound;
    float l2_eps;
    float rms_eps;
    float q_scale;
};

struct DecodeArgs {
    MixerConsts c;
    int B;
    const float *q, *k, *v, *z, *b, *g;
    const float *conv_w, *A_log, *dt_bias, *norm_w;
    float *state, *conv_state, *out;
};

struct PrefillArgs {
    MixerConsts c;
    int B, N;
    const int32_t *cu_seqlens;
    const uint16_t *q, *k, *v, *z, *b, *g;
    const float *conv_w, *A_log, *dt_bias, *norm_w;
    const float *initial_state, *initial_conv_state;
    float *out, *final_state, *final_conv_state;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

}  // namespace kda
