// Host-only driver for the address / undefined-behaviour sanitizer build of the C ABI's
// argument checks: kda_api.hip is linked with launchers that fail the test if reached,
// and every call below must be rejected (or accepted as empty) before any HIP call.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"
#include "kda_internal.hpp"

namespace kda {
static int reached = 0;
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { ++reached; return hipErrorInvalidValue; }
hipError_t launch_decode_multi(const DecodeMultiArgs &, hipStream_t) { ++reached; return hipErrorInvalidValue; }
hipError_t launch_decode_multi_seq(const DecodeMultiArgs &, hipStream_t) { ++reached; return hipErrorInvalidValue; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { ++reached; return hipErrorInvalidValue; }
hipError_t launch_carry(const PrefillArgs &, hipStream_t) { ++reached; return hipErrorInvalidValue; }
}  // namespace kda

static int failures = 0;
#define EXPECT(call, want)                                                               \
    do {                                                                                 \
        const int got_ = (int)(call);                                                    \
        if (got_ != (int)(want)) {                                                       \
            printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

int main() {
    float *F = reinterpret_cast<float *>(0x10000);  // aligned, never dereferenced
    float *Fm = reinterpret_cast<float *>(0x10004);
    const uint16_t *Hh = reinterpret_cast<const uint16_t *>(0x10000);
    const int32_t *I = reinterpret_cast<const int32_t *>(0x10000);
    kda_config c = kda_config_default();
    kda_config bad = c;
    bad.head_dim = 64;

    // decode, one token
    EXPECT(kda_decode_step(nullptr, 1, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_NULL_ARG);
    EXPECT(kda_decode_step(&bad, 1, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_BAD_CONFIG);
    EXPECT(kda_decode_step(&c, -1, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_BAD_SHAPE);
    EXPECT(kda_decode_step(&c, 0, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_OK);
    EXPECT(kda_decode_step(&c, 2, F, F, F, 0, nullptr, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_NULL_ARG);
    EXPECT(kda_decode_step(&c, 2, F, F, F, 0, F, F, F, F, F, F, F, F, Fm, F, nullptr), KDA_ERR_MISALIGNED);
    EXPECT(kda_decode_step_slots(&c, 2, nullptr, 4, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_NULL_ARG);
    EXPECT(kda_decode_step_slots(&c, 2, I, 0, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_OK);
    EXPECT(kda_decode_step_slots(&c, 2, I, -1, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_BAD_SHAPE);

    // decode, several tokens
    EXPECT(kda_decode_multi(&c, 2, 0, nullptr, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_BAD_SHAPE);
    EXPECT(kda_decode_multi(&c, 65536, 65536, nullptr, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, F, F, nullptr),
           KDA_ERR_BAD_SHAPE);
    EXPECT(kda_decode_multi(&c, 2, 3, nullptr, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, F, nullptr, nullptr),
           KDA_ERR_NULL_ARG);
    EXPECT(kda_decode_multi_slots(&c, 2, 3, nullptr, nullptr, 4, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, F, F, nullptr),
           KDA_ERR_NULL_ARG);
    EXPECT(kda_decode_multi_slots(&c, 2, 3, nullptr, I, 0, F, F, F, 0, F, F, F, F, F, F, F, F, F, F, F, F, nullptr),
           KDA_OK);

    // prefill
    c.prefill_path = 7;
    EXPECT(kda_prefill(&c, 1, 64, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F, nullptr, 0, nullptr),
           KDA_ERR_BAD_CONFIG);
    c.prefill_path = KDA_PREFILL_CHUNKED;
    EXPECT(kda_prefill(&c, 1, 64, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F, nullptr, 0, nullptr),
           KDA_ERR_WORKSPACE);
    EXPECT(kda_prefill(&c, -1, 64, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F, nullptr, 0, nullptr),
           KDA_ERR_BAD_SHAPE);
    EXPECT(kda_prefill(&c, 0, 0, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F, nullptr, 0, nullptr),
           KDA_OK);
    // one sequence: the ready words of the records (129 x 96 words, padded to 256 bytes)
    if (kda_prefill_workspace_bytes(&c, 1, 8192) != (size_t)256 + 49664 + (size_t)(128 + 1) * 96 * 111616) {
        printf("unexpected workspace size %zu\n", kda_prefill_workspace_bytes(&c, 1, 8192));
        ++failures;
    }
    c.prefill_path = KDA_PREFILL_AUTO;

    // state copies: slots outside the buffers, overlapping buffers
    const int32_t s0[1] = {0}, s9[1] = {9};
    float *A = reinterpret_cast<float *>(0x100000000ULL), *B = reinterpret_cast<float *>(0x200000000ULL);
    float *Ac = A + 8 * 96 * 128 * 128;
    EXPECT(kda_state_copy(&c, 1, A, Ac, 4, s9, B, B + 8 * 96 * 128 * 128, 4, s0, nullptr), KDA_ERR_BAD_SHAPE);
    EXPECT(kda_state_copy(&c, 1, A, Ac, 4, s0, A + 96 * 128 * 128, B, 4, s0, nullptr), KDA_ERR_OVERLAP);
    EXPECT(kda_state_copy(&c, 1, A, Ac, 4, nullptr, B, B, 4, s0, nullptr), KDA_ERR_NULL_ARG);
    EXPECT(kda_state_copy(&c, 0, A, Ac, 4, s0, B, B, 4, s0, nullptr), KDA_OK);

    // q/k/v row strides: below H*D, not a multiple of 8, past 2^24
    EXPECT(kda_decode_step(&c, 2, F, F, F, 96 * 128 - 8, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_BAD_SHAPE);
    EXPECT(kda_decode_step(&c, 2, F, F, F, 96 * 128 + 4, F, F, F, F, F, F, F, F, F, F, nullptr), KDA_ERR_BAD_SHAPE);
    EXPECT(kda_prefill(&c, 1, 64, I, Hh, Hh, Hh, (1 << 24) + 8, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F,
                       nullptr, 0, nullptr),
           KDA_ERR_BAD_SHAPE);
    // outputs over inputs: far-apart buffers with one output moved onto an input
    {
        const uintptr_t G = (uintptr_t)1 << 32;
        float *P[13];
        for (int i = 0; i < 13; ++i) P[i] = reinterpret_cast<float *>((i + 1) * G);
        EXPECT(kda_decode_step(&c, 4, P[0], P[1], P[2], 0, P[3], P[4], P[5], P[6], P[7], P[8], P[9], P[10], P[11],
                               P[0] + 4, nullptr),
               KDA_ERR_OVERLAP);
        EXPECT(kda_decode_multi(&c, 2, 3, nullptr, P[0], P[1], P[2], 0, P[3], P[4], P[5], P[6], P[7], P[8], P[9],
                                P[10], P[10] + 4, P[11], P[12], P[12] + 4096 * 1024, nullptr),
               KDA_ERR_OVERLAP);
        const uint16_t *Q[7];
        for (int i = 0; i < 7; ++i) Q[i] = reinterpret_cast<const uint16_t *>((i + 1) * G);
        const int32_t *cu = reinterpret_cast<const int32_t *>(8 * G);
        EXPECT(kda_prefill(&c, 2, 100, cu, Q[0], Q[1], Q[2], 0, Q[3], Q[4], Q[5], P[8], P[9], P[10], P[11], P[12],
                           P[12] + 8 * 96 * 128 * 128 * 4, reinterpret_cast<float *>(20 * G), P[12] + 4,
                           reinterpret_cast<float *>(22 * G), nullptr, 0, nullptr),
               KDA_ERR_OVERLAP);
    }
    EXPECT(kda_state_copy(&c, 1, A, Ac, 4, s0, A, Ac + 16, 4, s0, nullptr), KDA_ERR_OVERLAP);

    // the prefill with the decay projection inside: W_fb is required, and outputs may not
    // overlap it
    EXPECT(kda_prefill_gate_proj(&c, 1, 64, I, Hh, Hh, Hh, 0, Hh, nullptr, Hh, Hh, F, F, F, F, nullptr, nullptr, F,
                                 F, F, nullptr, 0, nullptr),
           KDA_ERR_NULL_ARG);
    EXPECT(kda_prefill_gate_proj(&c, 0, 0, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F,
                                 nullptr, 0, nullptr),
           KDA_OK);

    // the allocation-free prefill: the same checks; an explicit chunked layout past the
    // scratch array is rejected before the array is looked up
    EXPECT(kda_prefill_noalloc(&c, -1, 64, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F,
                               nullptr),
           KDA_ERR_BAD_SHAPE);
    EXPECT(kda_prefill_noalloc(&c, 0, 0, I, Hh, Hh, Hh, 0, Hh, Hh, Hh, F, F, F, F, nullptr, nullptr, F, F, F,
                               nullptr),
           KDA_OK);
    {
        const uintptr_t G = (uintptr_t)1 << 32;
        const uint16_t *Q[7];
        float *P[8];
        for (int i = 0; i < 7; ++i) Q[i] = reinterpret_cast<const uint16_t *>((i + 1) * G);
        for (int i = 0; i < 8; ++i) P[i] = reinterpret_cast<float *>((i + 10) * G);
        kda_config cc = c;
        cc.prefill_path = KDA_PREFILL_CHUNKED;
        EXPECT(kda_prefill_noalloc(&cc, 1, 4096, reinterpret_cast<const int32_t *>(Q[6]), Q[0], Q[1], Q[2], 0, Q[3],
                                   Q[4], Q[5], P[0], P[1], P[2], P[3], nullptr, nullptr, P[4], P[5], P[6], nullptr),
               KDA_ERR_WORKSPACE);
    }

    for (int s = 0; s <= 7; ++s)
        if (!kda_status_str((kda_status)s)[0]) ++failures;
    if (kda::reached) {
        printf("%d calls reached a launcher\n", kda::reached);
        ++failures;
    }
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
