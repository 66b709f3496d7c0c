// kda_prefill.hip -- chunked varlen prefill (placeholder until the chunk kernel lands).
#include "kda_internal.hpp"

namespace kda {
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
