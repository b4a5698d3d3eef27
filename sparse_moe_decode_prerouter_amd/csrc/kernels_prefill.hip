// Prefill path (grouped GEMV over the sorted token->expert assignments).
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

hipError_t launch_prefill_gateup(const PrefillArgs& a, hipStream_t s) { return launch_gateup(a.g, s); }
hipError_t launch_prefill_down(const PrefillArgs& a, hipStream_t s) { return launch_down(a.g, s); }

}  // namespace moe
