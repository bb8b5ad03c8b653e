// Placeholder until the fp8 top-k sparse kernel lands.
#include "mla_internal.h"

namespace mla {
hipError_t launch_split_fp8_topk(const Args&, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla
