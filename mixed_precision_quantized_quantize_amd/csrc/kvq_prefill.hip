// kvq_prefill.hip -- causal chunked prefill over the quantized cache.
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_prefill(int, int, int, const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvq
