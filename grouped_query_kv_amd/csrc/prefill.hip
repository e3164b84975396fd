#include "gqa_internal.h"
namespace gqa {
bool prefill_fast_supported(const Problem&) { return false; }
hipError_t launch_prefill_fast(const Problem&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace gqa
