#include "gqa_internal.h"
namespace gqa {
bool decode_fast_supported(const Problem&) { return false; }
hipError_t launch_decode_fast(const Problem&, void*, const WorkspaceLayout&, hipStream_t) {
  return hipErrorInvalidValue;
}
}  // namespace gqa
