// Backward kernels (being written): until they land, the launcher reports
// that the operation is not available rather than computing anything.
#include "fa_launch.h"

namespace fa {

hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const void*,
                           const float*, void*, void*, void*, void*, const Problem&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fa
