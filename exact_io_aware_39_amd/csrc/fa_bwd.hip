// fa_bwd.hip - backward of exact attention, bf16 (not yet implemented).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const void*,
                           const float*, void*, void*, void*, float*, const AttnShape&, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace fa
