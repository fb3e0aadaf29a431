// fa2_bwd.hip -- FlashAttention-2 backward pass for gfx950 (in progress).
#include "fa2_device.hpp"
#include "fa2_internal.hpp"

namespace fa2 {

hipError_t launch_bwd(const BwdParams& p) {
  (void)p;
  return hipErrorNotSupported;
}

}  // namespace fa2
