// fa2_fwd.hip -- FlashAttention-2 forward pass for gfx950: the kernel choice
// and launch.  The kernels, their design and their launch templates are in
// fa2_fwd_kernels.hpp; the 8-wave d = 128 configurations are instantiated in
// fa2_fwd_wide.hip.
#include "fa2_fwd_kernels.hpp"

namespace fa2 {

int fwd_resident_d128() { return resident_wgs<128, 64, 4, 2, true, false, true>(); }

hipError_t launch_fwd(const FwdParams& p) {
  const int variant =
      fwd_variant(p.B, p.H, p.N, p.d, p.causal, p.causal && p.d == 128 ? fwd_resident_d128() : 0);
  switch (variant) {
    case kFwdD64Nc4: return launch_fwd_dl<64, 64, 4, 2, false>(p);
    case kFwdD64Nc8: return launch_fwd_dl<64, 64, 8, 2, false>(p);
    case kFwdD128Sp4: return launch_fwd_sp<128, 64, 4>(p);
    case kFwdD64CausalDealt: return launch_fwd_dl<64, 64, 4, 2, true, false, true>(p);
    case kFwdD64CausalOne: return launch_fwd_dl<64, 64, 4, 2, true, false>(p);
    case kFwdD64CausalPair4: return launch_fwd_dl<64, 64, 4, 2, true>(p);
    case kFwdD64CausalPair8: return launch_fwd_dl<64, 64, 8, 2, true>(p);
    case kFwdD128CausalDealt: return launch_fwd_dl<128, 64, 4, 2, true, false, true>(p);
    case kFwdD128CausalOne: return launch_fwd_dl<128, 64, 4, 2, true, false>(p);
    case kFwdD128CausalPair4: return launch_fwd_dl<128, 64, 4, 2, true>(p);
    case kFwdD128Sp8:
    case kFwdD128CausalPair8: return launch_fwd_wide(p, variant);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_split_kv(const FwdParams& p) {
  if (p.d == 64) return p.causal ? launch_split_t<64, true>(p) : launch_split_t<64, false>(p);
  return p.causal ? launch_split_t<128, true>(p) : launch_split_t<128, false>(p);
}

}  // namespace fa2

