// fa2_fwd_wide.hip -- the 8-wave d = 128 forward configurations: the
// software-pipelined non-causal kernel (fwd_sp_kernel<128, 64, 8>) and the
// causal heavy/light pairs with 128-key K/V tiles (fwd_dl_kernel<128, 128,
// 8, 2, true>), the kernels of every d = 128 grid that fills the GPU.
//
// This translation unit is compiled with LLVM's ILP-first machine scheduler
// (-mllvm -amdgpu-sched-strategy=iterative-ilp; build.py sets it for this
// file alone).  In interleaved A/B runs on MI355X it made these kernels
// 1.1 to 1.9 % faster across eight workloads, while the same scheduler cost
// the 4-wave kernel of small grids 6 % and the backward pass 1.3 %, so every
// other source keeps the default scheduler.
#include "fa2_fwd_kernels.hpp"

namespace fa2 {

hipError_t launch_fwd_wide(const FwdParams& p, int variant) {
  switch (variant) {
    case kFwdD128Sp8: return launch_fwd_sp<128, 64, 8>(p);
    case kFwdD128CausalPair8: return launch_fwd_dl<128, 128, 8, 2, true>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
