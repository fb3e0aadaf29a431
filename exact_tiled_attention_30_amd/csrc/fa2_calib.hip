// fa2_calib.hip -- measurement helper: the bf16 MFMA throughput this GPU
// reaches at its running clock, the yardstick next to the nominal dense peak
// (256 CUs x 4096 FLOP/clk x 2.4 GHz) against which attention throughput is
// reported.  Not part of the attention path.
#include "fa2_device.hpp"
#include "fa2_internal.hpp"

namespace fa2 {
namespace {

constexpr int kCalibChains = 4;  // independent accumulators per wave

// Every wave issues iters x kCalibChains v_mfma_f32_32x32x16_bf16 with
// operands in registers and no other work, so the matrix pipes stay full.
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x % kWave;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.001f * (float)(lane - i));
  }
  f32x16 acc[kCalibChains];
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) s += acc[c][0] + acc[c][15];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace fa2
