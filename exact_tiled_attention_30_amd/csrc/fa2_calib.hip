// fa2_calib.hip -- measurement helper: the bf16 MFMA throughput this GPU
// reaches at its running clock, the yardstick next to the nominal dense peak
// (256 CUs x 4096 FLOP/clk x 2.4 GHz) against which attention throughput is
// reported.  Not part of the attention path.
#include "fa2_device.hpp"
#include "fa2_internal.hpp"

namespace fa2 {
namespace {

constexpr int kCalibChains = 4;  // independent accumulators per wave
constexpr int kCalibSets = 8;    // operand sets cycled by the random-operand mode

// Unit-variance pseudo-random value from a 32-bit counter: a 32-bit integer
// finaliser (xorshift-multiply) split into two 16-bit uniforms whose centred
// sum is triangular on (-1, 1), scaled by sqrt(6) to variance 1.
__device__ __forceinline__ float calib_value(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  const float u = (float)(x & 0xffffu) * (1.0f / 65536.0f) + (float)(x >> 16) * (1.0f / 65536.0f);
  return (u - 1.0f) * 2.4494897f;
}

// Every wave issues iters x kCalibChains v_mfma_f32_32x32x16_bf16 with
// operands in registers and no other work, so the matrix pipes stay full.
// RANDOM = false: one fixed operand pair (few bits toggle between MFMAs).
// RANDOM = true: kCalibSets pairs of unit-variance values, a different pair
// for every MFMA of a chain, as the operands of an attention tile change from
// one MFMA to the next.  The matrix cores' power grows with the bits that
// toggle, so under a power cap the second mode runs at a lower clock.
template <bool RANDOM>
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x % kWave;
  constexpr int kSets = RANDOM ? kCalibSets : 1;
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (RANDOM) {
        a[s][i] = (__bf16)calib_value(id * 2u * kSets * 8u + (uint32_t)(s * 8 + i));
        b[s][i] = (__bf16)calib_value(id * 2u * kSets * 8u + (uint32_t)(kSets * 8 + s * 8 + i));
      } else {
        a[s][i] = (__bf16)(0.001f * (float)(lane + i));
        b[s][i] = (__bf16)(0.001f * (float)(lane - i));
      }
    }
  f32x16 acc[kCalibChains];
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) acc[c] = f32x16{};
  int it = 0;
  for (; it <= iters - kSets; it += kSets) {  // iters >= 1: no overflow
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int c = 0; c < kCalibChains; ++c)
        acc[c] = mfma32(a[s], b[(s + c) % kSets], acc[c]);
  }
  for (; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c) acc[c] = mfma32(a[0], b[c % kSets], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) s += acc[c][0] + acc[c][15];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_calib_mfma(float* out, int blocks, int iters, bool random_operands,
                             hipStream_t stream) {
  (void)hipGetLastError();
  if (random_operands)
    hipLaunchKernelGGL(calib_mfma_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, out,
                       iters);
  else
    hipLaunchKernelGGL(calib_mfma_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, out,
                       iters);
  return hipGetLastError();
}

}  // namespace fa2
