// fa2_device.hpp -- gfx950 (CDNA4) device building blocks shared by the
// forward and backward kernels: vector types, MFMA wrappers, bf16 packing,
// wave-level exchanges and the workgroup -> tile map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Operand lanes: lane l supplies row (l % 32) of A and column (l % 32) of B,
// with 8 consecutive elements of the contraction in each lane; the two lane
// halves cover the two halves of the contraction.  Both operands use the same
// (lane half, slot) -> k assignment, so any consistent ordering of k is a
// valid contraction order.
// Accumulator: register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row index (within a 32x32 accumulator tile) held by register r of a lane
// in half `hi` (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int r, int hi) {
  return 8 * (r / 4) + 4 * hi + (r % 4);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// Round-to-nearest-even fp32 -> bf16 of 8 values (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) {
  return __builtin_convertvector(x, bf16x8);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  return __builtin_convertvector(x, bf16x4);
}
// Round-to-nearest-even fp32 -> bf16 bit pattern.
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Value of the same register in the partner lane l ^ 32 (the other half of
// the wave holds the other half of each 32x32 accumulator column).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, kWave);
}

// v_max3_f32 / v_max_f32 without the NaN-quieting canonicalisation the
// compiler wraps around fmaxf in IEEE mode (scores are finite or -inf; a NaN
// input still propagates through the exp).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max / sum of a value over the lane pair (l, l ^ 32) with one
// v_permlane32_swap: its two results are the two halves' values, in some
// order, in every lane -- the symmetric combinations below do not depend on
// which is which.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max2f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are dispatched round-robin over the eight XCDs (wg i runs on XCD
// i % 8).  Renumber them so that each XCD receives one contiguous range of
// logical ids; consecutive logical ids are Q tiles of the same (batch, head),
// which then share K/V through that XCD's L2.  Bijective for any grid size.
__device__ __forceinline__ int xcd_contiguous_id(int wg, int grid) {
  constexpr int kXcds = 8;
  const int per = grid / kXcds, rem = grid % kXcds;
  const int xcd = wg % kXcds, slot = wg / kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace fa2
