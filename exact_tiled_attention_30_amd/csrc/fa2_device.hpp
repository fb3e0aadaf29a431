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

// Max of a lane's scores.  It must stay compiler-visible: the hazard
// recognizer pads a VALU read of an MFMA result only when it can see the
// instruction, and a hand-written v_max reading an accumulator right after
// its MFMA was observed to see a partial sum (a race that only moved the
// rescale reference, so results differed from run to run by rounding).
// The NaN-propagating maximum lowers to a v_maximum3_f32 chain on gfx950
// with no operand canonicalisation (fmaxf's IEEE maxNum quiets the first
// operands with extra v_max instructions).  A NaN score makes the row max
// NaN, which never triggers a rescale; that row's P, l and O are NaN anyway.
__device__ __forceinline__ float fmax_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
template <int NV>
__device__ __forceinline__ float lane_max(const f32x16* s) {
  float mx = fmax_nan(s[0][0], s[0][1]);
#pragma unroll
  for (int i = 2; i < NV; i += 2)
    mx = fmax_nan(fmax_nan(mx, s[i / 16][i % 16]), s[i / 16][i % 16 + 1]);
  return mx;
}

// max / sum of a value over the lane pair (l, l ^ 32) with one
// v_permlane32_swap: its two results are the two halves' values, in some
// order, in every lane -- the symmetric combinations below do not depend on
// which is which.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// One output row in bf16, scaled by `mul`, from transposed accumulators
// (acc[dt], dt < D / 32: 32 columns x 32 rows, the row fixed per lane), stored 16 bytes
// per lane.  Accumulator register 4g + i of lane (row, half h) is column
// dt*32 + 8g + 4h + i: 8-byte pieces that alternate between the row's two
// lanes.  One v_permlane32_swap per register pair trades the lower lane's
// piece g = 2j+1 for the upper lane's piece g = 2j, so each lane holds the 8
// consecutive columns dt*32 + 16j + 8h .. +7 and every store instruction
// writes 32 contiguous bytes per row instead of 16: half the instructions and
// half the memory requests of an epilogue that every workgroup of a short
// launch runs at once.  All lanes must call it (the swap reads the partner
// lane); `valid` gates the store, `dst` points at the row's first column.
template <int D>
__device__ __forceinline__ void store_row_bf16(uint16_t* dst, const f32x16* acc, float mul,
                                               int hi, bool valid) {
  u32x4 row[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x16& a = acc[dt];
      const u32x2 even = __builtin_bit_cast(
          u32x2, to_bf16x4(f32x4{a[8 * j], a[8 * j + 1], a[8 * j + 2], a[8 * j + 3]} * mul));
      const u32x2 odd = __builtin_bit_cast(
          u32x2, to_bf16x4(f32x4{a[8 * j + 4], a[8 * j + 5], a[8 * j + 6], a[8 * j + 7]} * mul));
      // lower lane: (own even, partner's even); upper lane: (partner's odd, own odd)
      const auto w0 = __builtin_amdgcn_permlane32_swap(even[0], odd[0], false, false);
      const auto w1 = __builtin_amdgcn_permlane32_swap(even[1], odd[1], false, false);
      row[dt][j] = u32x4{w0[0], w1[0], w0[1], w1[1]};
    }
  if (valid) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 2; ++j) *(u32x4*)(dst + dt * 32 + 16 * j + 8 * hi) = row[dt][j];
  }
}

// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt in
// bits 6:4, lgkmcnt in bits 11:8).  Before a barrier after which another
// wave's global_load_lds may overwrite an LDS buffer, a wave must have both
// its own DMA landed (vmcnt) and its own LDS reads of that buffer returned
// (lgkmcnt): the workgroup fence of __syncthreads() orders LDS accesses
// among waves but not a read still in flight against a DMA write, and the
// compiler may schedule a read's consumer after the barrier.
constexpr int kWaitVmLgkm = 0x0070;  // vmcnt(0) lgkmcnt(0)
__device__ __forceinline__ void wait_dma_and_lds() { __builtin_amdgcn_s_waitcnt(kWaitVmLgkm); }

// Workgroups are dispatched round-robin over the eight XCDs (wg i runs on XCD
// i % 8).  Renumber them so that each XCD receives one contiguous range of
// logical ids; consecutive logical ids are Q tiles of the same (batch, head),
// which then share K/V through that XCD's L2.  Bijective for any grid size.
// Host-callable so the map can be checked on the CPU.
__host__ __device__ inline int xcd_contiguous_id(int wg, int grid) {
  constexpr int kXcds = 8;
  const int per = grid / kXcds, rem = grid % kXcds;
  const int xcd = wg % kXcds, slot = wg / kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Causal grids that are resident all at once (one Q tile per workgroup):
// workgroups are placed round-robin over the XCDs, and on an XCD local
// workgroup L lands on CU L mod 32 (32 CUs per XCD).  Ranking the XCD's Q
// tiles by their number of K/V tiles, heaviest first, and dealing them to
// the CUs in snake order (left to right, then right to left, ...) gives every
// CU the same total.  The host only selects this with whole heads per XCD
// (grid % 8 == 0 and (grid / 8) % n_qtiles == 0).  Item 0 of a head is its
// heaviest Q tile (the kernel reverses the tile order).  On a grid larger
// than the CUs hold, the first round is placed as above and the later
// workgroups, dispatched in rank order, take whichever slot frees first.
// Host-callable so the map can be checked on the CPU.
__host__ __device__ inline int dealt_id(int wg, int grid, int n_qtiles) {
  constexpr int kXcds = 8, kCusPerXcd = 32;
  const int per = grid / kXcds;
  const int xcd = wg % kXcds, local = wg / kXcds;
  const int round = local / kCusPerXcd, cu = local % kCusPerXcd;
  const int left = per - round * kCusPerXcd;
  const int width = left < kCusPerXcd ? left : kCusPerXcd;
  const int rank = round * kCusPerXcd + ((round & 1) ? width - 1 - cu : cu);
  const int heads = per / n_qtiles;
  return xcd * per + (rank % heads) * n_qtiles + rank / heads;
}

}  // namespace fa2
