// fa2_bwd.hip -- FlashAttention-2 backward pass for gfx950.
//
// Structure from infra-guide page "6.2 FlashAttention V2 in depth", section 7:
//   * P is not stored by the forward pass; it is recomputed from the saved
//     logsumexp L (section 7.1): P = exp(scale * q.k - L).
//   * The outer loop runs over key/value tiles: the workgroup that holds K_j,
//     V_j accumulates dK_j and dV_j by itself with no atomics.  dQ needs a sum
//     across those workgroups (section 7.2, "atomic add or a two-pass scan");
//     both are built: a separate Q-outer dQ pass (launch_bwd, the default:
//     deterministic and faster on MI355X) and fp32 atomics into a workspace
//     accumulator (launch_bwd_atomic_dq).
//   * D_i = rowsum(dO_i * O_i) is computed once per row (section 7.3), not
//     tile by tile: by the dQ pass, which runs first, on the two-pass path,
//     and by a separate pre-processing kernel on the atomic path.
// Gradient formulas (lost in the page's extraction; the standard softmax
// gradient): dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dK = scale dS^T Q,
// dQ = scale dS K.
//
// gfx950 mapping of the main kernel (bwd_dl_kernel):
//   * workgroup = 4 waves = 128 keys of one (batch, head); each wave owns 32
//     keys and keeps their K and V rows in VGPRs (MFMA B operands) and their
//     dK, dV accumulators in registers for the whole loop;
//   * it walks 64-query steps of Q, dO and the L / D rows, moved global ->
//     LDS by DMA one step ahead into a second buffer;
//   * S = K Q^T and dP = V dO^T put the key on the lane, so P and dS feed the
//     dV^T += dO^T P and dK^T += Q^T dS products straight from registers (as
//     B operands), with dO^T and Q^T read transposed from the same row-major
//     LDS tiles; the transposed accumulators keep the key on the lane, so the
//     dK and dV rows leave 16 bytes per lane; with the atomic dQ strategy,
//     dS also goes to LDS, from which
//     the workgroup forms its dQ partial = dS K over its 128 keys and adds it
//     atomically.
// For d = 128 the two-pass path runs bwd_kv_pair_kernel instead: the same
// products with two waves per 32-key block, each taking half of every query
// step, and V read from LDS, so that two waves fit per SIMD.
#include <limits.h>
#include <math.h>

#include "fa2_device.hpp"
#include "fa2_internal.hpp"

namespace fa2 {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdKeys = 128;    // keys per workgroup (4 waves x 32)
constexpr int kBwdQueries = 64;  // queries per inner step

// ---------------------------------------------------------------- B0 ----
// D[b, h, i] = sum_c dO[b, i, h, c] * O[b, i, h, c] (fp32), and zero the dQ
// accumulator row.  One 16-lane group per (b, i, h) row.
template <int D, bool ZERO_DQ>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    float* __restrict__ delta, float* __restrict__ dq_acc, int H, int N, long long rows) {
  constexpr int kLanesPerRow = 16;
  constexpr int kElemsPerLane = D / kLanesPerRow;  // 8 (d=128) or 4 (d=64)
  const long long row = (long long)blockIdx.x * (256 / kLanesPerRow) + threadIdx.x / kLanesPerRow;
  const int sub = threadIdx.x % kLanesPerRow;
  float acc = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * D + sub * kElemsPerLane;  // row = (b*N + i)*H + h
    if constexpr (kElemsPerLane == 8) {
      const u32x4 a = *(const u32x4*)(o + base);
      const u32x4 g = *(const u32x4*)(dout + base);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc += __uint_as_float(a[t] << 16) * __uint_as_float(g[t] << 16);
        acc += __uint_as_float(a[t] & 0xffff0000u) * __uint_as_float(g[t] & 0xffff0000u);
      }
      if (ZERO_DQ) {
        *(f32x4*)(dq_acc + base) = f32x4{};
        *(f32x4*)(dq_acc + base + 4) = f32x4{};
      }
    } else {
      const u32x2 a = *(const u32x2*)(o + base);
      const u32x2 g = *(const u32x2*)(dout + base);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc += __uint_as_float(a[t] << 16) * __uint_as_float(g[t] << 16);
        acc += __uint_as_float(a[t] & 0xffff0000u) * __uint_as_float(g[t] & 0xffff0000u);
      }
      if (ZERO_DQ) *(f32x4*)(dq_acc + base) = f32x4{};
    }
  }
  // reduce over the 16 lanes of the row
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off, kWave);
  if (row < rows && sub == 0) {
    const long long h = row % H;
    const long long i = (row / H) % N;
    const long long b = row / ((long long)H * N);
    delta[(b * H + h) * N + i] = acc;
  }
}

// ---------------------------------------------------------------- B2 ----
// dq = bf16(scale * dq_acc), 8 elements per thread.  The accumulator holds
// the unscaled sum of dS K, so the atomic adds work on O(1) values even when
// scale is tiny (a subnormal dQ is formed once, here, not summed).
__global__ __launch_bounds__(256) void bwd_convert_dq_kernel(const float* __restrict__ dq_acc,
                                                             uint16_t* __restrict__ dq,
                                                             long long n8, float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(dq_acc + 8 * i);
  const f32x4 b = *(const f32x4*)(dq_acc + 8 * i + 4);
  const bf16x8 r = to_bf16x8(f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]} * scale);
  *(u32x4*)(dq + 8 * i) = as_u32x4(r);
}

// ---------------------------------------------------------------- B1 ----
// Direct-to-LDS main kernel.  Every tile lives row-major in LDS, moved there
// with global_load_lds (no staging VGPRs, no transposing stores); the
// operands that need the transposed orientation -- Q^T and dO^T for dK and
// dV, K and dS for dQ -- are read with ds_read_b64_tr_b16 (within each group
// of 16 lanes, output lane 4a+b receives element b of the 8-byte chunks
// addressed by lanes a, 4+a, 8+a, 12+a).  Swizzles (XOR on the 16-byte chunk
// index of row r) keep every access pattern free of bank conflicts:
//   Q, dO tiles (row reads and transposed reads): 4*(r%4) + (r/4)%4 (d=128),
//                                                 4*((r/2)%2) + (r/4)%4 (d=64)
//   K tile (transposed reads only):              4*(r%4) (d=128), 4*((r/2)%2) (d=64)
//   dS tile [key][query] (8-byte stores, transposed reads):
//                                                4*((r/2)%2) ^ (r/4)%2 ^ 2*((r/8)%2)
// None of the transposed-read swizzles depends on row bits above 3, so a
// fragment's address is a per-lane base (computed once) plus a constant
// offset per 16-row block -- which keeps the compiler from holding one
// address register per fragment.
template <int D>
struct BwdSwz {
  __device__ static constexpr int qd(int r) {
    return D == 128 ? 4 * (r % 4) + (r / 4) % 4 : 4 * ((r / 2) % 2) + (r / 4) % 4;
  }
  __device__ static constexpr int k(int r) { return D == 128 ? 4 * (r % 4) : 4 * ((r / 2) % 2); }
  __device__ static constexpr int ds(int r) {
    return (4 * ((r / 2) % 2)) ^ ((r / 4) % 2) ^ (2 * ((r / 8) % 2));
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Per-lane byte offsets (row block 0, halves u = 0, 1, columns from 0) of a
// transposed fragment of a row-major, swizzled LDS tile.  Lane l ends up with
// src[16*blk + 8*(t/4) + 4*(l/32) + t%4][32*cb + l%32] in slot t -- the slot
// order the accumulator-derived operands use.  None of the swizzles here
// touches row bits above 3 or chunk bits above 1 for these lanes, so the
// fragment of 32-column block cb and 16-row block blk sits at
// (off ^ (cb << 6)) + blk * 16 * ROWBYTES.
template <int ROWBYTES, typename SWZ>
__device__ __forceinline__ void tr_offsets(int lane, SWZ swz, uint32_t (&off)[2]) {
  const int g = lane / 16, i = (lane % 16) / 4, a = lane % 4;
  const int col = 16 * (g % 2) + 4 * a;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int R = 8 * u + 4 * (g / 2) + i;
    off[u] = (uint32_t)(R * ROWBYTES + (((col / 8) ^ swz(R)) * 16) + (col % 8) * 2);
  }
}

template <int ROWBYTES>
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* tile, const uint32_t (&off)[2], int cb,
                                          int blk) {
  u32x2 part[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint8_t* addr = tile + (off[u] ^ (uint32_t)(cb << 6)) + blk * 16 * ROWBYTES;
    part[u] = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)addr));
  }
  return as_bf16x8(u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
}

// Scheduling request for an unrolled run of N_MFMA MFMAs, each fed by PER
// LDS reads: issue the reads AHEAD MFMAs early, then alternate, so the read
// latency hides behind the matrix pipe (one wave per SIMD here: no other
// wave covers it).
template <int N_MFMA, int PER, int AHEAD>
__device__ __forceinline__ void interleave_lds_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, PER * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N_MFMA - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Hides a value from loop-invariant code motion, so addresses derived from
// it are formed where they are used instead of being hoisted and held live.
// lgkmcnt(0) alone (vmcnt and expcnt at their maximum; gfx9 s_waitcnt
// layout): before a barrier at which no DMA is outstanding, so global stores
// still in flight need not drain first.
constexpr int kWaitLgkm = 0xC07F;
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(kWaitLgkm); }

__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, bool CAUSAL, bool ATOMIC_DQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void bwd_dl_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int H, int N, int n_ktiles, int grid,
    float c, float scale) {
  constexpr int RB = D * 2;                  // bytes per Q / dO / K row
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;             // rows per 1 KB DMA instruction
  constexpr int QT = kBwdQueries * RB;       // bytes of a Q or dO tile
  constexpr int KT = kBwdKeys * RB;          // bytes of the K tile
  constexpr int DSB = kBwdQueries * 2;       // bytes per dS row (64 queries)
  constexpr int NQI = QT / 1024 / 4;         // Q (and dO) DMA instructions per wave
  constexpr int NKI = KT / 1024 / 4;         // K DMA instructions per wave
  static_assert(NQI >= 1 && NKI >= 1, "tile split");
  using SW = BwdSwz<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kt_s[ATOMIC_DQ ? KT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t q_s0[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t q_s1[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t do_s0[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t do_s1[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t ds_s[ATOMIC_DQ ? kBwdKeys * DSB : 16];
  __shared__ __attribute__((aligned(256))) float st_s0[2 * kBwdQueries];  // lse | delta
  __shared__ __attribute__((aligned(256))) float st_s1[2 * kBwdQueries];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;

  // Work item: non-causal, one key tile; causal, the pair (p, n_ktiles-1-p)
  // of a heavy and a light key tile, so every workgroup walks about the same
  // number of query steps.
  const int logical = xcd_contiguous_id(blockIdx.x, grid);
  const int per_head = CAUSAL ? (n_ktiles + 1) / 2 : n_ktiles;
  const int bh = logical / per_head;
  const int item = logical % per_head;
  const int n_pass = (CAUSAL && item != n_ktiles - 1 - item) ? 2 : 1;
  const int b = bh / H, hh = bh % H;
  for (int pass = 0; pass < n_pass; ++pass) {
  const int kt_idx = pass == 0 ? item : n_ktiles - 1 - item;
  const int j0 = kt_idx * kBwdKeys;
  const int kw0 = j0 + wave * 32;
  const int my_key = kw0 + l32;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;
  const size_t rowstat = ((size_t)b * H + hh) * N;

  // K and V rows of this lane's key as B operands
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const size_t off = head + (size_t)min(my_key, N - 1) * tok + hi * 8;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 xk = *(const u32x4*)(k + off + cc * 16);
      u32x4 xv = *(const u32x4*)(v + off + cc * 16);
      if (my_key >= N) xk = xv = u32x4{0u, 0u, 0u, 0u};
      kf[cc] = as_bf16x8(xk);
      vf[cc] = as_bf16x8(xv);
    }
  }

  // LDS offsets, computed once per lane.  Q / dO row reads: row t*32 + l%32,
  // chunk 2*cc + hi at (row_base ^ (cc << 5)) + t * 32 * RB.  dS stores: row
  // wave*32 + l%32, queries t*32 + 8*g + 4*hi at dsw_base ^ ((4*t + g) << 4).
  uint32_t row_base = (uint32_t)(l32 * RB + ((hi ^ SW::qd(l32)) * 16));
  uint32_t trq[2], trk[2], trs[2];
  tr_offsets<RB>(lane, [](int r) { return SW::qd(r); }, trq);
  tr_offsets<RB>(lane, [](int r) { return SW::k(r); }, trk);
  tr_offsets<DSB>(lane, [](int r) { return SW::ds(r); }, trs);
  uint32_t dsw_base;
  {
    const int row = wave * 32 + l32;
    dsw_base = (uint32_t)(row * DSB + SW::ds(row) * 16 + 8 * hi);
  }

  // DMA helpers (rows past N repeat row N-1; those rows are masked out).
  // `ln` is the lane index passed through opaque() so that the per-lane
  // addresses are formed at each issue instead of being held in registers.
  auto dma_rows = [&](const uint16_t* src, int n0, uint8_t* dst, int m, int ln, auto swz)
      __attribute__((always_inline)) {
    const int r = m * RPI + ln / CPR, slot = ln % CPR;
    const uint32_t lane_off =
        (uint32_t)(min(r, N - 1 - n0) * (int)tok + (slot ^ swz(r)) * 8);
    const uint16_t* g = src + head + (size_t)n0 * tok + lane_off;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                     (void __attribute__((address_space(3)))*)(dst + m * 1024),
                                     16, 0, 0);
  };
  // Q / dO DMA: this lane's row in the tile and swizzled element offset
  int qd_row[NQI];
  uint32_t qd_col[NQI];
#pragma unroll
  for (int u = 0; u < NQI; ++u) {
    const unsigned ul = (unsigned)lane;
    qd_row[u] = (wave * NQI + u) * RPI + (int)(ul / CPR);
    qd_col[u] = (uint32_t)(((int)(ul % CPR) ^ SW::qd(qd_row[u])) * 8);
  }
  auto issue_step = [&](int it, uint8_t* qd, uint8_t* dod, float* st)
      __attribute__((always_inline)) {
    const int q0 = it * kBwdQueries;
    const int lim = N - 1 - q0;
    const uint16_t* qb = q + head + (size_t)q0 * tok;
    const uint16_t* db = dout + head + (size_t)q0 * tok;
#pragma unroll
    for (int u = 0; u < NQI; ++u) {
      const int m = wave * NQI + u;
      const uint32_t off = (uint32_t)(min(qd_row[u], lim) * (int)tok) + qd_col[u];
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(qb + off),
                                       (void __attribute__((address_space(3)))*)(qd + m * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(db + off),
                                       (void __attribute__((address_space(3)))*)(dod + m * 1024),
                                       16, 0, 0);
    }
    if (wave < 2) {
      const float* src = (wave == 0 ? lse : delta) + rowstat + q0 + min(lane, lim);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)(st + wave * kBwdQueries),
                                       4, 0, 0);
    }
  };

  // The accumulators start as the result of an MFMA (0 * 0 + 0) rather than
  // as literal zeros, so the register allocator places them, and keeps them
  // across the loop, in accumulation registers instead of shuttling them
  // between register files on every iteration.
  f32x16 dk_acc[D / 32], dv_acc[D / 32];
  {
    const bf16x8 z = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      dk_acc[dt] = mfma32(z, z, f32x16{});
      dv_acc[dt] = mfma32(z, z, f32x16{});
    }
  }

  const int n_qtiles = (N + kBwdQueries - 1) / kBwdQueries;
  const int it0 = CAUSAL ? j0 / kBwdQueries : 0;

#pragma unroll
  for (int u = 0; u < NKI; ++u)
    if constexpr (ATOMIC_DQ) dma_rows(k, j0, kt_s, wave * NKI + u, lane, [](int r) { return SW::k(r); });
  if (it0 < n_qtiles) issue_step(it0, q_s0, do_s0, st_s0);
  wait_dma_and_lds();  // the first tiles have landed
  __syncthreads();

  constexpr int kTilesPerWave = D / 64;  // 32x32 dQ tiles per wave per step
  f32x16 dq_pend[kTilesPerWave];
  int q0_pend = -1;  // first query of the pending dQ partial (-1: none)
  auto flush_dq = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) {
      const int tile = wave * kTilesPerWave + u;
      const int t = tile % 2, dt = tile / 2;
      float* dst = dq_acc + head + (size_t)(q0_pend + t * 32) * tok + dt * 32;
      const int lane_off = 4 * hi * (int)tok + l32;
      if (q0_pend + kBwdQueries <= N) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          atomicAdd(dst + (8 * (r / 4) + r % 4) * tok + lane_off, dq_pend[u][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (q0_pend + t * 32 + acc_row(r, hi) < N)
            atomicAdd(dst + (8 * (r / 4) + r % 4) * tok + lane_off, dq_pend[u][r]);
      }
    }
  };

  auto step = [&](int it, const uint8_t* qs, const uint8_t* dos, const float* st, uint8_t* qn,
                  uint8_t* don, float* stn) __attribute__((always_inline)) {
    const int q0 = it * kBwdQueries;
    if (it + 1 < n_qtiles) issue_step(it + 1, qn, don, stn);
    if constexpr (ATOMIC_DQ) if (q0_pend >= 0) flush_dq();
    row_base = opaque(row_base);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      trq[u] = opaque(trq[u]);
      trk[u] = opaque(trk[u]);
      trs[u] = opaque(trs[u]);
    }
    dsw_base = opaque(dsw_base);

    // The 64 queries of the step go in two halves of 32, so only one half's
    // S and dP accumulators are live at a time.
    const bool need_mask =
        (CAUSAL && kw0 + 31 > q0) || (q0 + kBwdQueries > N) || (kw0 + 32 > N);
    const int lo = CAUSAL ? my_key - q0 - 4 * hi : INT_MIN;
    const int hi_lim = my_key < N ? N - q0 - 4 * hi : INT_MIN;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // S = Q K^T and dP = dO V^T for queries t*32 .. t*32+31 x this wave's 32 keys
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const uint32_t off = (row_base ^ (uint32_t)(cc << 5)) + t * 32 * RB;
        s = mfma32(*(const bf16x8*)(qs + off), kf[cc], s);
        dp = mfma32(*(const bf16x8*)(dos + off), vf[cc], dp);
      }
      interleave_lds_mfma<2 * (D / 16), 1, 4>();

      // P = exp2(S*c - L*log2e), dS = P * (dP - D)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = t * 32 + 8 * g + 4 * hi;
        const f32x4 l4 = *(const f32x4*)(st + qr);
        const f32x4 d4 = *(const f32x4*)(st + kBwdQueries + qr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          s[r] = fast_exp2(fmaf(s[r], c, -l4[e] * kLog2e));
          dp[r] = s[r] * (dp[r] - d4[e]);
        }
      }
      // Entry (g, e) is query q0 + 4*hi + C with C = t*32 + 8*g + e, visible
      // iff lo <= C < hi_lim.  Masked entries are set to 0 afterwards, on the
      // diagonal and ragged steps only; the empty volatile asm keeps this a
      // branch (the compiler would otherwise turn it into selects evaluated
      // on every step).
      if (need_mask) {
        asm volatile("");
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int C = t * 32 + 8 * (r / 4) + r % 4;
          if (!(lo <= C && C < hi_lim)) {
            s[r] = 0.f;
            dp[r] = 0.f;
          }
        }
      }
      // dV += P^T dO and dK += dS^T Q: B operands dO^T and Q^T read transposed
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int r0 = 8 * c2;
        const bf16x8 pf = to_bf16x8(f32x8{s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4],
                                          s[r0 + 5], s[r0 + 6], s[r0 + 7]});
        const bf16x8 dsf = to_bf16x8(f32x8{dp[r0], dp[r0 + 1], dp[r0 + 2], dp[r0 + 3],
                                           dp[r0 + 4], dp[r0 + 5], dp[r0 + 6], dp[r0 + 7]});
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          // dV^T += dO^T P, dK^T += Q^T dS: the key on the lane, d down the
          // registers, so the rows leave 16 bytes per lane (store_row_bf16)
          dv_acc[dt] = mfma32(tr_frag<RB>(dos, trq, dt, 2 * t + c2), pf, dv_acc[dt]);
          dk_acc[dt] = mfma32(tr_frag<RB>(qs, trq, dt, 2 * t + c2), dsf, dk_acc[dt]);
        }
      }
      interleave_lds_mfma<2 * 2 * (D / 32), 2, 3>();

      if constexpr (ATOMIC_DQ) {
        // dS (bf16) -> LDS [key][query], 4 consecutive queries per 8-byte store
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x4 x = to_bf16x4(f32x4{dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3]});
          *(u32x2*)(ds_s + (dsw_base ^ (uint32_t)((4 * t + g) << 4))) = __builtin_bit_cast(u32x2, x);
        }
      }
    }

    if constexpr (ATOMIC_DQ) {
    wait_dma_and_lds();
    __syncthreads();

    // dQ partial = dS K over this workgroup's 128 keys (scale is applied
    // when the accumulator is rounded to bf16).  Its atomic
    // adds are issued at the start of the next step (flush_dq), so their
    // round trips overlap that step's work instead of the wait below.
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) {
      const int tile = wave * kTilesPerWave + u;
      const int t = tile % 2, dt = tile / 2;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int cc = 0; cc < kBwdKeys / 16; ++cc) {
        const bf16x8 a = tr_frag<DSB>(ds_s, trs, t, cc);
        const bf16x8 bk = tr_frag<RB>(kt_s, trk, dt, cc);
        acc = mfma32(a, bk, acc);
      }
      interleave_lds_mfma<kBwdKeys / 16, 4, 2>();
      dq_pend[u] = acc;
    }
    q0_pend = q0;
    }
    wait_dma_and_lds();  // next step's tiles have landed
    __syncthreads();
  };
  for (int it = it0; it < n_qtiles; it += 2) {
    step(it, q_s0, do_s0, st_s0, q_s1, do_s1, st_s1);
    if (it + 1 < n_qtiles) step(it + 1, q_s1, do_s1, st_s1, q_s0, do_s0, st_s0);
  }
  if constexpr (ATOMIC_DQ) if (q0_pend >= 0) flush_dq();

  store_row_bf16<D>(dk + head + (size_t)min(my_key, N - 1) * tok, dk_acc, scale, hi, my_key < N);
  store_row_bf16<D>(dv + head + (size_t)min(my_key, N - 1) * tok, dv_acc, 1.0f, hi, my_key < N);
  }
}

// ----------------------------------------------------------- B2 (dQ) ----
// Q-outer dQ pass, the two-pass alternative to the atomic dQ sum (infra-guide
// page "6.2 FlashAttention V2 in depth", section 7.2, "a two-pass scan", read
// as a separate pass over Q tiles).  Shaped like the forward pass: a wave
// owns 32 query rows (Q and dO rows held in VGPRs as MFMA B operands, L and D
// as per-lane scalars) and walks the visible K/V tiles, double-buffered in
// LDS by DMA.  Per tile it recomputes S^T = K Q^T and dP^T = V dO^T, forms
// P^T = exp2(S^T c - L log2 e) and dS^T = P^T (dP^T - D) with the query on
// the lane, and accumulates dQ^T += K^T dS^T, reading K^T transposed from the
// same row-major K tile.  No atomics and no fp32 workspace: each dQ row is
// written once, in bf16, so the result is deterministic.
template <int D>
struct DqSwz {
  // K tile: row reads (A of S^T) and transposed reads (A of dQ^T)
  __device__ static constexpr int k(int r) { return BwdSwz<D>::qd(r); }
  // V tile: row reads only
  __device__ static constexpr int v(int r) { return D == 128 ? (r % 16) : ((r / 2) % 8); }
};

template <int D, int W, bool CAUSAL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(8 / W))) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ o, const float* __restrict__ lse, float* __restrict__ delta,
    uint16_t* __restrict__ dq, int H, int N, int n_qtiles, int grid, float c, float scale) {
  constexpr int BC = 64;                    // keys per K/V tile
  constexpr int BR = W * 32;                // query rows per Q tile
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPI = 1024 / RB;
  constexpr int TILE = BC * RB;
  constexpr int NI = TILE / 1024;
  constexpr int NIW = NI / W;
  static_assert(NI % W == 0 && NIW >= 1, "tile split");
  using SW = DqSwz<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;

  // causal work items pair a heavy and a light Q tile, as in the forward pass
  const int logical = xcd_contiguous_id(blockIdx.x, grid);
  const int per_head = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;
  const int bh = logical / per_head;
  const int item = logical % per_head;
  const int n_pass = (CAUSAL && item != n_qtiles - 1 - item) ? 2 : 1;
  const int b = bh / H, hh = bh % H;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;
  const size_t rowstat = ((size_t)b * H + hh) * N;

  uint32_t koff[NIW], voff[NIW];
  int lrow[NIW];
#pragma unroll
  for (int u = 0; u < NIW; ++u) {
    const int m = wave * NIW + u;
    const int r = m * RPI + lane / CPR, slot = lane % CPR;
    lrow[u] = r;
    koff[u] = (uint32_t)(r * tok * 2) + (uint32_t)((slot ^ SW::k(r)) * 16);
    voff[u] = (uint32_t)(r * tok * 2) + (uint32_t)((slot ^ SW::v(r)) * 16);
  }
  auto issue = [&](int jt, uint8_t* kd, uint8_t* vd) __attribute__((always_inline)) {
    const int kv0 = jt * BC;
    const uint8_t* kbase = (const uint8_t*)(k + head + (size_t)kv0 * tok);
    const uint8_t* vbase = (const uint8_t*)(v + head + (size_t)kv0 * tok);
    const bool whole = kv0 + BC <= N;
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
      const int m = wave * NIW + u;
      uint32_t ko = koff[u], vo = voff[u];
      if (!whole) {
        const uint32_t back = (uint32_t)(max(kv0 + lrow[u] - (N - 1), 0) * tok * 2);
        ko -= back;
        vo -= back;
      }
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(kbase + ko),
                                       (void __attribute__((address_space(3)))*)(kd + m * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(vbase + vo),
                                       (void __attribute__((address_space(3)))*)(vd + m * 1024), 16, 0, 0);
    }
  };

  // LDS read offsets: K / V row kt*32 + l%32, chunk 2*cc + hi at
  // (base ^ (cc << 5)) + kt*32*RB; K^T fragment (cc, dt), half u at
  // (ktr[u] ^ (dt << 6)) + cc*16*RB.
  uint32_t k_row = (uint32_t)(l32 * RB + ((hi ^ SW::k(l32)) * 16));
  uint32_t v_row = (uint32_t)(l32 * RB + ((hi ^ SW::v(l32)) * 16));
  uint32_t ktr[2];
  tr_offsets<RB>(lane, [](int r) { return SW::k(r); }, ktr);

  for (int pass = 0; pass < n_pass; ++pass) {
    const int qt = CAUSAL ? (pass == 0 ? n_qtiles - 1 - item : item) : item;
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + l32;
    const int qc = min(my_q, N - 1);

    bf16x8 qf[D / 16], dof[D / 16];
    {
      const uint16_t* qp = q + head + (size_t)qc * tok + 8 * hi;
      const uint16_t* dp_ = dout + head + (size_t)qc * tok + 8 * hi;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        u32x4 x = *(const u32x4*)(qp + 16 * cc);
        u32x4 y = *(const u32x4*)(dp_ + 16 * cc);
        if (my_q >= N) x = y = u32x4{0u, 0u, 0u, 0u};
        qf[cc] = as_bf16x8(x);
        dof[cc] = as_bf16x8(y);
      }
    }
    const float l2 = lse[rowstat + qc] * kLog2e;
    // D_i = rowsum(dO_i * O_i) (section 7.3), computed here from the rows
    // this wave already holds and written once for the KV-outer pass: the
    // two lane halves hold the two halves of the row
    float dd;
    {
      const uint16_t* op = o + head + (size_t)qc * tok + 8 * hi;
      float part = 0.f;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const u32x4 ox = *(const u32x4*)(op + 16 * cc);
        const u32x4 gx = as_u32x4(dof[cc]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          part += __uint_as_float(ox[t] << 16) * __uint_as_float(gx[t] << 16);
          part += __uint_as_float(ox[t] & 0xffff0000u) * __uint_as_float(gx[t] & 0xffff0000u);
        }
      }
      dd = pair_sum(part);
      if (my_q < N && hi == 0) delta[rowstat + my_q] = dd;
    }

    const int kv_len = CAUSAL ? min(N, q0 + BR) : N;
    const int n_kv = (kv_len + BC - 1) / BC;

    f32x16 dqa[D / 32];
    {
      const bf16x8 z = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) dqa[dt] = mfma32(z, z, f32x16{});
    }

    auto tile = [&](int jt, const uint8_t* kb, const uint8_t* vb) __attribute__((always_inline)) {
      const int kv0 = jt * BC;
      k_row = opaque(k_row);
      v_row = opaque(v_row);
      ktr[0] = opaque(ktr[0]);
      ktr[1] = opaque(ktr[1]);
      f32x16 s[BC / 32], dp[BC / 32];
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt) {
        s[kt] = f32x16{};
        dp[kt] = f32x16{};
      }
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc)
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt) {
          const uint32_t ko = (k_row ^ (uint32_t)(cc << 5)) + kt * 32 * RB;
          const uint32_t vo = (v_row ^ (uint32_t)(cc << 5)) + kt * 32 * RB;
          s[kt] = mfma32(*(const bf16x8*)(kb + ko), qf[cc], s[kt]);
          dp[kt] = mfma32(*(const bf16x8*)(vb + vo), dof[cc], dp[kt]);
        }
      interleave_lds_mfma<2 * (D / 16) * (BC / 32), 1, 4>();

      // P^T, dS^T (query on the lane); keys past the diagonal or N give 0
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > qw0) || (kv0 + BC > N);
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(s[kt][r], c, -l2));
          dp[kt][r] = pr * (dp[kt][r] - dd);
        }
      // masked entries of dS are set to 0 afterwards, on the diagonal and
      // ragged tiles only; the empty volatile asm keeps this a branch
      if (need_mask) {
        asm volatile("");
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kt * 32 + acc_row(r, hi);
            if (!(key < N && (!CAUSAL || key <= my_q))) dp[kt][r] = 0.f;
          }
      }

      // dQ^T += K^T dS^T
#pragma unroll
      for (int cc = 0; cc < BC / 16; ++cc) {
        const f32x16& sv = dp[cc / 2];
        const int r0 = 8 * (cc % 2);
        const bf16x8 dsf = to_bf16x8(f32x8{sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3], sv[r0 + 4],
                                           sv[r0 + 5], sv[r0 + 6], sv[r0 + 7]});
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) dqa[dt] = mfma32(tr_frag<RB>(kb, ktr, dt, cc), dsf, dqa[dt]);
      }
      interleave_lds_mfma<(BC / 16) * (D / 32), 2, 3>();
    };

    if (n_kv > 0) issue(0, kb0, vb0);
    wait_dma_and_lds();  // tile 0 has landed
    __syncthreads();
    auto step = [&](int jt, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn)
        __attribute__((always_inline)) {
      issue(min(jt + 1, n_kv - 1), kn, vn);
      if (!CAUSAL || jt * BC <= qw0 + 31) tile(jt, kc, vc);
      wait_dma_and_lds();  // tile jt+1 has landed
      __syncthreads();
    };
    for (int jt = 0; jt < n_kv; jt += 2) {
      step(jt, kb0, vb0, kb1, vb1);
      if (jt + 1 < n_kv) step(jt + 1, kb1, vb1, kb0, vb0);
    }

    store_row_bf16<D>(dq + head + (size_t)qc * tok, dqa, scale, hi, my_q < N);
  }
}

// ----------------------------------------------------- B1, d = 128 ----
// KV-outer dK/dV pass of the two-pass backward for d = 128, with two waves
// per SIMD.  bwd_dl_kernel keeps K and V of its 32 keys in VGPRs and both
// 32-query halves of a step in one wave: about 360 registers, so one wave per
// SIMD and no other wave to run while it waits.  Here a workgroup has 8 waves
// over the same 128 keys: wave w owns key block w % 4 and, of every 64-query
// step, the half w / 4.  K rows stay in VGPRs (B operand of S); the V rows of
// the 128 keys go to LDS once per work item and are read as the B operand of
// dP (row reads, swizzled like the dQ pass's V tile).  That brings a wave
// under 256 registers.  The two waves of a key block each hold a dK/dV partial
// over their query halves; at the end one adds the other's through LDS and
// writes the result, so each element is still written once and the pass stays
// deterministic.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int H, int N, int n_ktiles, int grid, float c, float scale) {
  constexpr int kWaves = 8;
  constexpr int RB = D * 2;                  // bytes per row
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;             // rows per 1 KB DMA instruction
  constexpr int QT = kBwdQueries * RB;       // bytes of a Q or dO tile
  constexpr int VT = kBwdKeys * RB;          // bytes of the V tile
  constexpr int NQI = QT / 1024 / kWaves;    // Q (and dO) DMA instructions per wave
  constexpr int NVI = VT / 1024 / kWaves;    // V DMA instructions per wave
  constexpr int DT = D / 32;
  static_assert(NQI >= 1 && NVI >= 1, "tile split");
  static_assert(16 * DT * 64 * 4 <= QT, "a wave's dK or dV partial fits one Q/dO buffer");
  using SW = BwdSwz<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t v_s[VT];
  __shared__ __attribute__((aligned(1024))) uint8_t q_s0[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t q_s1[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t do_s0[QT];
  __shared__ __attribute__((aligned(1024))) uint8_t do_s1[QT];
  __shared__ __attribute__((aligned(256))) float st_s0[2 * kBwdQueries];  // lse | delta
  __shared__ __attribute__((aligned(256))) float st_s1[2 * kBwdQueries];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;
  const int kb = wave % 4;   // key block of the wave
  const int qh = wave / 4;   // query half of every step

  const int logical = xcd_contiguous_id(blockIdx.x, grid);
  const int per_head = CAUSAL ? (n_ktiles + 1) / 2 : n_ktiles;
  const int bh = logical / per_head;
  const int item = logical % per_head;
  const int n_pass = (CAUSAL && item != n_ktiles - 1 - item) ? 2 : 1;
  const int b = bh / H, hh = bh % H;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;
  const size_t rowstat = ((size_t)b * H + hh) * N;

  // Q / dO DMA: this lane's row in the tile and swizzled element offset
  int qd_row[NQI];
  uint32_t qd_col[NQI];
#pragma unroll
  for (int u = 0; u < NQI; ++u) {
    const unsigned ul = (unsigned)lane;
    qd_row[u] = (wave * NQI + u) * RPI + (int)(ul / CPR);
    qd_col[u] = (uint32_t)(((int)(ul % CPR) ^ SW::qd(qd_row[u])) * 8);
  }
  auto issue_step = [&](int it, uint8_t* qd, uint8_t* dod, float* st)
      __attribute__((always_inline)) {
    const int q0 = it * kBwdQueries;
    const int lim = N - 1 - q0;
    const uint16_t* qb = q + head + (size_t)q0 * tok;
    const uint16_t* db = dout + head + (size_t)q0 * tok;
#pragma unroll
    for (int u = 0; u < NQI; ++u) {
      const int m = wave * NQI + u;
      const uint32_t off = (uint32_t)(min(qd_row[u], lim) * (int)tok) + qd_col[u];
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(qb + off),
                                       (void __attribute__((address_space(3)))*)(qd + m * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(db + off),
                                       (void __attribute__((address_space(3)))*)(dod + m * 1024),
                                       16, 0, 0);
    }
    if (wave < 2) {
      const float* src = (wave == 0 ? lse : delta) + rowstat + q0 + min(lane, lim);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)(st + wave * kBwdQueries),
                                       4, 0, 0);
    }
  };

  // LDS read offsets, once per lane.  Q / dO rows: row t*32 + l%32, chunk
  // 2*cc + hi at (row_base ^ (cc << 5)) + t * 32 * RB.  V rows (B operand of
  // dP): key kb*32 + l%32, chunk 2*cc + hi at vrow_base ^ (cc << 5); the V
  // swizzle depends on the row's low bits only.
  uint32_t row_base = (uint32_t)(l32 * RB + ((hi ^ SW::qd(l32)) * 16));
  uint32_t vrow_base = (uint32_t)(kb * 32 * RB + l32 * RB + ((hi ^ DqSwz<D>::v(l32)) * 16));
  uint32_t trq[2];
  tr_offsets<RB>(lane, [](int r) { return SW::qd(r); }, trq);

  for (int pass = 0; pass < n_pass; ++pass) {
    const int kt_idx = pass == 0 ? item : n_ktiles - 1 - item;
    const int j0 = kt_idx * kBwdKeys;
    const int kw0 = j0 + kb * 32;
    const int my_key = kw0 + l32;

    // V rows of the workgroup's 128 keys -> LDS (rows past N repeat row N-1)
#pragma unroll
    for (int u = 0; u < NVI; ++u) {
      const int m = wave * NVI + u;
      const int r = m * RPI + lane / CPR, slot = lane % CPR;
      const uint32_t off =
          (uint32_t)(min(r, N - 1 - j0) * (int)tok) + (uint32_t)((slot ^ DqSwz<D>::v(r)) * 8);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(v + head + (size_t)j0 * tok + off),
          (void __attribute__((address_space(3)))*)(v_s + m * 1024), 16, 0, 0);
    }
    const int n_qtiles = (N + kBwdQueries - 1) / kBwdQueries;
    const int it0 = CAUSAL ? j0 / kBwdQueries : 0;
    if (it0 < n_qtiles) issue_step(it0, q_s0, do_s0, st_s0);

    // K rows of this lane's key as B operands of S
    bf16x8 kf[D / 16];
    {
      const size_t off = head + (size_t)min(my_key, N - 1) * tok + hi * 8;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        u32x4 xk = *(const u32x4*)(k + off + cc * 16);
        if (my_key >= N) xk = u32x4{0u, 0u, 0u, 0u};
        kf[cc] = as_bf16x8(xk);
      }
    }

    f32x16 dk_acc[DT], dv_acc[DT];
    {
      const bf16x8 z = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dk_acc[dt] = mfma32(z, z, f32x16{});
        dv_acc[dt] = mfma32(z, z, f32x16{});
      }
    }
    wait_dma_and_lds();  // the first tiles have landed
    __syncthreads();

    auto step = [&](int it, const uint8_t* qs, const uint8_t* dos, const float* st, uint8_t* qn,
                    uint8_t* don, float* stn) __attribute__((always_inline)) {
      const int q0 = it * kBwdQueries;
      if (it + 1 < n_qtiles) issue_step(it + 1, qn, don, stn);
      row_base = opaque(row_base);
      vrow_base = opaque(vrow_base);
      trq[0] = opaque(trq[0]);
      trq[1] = opaque(trq[1]);
      const int qw = q0 + qh * 32;  // first query of this wave's half
      {
        const bool need_mask = (CAUSAL && kw0 + 31 > qw) || (qw + 32 > N) || (kw0 + 32 > N);
        const int lo = CAUSAL ? my_key - q0 - 4 * hi : INT_MIN;
        const int hi_lim = my_key < N ? N - q0 - 4 * hi : INT_MIN;
        const int t = qh;
        f32x16 s = f32x16{}, dp = f32x16{};
        // Q, dO and V fragments two chunks ahead, fenced so the compiler
        // neither hoists every read nor holds their registers
        bf16x8 qa[2], da[2], va[2];
        auto load = [&](int cc, int slot) __attribute__((always_inline)) {
          const uint32_t off = (row_base ^ (uint32_t)(cc << 5)) + t * 32 * RB;
          qa[slot] = *(const bf16x8*)(qs + off);
          da[slot] = *(const bf16x8*)(dos + off);
          va[slot] = *(const bf16x8*)(v_s + (vrow_base ^ (uint32_t)(cc << 5)));
        };
        load(0, 0);
        load(1, 1);
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          s = mfma32(qa[cc % 2], kf[cc], s);
          dp = mfma32(da[cc % 2], va[cc % 2], dp);
          if (cc + 2 < D / 16) load(cc + 2, cc % 2);
          __builtin_amdgcn_sched_barrier(0);
        }

        // P = exp2(S*c - L*log2e), dS = P * (dP - D)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qr = t * 32 + 8 * g + 4 * hi;
          const f32x4 l4 = *(const f32x4*)(st + qr);
          const f32x4 d4 = *(const f32x4*)(st + kBwdQueries + qr);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            s[r] = fast_exp2(fmaf(s[r], c, -l4[e] * kLog2e));
            dp[r] = s[r] * (dp[r] - d4[e]);
          }
        }
        // Masked entries (C = t*32 + 8g + e outside [lo, hi_lim)) are set to 0
        // afterwards, on the diagonal and ragged steps only.  The empty
        // volatile asm keeps this a branch: the compiler would otherwise
        // turn it into selects evaluated on every step.
        if (need_mask) {
          asm volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int C = t * 32 + 8 * (r / 4) + r % 4;
            if (!(lo <= C && C < hi_lim)) {
              s[r] = 0.f;
              dp[r] = 0.f;
            }
          }
        }

        // dV^T += dO^T P and dK^T += Q^T dS over the wave's 32 queries: the
        // same fragments as dV = P^T dO with the operands swapped (the
        // 32x32x16 MFMA's A rows and B columns take the same lane layout),
        // so the key stays on the lane and d runs down the registers; the
        // transposed dO / Q fragments run one product pair ahead
        bf16x8 pf[2], dsf[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int r0 = 8 * c2;
          pf[c2] = to_bf16x8(f32x8{s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4], s[r0 + 5],
                                   s[r0 + 6], s[r0 + 7]});
          dsf[c2] = to_bf16x8(f32x8{dp[r0], dp[r0 + 1], dp[r0 + 2], dp[r0 + 3], dp[r0 + 4],
                                    dp[r0 + 5], dp[r0 + 6], dp[r0 + 7]});
        }
        constexpr int kPairs = 2 * DT;  // (c2, dt) pairs
        bf16x8 ofr[2], qfr[2];
        auto tload = [&](int i, int slot) __attribute__((always_inline)) {
          const int c2 = i / DT, dt = i % DT;
          ofr[slot] = tr_frag<RB>(dos, trq, dt, 2 * t + c2);
          qfr[slot] = tr_frag<RB>(qs, trq, dt, 2 * t + c2);
        };
        tload(0, 0);
        tload(1, 1);
#pragma unroll
        for (int i = 0; i < kPairs; ++i) {
          const int c2 = i / DT, dt = i % DT;
          dv_acc[dt] = mfma32(ofr[i % 2], pf[c2], dv_acc[dt]);
          dk_acc[dt] = mfma32(qfr[i % 2], dsf[c2], dk_acc[dt]);
          if (i + 2 < kPairs) tload(i + 2, i % 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_dma_and_lds();  // next step's tiles have landed
      __syncthreads();
    };
    for (int it = it0; it < n_qtiles; it += 2) {
      step(it, q_s0, do_s0, st_s0, q_s1, do_s1, st_s1);
      if (it + 1 < n_qtiles) step(it + 1, q_s1, do_s1, st_s1, q_s0, do_s0, st_s0);
    }

    // The two waves of a key block add their partials through LDS (the Q/dO
    // buffers are free now): the upper half stores, the lower half adds and
    // writes out.  The accumulators hold dK^T and dV^T (the key on the lane,
    // d in the registers, as O^T in the forward pass), so a partial moves as
    // 16-byte chunks in [chunk][lane] order (conflict-free), and the sum
    // leaves through store_row_bf16: 16 bytes of a key's row per lane.
    uint8_t* const red = kb == 0 ? q_s0 : kb == 1 ? q_s1 : kb == 2 ? do_s0 : do_s1;
    auto put = [&](const f32x16* acc) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          ((f32x4*)red)[(dt * 4 + g) * 64 + lane] =
              f32x4{acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]};
    };
    auto add_store = [&](f32x16* acc, uint16_t* dst, float mul) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 other = ((const f32x4*)red)[(dt * 4 + g) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[dt][4 * g + i] += other[i];
        }
      store_row_bf16<D>(dst + head + (size_t)min(my_key, N - 1) * tok, acc, mul, hi, my_key < N);
    };
    // No DMA is in flight here (the last step issued none), so the barriers
    // wait for LDS accesses only and the dK/dV stores drain in the background.
    if (qh == 1) put(dk_acc);
    wait_lds();
    __syncthreads();
    if (qh == 0) add_store(dk_acc, dk, scale);
    wait_lds();
    __syncthreads();
    if (qh == 1) put(dv_acc);
    wait_lds();
    __syncthreads();
    if (qh == 0) add_store(dv_acc, dv, 1.0f);
    wait_lds();
    __syncthreads();
  }
}

template <int D, bool CAUSAL>
void launch_kv_pair(const BwdParams& p) {
  const int n_ktiles = (p.N + kBwdKeys - 1) / kBwdKeys;
  const long long grid = (long long)p.B * p.H * (CAUSAL ? (n_ktiles + 1) / 2 : n_ktiles);
  const float c = (float)((double)p.scale * 1.4426950408889634);
  hipLaunchKernelGGL((bwd_kv_pair_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(512), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (const uint16_t*)p.dout, p.lse, p.delta, (uint16_t*)p.dk, (uint16_t*)p.dv,
                     p.H, p.N, n_ktiles, (int)grid, c, p.scale);
}


// B0 launch: D (and, for the atomic dQ sum, the zeroed accumulator)
template <int D, bool ZERO_DQ>
void launch_preprocess(const BwdParams& p) {
  const long long rows = (long long)p.B * p.N * p.H;
  const long long blocks = (rows + 15) / 16;
  hipLaunchKernelGGL((bwd_preprocess_kernel<D, ZERO_DQ>), dim3((unsigned)blocks), dim3(256), 0,
                     p.stream, (const uint16_t*)p.o, (const uint16_t*)p.dout, p.delta, p.dq_acc,
                     p.H, p.N, rows);
}

template <int D, bool CAUSAL, bool ATOMIC_DQ>
void launch_kv_outer(const BwdParams& p) {
  const int n_ktiles = (p.N + kBwdKeys - 1) / kBwdKeys;
  const long long grid = (long long)p.B * p.H * (CAUSAL ? (n_ktiles + 1) / 2 : n_ktiles);
  const float c = (float)((double)p.scale * 1.4426950408889634);
  hipLaunchKernelGGL((bwd_dl_kernel<D, CAUSAL, ATOMIC_DQ>), dim3((unsigned)grid), dim3(kBwdThreads),
                     0, p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (const uint16_t*)p.dout, p.lse, p.delta, p.dq_acc, (uint16_t*)p.dk,
                     (uint16_t*)p.dv, p.H, p.N, n_ktiles, (int)grid, c, p.scale);
}

template <int D, int W, bool CAUSAL>
void launch_dq_pass(const BwdParams& p) {
  constexpr int BR = W * 32;
  const int n_qtiles = (p.N + BR - 1) / BR;
  const long long grid = (long long)p.B * p.H * (CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles);
  const float c = (float)((double)p.scale * 1.4426950408889634);
  hipLaunchKernelGGL((bwd_dq_kernel<D, W, CAUSAL>), dim3((unsigned)grid), dim3(W * 64), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (const uint16_t*)p.dout, (const uint16_t*)p.o, p.lse, p.delta,
                     (uint16_t*)p.dq, p.H, p.N, n_qtiles, (int)grid, c, p.scale);
}

// dQ summed with fp32 atomics across the KV-outer workgroups, then converted
template <int D, bool CAUSAL>
hipError_t launch_bwd_atomic(const BwdParams& p) {
  (void)hipGetLastError();
  launch_preprocess<D, true>(p);
  launch_kv_outer<D, CAUSAL, true>(p);
  const long long n8 = (long long)p.B * p.N * p.H * D / 8;
  hipLaunchKernelGGL(bwd_convert_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                     p.stream, p.dq_acc, (uint16_t*)p.dq, n8, p.scale);
  return hipGetLastError();
}

// dQ from its own Q-outer pass (no atomics, no fp32 accumulator).  That pass
// runs first and also computes D (the pre-processing step folded into it),
// which the KV-outer dK/dV pass then reads.
template <int D, bool CAUSAL>
hipError_t launch_bwd_two_pass(const BwdParams& p) {
  (void)hipGetLastError();
  if (bwd_dq_waves(p.B, p.H, p.N, p.causal) == 4) launch_dq_pass<D, 4, CAUSAL>(p);
  else launch_dq_pass<D, 8, CAUSAL>(p);
  // d = 128: the 8-wave pass (two waves per SIMD); d = 64 fits two 4-wave
  // workgroups per CU already, where the 4-wave pass measures faster
  if constexpr (D == 128) launch_kv_pair<D, CAUSAL>(p);
  else launch_kv_outer<D, CAUSAL, false>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p) {
  if (p.d == 64)
    return p.causal ? launch_bwd_two_pass<64, true>(p) : launch_bwd_two_pass<64, false>(p);
  return p.causal ? launch_bwd_two_pass<128, true>(p) : launch_bwd_two_pass<128, false>(p);
}

hipError_t launch_bwd_atomic_dq(const BwdParams& p) {
  if (p.d == 64)
    return p.causal ? launch_bwd_atomic<64, true>(p) : launch_bwd_atomic<64, false>(p);
  return p.causal ? launch_bwd_atomic<128, true>(p) : launch_bwd_atomic<128, false>(p);
}

}  // namespace fa2
