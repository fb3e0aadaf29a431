// fa2_fa1_order.hip -- an ablation of the forward pass in FlashAttention-1's
// loop order, to measure on gfx950 what FlashAttention-2's changes buy.
//
// Pages: "FlashAttention Implementation > FlashAttention-2 Improvements"
// ("Reduced Non-Matrix-Multiply FLOPs", "Improved Memory Access") and infra
// guide "6.2 FlashAttention V2 in depth", sections 2.1 and 3.1-3.3: the first
// version walks K/V tiles in the outer loop and Q tiles in the inner loop, so
// every (K/V tile, Q tile) step reloads the Q tile and reads and writes back
// the O tile and its row statistics; it keeps O normalised after every step
// (rescale by the old sum, add P V, divide by the new sum); and it can only
// spread work over batch x heads.  This kernel does exactly that, and nothing
// else differently from the shipping forward kernel: same MFMA mapping, same
// LDS layout and DMA, the same exp2 softmax, 32
// query rows per wave (the warp partition of section 4 is not part of this
// ablation).  The O state
// between steps is kept in fp32 in a caller workspace, so the result matches
// the shipping kernel's to rounding.
#include <math.h>

#include "fa2_device.hpp"
#include "fa2_internal.hpp"

namespace fa2 {
namespace {

template <int D>
struct Fa1Swz {
  __device__ static constexpr int k(int r) { return D == 128 ? (r % 16) : ((r / 2) % 8); }
  __device__ static constexpr int v(int r) { return D == 128 ? 4 * (r % 4) : 4 * ((r / 2) % 2); }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void fa1_order_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ o_state, float* __restrict__ ml_state, int H, int N, float c,
    uint32_t q_and, uint32_t q_xor) {
  constexpr int W = 8;
  constexpr int BR = W * 32;                // Q tile rows (inner loop)
  constexpr int BC = 64;                    // K/V tile keys (outer loop)
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPI = 1024 / RB;
  constexpr int TILE = BC * RB;
  constexpr int NIW = TILE / 1024 / W;
  static_assert(NIW >= 1, "tile split");
  using SW = Fa1Swz<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;

  // one workgroup per (batch, head): the first version's parallelism
  const int bh = blockIdx.x;
  const int b = bh / H, hh = bh % H;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;
  const size_t rowstat = ((size_t)b * H + hh) * N;
  const int n_kv = (N + BC - 1) / BC;
  const int n_qt = (N + BR - 1) / BR;

  for (int jt = 0; jt < n_kv; ++jt) {
    const int kv0 = jt * BC;
    // load K_j, V_j (every wave is done with the previous tile)
    wait_dma_and_lds();
    __syncthreads();
    {
      const uint8_t* kbase = (const uint8_t*)(k + head + (size_t)kv0 * tok);
      const uint8_t* vbase = (const uint8_t*)(v + head + (size_t)kv0 * tok);
#pragma unroll
      for (int u = 0; u < NIW; ++u) {
        const int m = wave * NIW + u;
        const int r = m * RPI + lane / CPR, slot = lane % CPR;
        const size_t row = (size_t)min(kv0 + r, N - 1) - kv0;
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(kbase + row * tok * 2 +
                                                            (slot ^ SW::k(r)) * 16),
            (void __attribute__((address_space(3)))*)(kb + m * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(vbase + row * tok * 2 +
                                                            (slot ^ SW::v(r)) * 16),
            (void __attribute__((address_space(3)))*)(vb + m * 1024), 16, 0, 0);
      }
    }
    wait_dma_and_lds();  // the first tiles have landed
    __syncthreads();

    const int it0 = CAUSAL ? kv0 / BR : 0;  // first Q tile that sees this K/V tile
    for (int it = it0; it < n_qt; ++it) {
      const int qw0 = it * BR + wave * 32;
      const int my_q = qw0 + l32;
      if (CAUSAL && kv0 > qw0 + 31) continue;  // the whole tile is above these rows
      const int last_jt = CAUSAL ? min(n_kv - 1, (qw0 + 31) / BC) : n_kv - 1;
      const int qc = min(my_q, N - 1);

      // reload the Q rows and the O state of these rows
      bf16x8 qf[D / 16];
      {
        const uint16_t* qp = q + head + (size_t)qc * tok + 8 * hi;
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          u32x4 x = *(const u32x4*)(qp + 16 * cc);
          if (my_q >= N) x = u32x4{0u, 0u, 0u, 0u};
          x = (x & q_and) ^ q_xor;
          qf[cc] = as_bf16x8(x);
        }
      }
      f32x16 oacc[D / 32];
      float m_old = -INFINITY, l_old = 0.f;
      float* os = o_state + head + (size_t)qc * tok;
      float* ms = ml_state + 2 * (rowstat + qc);
      if (jt == 0) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
      } else {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 x = *(const f32x4*)(os + dt * 32 + 8 * g + 4 * hi);
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[dt][4 * g + e] = x[e];
          }
        m_old = ms[0];
        l_old = ms[1];
      }

      // S^T = K Q^T
      f32x16 s[BC / 32];
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt) s[kt] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc)
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt) {
          const int r = kt * 32 + l32;
          const bf16x8 a = *(const bf16x8*)(kb + r * RB + ((cc * 2 + hi) ^ SW::k(r)) * 16);
          s[kt] = mfma32(a, qf[cc], s[kt]);
        }
      if ((CAUSAL && kv0 + BC - 1 > qw0) || kv0 + BC > N) {
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kt * 32 + acc_row(r, hi);
            if (!(key < N && (!CAUSAL || key <= my_q))) s[kt][r] = -INFINITY;
          }
      }
      float mx = lane_max<BC / 2>(s);
      mx = pair_max(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
      const float m_new = fmaxf(m_old, mt);
      const float mref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - mref);

      // un-normalise the old O (times l_old * alpha), add P V, normalise again
      const float undo = l_old * alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= undo;
      const int g16 = lane / 16, i4 = (lane % 16) / 4, a4 = lane % 4;
      float rs = 0.f;
#pragma unroll
      for (int cc = 0; cc < BC / 16; ++cc) {
        const f32x16& sv = s[cc / 2];
        const int r0 = 8 * (cc % 2);
        f32x8 p8;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p8[t] = fast_exp2(fmaf(sv[r0 + t], c, -mref));
          rs += p8[t];
        }
        const bf16x8 pcur = to_bf16x8(p8);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int col = dt * 32 + 16 * (g16 % 2) + 4 * a4;
          u32x2 part[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int R = 16 * cc + 8 * u + 4 * hi + i4;
            const uint8_t* addr = vb + R * RB + (((col / 8) ^ SW::v(R)) * 16) + (col % 8) * 2;
            part[u] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (short __attribute__((ext_vector_type(4))) __attribute__((address_space(3)))*)addr));
          }
          oacc[dt] = mfma32(as_bf16x8(u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}),
                            pcur, oacc[dt]);
        }
      }
      const float l_new = undo + pair_sum(rs);
      const float inv = 1.0f / l_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= inv;

      if (my_q < N) {
        if (jt == last_jt) {  // these rows have seen every visible key: final O and L
          uint16_t* op = o + head + (size_t)my_q * tok;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 x = f32x4{oacc[dt][4 * g + 0], oacc[dt][4 * g + 1], oacc[dt][4 * g + 2],
                                    oacc[dt][4 * g + 3]};
              *(u32x2*)(op + dt * 32 + 8 * g + 4 * hi) = __builtin_bit_cast(u32x2, to_bf16x4(x));
            }
          if (hi == 0) lse[rowstat + my_q] = (m_new + log2f(l_new)) * kLn2;
        } else {  // write the normalised O and the row statistics back
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *(f32x4*)(os + dt * 32 + 8 * g + 4 * hi) =
                  f32x4{oacc[dt][4 * g + 0], oacc[dt][4 * g + 1], oacc[dt][4 * g + 2],
                        oacc[dt][4 * g + 3]};
          if (hi == 0) {
            ms[0] = m_new;
            ms[1] = l_new;
          }
        }
      }
    }
  }
}

// FlashAttention-1's warp partition on top of its loop order ("6.2
// FlashAttention V2 in depth", sections 4.1-4.3; "FlashAttention
// Implementation", "Better Work Partitioning"): the waves of a workgroup do
// not own query rows; they share the Q tile and split each K/V tile between
// them ("split-K").  Each wave forms the scores of the 32 Q rows against its
// own 32 keys, a partial softmax over those keys (its max m_w, sum l_w) and a
// partial output O_w = P_w V_w; the partials then meet in LDS, where
//   m = max(m_old, max_w m_w),  l = l_old 2^(m_old - m) + sum_w l_w 2^(m_w - m),
//   O = (l_old 2^(m_old - m) O_old + sum_w 2^(m_w - m) O_w) / l,
// with O_old (normalised), m_old and l_old read from and written back to the
// workspace at every step, as in fa1_order_kernel.  4 waves = 128 keys per
// K/V tile (outer loop), 32 Q rows per step (inner loop), one workgroup per
// (batch, head).  The merge is the cross-wave communication the split-Q
// partition of FlashAttention-2 removes.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void fa1_splitk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ o_state, float* __restrict__ ml_state, int H, int N, float c,
    uint32_t q_and, uint32_t q_xor) {
  constexpr int W = 4;
  constexpr int BC = W * 32;                // K/V tile keys (outer loop), 32 per wave
  constexpr int BQ = 32;                    // Q rows per step (inner loop), shared by the waves
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPI = 1024 / RB;
  constexpr int TILE = BC * RB;
  constexpr int NIW = TILE / 1024 / W;
  constexpr int DT = D / 32;
  constexpr int OSTRIDE = D + 4;            // floats per row of a wave's partial O (padded)
  static_assert(NIW >= 1, "tile split");
  using SW = Fa1Swz<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb[TILE];
  __shared__ __attribute__((aligned(16))) float ob[W * BQ * OSTRIDE];  // O_w[query][d]
  __shared__ __attribute__((aligned(16))) float mb[W * BQ];            // m_w (log2 units)
  __shared__ __attribute__((aligned(16))) float lb[W * BQ];            // l_w

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;

  const int bh = blockIdx.x;
  const int b = bh / H, hh = bh % H;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;
  const size_t rowstat = ((size_t)b * H + hh) * N;
  const int n_kv = (N + BC - 1) / BC;
  const int n_qt = (N + BQ - 1) / BQ;
  const int g16 = lane / 16, i4 = (lane % 16) / 4, a4 = lane % 4;

  for (int jt = 0; jt < n_kv; ++jt) {
    const int kv0 = jt * BC;
    const int kw0 = kv0 + wave * 32;  // this wave's keys: kw0 .. kw0 + 31
    wait_dma_and_lds();
    __syncthreads();  // every wave is done with the previous K/V tile
    {
      const uint8_t* kbase = (const uint8_t*)(k + head + (size_t)kv0 * tok);
      const uint8_t* vbase = (const uint8_t*)(v + head + (size_t)kv0 * tok);
#pragma unroll
      for (int u = 0; u < NIW; ++u) {
        const int m = wave * NIW + u;
        const int r = m * RPI + lane / CPR, slot = lane % CPR;
        const size_t row = (size_t)min(kv0 + r, N - 1) - kv0;
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(kbase + row * tok * 2 +
                                                            (slot ^ SW::k(r)) * 16),
            (void __attribute__((address_space(3)))*)(kb + m * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(vbase + row * tok * 2 +
                                                            (slot ^ SW::v(r)) * 16),
            (void __attribute__((address_space(3)))*)(vb + m * 1024), 16, 0, 0);
      }
    }
    wait_dma_and_lds();
    __syncthreads();

    const int it0 = CAUSAL ? kv0 / BQ : 0;  // first Q tile that sees this K/V tile
    for (int it = it0; it < n_qt; ++it) {
      const int q0 = it * BQ;
      const int my_q = q0 + l32;
      const int qc = min(my_q, N - 1);
      const int last_jt = CAUSAL ? min(n_kv - 1, (q0 + BQ - 1) / BC) : n_kv - 1;

      // every wave reloads the same Q rows (B operand: this lane's query)
      bf16x8 qf[D / 16];
      {
        const uint16_t* qp = q + head + (size_t)qc * tok + 8 * hi;
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          u32x4 x = *(const u32x4*)(qp + 16 * cc);
          if (my_q >= N) x = u32x4{0u, 0u, 0u, 0u};
          x = (x & q_and) ^ q_xor;
          qf[cc] = as_bf16x8(x);
        }
      }
      // S_w^T = K_w Q^T for this wave's 32 keys
      f32x16 s = f32x16{};
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const int r = wave * 32 + l32;
        const bf16x8 a = *(const bf16x8*)(kb + r * RB + ((cc * 2 + hi) ^ SW::k(r)) * 16);
        s = mfma32(a, qf[cc], s);
      }
      if ((CAUSAL && kw0 + 31 > q0) || kw0 + 32 > N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kw0 + acc_row(r, hi);
          if (!(key < N && (!CAUSAL || key <= my_q))) s[r] = -INFINITY;
        }
      }
      // the wave's partial softmax over its keys
      float mx = lane_max<16>(&s);
      mx = pair_max(mx);
      const float m_w = mx * c;  // -inf if none of the wave's keys is visible
      const float mref = (m_w == -INFINITY) ? 0.f : m_w;
      f32x16 ow[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ow[dt] = f32x16{};
      float l_part = 0.f;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        f32x8 p8;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p8[t] = fast_exp2(fmaf(s[8 * cc + t], c, -mref));
          l_part += p8[t];
        }
        const bf16x8 pcur = to_bf16x8(p8);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int col = dt * 32 + 16 * (g16 % 2) + 4 * a4;
          u32x2 part[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int R = wave * 32 + 16 * cc + 8 * u + 4 * hi + i4;
            const uint8_t* addr = vb + R * RB + (((col / 8) ^ SW::v(R)) * 16) + (col % 8) * 2;
            part[u] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (short __attribute__((ext_vector_type(4))) __attribute__((address_space(3)))*)addr));
          }
          ow[dt] = mfma32(as_bf16x8(u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}), pcur,
                          ow[dt]);
        }
      }
      const float l_w = pair_sum(l_part);
      // partials to LDS: O_w^T register r of lane l is d = dt*32 + 8(r/4) + 4hi + r%4
      // of query l32; store rows [query][d]
      float* orow = ob + (wave * BQ + l32) * OSTRIDE;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(orow + dt * 32 + 8 * g + 4 * hi) =
              f32x4{ow[dt][4 * g + 0], ow[dt][4 * g + 1], ow[dt][4 * g + 2], ow[dt][4 * g + 3]};
      if (hi == 0) {
        mb[wave * BQ + l32] = m_w;
        lb[wave * BQ + l32] = l_w;
      }
      wait_dma_and_lds();
      __syncthreads();

      // merge: each thread takes (query, 8 consecutive d) pieces of the tile
      constexpr int CH = D / 8;
      for (int item = tid; item < BQ * CH; item += W * 64) {
        const int qi = item / CH, ch = item % CH;
        const int row = q0 + qi;
        if (row < N) {
          float* os = o_state + head + (size_t)row * tok + ch * 8;
          float* ms = ml_state + 2 * (rowstat + row);
          const float m_old = jt == 0 ? -INFINITY : ms[0];
          const float l_old = jt == 0 ? 0.f : ms[1];
          float m_new = m_old;
#pragma unroll
          for (int w = 0; w < W; ++w) m_new = fmaxf(m_new, mb[w * BQ + qi]);
          const float mr = (m_new == -INFINITY) ? 0.f : m_new;
          const float a_old = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - mr);
          float l_new = l_old * a_old;
          f32x8 acc = f32x8{};
          if (jt != 0) {
            const f32x4 x0 = *(const f32x4*)os, x1 = *(const f32x4*)(os + 4);
            acc = f32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]} * l_new;
          }
#pragma unroll
          for (int w = 0; w < W; ++w) {
            const float mw = mb[w * BQ + qi];
            const float aw = (mw == -INFINITY) ? 0.f : fast_exp2(mw - mr);
            l_new += aw * lb[w * BQ + qi];
            const float* src = ob + (w * BQ + qi) * OSTRIDE + ch * 8;
            const f32x4 y0 = *(const f32x4*)src, y1 = *(const f32x4*)(src + 4);
            acc += aw * f32x8{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
          }
          acc *= 1.0f / l_new;
          if (jt == last_jt) {  // every visible key seen: final O and L
            *(u32x4*)(o + head + (size_t)row * tok + ch * 8) = as_u32x4(to_bf16x8(acc));
            if (ch == 0) lse[rowstat + row] = (m_new + log2f(l_new)) * kLn2;
          } else {
            *(f32x4*)os = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *(f32x4*)(os + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
            if (ch == 0) {
              ms[0] = m_new;
              ms[1] = l_new;
            }
          }
        }
      }
      wait_dma_and_lds();
      __syncthreads();  // the partials have been merged: the buffers are free
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_splitk_t(const Fa1Params& p) {
  const long long grid = (long long)p.B * p.H;
  const FwdScale sc = fwd_scale(p.scale);
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa1_splitk_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (uint16_t*)p.o, p.lse, p.o_state, p.ml_state, p.H, p.N, sc.c, sc.q_and,
                     sc.q_xor);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_t(const Fa1Params& p) {
  const long long grid = (long long)p.B * p.H;
  const FwdScale sc = fwd_scale(p.scale);
  const float c = sc.c;
  const uint32_t q_and = sc.q_and, q_xor = sc.q_xor;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa1_order_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(512), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (uint16_t*)p.o, p.lse, p.o_state, p.ml_state, p.H, p.N, c, q_and, q_xor);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fa1_order_fwd(const Fa1Params& p) {
  if (p.split_k) {
    if (p.d == 64) return p.causal ? launch_splitk_t<64, true>(p) : launch_splitk_t<64, false>(p);
    return p.causal ? launch_splitk_t<128, true>(p) : launch_splitk_t<128, false>(p);
  }
  if (p.d == 64) return p.causal ? launch_t<64, true>(p) : launch_t<64, false>(p);
  return p.causal ? launch_t<128, true>(p) : launch_t<128, false>(p);
}

}  // namespace fa2
