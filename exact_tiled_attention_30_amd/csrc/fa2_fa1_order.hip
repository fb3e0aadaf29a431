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
  if (p.d == 64) return p.causal ? launch_t<64, true>(p) : launch_t<64, false>(p);
  return p.causal ? launch_t<128, true>(p) : launch_t<128, false>(p);
}

}  // namespace fa2
