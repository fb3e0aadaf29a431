// fa2_fwd_kernels.hpp -- FlashAttention-2 forward pass for gfx950: the kernels and
// their launch templates, instantiated by fa2_fwd.hip and fa2_fwd_wide.hip.
//
// Algorithm: infra-guide page "6.2 FlashAttention V2 in depth", section 6.1
// (Q-tile outer loop, K/V-tile inner loop, running max m and sum l, one
// division by l after the loop, logsumexp saved for the backward), with the
// causal block skipping of section 5.3 and the split-Q warp partition of
// section 4.2.  Design for CDNA4, not a port of the A100 kernel:
//
//  * A workgroup of W waves (64 lanes) owns a Q tile of 32*W rows of one
//    (batch, head); each wave owns 32 query rows and their softmax rows
//    outright (no cross-wave merge).  Causal workgroups take a heavy and a
//    light Q tile in turn so all stream the same number of K/V tiles, or,
//    when the whole grid fits on the CUs at once, one Q tile each, dealt to
//    the CUs so that every CU's tiles add up to the same work.  Work items
//    are renumbered so each XCD runs contiguous Q tiles of the same heads
//    (shared K/V in its L2).
//  * Both products run on v_mfma_f32_32x32x16_bf16 in transposed form:
//    S^T = K Q^T (A = K rows from LDS, B = Q held in VGPRs for the whole
//    loop) and O^T = V^T P^T (A = V^T read transposed from LDS, B = P^T
//    straight from the S^T accumulators after an in-register bf16
//    conversion).  In both, the accumulator column -- one query -- is fixed
//    per lane, so row max, row sum, rescale and the final 1/l are per-lane
//    scalars plus one exchange between the two lane halves.
//  * K/V tiles move global -> LDS by DMA (global_load_lds), double-buffered,
//    one barrier per tile; see the kernel's comment for the LDS layout.
//  * Softmax in base 2: t = s * scale*log2(e) in fp32 on the MFMA output
//    (never folded into bf16 Q), P = exp2(t - m).  l is summed from the fp32
//    P before the bf16 conversion.  The reference m of P = exp2(t - m) is
//    the running row max, moved (with the O rescale: a multiply of every
//    accumulator by exp2(m_old - m_new)) when a tile's max exceeds it -- with
//    one exception that saves most rescales: a new max that would give a key
//    at most 1/16 of the row's running sum, P <= l/16 (and at most 2^8), is
//    left in P instead.  Any key that carries more of the row's mass moves m
//    to its own score, so the largest P of a row dominated by a few keys is
//    exactly 1, free of bf16 rounding, and O stays within rounding of those
//    keys' V rows; a skipped key's P may be inexact in bf16 (2^-9
//    relative), but its weight is at most 1/16.  (A reference allowed to
//    trail the max by a fixed 8 whatever the mass put the dominant P's
//    rounding into O: on the peaked N = 32768 workload that exceeded the O
//    tolerance.)  O/l and L = ln2 * (m + log2 l) are mathematically the same
//    for any reference.
//  * Causal: K/V tiles past the Q tile's last row are never loaded; a wave
//    skips tiles entirely above its rows; only tiles crossing the diagonal (or
//    the ragged end of the sequence) run the element mask.
#pragma once

#include <math.h>


#include "fa2_device.hpp"
#include "fa2_internal.hpp"

namespace fa2 {
namespace {

// Threshold of the next rescale: the running max plus log2 of the lane's
// running sum minus kMassShift (a new key of P <= l_lane / 2^kMassShift does
// not move the reference), clamped to [0, kMaxSlack] so P stays <= 2^8.
constexpr float kMassShift = 4.0f, kMaxSlack = 8.0f;
__device__ __forceinline__ float next_threshold(float m_run, float l_lane) {
  return m_run + __builtin_amdgcn_fmed3f(__builtin_amdgcn_logf(l_lane) - kMassShift, 0.0f,
                                         kMaxSlack);
}

// ---------------------------------------------------------------------------
// K and V tiles move HBM/L2 -> LDS with global_load_lds_dwordx4: lane L of a
// wave deposits its 16 bytes at LDS base + 16*L, so no VGPRs, no ds_write and
// no VALU packing are spent on staging.  Rows are stored unpadded (D*2 bytes)
// with the 16-byte chunks of each row permuted by an XOR swizzle, chosen per
// tensor so the MFMA operand reads below are free of bank conflicts; the
// loading lane fetches whichever global chunk belongs at its LDS slot.
//  * K operand (S^T = K Q^T): lane reads 16 bytes of key row kt*32 + l%32.
//  * V^T operand (O^T = V^T P^T): two ds_read_b64_tr_b16.  Within each group
//    of 16 lanes, output lane 4a+b receives element b of the 8-byte chunks
//    addressed by lanes a, 4+a, 8+a, 12+a (pinned by a probe on gfx950); so
//    when lane 4i+a addresses 4 consecutive d of key row key_i, every output
//    lane holds one d column across 4 keys -- the transposed fragment -- read
//    straight from the row-major V tile.
// LDS buffers are separate arrays picked at compile time (the tile loop is
// unrolled by two) so the compiler can tell the in-flight LDS DMA into one
// buffer from the reads of the other.
template <int D>
struct DlSwz {
  // XOR applied to the 16-byte chunk index of row r
  __device__ static constexpr int k(int r) { return D == 128 ? (r % 16) : ((r / 2) % 8); }
  __device__ static constexpr int v(int r) { return D == 128 ? 4 * (r % 4) : 4 * ((r / 2) % 2); }
};

// SPLIT: the key range of every Q tile is cut into n_split slices, one work
// item each; a slice's normalised O (fp32) and its logsumexp (log2 units) go
// to o_part / lse_part, and fwd_combine_kernel merges them.
// PAIR (causal): a work item is a heavy + light pair of Q tiles; without it,
// one Q tile, heaviest first -- for grids too small to fill the GPU, where
// twice the workgroups beat the balance.
// DEAL (causal, unpaired): the whole grid is resident at once, so the tiles
// are dealt to CUs by weight (dealt_id) instead of heaviest first per head.
template <int D, int BC, int W, int STAGES, bool CAUSAL, bool SPLIT = false, bool PAIR = true,
          bool DEAL = false>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(8 / W * 1))) void fwd_dl_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int H, int N, int n_qtiles, int grid, float c, uint32_t q_and, uint32_t q_xor,
    int n_split = 1, float* __restrict__ o_part = nullptr, float* __restrict__ lse_part = nullptr) {
  constexpr int kWaves = W;
  constexpr int BR = kWaves * 32;
  constexpr int RB = D * 2;                 // bytes per LDS row
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;            // rows per 1 KB load instruction
  constexpr int TILE = BC * RB;             // bytes per K or V tile
  constexpr int NI = TILE / 1024;           // load instructions per tile and tensor
  constexpr int NIW = NI / kWaves;          // ... per wave
  static_assert(NI % kWaves == 0 && NIW >= 1, "tile must split evenly over the waves");
  using SW = DlSwz<D>;
  static_assert(STAGES == 2 || STAGES == 3, "pipeline depth");
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb2[STAGES > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb2[STAGES > 2 ? TILE : 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;

  // Work item: non-causal, one Q tile; causal, the pair (n_qtiles-1-p, p)
  // of a heavy and a light Q tile, so every workgroup streams the same
  // number of K/V tiles (n_qtiles + 1 tile rows of keys) whatever p is.
  const int logical0 = DEAL ? dealt_id(blockIdx.x, grid, n_qtiles) : xcd_contiguous_id(blockIdx.x, grid);
  const int split = SPLIT ? logical0 % n_split : 0;  // slices of one Q tile are adjacent
  const int logical = SPLIT ? logical0 / n_split : logical0;
  const int per_head = (CAUSAL && !SPLIT && PAIR) ? (n_qtiles + 1) / 2 : n_qtiles;
  const int bh = logical / per_head;
  const int item = logical % per_head;
  const int n_pass = (CAUSAL && !SPLIT && PAIR && item != n_qtiles - 1 - item) ? 2 : 1;
  const int b = bh / H, hh = bh % H;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;

  // Per-lane byte offsets of the chunks this lane deposits, relative to the
  // tile's first key row; the tile base is a scalar pointer.
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
  // issue the direct loads of tile jt (rows past N repeat row N-1)
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
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(kbase + ko),
          (void __attribute__((address_space(3)))*)(kd + m * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(vbase + vo),
          (void __attribute__((address_space(3)))*)(vd + m * 1024), 16, 0, 0);
    }
  };

  for (int pass = 0; pass < n_pass; ++pass) {
  const int qt = (CAUSAL && !SPLIT) ? ((PAIR && pass != 0) ? item : n_qtiles - 1 - item) : item;
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;

  const int kv_len = CAUSAL ? min(N, q0 + BR) : N;
  const int n_kv_all = (kv_len + BC - 1) / BC;
  // this work item's K/V tiles: [jt_begin, n_kv)
  const int chunk = SPLIT ? (n_kv_all + n_split - 1) / n_split : n_kv_all;
  const int jt_begin = SPLIT ? min(n_kv_all, split * chunk) : 0;
  const int n_kv = SPLIT ? min(n_kv_all, jt_begin + chunk) : n_kv_all;

  // The first K/V tiles' DMA goes out before the Q loads, so the two
  // latencies overlap under the one wait below.
  if (n_kv > jt_begin) {
    issue(jt_begin, kb0, vb0);
    if constexpr (STAGES > 2) issue(min(jt_begin + 1, n_kv - 1), kb1, vb1);
  }

  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = q + head + (size_t)min(my_q, N - 1) * tok + 8 * hi;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 x = *(const u32x4*)(qp + 16 * cc);
      if (my_q >= N) x = u32x4{0u, 0u, 0u, 0u};
      x = (x & q_and) ^ q_xor;
      qf[cc] = as_bf16x8(x);
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // reference max of P (log2 units)
  float m_thr = -INFINITY;  // a tile max above this moves the reference
  float neg_mref = 0.f;     // -m_run, or 0 while m_run is -inf
  float l_part = 0.f;

  auto tile = [&](int jt, const uint8_t* kb, const uint8_t* vb) __attribute__((always_inline)) {
    const int kv0 = jt * BC;
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
    {
      // keep four K reads in flight ahead of the MFMAs that consume them
      constexpr int kSteps = (D / 16) * (BC / 32), kAhead = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int i = 0; i < kSteps - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    }

    const bool need_mask = (CAUSAL && kv0 + BC - 1 > qw0) || (kv0 + BC > N);
    if (need_mask) {
      // key kv0 + kt*32 + acc_row(r, hi) is visible iff it is below N and, if
      // causal, at most my_q: iff kt*32 + acc_row(r, 0) <= lim, a compile-time
      // constant against one per-lane bound
      const int lim = (CAUSAL ? min(my_q, N - 1) : N - 1) - kv0 - 4 * hi;
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + acc_row(r, 0) > lim) s[kt][r] = -INFINITY;
    }
    float mx = lane_max<BC / 2>(s);
    mx = pair_max(mx);
    const float mt = mx * c;  // c > 0: a row with no visible key stays -inf
    if (wave_any(mt > m_thr)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
      neg_mref = (m_run == -INFINITY) ? 0.f : -m_run;
    }

    // V^T fragment addresses: this lane supplies row 16*cc + 8*u + 4*hi + i,
    // columns dt*32 + 16*(g%2) + 4*a .. +3 (g = lane/16, i = (lane%16)/4, a = lane%4)
    const int g16 = lane / 16, i4 = (lane % 16) / 4, a4 = lane % 4;
    float rs = 0.f;
#pragma unroll
    for (int cc = 0; cc < BC / 16; ++cc) {
      const f32x16& sv = s[cc / 2];
      const int r0 = 8 * (cc % 2);
      f32x8 p8;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        p8[t] = fast_exp2(fmaf(sv[r0 + t], c, neg_mref));
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
        oacc[dt] = mfma32(as_bf16x8(u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}), pcur,
                          oacc[dt]);
      }
    }
    if constexpr (D == 128) {
      // four LDS reads ahead, then one MFMA per two V^T reads (causal d = 128
      // on MI355X: about +2 to +4 % against no such schedule; at d = 64 every
      // depth tried measured within noise, so it is not used there)
      constexpr int kM = (BC / 16) * (D / 32), kAhead = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int i = 0; i < (2 * kM - kAhead) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kM - (2 * kM - kAhead) / 2, 0);
    }
    l_part += rs;
    m_thr = next_threshold(m_run, l_part);
  };

  // STAGES-deep LDS pipeline.  At step jt the DMA for tile jt+STAGES-1 is
  // issued into the buffer tile jt-1 used (its readers passed the barrier
  // that ended step jt-1); every step issues one batch (the tile index is
  // clamped at the end), so the wait before each barrier is "all but the
  // newest STAGES-2 batches" -- which leaves tile jt+1 landed.
  static_assert(2 * NIW * (STAGES - 1) <= 15, "vmcnt immediate");
  constexpr int kWaitStep = kWaitVmLgkm | (2 * NIW * (STAGES - 2));  // lgkmcnt(0) too
  __builtin_amdgcn_s_waitcnt(kWaitStep);  // tile 0 (and Q) have landed
  __syncthreads();

  auto step = [&](int jt, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn)
      __attribute__((always_inline)) {
    issue(min(jt + STAGES - 1, n_kv - 1), kn, vn);
    if (!CAUSAL || jt * BC <= qw0 + 31) tile(jt, kc, vc);
    __builtin_amdgcn_s_waitcnt(kWaitStep);  // tile jt+1 has landed
    __syncthreads();
  };
  if constexpr (STAGES == 3) {
    for (int jt = jt_begin; jt < n_kv; jt += 3) {
      step(jt, kb0, vb0, kb2, vb2);
      if (jt + 1 < n_kv) step(jt + 1, kb1, vb1, kb0, vb0);
      if (jt + 2 < n_kv) step(jt + 2, kb2, vb2, kb1, vb1);
    }
  } else {
    for (int jt = jt_begin; jt < n_kv; jt += 2) {
      step(jt, kb0, vb0, kb1, vb1);
      if (jt + 1 < n_kv) step(jt + 1, kb1, vb1, kb0, vb0);
    }
  }
  wait_dma_and_lds();  // drain the LDS DMA before exit

  const float l = pair_sum(l_part);
  if constexpr (SPLIT) {
    // partial result of this slice: O / l in fp32 and log2(sum) + m; a
    // slice with no visible key for a row has l == 0, so it writes O = 0 and
    // -inf, which weighs nothing in the merge
    if (my_q < N) {
      const size_t rows_all = (size_t)(grid / n_split / per_head) * (size_t)N;  // B * H * N
      float* opp = o_part + (size_t)split * rows_all * D + head + (size_t)my_q * tok;
      const float inv_p = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(opp + dt * 32 + 8 * g + 4 * hi) =
              f32x4{oacc[dt][4 * g + 0], oacc[dt][4 * g + 1], oacc[dt][4 * g + 2],
                    oacc[dt][4 * g + 3]} * inv_p;
      if (hi == 0)
        lse_part[(size_t)split * rows_all + ((size_t)b * H + hh) * N + my_q] =
            l > 0.f ? m_run + log2f(l) : -INFINITY;
    }
  } else {
  store_row_bf16<D>(o + head + (size_t)min(my_q, N - 1) * tok, oacc, 1.0f / l, hi, my_q < N);
  if (my_q < N && hi == 0) lse[((size_t)b * H + hh) * N + my_q] = (m_run + log2f(l)) * kLn2;
  }
  if (pass + 1 < n_pass) {
    wait_dma_and_lds();
    __syncthreads();  // every wave is done with the LDS tiles
  }
  }
}

// Workgroups of this kernel one CU holds at once (its occupancy), queried
// once per process; 0 if the query fails, which turns the dealt path off.
template <int D, int BC, int W, int STAGES, bool CAUSAL, bool PAIR, bool DEAL>
int resident_wgs() {
  static const int n = [] {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, fwd_dl_kernel<D, BC, W, STAGES, CAUSAL, false, PAIR, DEAL>, W * 64, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    return blocks;
  }();
  return n;
}

template <int D, int BC, int W, int STAGES, bool CAUSAL, bool PAIR = true, bool DEAL = false>
hipError_t launch_fwd_dl(const FwdParams& p) {
  constexpr int BR = W * 32;
  const int n_qtiles = (p.N + BR - 1) / BR;
  const long long grid = (long long)p.B * p.H * ((CAUSAL && PAIR) ? (n_qtiles + 1) / 2 : n_qtiles);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const FwdScale sc = fwd_scale(p.scale);
  const float c = sc.c;
  const uint32_t q_and = sc.q_and, q_xor = sc.q_xor;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fwd_dl_kernel<D, BC, W, STAGES, CAUSAL, false, PAIR, DEAL>), dim3((unsigned)grid), dim3(W * 64), 0,
                     p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (uint16_t*)p.o, p.lse, p.H, p.N, n_qtiles, (int)grid, c, q_and, q_xor);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Software-pipelined variant for non-causal d = 128.  Per wave and K/V tile
// the loop body is the same arithmetic as fwd_dl_kernel's, reordered so the
// matrix cores and the vector ALUs work on different tiles: iteration j
// issues the MFMAs of S(j+1) = K(j+1) Q^T while the VALU forms
// P(j) = exp2(S(j) c - m), then the MFMAs of O += V(j)^T P(j)^T while the VALU
// takes the max of S(j+1).  K therefore runs one tile ahead of V: at step j the
// DMA fills K(j+2) into the buffer K(j) used and V(j+1) into the one V(j-1)
// used.  Tiles that need the element mask (the ragged end) take the plain
// one-tile-per-step path after the pipelined loop.
template <int D, int BC, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(8 / W))) void fwd_sp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int H, int N, int n_qtiles, int grid, float c, uint32_t q_and, uint32_t q_xor) {
  constexpr int BR = W * 32;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPI = 1024 / RB;
  constexpr int TILE = BC * RB;
  constexpr int NI = TILE / 1024;
  constexpr int NIW = NI / W;
  static_assert(NI % W == 0 && NIW >= 1, "tile must split evenly over the waves");
  using SW = DlSwz<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, hi = lane / 32;

  const int logical = xcd_contiguous_id(blockIdx.x, grid);
  const int bh = logical / n_qtiles;
  const int qt = logical % n_qtiles;
  const int b = bh / H, hh = bh % H;
  const size_t tok = (size_t)H * D;
  const size_t head = (size_t)b * N * tok + (size_t)hh * D;
  const int qw0 = qt * BR + wave * 32;
  const int my_q = qw0 + l32;

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
  // DMA of one tensor's tile jt into dst (rows past N repeat row N-1)
  auto issue_one = [&](const uint16_t* src, const uint32_t* off, int jt, uint8_t* dst)
      __attribute__((always_inline)) {
    const int kv0 = jt * BC;
    const uint8_t* base = (const uint8_t*)(src + head + (size_t)kv0 * tok);
    const bool whole = kv0 + BC <= N;
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
      const int m = wave * NIW + u;
      uint32_t x = off[u];
      if (!whole) x -= (uint32_t)(max(kv0 + lrow[u] - (N - 1), 0) * tok * 2);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(base + x),
                                       (void __attribute__((address_space(3)))*)(dst + m * 1024),
                                       16, 0, 0);
    }
  };

  const int n_kv = (N + BC - 1) / BC;
  const int n_main = N / BC;  // tiles with no masked key
  issue_one(k, koff, 0, kb0);
  issue_one(v, voff, 0, vb0);
  if (n_kv > 1) issue_one(k, koff, 1, kb1);

  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = q + head + (size_t)min(my_q, N - 1) * tok + 8 * hi;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 x = *(const u32x4*)(qp + 16 * cc);
      if (my_q >= N) x = u32x4{0u, 0u, 0u, 0u};
      x = (x & q_and) ^ q_xor;
      qf[cc] = as_bf16x8(x);
    }
  }

  // S^T = K Q^T for the tile in kb; row kt*32 + l32's swizzle depends on l32
  // only, so chunk cc*2+hi sits at kbase ^ (cc << 5) in every kt block
  const uint32_t kbase = (uint32_t)(l32 * RB) + (uint32_t)((hi ^ SW::k(l32)) * 16);
  auto scores = [&](const uint8_t* kb, f32x16* s) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      const uint32_t off = kbase ^ (uint32_t)(cc << 5);
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt) {
        const bf16x8 a = *(const bf16x8*)(kb + kt * 32 * RB + off);
        s[kt] = mfma32(a, qf[cc], cc == 0 ? f32x16{} : s[kt]);
      }
    }
  };
  // tile max in log2 units (-inf for a row with no visible key)
  auto tile_max = [&](const f32x16* s) __attribute__((always_inline)) {
    float mx = lane_max<BC / 2>(s);
    mx = pair_max(mx);
    return mx * c;  // c > 0: a row with no visible key stays -inf
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // reference max of P (log2 units)
  float m_thr = -INFINITY;  // a tile max above this moves the reference
  float neg_mref = 0.f;     // -m_run, or 0 while m_run is -inf
  float l_part = 0.f;
  // move the reference when the tile's max passes the threshold (see the
  // file comment); returns minus the reference the tile's P uses
  auto rescale_to = [&](float mt) __attribute__((always_inline)) {
    if (wave_any(mt > m_thr)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
      neg_mref = (m_run == -INFINITY) ? 0.f : -m_run;
    }
    return neg_mref;
  };
  // P = exp2(S c - mref) in bf16, and its fp32 row sum
  auto probs = [&](const f32x16* sc, float nm, bf16x8* pf) __attribute__((always_inline)) {
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < BC / 16; ++cc) {
      f32x8 p8;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        p8[t] = fast_exp2(fmaf(sc[cc / 2][8 * (cc % 2) + t], c, nm));
        if (t % 2) rs1 += p8[t];
        else rs0 += p8[t];
      }
      pf[cc] = to_bf16x8(p8);
    }
    return rs0 + rs1;
  };
  // O^T += V^T P^T; the V^T fragment of row 16cc + 8u + 4hi + i4, columns
  // dt*32 + 16(g16%2) + 4a4 .. +3 sits at vbase ^ (dt << 6) + (16cc + 8u) RB
  const int g16 = lane / 16, i4 = (lane % 16) / 4, a4 = lane % 4;
  const uint32_t vbase = (uint32_t)((4 * hi + i4) * RB) +
                         (uint32_t)(((2 * (g16 % 2) + a4 / 2) ^ SW::v(4 * hi + i4)) * 16) +
                         (uint32_t)((4 * a4) % 8 * 2);
  auto pv = [&](const uint8_t* vb, const bf16x8* pf) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < BC / 16; ++cc)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint32_t off = vbase ^ (uint32_t)(dt << 6);
        u32x2 part[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
          part[u] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (short __attribute__((ext_vector_type(4))) __attribute__((address_space(3)))*)(
                             vb + (16 * cc + 8 * u) * RB + off)));
        oacc[dt] = mfma32(as_bf16x8(u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}), pf[cc],
                          oacc[dt]);
      }
    if constexpr (W == 8) {
      // Schedule of the block this lands in (in a pipelined step: the S
      // products of the next tile, P of this one and these PV products):
      // four LDS reads, then one MFMA per two reads, so the V^T reads are
      // issued under the S MFMAs instead of just before their own MFMAs.
      // Depth 4 measured best of 2, 3, 4, 6, 8 and 12 (8: 1-2 % slower, 12:
      // about 4 % slower); the 4-wave variant was 13 % slower with the
      // schedule at all
      constexpr int kM = (BC / 16) * (D / 32), kAhead = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int i = 0; i < (2 * kM - kAhead) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kM - (2 * kM - kAhead) / 2, 0);
    }
  };

  wait_dma_and_lds();  // K(0), V(0), K(1) and Q have landed
  __syncthreads();
  f32x16 sa[BC / 32], sb[BC / 32];
  float mt = -INFINITY;
  if (n_main > 0) {
    scores(kb0, sa);
    mt = tile_max(sa);
  }
  wait_dma_and_lds();
  __syncthreads();  // every wave has read K(0): kb0 may take K(2)

  // pipelined step jt < n_main - 1: S(jt+1) and P(jt), then O += V(jt) P(jt)
  // and the max of S(jt+1)
  auto full = [&](int jt, const f32x16* sc, f32x16* sn, const uint8_t* k_next, const uint8_t* v_cur,
                  uint8_t* k_dma, uint8_t* v_dma) __attribute__((always_inline)) {
    if (jt + 2 < n_kv) issue_one(k, koff, jt + 2, k_dma);
    issue_one(v, voff, jt + 1, v_dma);
    const float nm = rescale_to(mt);
    bf16x8 pf[BC / 16];
    scores(k_next, sn);
    const float rs = probs(sc, nm, pf);
    pv(v_cur, pf);
    mt = tile_max(sn);
    l_part += rs;
    m_thr = next_threshold(m_run, l_part);
    wait_dma_and_lds();
    __syncthreads();
  };
  // last unmasked tile: P and O only; starts the loads the ragged tile needs
  auto drain = [&](int jt, const f32x16* sc, const uint8_t* v_cur, uint8_t* k_dma, uint8_t* v_dma)
      __attribute__((always_inline)) {
    if (jt + 2 < n_kv) issue_one(k, koff, jt + 2, k_dma);
    if (jt + 1 < n_kv) issue_one(v, voff, jt + 1, v_dma);
    const float nm = rescale_to(mt);
    bf16x8 pf[BC / 16];
    const float rs = probs(sc, nm, pf);
    pv(v_cur, pf);
    l_part += rs;
    m_thr = next_threshold(m_run, l_part);
    wait_dma_and_lds();
    __syncthreads();
  };
  int jt = 0;
  for (; jt + 2 < n_main; jt += 2) {
    full(jt, sa, sb, kb1, vb0, kb0, vb1);
    full(jt + 1, sb, sa, kb0, vb1, kb1, vb0);
  }
  if (jt + 1 < n_main) {
    full(jt, sa, sb, kb1, vb0, kb0, vb1);
    drain(jt + 1, sb, vb1, kb1, vb0);
    jt += 2;
  } else if (jt < n_main) {
    drain(jt, sa, vb0, kb0, vb1);
    jt += 1;
  }
  // the ragged last tile (keys past N masked); K(jt), V(jt) are in buffer jt % 2
  if (jt < n_kv) {
    const uint8_t* kc = (jt % 2) ? kb1 : kb0;
    const uint8_t* vc = (jt % 2) ? vb1 : vb0;
    f32x16 st[BC / 32];
    scores(kc, st);
    const int kv0 = jt * BC;
#pragma unroll
    for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kv0 + kt * 32 + acc_row(r, hi) >= N) st[kt][r] = -INFINITY;
    const float nm = rescale_to(tile_max(st));
    bf16x8 pf[BC / 16];
    const float rs = probs(st, nm, pf);
    pv(vc, pf);
    l_part += rs;
  }

  const float l = pair_sum(l_part);
  store_row_bf16<D>(o + head + (size_t)min(my_q, N - 1) * tok, oacc, 1.0f / l, hi, my_q < N);
  if (my_q < N && hi == 0) lse[((size_t)b * H + hh) * N + my_q] = (m_run + log2f(l)) * kLn2;
}

template <int D, int BC, int W>
hipError_t launch_fwd_sp(const FwdParams& p) {
  constexpr int BR = W * 32;
  const int n_qtiles = (p.N + BR - 1) / BR;
  const long long grid = (long long)p.B * p.H * n_qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const FwdScale sc = fwd_scale(p.scale);
  const float c = sc.c;
  const uint32_t q_and = sc.q_and, q_xor = sc.q_xor;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fwd_sp_kernel<D, BC, W>), dim3((unsigned)grid), dim3(W * 64), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (uint16_t*)p.o, p.lse, p.H, p.N, n_qtiles, (int)grid, c, q_and, q_xor);
  return hipGetLastError();
}

// Split-KV merge: for every row, L = log2 sum_s 2^{L_s} and
// O = sum_s 2^{L_s - L} O_s, i.e. the slices' softmax sums re-weighted to the
// whole key range (each O_s was normalised by its own sum).  One thread per
// 8 consecutive elements of a row; rows in [B, N, H] order.
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float* __restrict__ o_part,
                                                          const float* __restrict__ lse_part,
                                                          uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, int H, int N,
                                                          long long rows, int n_split) {
  constexpr int CH = D / 8;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / CH;
  const int ch = (int)(t % CH);
  if (row >= rows) return;
  const long long h = row % H, n = (row / H) % N, b = row / ((long long)H * N);
  const size_t li = ((size_t)b * H + h) * N + n;
  float m = -INFINITY;
  for (int sl = 0; sl < n_split; ++sl) m = fmaxf(m, lse_part[(size_t)sl * rows + li]);
  f32x8 acc = f32x8{};
  float wsum = 0.f;
  for (int sl = 0; sl < n_split; ++sl) {
    const float ls = lse_part[(size_t)sl * rows + li];
    const float w = (ls == -INFINITY) ? 0.f : fast_exp2(ls - m);
    wsum += w;
    const float* src = o_part + ((size_t)sl * rows + row) * D + ch * 8;
    const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
    acc += w * f32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  }
  const float inv = 1.0f / wsum;
  *(u32x4*)(o + row * D + ch * 8) = as_u32x4(to_bf16x8(acc * inv));
  if (ch == 0) lse[li] = (m + log2f(wsum)) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch_split_t(const FwdParams& p) {
  constexpr int W = 4, BR = W * 32;
  const int n_qtiles = (p.N + BR - 1) / BR;
  const long long grid = (long long)p.B * p.H * n_qtiles * p.n_split;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const FwdScale sc = fwd_scale(p.scale);
  const float c = sc.c;
  const uint32_t q_and = sc.q_and, q_xor = sc.q_xor;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fwd_dl_kernel<D, 64, W, 2, CAUSAL, true>), dim3((unsigned)grid), dim3(W * 64),
                     0, p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (uint16_t*)p.o, p.lse, p.H, p.N, n_qtiles, (int)grid, c, q_and, q_xor,
                     p.n_split, p.o_part, p.lse_part);
  const long long rows = (long long)p.B * p.N * p.H;
  const long long threads = rows * (D / 8);
  hipLaunchKernelGGL((fwd_combine_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     p.stream, p.o_part, p.lse_part, (uint16_t*)p.o, p.lse, p.H, p.N, rows,
                     p.n_split);
  return hipGetLastError();
}

}  // namespace

// The 8-wave d = 128 configurations (kFwdD128Sp8, kFwdD128CausalPair8),
// launched from fa2_fwd_wide.hip, which is compiled with another machine
// scheduler (see there).
hipError_t launch_fwd_wide(const FwdParams& p, int variant);

}  // namespace fa2
