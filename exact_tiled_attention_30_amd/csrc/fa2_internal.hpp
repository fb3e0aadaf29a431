// fa2_internal.hpp -- host-side interface between the C ABI layer and the
// kernel translation units.  Not installed; callers use include/fa2.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa2 {

// Softmax constants of the forward kernels for a given scale: the kernels
// form exp2(s * c - m) with c = |scale| * log2(e) > 0, flip the bf16 sign bits
// of Q (exact) for a negative scale, and zero Q (q_and = 0, c = 1) for a zero
// scale -- or one so small that c is not a normal fp32 number, where every
// scaled score is 0 to fp32 precision anyway and a zero or subnormal c would
// turn the masked scores' -inf * c into NaN.
struct FwdScale {
  float c;
  uint32_t q_and, q_xor;
};
inline FwdScale fwd_scale(float scale) {
  const float c = (float)((scale < 0.f ? -(double)scale : (double)scale) * 1.4426950408889634);
  FwdScale r;
  r.q_xor = scale < 0.f ? 0x80008000u : 0u;
  if (c >= 1.17549435e-38f) {  // FLT_MIN, the smallest normal fp32
    r.c = c;
    r.q_and = 0xffffffffu;
  } else {
    r.c = 1.0f;
    r.q_and = 0u;
  }
  return r;
}

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  bool causal;
  float scale;
  hipStream_t stream;
  // split-KV only (launch_fwd_split_kv): slices per Q tile and the partials
  int n_split = 1;
  float* o_part = nullptr;    // fp32 [n_split][B, N, H, d] (workspace)
  float* lse_part = nullptr;  // fp32 [n_split][B, H, N], log2 units (workspace)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // D vector, fp32 [B, H, N] (workspace)
  float* dq_acc;  // fp32 [B, N, H, d] (workspace; atomic dQ strategy only)
  int B, H, N, d;
  bool causal;
  float scale;
  hipStream_t stream;
};

// The forward pass in FlashAttention-1's loop order (an ablation).
struct Fa1Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* o_state;   // fp32 [B, N, H, d] (workspace)
  float* ml_state;  // fp32 [B, H, N, 2]: running max, running sum (workspace)
  int B, H, N, d;
  bool causal;
  float scale;
  hipStream_t stream;
  bool split_k = false;  // FlashAttention-1's split-K wave partition (else split-Q)
};

// Host argument checks of a backward call (fa2_api.cpp); need_ws is the
// workspace size the call requires, or kNoWorkspace when it takes none.
constexpr size_t kNoWorkspace = ~(size_t)0;
int bwd_checks(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, size_t need_ws, int B, int H, int N, int d, float scale,
               size_t* rows_out);

// Workspace layout of the backward pass (offsets in bytes, 256-aligned).
size_t bwd_delta_bytes(int B, int H, int N);
size_t bwd_dq_acc_bytes(int B, int H, int N, int d);
size_t fa1_ml_bytes(int B, int H, int N);

// Kernel configurations the host dispatch picks from (diagnostic ids, also
// exported through fa2_fwd_variant / fa2_bwd_variant).
enum Variant {
  kFwdD64Nc4 = 0, kFwdD64Nc8, kFwdD128Sp4, kFwdD128Sp8,
  kFwdD64CausalDealt, kFwdD64CausalOne, kFwdD64CausalPair4, kFwdD64CausalPair8,
  kFwdD128CausalDealt, kFwdD128CausalOne, kFwdD128CausalPair4, kFwdD128CausalPair8,
  kFwdCount,
  kBwdFirst = 16,  // 16 + 4*(d == 128) + 2*causal + (dQ pass has 8 waves)
  kBwdCount = 8,
};
int fwd_variant(int B, int H, int N, int d, bool causal, int resident_d128);
const char* fwd_variant_name(int v);
int fwd_resident_d128();  // occupancy query of the d = 128 dealt causal kernel
int bwd_dq_waves(int B, int H, int N, bool causal);
int bwd_variant(int B, int H, int N, int d, bool causal);
const char* bwd_variant_name(int v);

hipError_t launch_fwd(const FwdParams& p);
hipError_t launch_fwd_split_kv(const FwdParams& p);
int split_kv_slices(int B, int H, int N, int requested);
hipError_t launch_fa1_order_fwd(const Fa1Params& p);
hipError_t launch_bwd(const BwdParams& p);             // dQ from a Q-outer pass
hipError_t launch_bwd_atomic_dq(const BwdParams& p);   // dQ summed with fp32 atomics
hipError_t launch_calib_mfma(float* out, int blocks, int iters, bool random_operands,
                             hipStream_t stream);

}  // namespace fa2
