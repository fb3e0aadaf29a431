// fa2_dispatch.cpp -- the host side of the kernel choice: which kernel
// configuration (tile shape, waves per workgroup, causal work assignment,
// split-KV slice count) a problem of a given size runs.  Pure arithmetic on
// the sizes, shared by the launchers (fa2_fwd.hip, fa2_bwd.hip) and the C
// ABI's diagnostics; no device code, so it also builds with a host compiler
// alone (the sanitizer build of the argument checks).
#include "fa2_internal.hpp"

namespace fa2 {

// Kernel configuration of the forward pass for a problem.  Tile shapes (K/V
// tile 64 keys, 128 for the 8-wave causal d = 128 pairs; 8 waves = 256-row Q
// tiles, or 4 waves = 128 rows) chosen by measurement on MI355X, each
// parity-tested.  Grids of fewer 8-wave Q tiles
// than CUs use 4-wave tiles (twice the workgroups); causal grids of fewer
// than two 8-wave workgroups per CU use the 4-wave tiles too, and grids of
// fewer 4-wave pairs than CUs drop the pairing.  Causal grids with whole
// heads per XCD run one 4-wave workgroup per Q tile, dealt to the CUs by
// weight (d = 128: only when the CUs hold the whole grid at once, i.e. when
// B*H*ceil(N/128) <= 256 * resident_d128, the workgroups of that kernel one
// CU holds).  Host-only arithmetic: the same answer with or without a GPU.
int fwd_variant(int B, int H, int N, int d, bool causal, int resident_d128) {
  constexpr long long kCus = 256;
  if (!causal) {
    // d = 128: the software-pipelined kernel (the VALU work of one tile under
    // the MFMAs of the next); at d = 64 the plain kernel measures faster
    const bool tiny = (long long)B * H * ((N + 255) / 256) < kCus;
    if (d == 64) return tiny ? kFwdD64Nc4 : kFwdD64Nc8;
    return tiny ? kFwdD128Sp4 : kFwdD128Sp8;
  }
  const long long pairs8 = (long long)B * H * (((N + 255) / 256 + 1) / 2);
  const long long nq4 = (N + 127) / 128;
  const long long pairs4 = (long long)B * H * ((nq4 + 1) / 2);
  const long long tiles4 = (long long)B * H * nq4;
  const bool small = pairs8 < 2 * kCus;
  const bool tiny = pairs4 < kCus;  // 4-wave pairs would leave CUs idle: one tile each
  // One 4-wave workgroup per Q tile, dealt to the CUs by weight: twice the
  // waves of the pairs with the same balance when the grid is resident at
  // once; on larger grids the first round is dealt the same way and later
  // workgroups, still heaviest first, go wherever a slot frees.  At d = 64
  // that beats the pairs on every causal workload measured (1-5 % past one
  // round); at d = 128 only within one round (past it, 4-5 % slower at
  // N >= 8192).
  const bool whole_heads = nq4 > 0 && tiles4 % 8 == 0 && (tiles4 / 8) % nq4 == 0;
  if (d == 64) {
    if (whole_heads) return kFwdD64CausalDealt;
    if (tiny) return kFwdD64CausalOne;
    return small ? kFwdD64CausalPair4 : kFwdD64CausalPair8;
  }
  if (whole_heads && tiles4 <= kCus * resident_d128) return kFwdD128CausalDealt;
  if (tiny) return kFwdD128CausalOne;
  return small ? kFwdD128CausalPair4 : kFwdD128CausalPair8;
}

const char* fwd_variant_name(int v) {
  switch (v) {
    case kFwdD64Nc4: return "fwd_dl_kernel<64,64,4,2,false>";
    case kFwdD64Nc8: return "fwd_dl_kernel<64,64,8,2,false>";
    case kFwdD128Sp4: return "fwd_sp_kernel<128,64,4>";
    case kFwdD128Sp8: return "fwd_sp_kernel<128,64,8>";
    case kFwdD64CausalDealt: return "fwd_dl_kernel<64,64,4,2,true,false,false,true>";
    case kFwdD64CausalOne: return "fwd_dl_kernel<64,64,4,2,true,false,false>";
    case kFwdD64CausalPair4: return "fwd_dl_kernel<64,64,4,2,true>";
    case kFwdD64CausalPair8: return "fwd_dl_kernel<64,64,8,2,true>";
    case kFwdD128CausalDealt: return "fwd_dl_kernel<128,64,4,2,true,false,false,true>";
    case kFwdD128CausalOne: return "fwd_dl_kernel<128,64,4,2,true,false,false>";
    case kFwdD128CausalPair4: return "fwd_dl_kernel<128,64,4,2,true>";
    case kFwdD128CausalPair8: return "fwd_dl_kernel<128,128,8,2,true>";
    default: return nullptr;
  }
}

// Waves per workgroup of the dQ pass: 8 (256-row Q tiles), or 4 when the
// 8-wave grid would give fewer than two workgroups per CU.
int bwd_dq_waves(int B, int H, int N, bool causal) {
  constexpr long long kCus = 256;
  const long long items8 =
      (long long)B * H * (causal ? ((N + 255) / 256 + 1) / 2 : (N + 255) / 256);
  return items8 < 2 * kCus ? 4 : 8;
}

int bwd_variant(int B, int H, int N, int d, bool causal) {
  const int w8 = bwd_dq_waves(B, H, N, causal) == 8;
  return kBwdFirst + ((d == 128) << 2) + ((int)causal << 1) + w8;
}

const char* bwd_variant_name(int v) {
  static const char* const names[8] = {
      "bwd_dq_kernel<64,4,false>+bwd_dl_kernel<64,false,false>",
      "bwd_dq_kernel<64,8,false>+bwd_dl_kernel<64,false,false>",
      "bwd_dq_kernel<64,4,true>+bwd_dl_kernel<64,true,false>",
      "bwd_dq_kernel<64,8,true>+bwd_dl_kernel<64,true,false>",
      "bwd_dq_kernel<128,4,false>+bwd_kv_pair_kernel<128,false>",
      "bwd_dq_kernel<128,8,false>+bwd_kv_pair_kernel<128,false>",
      "bwd_dq_kernel<128,4,true>+bwd_kv_pair_kernel<128,true>",
      "bwd_dq_kernel<128,8,true>+bwd_kv_pair_kernel<128,true>"};
  return v >= kBwdFirst && v < kBwdFirst + 8 ? names[v - kBwdFirst] : nullptr;
}

int split_kv_slices(int B, int H, int N, int requested) {
  if (requested > 0) return requested;
  // enough work items for two 4-wave workgroups per CU, at most 16 slices,
  // and at least two 64-key tiles per slice
  constexpr long long kCus = 256;
  const long long items = (long long)B * H * ((N + 127) / 128);
  long long s = (2 * kCus + items - 1) / items;
  const long long max_by_keys = ((N + 63) / 64) / 2;
  s = s < 16 ? s : 16;
  s = s < max_by_keys ? s : max_by_keys;
  return (int)(s < 1 ? 1 : s);
}

}  // namespace fa2
