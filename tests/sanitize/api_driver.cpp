// Drives the C ABI's host-side argument checks (fa2_api.cpp) and the kernel
// choice (fa2_dispatch.cpp), and the backward checks fa2_bwd_noalloc
// shares, under the host AddressSanitizer and
// UndefinedBehaviorSanitizer.  The kernel launchers are replaced by stubs
// that abort: every call below must be refused, or be an empty no-op,
// before any launch.  Sizes reach the limits of the checks (overflowing
// products, the 2^31 row and grid limits, the static scratch limit).
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "fa2.h"
#include "fa2_internal.hpp"

namespace fa2 {
static hipError_t never(const char* what) {
  std::fprintf(stderr, "launcher reached: %s\n", what);
  std::abort();
}
hipError_t launch_fwd(const FwdParams&) { return never("fwd"); }
hipError_t launch_fwd_split_kv(const FwdParams&) { return never("split_kv"); }
hipError_t launch_fa1_order_fwd(const Fa1Params&) { return never("fa1_order"); }
hipError_t launch_bwd(const BwdParams&) { return never("bwd"); }
hipError_t launch_bwd_atomic_dq(const BwdParams&) { return never("bwd_atomic"); }
hipError_t launch_calib_mfma(float*, int, int, bool, hipStream_t) { return never("calib"); }
int fwd_resident_d128() { return 2; }
}  // namespace fa2

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  // fake, aligned, far-apart "device" addresses: only the checks read them
  const uintptr_t G = (uintptr_t)1 << 40;
  void* P[12];
  for (int i = 0; i < 12; ++i) P[i] = (void*)(G * (i + 1));
  float* L = (float*)P[4];
  const int sizes[][3] = {{-1, 1, 1}, {1, -1, 1}, {1, 1, -1}, {INT_MAX, INT_MAX, INT_MAX},
                          {65536, 65536, 2}, {1, 1 << 20, 1 << 12}, {1, 1, INT_MAX}};
  for (auto& s : sizes) {
    for (int d : {64, 128}) {
      const int st = fa2_fwd(P[0], P[1], P[2], P[3], L, s[0], s[1], s[2], d, 1, 0.1f, nullptr);
      if (st == FA2_OK) expect(st, FA2_ERR_SHAPE, "fwd accepted an out-of-range shape");
      expect(fa2_bwd_workspace_bytes(s[0], s[1], s[2], d, 1) == 0, 1, "bwd workspace size");
      expect(fa2_fwd_variant(s[0], s[1], s[2], d, 1, 0), -1, "fwd variant of a bad shape");
      expect(fa2_bwd_variant(s[0], s[1], s[2], d, 0), -1, "bwd variant of a bad shape");
      expect(fa2_fwd_split_kv_workspace_bytes(s[0], s[1], s[2], d, 0, 0) == 0, 1, "split size");
      expect(fa2_fwd_fa1_order_workspace_bytes(s[0], s[1], s[2], d, 0) == 0, 1, "fa1 size");
      // fa2_bwd_noalloc's checks before its scratch limit (the rest of that
      // entry point needs the device)
      size_t rows = 0;
      const int sb = fa2::bwd_checks(P[0], P[1], P[2], P[3], L, P[5], P[6], P[7], P[8], nullptr,
                                     0, fa2::kNoWorkspace, s[0], s[1], s[2], d, 0.1f, &rows);
      if (sb == FA2_OK) expect(sb, FA2_ERR_SHAPE, "bwd checks accepted an out-of-range shape");
    }
  }
  expect(fa2_fwd(P[0], P[1], P[2], P[3], L, 1, 1, (1 << 30) + 1, 64, 1, 0.1f, nullptr),
         FA2_ERR_SHAPE, "N above 2^30");
  expect(fa2_fwd_variant(1, 1, 1 << 30, 64, 1, 0) >= 0, 1, "N = 2^30 has a kernel");
  // every check in turn, on a valid shape
  expect(fa2_fwd(P[0], P[1], P[2], P[3], L, 2, 3, 100, 96, 0, 0.1f, nullptr), FA2_ERR_HEADDIM, "d");
  expect(fa2_fwd(P[0], P[1], P[2], P[3], L, 2, 3, 100, 64, 0, NAN, nullptr), FA2_ERR_SCALE, "nan");
  expect(fa2_fwd(P[0], P[1], P[2], P[3], L, 2, 3, 100, 64, 0, 3e38f, nullptr), FA2_ERR_SCALE,
         "scale*log2e overflows");
  expect(fa2_fwd(nullptr, P[1], P[2], P[3], L, 2, 3, 100, 64, 0, 0.1f, nullptr), FA2_ERR_NULLPTR,
         "null q");
  expect(fa2_fwd((char*)P[0] + 2, P[1], P[2], P[3], L, 2, 3, 100, 64, 0, 0.1f, nullptr),
         FA2_ERR_ALIGN, "misaligned q");
  expect(fa2_fwd(P[0], P[1], P[2], P[1], L, 2, 3, 100, 64, 0, 0.1f, nullptr), FA2_ERR_ALIAS,
         "o aliases k");
  expect(fa2_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 3, 100, 64, 0, 0.1f, nullptr),
         FA2_OK, "empty");
  const size_t ws = fa2_bwd_workspace_bytes(2, 3, 100, 64, 1);
  expect(fa2_bwd(P[0], P[1], P[2], P[3], L, P[5], P[6], P[7], P[8], P[9], ws - 1, 2, 3, 100, 64,
                 1, 0.1f, nullptr), FA2_ERR_WORKSPACE, "short workspace");
  expect(fa2_bwd(P[0], P[1], P[2], P[3], L, P[5], P[6], P[7], P[8], P[2], ws, 2, 3, 100, 64, 1,
                 0.1f, nullptr), FA2_ERR_ALIAS, "workspace aliases v");
  expect(fa2_bwd_atomic_dq(P[0], P[1], P[2], P[3], L, P[5], P[6], P[7], P[8], P[9], ws, 2, 3, 100,
                           64, 1, 0.1f, nullptr), FA2_ERR_WORKSPACE, "atomic needs more");
  {
    size_t rows = 0;
    expect(fa2::bwd_checks(P[0], P[1], P[2], P[3], L, P[5], P[6], P[7], P[8], nullptr, 0,
                           fa2::kNoWorkspace, 2, 3, 100, 64, 0.1f, &rows), FA2_OK,
           "checks without a workspace");
    expect((int)rows, 600, "rows");
    expect(fa2::bwd_checks(P[0], P[1], P[2], P[3], L, P[5], P[6], P[7], P[2], nullptr, 0,
                           fa2::kNoWorkspace, 2, 3, 100, 64, 0.1f, &rows), FA2_ERR_ALIAS,
           "dv aliases v");
  }
  expect(fa2_fwd_split_kv(P[0], P[1], P[2], P[3], L, P[9], 1 << 30, 2, 3, 1000, 64, 0, 0.1f, 65,
                          nullptr), FA2_ERR_SHAPE, "too many slices");
  expect(fa2_fwd_fa1_order(P[0], P[1], P[2], P[3], L, nullptr, 0, 2, 3, 100, 64, 0, 0.1f, 1,
                           nullptr), FA2_ERR_WORKSPACE, "fa1 without workspace");
  expect(fa2_calibrate_mfma(nullptr, 1, 1, nullptr), FA2_ERR_NULLPTR, "calib null");
  expect(fa2_calibrate_mfma_random((float*)P[9], 0, 1, nullptr), FA2_ERR_SHAPE,
         "calib random blocks");
  // the dispatch over a range of valid shapes: every id names a kernel
  for (int B : {1, 2, 3, 8, 80})
    for (int H : {1, 2, 9, 16, 64})
      for (int N : {1, 63, 64, 65, 1000, 4096, 32768, 1 << 20})
        for (int d : {64, 128})
          for (int c : {0, 1}) {
            if ((long long)B * H * N > INT_MAX) continue;  // refused, as checked above
            const int fv = fa2_fwd_variant(B, H, N, d, c, 0);
            const int bv = fa2_bwd_variant(B, H, N, d, c);
            if (fv < 0 || !*fa2_variant_name(fv) || bv < 0 || !*fa2_variant_name(bv)) {
              std::fprintf(stderr, "no kernel for B=%d H=%d N=%d d=%d causal=%d\n", B, H, N, d, c);
              ++failures;
            }
            expect(fa2_fwd_split_kv_workspace_bytes(B, H, N, d, c, 0) > 0, 1, "split size");
          }
  for (int s = -2; s < 12; ++s) (void)fa2_status_string(s);
  if (failures) return 1;
  std::printf("api sanitizer run: ok\n");
  return 0;
}
