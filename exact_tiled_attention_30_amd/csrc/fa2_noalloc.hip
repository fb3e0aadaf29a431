// fa2_noalloc.hip -- fa2_bwd_noalloc: the backward pass for callers that
// cannot allocate device memory (HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// fa2_bwd's only device scratch is the D vector (fp32, one value per row,
// written by the dQ pass and read by the dK/dV pass).  Here it lives in a
// file-scope device array that comes with the code object instead of in a
// caller workspace.  In host code `scratch` names a host-side stand-in, not
// the device memory: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever passed to kernels.
#include <mutex>

#include "fa2.h"
#include "fa2_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)FA2_BWD_NOALLOC_MAX_ROWS * sizeof(float);  // 16 MiB
static_assert(kScratchBytes == ((size_t)16 << 20), "scratch size as documented");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// Device address of this device's `scratch`, looked up on the first call for
// `dev` with `dev` current (the caller's current device is restored).
hipError_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int H, int N, int d, int causal, float scale,
                               void* stream) {
  size_t rows = 0;
  int st = fa2::bwd_checks(q, k, v, o, lse, dout, dq, dk, dv, nullptr, 0, fa2::kNoWorkspace, B,
                           H, N, d, scale, &rows);
  if (st != FA2_OK || rows == 0) return st;
  if (rows > (size_t)FA2_BWD_NOALLOC_MAX_ROWS) return FA2_ERR_SCRATCH;
  // the kernels run on the stream's device, so its scratch is the one to use
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  void* delta = nullptr;
  if (e == hipSuccess) e = scratch_on(dev, &delta);
  if (e != hipSuccess) return FA2_ERR_LAUNCH;
  fa2::BwdParams p{q, k, v, o, lse, dout, dq, dk, dv, (float*)delta, nullptr,
                   B, H, N, d, causal != 0, scale, (hipStream_t)stream};
  return fa2::launch_bwd(p) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}
