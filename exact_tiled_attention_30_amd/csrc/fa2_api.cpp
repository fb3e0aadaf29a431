// fa2_api.cpp -- the C ABI of libfa2.so (declared in include/fa2.h).
//
// Every argument is checked on the host before any HIP runtime call, so each
// error path is reachable without a GPU; only then is the kernel for the
// requested (d, causal) enqueued on the caller's stream.
#include "fa2.h"

#include <math.h>
#include <stdint.h>

#include "fa2_internal.hpp"

namespace {

constexpr size_t kMaxElems = (size_t)1 << 62;
constexpr long long kMaxTokenElems = 1LL << 23;  // H * d of one token
constexpr int kMaxN = 1 << 30;                   // tokens per sequence
constexpr int kMaxSplits = 64;  // split-KV slices per Q tile

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = (uintptr_t)p;
  return Range{a, a + bytes};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Shape checks shared by both passes.  *elems receives B*N*H*d.
int check_shape(int B, int H, int N, int d, float scale, size_t* elems, size_t* rows) {
  // N <= 2^30 keeps every token index the kernels and launchers form (a
  // tile's first row plus a tile, N rounded up to a tile) inside int
  if (B < 0 || H < 0 || N < 0 || N > kMaxN) return FA2_ERR_SHAPE;
  if (d != 64 && d != 128) return FA2_ERR_HEADDIM;
  // the kernels work with scale * log2(e), which must be a finite fp32 too
  if (!isfinite(scale) || !isfinite((float)((double)scale * 1.4426950408889634)))
    return FA2_ERR_SCALE;
  const long double e = (long double)B * H * N * d;
  if (e > (long double)kMaxElems) return FA2_ERR_SHAPE;
  // every launch size derived from the row count must fit 32-bit grids
  if ((long double)B * H * N > 2147483647.0L) return FA2_ERR_SHAPE;
  // the kernels address rows within a tile of up to 128 tokens with 32-bit
  // offsets: 128 tokens of H*d bf16 elements must stay below 2^31 bytes
  if ((long long)H * d > kMaxTokenElems) return FA2_ERR_SHAPE;
  // grid = B * H * ceil(N / 128) workgroups must fit the launch limit
  const long double grid = (long double)B * H * ((N + 127) / 128);
  if (grid > 2147483647.0L) return FA2_ERR_SHAPE;
  *elems = (size_t)B * H * N * d;
  *rows = (size_t)B * H * N;
  return FA2_OK;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace fa2 {
size_t bwd_delta_bytes(int B, int H, int N) { return align256((size_t)B * H * N * sizeof(float)); }
size_t bwd_dq_acc_bytes(int B, int H, int N, int d) {
  return align256((size_t)B * H * N * d * sizeof(float));
}
size_t fa1_ml_bytes(int B, int H, int N) { return align256((size_t)B * H * N * 2 * sizeof(float)); }
}  // namespace fa2

extern "C" {

const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "FA2_OK";
    case FA2_ERR_NULLPTR: return "FA2_ERR_NULLPTR: a required pointer is NULL";
    case FA2_ERR_SHAPE:
      return "FA2_ERR_SHAPE: negative or too large B, H or N (N above 2^30), or H*d above 2^23";
    case FA2_ERR_HEADDIM: return "FA2_ERR_HEADDIM: head dimension must be 64 or 128";
    case FA2_ERR_SCALE: return "FA2_ERR_SCALE: scale and scale*log2(e) must be finite fp32 values";
    case FA2_ERR_ALIGN: return "FA2_ERR_ALIGN: tensor base pointer misaligned";
    case FA2_ERR_ALIAS: return "FA2_ERR_ALIAS: an output overlaps another tensor";
    case FA2_ERR_WORKSPACE: return "FA2_ERR_WORKSPACE: workspace missing or too small";
    case FA2_ERR_LAUNCH: return "FA2_ERR_LAUNCH: the HIP runtime rejected a launch";
    case FA2_ERR_SCRATCH:
      return "FA2_ERR_SCRATCH: B*H*N exceeds FA2_BWD_NOALLOC_MAX_ROWS, the rows the static "
             "scratch of fa2_bwd_noalloc holds";
    default: return "unknown fa2 status";
  }
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
            int N, int d, int causal, float scale, void* stream) {
  size_t elems = 0, rows = 0;
  const int st = check_shape(B, H, N, d, scale, &elems, &rows);
  if (st != FA2_OK) return st;
  if (elems == 0) return FA2_OK;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA2_ERR_ALIGN;
  const size_t tb = elems * 2, lb = rows * sizeof(float);
  const Range rq = range_of(q, tb), rk = range_of(k, tb), rv = range_of(v, tb);
  const Range ro = range_of(o, tb), rl = range_of(lse, lb);
  for (const Range& out : {ro, rl})
    for (const Range& in : {rq, rk, rv})
      if (overlap(out, in)) return FA2_ERR_ALIAS;
  if (overlap(ro, rl)) return FA2_ERR_ALIAS;

  fa2::FwdParams p{q, k, v, o, lse, B, H, N, d, causal != 0, scale, (hipStream_t)stream};
  return fa2::launch_fwd(p) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

size_t fa2_fwd_split_kv_workspace_bytes(int B, int H, int N, int d, int causal, int n_split) {
  (void)causal;
  size_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, 1.0f, &elems, &rows) != FA2_OK || elems == 0) return 0;
  if (n_split > kMaxSplits) return 0;
  const size_t s = (size_t)fa2::split_kv_slices(B, H, N, n_split);
  return s * (align256(elems * sizeof(float)) + align256(rows * sizeof(float)));
}

int fa2_fwd_split_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     int causal, float scale, int n_split, void* stream) {
  size_t elems = 0, rows = 0;
  const int st = check_shape(B, H, N, d, scale, &elems, &rows);
  if (st != FA2_OK) return st;
  if (n_split > kMaxSplits) return FA2_ERR_SHAPE;
  if (elems == 0) return FA2_OK;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
  if (!workspace ||
      workspace_bytes < fa2_fwd_split_kv_workspace_bytes(B, H, N, d, causal, n_split))
    return FA2_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return FA2_ERR_ALIGN;
  const size_t tb = elems * 2, lb = rows * sizeof(float);
  const Range ins[] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
  const Range outs[] = {range_of(o, tb), range_of(lse, lb), range_of(workspace, workspace_bytes)};
  for (const Range& out : outs)
    for (const Range& in : ins)
      if (overlap(out, in)) return FA2_ERR_ALIAS;
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FA2_ERR_ALIAS;
  const int s = fa2::split_kv_slices(B, H, N, n_split);
  char* ws = (char*)workspace;
  fa2::FwdParams p{q, k, v, o, lse, B, H, N, d, causal != 0, scale, (hipStream_t)stream};
  p.n_split = s;
  p.o_part = (float*)ws;
  p.lse_part = (float*)(ws + (size_t)s * align256(elems * sizeof(float)));
  return fa2::launch_fwd_split_kv(p) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

size_t fa2_fwd_fa1_order_workspace_bytes(int B, int H, int N, int d, int causal) {
  (void)causal;
  size_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, 1.0f, &elems, &rows) != FA2_OK || elems == 0) return 0;
  return fa2::bwd_dq_acc_bytes(B, H, N, d) + fa2::fa1_ml_bytes(B, H, N);
}

int fa2_fwd_fa1_order(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                      int causal, float scale, int split_k, void* stream) {
  size_t elems = 0, rows = 0;
  const int st = check_shape(B, H, N, d, scale, &elems, &rows);
  if (st != FA2_OK) return st;
  if (elems == 0) return FA2_OK;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULLPTR;
  if (!workspace || workspace_bytes < fa2_fwd_fa1_order_workspace_bytes(B, H, N, d, causal))
    return FA2_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return FA2_ERR_ALIGN;
  const size_t tb = elems * 2, lb = rows * sizeof(float);
  const Range ins[] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
  const Range outs[] = {range_of(o, tb), range_of(lse, lb), range_of(workspace, workspace_bytes)};
  for (const Range& out : outs)
    for (const Range& in : ins)
      if (overlap(out, in)) return FA2_ERR_ALIAS;
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return FA2_ERR_ALIAS;
  char* ws = (char*)workspace;
  fa2::Fa1Params p{q, k, v, o, lse, (float*)ws,
                   (float*)(ws + fa2::bwd_dq_acc_bytes(B, H, N, d)), B, H, N, d, causal != 0,
                   scale, (hipStream_t)stream};
  p.split_k = split_k != 0;
  return fa2::launch_fa1_order_fwd(p) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

size_t fa2_bwd_workspace_bytes(int B, int H, int N, int d, int causal) {
  (void)causal;
  size_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, 1.0f, &elems, &rows) != FA2_OK || elems == 0) return 0;
  return fa2::bwd_delta_bytes(B, H, N);
}

size_t fa2_bwd_atomic_dq_workspace_bytes(int B, int H, int N, int d, int causal) {
  (void)causal;
  size_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, 1.0f, &elems, &rows) != FA2_OK || elems == 0) return 0;
  return fa2::bwd_delta_bytes(B, H, N) + fa2::bwd_dq_acc_bytes(B, H, N, d);
}

}  // extern "C"

namespace fa2 {

// Host checks of a backward call, in the order fa2_bwd makes them: shapes,
// then (for a non-empty problem) pointers, the workspace (need_ws bytes;
// kNoWorkspace when the call takes none), alignment and overlaps.
int bwd_checks(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, size_t need_ws, int B, int H, int N, int d, float scale,
               size_t* rows_out) {
  size_t elems = 0, rows = 0;
  const int st = check_shape(B, H, N, d, scale, &elems, &rows);
  *rows_out = rows;
  if (st != FA2_OK) return st;
  if (elems == 0) return FA2_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA2_ERR_NULLPTR;
  const bool has_ws = need_ws != kNoWorkspace;
  if (has_ws && (!workspace || workspace_bytes < need_ws)) return FA2_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || (has_ws && !aligned(workspace, 16)))
    return FA2_ERR_ALIGN;
  const size_t tb = elems * 2, lb = rows * sizeof(float);
  const Range ins[] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), range_of(o, tb),
                       range_of(lse, lb), range_of(dout, tb)};
  const Range outs[] = {range_of(dq, tb), range_of(dk, tb), range_of(dv, tb),
                        has_ws ? range_of(workspace, workspace_bytes) : Range{0, 0}};
  for (const Range& out : outs)
    for (const Range& in : ins)
      if (overlap(out, in)) return FA2_ERR_ALIAS;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FA2_ERR_ALIAS;
  return FA2_OK;
}

}  // namespace fa2

namespace {

// Shared argument checks and launch of the two backward entry points.
int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
               void* stream, bool atomic_dq) {
  const size_t need = atomic_dq ? fa2_bwd_atomic_dq_workspace_bytes(B, H, N, d, causal)
                                : fa2_bwd_workspace_bytes(B, H, N, d, causal);
  size_t rows = 0;
  const int st = fa2::bwd_checks(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                                 need, B, H, N, d, scale, &rows);
  if (st != FA2_OK || rows == 0) return st;
  char* ws = (char*)workspace;
  fa2::BwdParams p{q, k, v, o, lse, dout, dq, dk, dv,
                   (float*)ws, atomic_dq ? (float*)(ws + fa2::bwd_delta_bytes(B, H, N)) : nullptr,
                   B, H, N, d, causal != 0, scale, (hipStream_t)stream};
  const hipError_t e = atomic_dq ? fa2::launch_bwd_atomic_dq(p) : fa2::launch_bwd(p);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int calibrate(float* out, int blocks, int iters, bool random_operands, void* stream) {
  if (out == nullptr) return FA2_ERR_NULLPTR;
  if (blocks < 1 || iters < 1) return FA2_ERR_SHAPE;
  return fa2::launch_calib_mfma(out, blocks, iters, random_operands, (hipStream_t)stream) ==
                 hipSuccess
             ? FA2_OK
             : FA2_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, void* workspace,
            size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
            void* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    causal, scale, stream, false);
}

int fa2_fwd_variant(int B, int H, int N, int d, int causal, int resident_wgs) {
  size_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, 1.0f, &elems, &rows) != FA2_OK || elems == 0) return -1;
  if (resident_wgs <= 0 && causal && d == 128) resident_wgs = fa2::fwd_resident_d128();
  return fa2::fwd_variant(B, H, N, d, causal != 0, resident_wgs);
}

int fa2_bwd_variant(int B, int H, int N, int d, int causal) {
  size_t elems = 0, rows = 0;
  if (check_shape(B, H, N, d, 1.0f, &elems, &rows) != FA2_OK || elems == 0) return -1;
  return fa2::bwd_variant(B, H, N, d, causal != 0);
}

const char* fa2_variant_name(int variant) {
  const char* n = fa2::fwd_variant_name(variant);
  if (!n) n = fa2::bwd_variant_name(variant);
  return n ? n : "";
}

int fa2_calibrate_mfma(float* out, int blocks, int iters, void* stream) {
  return calibrate(out, blocks, iters, false, stream);
}

int fa2_calibrate_mfma_random(float* out, int blocks, int iters, void* stream) {
  return calibrate(out, blocks, iters, true, stream);
}

int fa2_bwd_atomic_dq(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                      int causal, float scale, void* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    causal, scale, stream, true);
}

}  // extern "C"
