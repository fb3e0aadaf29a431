/*
 * fa2.h -- C ABI of the MI355X (gfx950) FlashAttention-2 library, libfa2.so.
 *
 * Exact attention, computed tile by tile without forming the N x N score
 * matrix:
 *
 *     O  = softmax(scale * Q K^T + M) V,     L = rowwise logsumexp of the same
 *                                                scaled, masked scores
 *
 * with M = 0 (non-causal) or M_ij = -inf for j > i (causal).  The problem
 * statement, the saved logsumexp and the causal mask follow the infra-guide
 * page "6.2 FlashAttention V2 in depth": section 6.1 (forward algorithm and
 * its outputs O and L), section 5.1 (the mask keeps the lower triangle,
 * diagonal included) and section 7 (backward inputs Q, K, V, O, L, dO;
 * outputs dQ, dK, dV; the D vector of section 7.3).  The abstract of
 * "FlashAttention-2: Faster Attention with Better Parallelism and Work
 * Partitioning" fixes that the result is exact, not an approximation.
 *
 * Common conventions
 *  - Self-attention: queries and keys share one sequence length N.
 *  - Q, K, V, O, dO, dQ, dK, dV: bfloat16, [B, N, H, d] contiguous row-major
 *    (element (b, n, h, c) at ((b*N + n)*H + h)*d + c).
 *  - L (lse): float32, [B, H, N] contiguous; natural-log logsumexp of the
 *    scaled, masked scores of each query row.
 *  - d must be 64 or 128.  B, H, N >= 0, N <= 2^30; B*H*N == 0 is a
 *    successful no-op.
 *  - scale: any finite float with |scale| * log2(e) finite in fp32, i.e.
 *    |scale| <= 2.35e38 (usually 1/sqrt(d)).
 *  - Every pointer is a DEVICE pointer owned by the caller; the library keeps
 *    no reference after the call returns and allocates no device memory.
 *    Tensor base pointers must be 16-byte aligned (lse 4-byte aligned).
 *    Outputs must not overlap inputs or each other.
 *  - stream is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; device-side faults surface at the caller's next
 *    synchronisation.
 *  - Argument checking happens on the host before any HIP call; on error
 *    nothing is enqueued and a nonzero fa2_status is returned.
 *  - No global mutable state: concurrent calls on different streams are safe.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
  FA2_OK = 0,
  FA2_ERR_NULLPTR = 1,   /* a required pointer is NULL and the problem is non-empty */
  FA2_ERR_SHAPE = 2,     /* B, H or N negative, N above 2^30, B*H*N above         */
                         /* 2^31 - 1, or H*d (elements of one token) above 2^23   */
  FA2_ERR_HEADDIM = 3,   /* d is not 64 or 128                                    */
  FA2_ERR_SCALE = 4,     /* scale is NaN or infinite, or |scale| > 2.35e38        */
  FA2_ERR_ALIGN = 5,     /* a base pointer is not 16-byte (lse: 4-byte) aligned   */
  FA2_ERR_ALIAS = 6,     /* an output range overlaps an input or another output   */
  FA2_ERR_WORKSPACE = 7, /* backward workspace missing or smaller than required   */
  FA2_ERR_LAUNCH = 8,    /* the HIP runtime rejected a kernel launch              */
  FA2_ERR_SCRATCH = 9    /* fa2_bwd_noalloc: B*H*N above FA2_BWD_NOALLOC_MAX_ROWS */
} fa2_status;

/*
 * Forward pass ("6.2 FlashAttention V2 in depth", section 6.1; causal block
 * skipping of section 5.3).
 *   q, k, v : inputs, bf16 [B, N, H, d]
 *   o       : output, bf16 [B, N, H, d]; O = softmax(scale*QK^T + M) V,
 *             rounded to nearest even
 *   lse     : output, fp32 [B, H, N]; L_i = log sum_j exp(scale*q_i.k_j + M_ij)
 *   causal  : nonzero applies the lower-triangular mask (key j visible to
 *             query i iff j <= i)
 * Returns FA2_OK or an fa2_status error code.
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * Bytes of device workspace fa2_bwd needs for these sizes (0 if the problem
 * is empty or the arguments are invalid): the D vector, fp32 [B, H, N].
 */
size_t fa2_bwd_workspace_bytes(int B, int H, int N, int d, int causal);

/*
 * Backward pass ("6.2 FlashAttention V2 in depth", section 7: P is recovered
 * from the saved logsumexp, dK and dV are owned by the block that holds a
 * key/value tile, and D_i = rowsum(dO_i * O_i) is computed once per row
 * rather than per tile).  dQ, which section 7.2 says must be summed across
 * the blocks of different key/value tiles, comes from a separate pass over Q
 * tiles (the page's "two-pass" option), which runs first and also computes
 * D: no atomics, and the result is bitwise reproducible run to run.
 *   q, k, v : forward inputs, bf16 [B, N, H, d]
 *   o, lse  : forward outputs of fa2_fwd for the same q, k, v, causal, scale
 *   dout    : gradient of the loss w.r.t. o, bf16 [B, N, H, d]
 *   dq, dk, dv : outputs, bf16 [B, N, H, d]
 *   workspace  : device scratch of at least fa2_bwd_workspace_bytes() bytes,
 *                16-byte aligned; its contents on entry are ignored and are
 *                overwritten.  Calls that share one workspace must be ordered
 *                on one stream.
 * Returns FA2_OK or an fa2_status error code.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o,
            const float* lse, const void* dout, void* dq, void* dk, void* dv,
            void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
            int causal, float scale, void* stream);

/* Rows B*H*N fa2_bwd_noalloc serves: its static scratch holds one fp32 D
 * value per row (16 MiB on each GPU the library runs on). */
#define FA2_BWD_NOALLOC_MAX_ROWS 4194304

/*
 * fa2_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and results as fa2_bwd (bitwise), but the D vector lives in a
 * scratch array of the library's own, allocated with the code object
 * (FA2_BWD_NOALLOC_MAX_ROWS fp32 values per GPU, held until the process
 * ends), so the caller passes no workspace and nothing is allocated:
 * no hipMalloc, hipFree or allocating library call on any path.
 *   Arguments, layouts, ownership and errors as for fa2_bwd, without the
 *   workspace; B*H*N > FA2_BWD_NOALLOC_MAX_ROWS returns FA2_ERR_SCRATCH
 *   before any HIP call.  The scratch of a GPU is looked up once per device
 *   (hipGetSymbolAddress, with the stream's device current).
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (on different streams, or from several threads) race and
 *   must be ordered by the caller.  Nothing in the scratch needs to start at
 *   zero (each call writes every D value it reads); its contents after a
 *   call are the last call's D.
 */
int fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * Bytes of device workspace fa2_bwd_atomic_dq needs (0 if the problem is
 * empty or the arguments are invalid): the D vector (fp32 [B, H, N]) and an
 * fp32 dQ accumulator ([B, N, H, d]), each 256-byte aligned.
 */
size_t fa2_bwd_atomic_dq_workspace_bytes(int B, int H, int N, int d, int causal);

/*
 * The same backward pass with section 7.2's other option for dQ: every
 * key/value block adds its dQ partial into the fp32 accumulator in the
 * workspace with atomic adds, and a final kernel rounds it to bf16.  dK and
 * dV are bitwise reproducible; dQ may differ in the last bits between runs
 * (the order of the fp32 additions varies).  Arguments, layouts, ownership
 * and errors as for fa2_bwd, except that the workspace must hold at least
 * fa2_bwd_atomic_dq_workspace_bytes() bytes.
 */
int fa2_bwd_atomic_dq(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                      int causal, float scale, void* stream);

/*
 * Bytes of device workspace fa2_fwd_split_kv needs for these sizes and
 * n_split (0 if the problem is empty or the arguments are invalid): per
 * slice, an fp32 partial O ([B, N, H, d]) and an fp32 partial logsumexp
 * ([B, H, N]).  n_split <= 0 asks for the library's choice, the same one
 * fa2_fwd_split_kv makes.
 */
size_t fa2_fwd_split_kv_workspace_bytes(int B, int H, int N, int d, int causal, int n_split);

/*
 * The forward pass with the key range of every Q tile cut into n_split
 * slices that run as separate workgroups, for problems whose
 * B * H * ceil(N / 128) workgroups cannot fill the GPU ("FlashAttention
 * Implementation > FlashAttention-2 Improvements", "Better Work
 * Partitioning": work split across blocks even for a single head).  Each
 * slice leaves its normalised partial O and logsumexp in the workspace; a
 * second kernel merges them with logsumexp weights into O and L.  Inputs,
 * outputs, layouts and errors as for fa2_fwd; n_split <= 0 lets the library
 * choose (enough work items for the GPU, at most 16, at least two 64-key
 * tiles per slice), n_split > 64 is FA2_ERR_SHAPE.  workspace: at least
 * fa2_fwd_split_kv_workspace_bytes() bytes for the same n_split, 16-byte
 * aligned, contents on entry ignored and overwritten.
 */
int fa2_fwd_split_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     int causal, float scale, int n_split, void* stream);

/*
 * Bytes of device workspace fa2_fwd_fa1_order needs (0 if the problem is
 * empty or the arguments are invalid): the fp32 O state ([B, N, H, d]) and
 * the running max and sum of every row (fp32 [B, H, N, 2]), each 256-byte
 * aligned.
 */
size_t fa2_fwd_fa1_order_workspace_bytes(int B, int H, int N, int d, int causal);

/*
 * The forward pass in FlashAttention-1's loop order, kept to measure what
 * FlashAttention-2's changes buy ("FlashAttention Implementation >
 * FlashAttention-2 Improvements"; "6.2 FlashAttention V2 in depth", sections
 * 2.1 and 3.1-3.4): K/V tiles in the outer loop and Q tiles in the inner
 * one, the Q tile reloaded and the O tile and its row statistics read and
 * written back (in the fp32 workspace) at every step, O renormalised after
 * every step, and one workgroup per (batch, head).
 *   split_k = 0: the waves of a workgroup own query rows (FlashAttention-2's
 *                split-Q partition, section 4.2), so only the loop order and
 *                the per-step renormalisation differ from fa2_fwd;
 *   split_k != 0: FlashAttention-1's own partition (sections 4.1, 4.3): the
 *                waves share the Q rows and split each K/V tile, and their
 *                partial softmax results (max, sum, P V) are merged through
 *                LDS at every step.
 * Same inputs, outputs, layouts, ownership and errors as fa2_fwd, plus the
 * workspace (at least fa2_fwd_fa1_order_workspace_bytes() bytes, 16-byte
 * aligned, contents on entry ignored and overwritten).
 */
int fa2_fwd_fa1_order(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                      int causal, float scale, int split_k, void* stream);

/* Measurement helper, not part of the attention path: runs `blocks`
 * workgroups of 256 threads in which every wave issues iters x 4
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) from registers, so the caller
 * can time it and read the bf16 MFMA throughput at the GPU's running clock,
 * the yardstick for the nominal dense peak (MI355X data sheet: 256 CUs x
 * 4096 FLOP/clk x 2.4 GHz).  FLOPs per call = blocks x 4 x iters x 4 x 32768.
 * out: device buffer of at least blocks x 256 floats (caller-owned; the
 * values are meaningless, they keep the work alive).  Errors: FA2_ERR_NULLPTR
 * if out is NULL, FA2_ERR_SHAPE if blocks < 1 or iters < 1, FA2_ERR_LAUNCH.
 * Asynchronous on `stream`.
 */
int fa2_calibrate_mfma(float* out, int blocks, int iters, void* stream);

/* Measurement helper, not part of the attention path: as fa2_calibrate_mfma
 * (same grid, same FLOPs per call, same `out` contract and errors), but each
 * wave cycles through 8 operand pairs of unit-variance pseudo-random bf16
 * values, a different pair for every MFMA of a chain, as the operands of an
 * attention tile change from one MFMA to the next.  The matrix cores draw
 * more power when more operand bits toggle, so on a power-capped GPU this
 * mode settles at a lower clock than the fixed-operand one: its throughput is
 * the bf16 MFMA rate attainable on real data.
 */
int fa2_calibrate_mfma_random(float* out, int blocks, int iters, void* stream);

/*
 * Diagnostics, not part of the attention path: which kernel configuration
 * (tile shape, waves per workgroup, causal work assignment) fa2_fwd and
 * fa2_bwd launch for a problem, so tests can show that every configuration
 * the dispatch can pick is exercised, and profiles can name the kernel they
 * time.  Pure host arithmetic on the sizes, with no device work and no
 * allocation.
 *   fa2_fwd_variant: an id in [0, 12); resident_wgs is the number of
 *     workgroups of the 4-wave d = 128 causal kernel one CU holds at once,
 *     which decides whether a causal d = 128 grid is dealt to the CUs by
 *     weight; resident_wgs <= 0 asks the current device (the occupancy query
 *     fa2_fwd itself makes; 0 without a usable device).  Ignored unless
 *     causal and d == 128.
 *   fa2_bwd_variant: an id in [16, 24), the dQ pass and dK/dV pass fa2_bwd
 *     launches.
 * Both return -1 for arguments fa2_fwd / fa2_bwd would reject or an empty
 * problem.  fa2_variant_name returns the kernel template(s) of an id as a
 * static string, or "" for an unknown id.
 */
int fa2_fwd_variant(int B, int H, int N, int d, int causal, int resident_wgs);
int fa2_bwd_variant(int B, int H, int N, int d, int causal);
const char* fa2_variant_name(int variant);

/* Static, human-readable name of a status code (never NULL). */
const char* fa2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
