/*
 * oracle.c -- plain, slow fp64 reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * What it computes is the definition that FlashAttention-2 reaches exactly
 * (the abstract of "FlashAttention-2: Faster Attention with Better Parallelism
 * and Work Partitioning" states the result carries no approximation; the
 * infra-guide page "6.2 FlashAttention V2 in depth", section 3.2, shows that
 * delaying the normalisation leaves the result unchanged).  So there is no
 * tiling, no online softmax and no delayed rescale here: every query row is
 * evaluated on its own, in double precision, straight from the definition
 *
 *     s_ij  = scale * <q_i, k_j>                    (section 6.1, score line)
 *     mask:  key j visible to query i iff j <= i    (section 5.1, causal mask:
 *            lower triangle including the diagonal)
 *     P_ij  = exp(s_ij - m_i) / l_i,  m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i)
 *     O_i   = sum_j P_ij v_j
 *     L_i   = m_i + log(l_i)                        (section 6.1, the saved
 *                                                    logsumexp for backward)
 *
 * Backward (section 7 of the same page; its formulas were lost in extraction,
 * so the standard softmax-gradient identities are written out):
 *
 *     P_ij  = exp(s_ij - L_i)            (section 7.1: P recovered from L)
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = <dO_i, v_j>
 *     D_i   = sum_j P_ij dP_ij           (section 7.3; equal to <dO_i, O_i>)
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j  = scale * sum_i dS_ij q_i
 *
 * Tensor layout: q, k, v, o, dout are [B, N, H, d] row-major (token row
 * stride H*d); lse is [B, H, N].  All arrays are double.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* flat offset of element (b, n, h, c) of a [B, N, H, d] tensor */
static inline size_t at_bnhd(int64_t b, int64_t n, int64_t h, int64_t c,
                             int64_t N, int64_t H, int64_t d) {
  return (size_t)(((b * N + n) * H + h) * d + c);
}

static int bad_sizes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return B < 0 || H < 0 || N < 0 || d < 1;
}

/* Number of keys query i may see: all N, or i+1 under the causal mask. */
static inline int64_t visible_keys(int64_t i, int64_t N, int causal) {
  return causal ? i + 1 : N;
}

/*
 * One query row (b, h, i) of the forward pass, written out from the
 * definition.  `e` is caller scratch of N doubles.
 */
static void forward_row(const double* q, const double* k, const double* v,
                        int64_t H, int64_t N, int64_t d, int causal,
                        double scale, int64_t b, int64_t h, int64_t i,
                        double* e, double* o_row, double* lse_out) {
  const int64_t n_vis = visible_keys(i, N, causal);
  const double* qi = q + at_bnhd(b, i, h, 0, N, H, d);

  /* scores and their maximum */
  double m = -INFINITY;
  for (int64_t j = 0; j < n_vis; ++j) {
    const double* kj = k + at_bnhd(b, j, h, 0, N, H, d);
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
    e[j] = scale * dot;
    if (e[j] > m) m = e[j];
  }
  /* unnormalised weights and their sum */
  double l = 0.0;
  for (int64_t j = 0; j < n_vis; ++j) {
    e[j] = exp(e[j] - m);
    l += e[j];
  }
  /* weighted sum of value rows, then normalise */
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < n_vis; ++j) {
    const double* vj = v + at_bnhd(b, j, h, 0, N, H, d);
    for (int64_t c = 0; c < d; ++c) o_row[c] += e[j] * vj[c];
  }
  for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
  *lse_out = m + log(l);
}

/*
 * Full forward pass: o [B,N,H,d], lse [B,H,N].  Returns 0, or -1 on bad
 * sizes / allocation failure.
 */
int oracle_attention_forward(const double* q, const double* k, const double* v,
                             int64_t B, int64_t H, int64_t N, int64_t d,
                             int causal, double scale, double* o, double* lse) {
  if (bad_sizes(B, H, N, d)) return -1;
  const int64_t rows = B * H * N;
  int failed = 0;
#pragma omp parallel
  {
    double* e = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!e) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r / (H * N), h = (r / N) % H, i = r % N;
        forward_row(q, k, v, H, N, d, causal, scale, b, h, i, e,
                    o + at_bnhd(b, i, h, 0, N, H, d), lse + (b * H + h) * N + i);
      }
      free(e);
    }
  }
  return failed ? -1 : 0;
}

/*
 * Forward pass for selected rows only.  rows holds n_rows triples (b, h, i);
 * o_rows is [n_rows, d], lse_rows is [n_rows].  Rows are independent, so a
 * sample of rows is exactly the corresponding part of the full result.
 */
int oracle_attention_forward_rows(const double* q, const double* k, const double* v,
                                  int64_t B, int64_t H, int64_t N, int64_t d,
                                  int causal, double scale, int64_t n_rows,
                                  const int64_t* rows, double* o_rows,
                                  double* lse_rows) {
  if (bad_sizes(B, H, N, d) || n_rows < 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N) return -1;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* e = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!e) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < n_rows; ++r) {
        forward_row(q, k, v, H, N, d, causal, scale, rows[3 * r], rows[3 * r + 1],
                    rows[3 * r + 2], e, o_rows + r * d, lse_rows + r);
      }
      free(e);
    }
  }
  return failed ? -1 : 0;
}

/*
 * Backward pass of one head (b, h).  Outputs dq, dk, dv as [N, d] slabs for
 * this head, plus lse[N] and D[N].  s and p are caller scratch of N doubles.
 */
static void backward_head(const double* q, const double* k, const double* v,
                          const double* dout, int64_t H, int64_t N, int64_t d,
                          int causal, double scale, int64_t b, int64_t h,
                          double* s, double* dp, double* dq, double* dk,
                          double* dv, double* lse, double* D) {
  memset(dq, 0, sizeof(double) * (size_t)(N * d));
  memset(dk, 0, sizeof(double) * (size_t)(N * d));
  memset(dv, 0, sizeof(double) * (size_t)(N * d));
  for (int64_t i = 0; i < N; ++i) {
    const int64_t n_vis = visible_keys(i, N, causal);
    const double* qi = q + at_bnhd(b, i, h, 0, N, H, d);
    const double* doi = dout + at_bnhd(b, i, h, 0, N, H, d);

    /* scores and the row logsumexp */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) {
      const double* kj = k + at_bnhd(b, j, h, 0, N, H, d);
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
      s[j] = scale * dot;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) l += exp(s[j] - m);
    const double L = m + log(l);
    lse[i] = L;

    /* P from the logsumexp, dP = dO v^T, and D = sum_j P dP */
    double Di = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
      const double* vj = v + at_bnhd(b, j, h, 0, N, H, d);
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c) dot += doi[c] * vj[c];
      s[j] = exp(s[j] - L); /* s now holds P_ij */
      dp[j] = dot;
      Di += s[j] * dp[j];
    }
    D[i] = Di;

    /* dS and the three gradient accumulations */
    for (int64_t j = 0; j < n_vis; ++j) {
      const double pij = s[j];
      const double dsij = pij * (dp[j] - Di);
      const double* kj = k + at_bnhd(b, j, h, 0, N, H, d);
      double* dqi = dq + i * d;
      double* dkj = dk + j * d;
      double* dvj = dv + j * d;
      for (int64_t c = 0; c < d; ++c) {
        dqi[c] += scale * dsij * kj[c];
        dkj[c] += scale * dsij * qi[c];
        dvj[c] += pij * doi[c];
      }
    }
  }
}

/*
 * Backward pass for selected heads.  heads holds n_heads pairs (b, h); every
 * per-head output is a slab: dq, dk, dv [n_heads, N, d]; lse, D [n_heads, N].
 */
int oracle_attention_backward(const double* q, const double* k, const double* v,
                              const double* dout, int64_t B, int64_t H, int64_t N,
                              int64_t d, int causal, double scale, int64_t n_heads,
                              const int64_t* heads, double* dq, double* dk,
                              double* dv, double* lse, double* D) {
  if (bad_sizes(B, H, N, d) || n_heads < 0) return -1;
  for (int64_t t = 0; t < n_heads; ++t) {
    const int64_t b = heads[2 * t], h = heads[2 * t + 1];
    if (b < 0 || b >= B || h < 0 || h >= H) return -1;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!s || !dp) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < n_heads; ++t) {
        const size_t slab = (size_t)(t * N * d);
        backward_head(q, k, v, dout, H, N, d, causal, scale, heads[2 * t],
                      heads[2 * t + 1], s, dp, dq + slab, dk + slab, dv + slab,
                      lse + t * N, D + t * N);
      }
    }
    free(s);
    free(dp);
  }
  return failed ? -1 : 0;
}

int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
