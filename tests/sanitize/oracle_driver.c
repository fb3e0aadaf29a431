/* Drives oracle.c under the host AddressSanitizer and UndefinedBehaviorSanitizer:
 * every entry point on small problems (both masks, several scales, ragged
 * sizes, a single token, row subsets, a subset of heads) and on invalid
 * arguments.  Exit status 0 when every call returns what it should and every
 * output is finite; any sanitizer report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention_forward(const double* q, const double* k, const double* v, int64_t B,
                             int64_t H, int64_t N, int64_t d, int causal, double scale,
                             double* o, double* lse);
int oracle_attention_forward_rows(const double* q, const double* k, const double* v, int64_t B,
                                  int64_t H, int64_t N, int64_t d, int causal, double scale,
                                  int64_t n_rows, const int64_t* rows, double* o, double* lse);
int oracle_attention_backward(const double* q, const double* k, const double* v,
                              const double* dout, int64_t B, int64_t H, int64_t N, int64_t d,
                              int causal, double scale, int64_t n_heads, const int64_t* heads,
                              double* dq, double* dk, double* dv, double* lse, double* D);

static uint64_t state = 88172645463325252ull;
static double uniform(void) { /* xorshift64, mapped to [-2, 2) */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / 9007199254740992.0 * 4.0 - 2.0;
}

static double* filled(size_t n) {
  double* p = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = uniform();
  return p;
}

static int all_finite(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run(int64_t B, int64_t H, int64_t N, int64_t d, int causal, double scale) {
  const size_t e = (size_t)(B * H * N * d), r = (size_t)(B * H * N);
  double *q = filled(e), *k = filled(e), *v = filled(e), *g = filled(e);
  double* o = (double*)malloc((e ? e : 1) * sizeof(double));
  double* lse = (double*)malloc((r ? r : 1) * sizeof(double));
  int bad = oracle_attention_forward(q, k, v, B, H, N, d, causal, scale, o, lse) != 0 ||
            !all_finite(o, e) || !all_finite(lse, r);
  /* a few rows, the first and last included */
  int64_t rows[3 * 4];
  int64_t n_rows = 0;
  if (r) {
    const int64_t pick[4][3] = {{0, 0, 0}, {B - 1, H - 1, N - 1}, {0, H - 1, N / 2}, {B - 1, 0, 1 % N}};
    for (int t = 0; t < 4; ++t, ++n_rows)
      for (int c = 0; c < 3; ++c) rows[3 * t + c] = pick[t][c];
  }
  double* orow = (double*)malloc(4 * (size_t)d * sizeof(double));
  double lrow[4];
  bad |= oracle_attention_forward_rows(q, k, v, B, H, N, d, causal, scale, n_rows, rows, orow,
                                       lrow) != 0;
  bad |= !all_finite(orow, (size_t)n_rows * (size_t)d);
  /* backward of every head, then of one head */
  const int64_t nh = B * H;
  int64_t* heads = (int64_t*)malloc((size_t)(2 * (nh ? nh : 1)) * sizeof(int64_t));
  for (int64_t t = 0; t < nh; ++t) {
    heads[2 * t] = t / H;
    heads[2 * t + 1] = t % H;
  }
  double *dq = (double*)malloc((e ? e : 1) * sizeof(double)),
         *dk = (double*)malloc((e ? e : 1) * sizeof(double)),
         *dv = (double*)malloc((e ? e : 1) * sizeof(double)),
         *l2 = (double*)malloc((r ? r : 1) * sizeof(double)),
         *D = (double*)malloc((r ? r : 1) * sizeof(double));
  bad |= oracle_attention_backward(q, k, v, g, B, H, N, d, causal, scale, nh, heads, dq, dk, dv,
                                   l2, D) != 0;
  bad |= !all_finite(dq, e) || !all_finite(dk, e) || !all_finite(dv, e) || !all_finite(D, r);
  if (nh > 1) bad |= oracle_attention_backward(q, k, v, g, B, H, N, d, causal, scale, 1,
                                               heads + 2 * (nh - 1), dq, dk, dv, l2, D) != 0;
  free(q); free(k); free(v); free(g); free(o); free(lse); free(orow); free(heads);
  free(dq); free(dk); free(dv); free(l2); free(D);
  if (bad) fprintf(stderr, "failed: B=%ld H=%ld N=%ld d=%ld causal=%d scale=%g\n", (long)B,
                   (long)H, (long)N, (long)d, causal, scale);
  return bad;
}

int main(void) {
  int bad = 0;
  const double scales[] = {0.125, 0.0, -0.3, 20.0};
  for (int c = 0; c < 2; ++c)
    for (int s = 0; s < 4; ++s) {
      bad |= run(2, 3, 37, 8, c, scales[s]);
      bad |= run(1, 1, 1, 16, c, scales[s]);
      bad |= run(1, 2, 130, 64, c, scales[s]);
    }
  /* invalid arguments are refused, not read past */
  double x = 0.0;
  int64_t badrow[3] = {0, 0, 5};
  int64_t badhead[2] = {1, 0};
  bad |= oracle_attention_forward(&x, &x, &x, -1, 1, 1, 1, 0, 1.0, &x, &x) == 0;
  bad |= oracle_attention_forward_rows(&x, &x, &x, 1, 1, 1, 1, 0, 1.0, 1, badrow, &x, &x) == 0;
  bad |= oracle_attention_backward(&x, &x, &x, &x, 1, 1, 1, 1, 0, 1.0, 1, badhead, &x, &x, &x,
                                   &x, &x) == 0;
  if (bad) return 1;
  printf("oracle sanitizer run: ok\n");
  return 0;
}
