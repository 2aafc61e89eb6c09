/*
 * Drives every entry point of the CPU oracle (oracle/llref.c) on small
 * inputs, including the degenerate shapes (one token, one level more than
 * needed, dk != dv, an empty row set, rejected arguments), so that an
 * AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle can check
 * its memory accesses and arithmetic.  Test infrastructure: built and run by
 * tests/test_sanitize.py, never part of the library.  Exit status 0 = every
 * call returned what it should; a sanitizer finding aborts with its report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int llref_threads(void);
int llref_level(int64_t t, int64_t s);
void llref_levels_row(int64_t t, int32_t *out);
int llref_fwd_direct(int B, int T, int H, int dk, int dv, int L, int rule, const float *q, const float *k,
                     const float *v, const float *log_gate, const float *lambda, const float *beta, int nheads,
                     const int32_t *heads, int64_t t_lo, int64_t t_hi, double *o);
int llref_state_direct(int B, int T, int H, int dk, int dv, int L, int rule, const float *k, const float *v,
                       const float *log_gate, const float *beta, int nheads, const int32_t *heads, double *state);
int llref_fwd_recurrent(int B, int T, int H, int dk, int dv, int L, int rule, const float *q, const float *k,
                        const float *v, const float *log_gate, const float *lambda, const float *beta, int nheads,
                        const int32_t *heads, double *o, double *state_out);
int llref_decode_step(int B, int H, int dk, int dv, int L, int rule, int64_t pos, const float *q, const float *k,
                      const float *v, const float *log_gate, const float *lambda, const float *beta, double *o,
                      double *state);
int llref_lambda_mlp(int64_t rows, int L, int hidden, const float *d, const float *w1, const float *w2,
                     const float *bias, double *lambda);
int llref_ccq_query(int B, int T, int H, int dk, const float *q, const float *k, const float *w, const float *b,
                    double *q_clean);
int llref_bwd_direct(int B, int T, int H, int dk, int dv, int L, const float *q, const float *k, const float *v,
                     const float *log_gate, const float *lambda, const float *dO, double *dq, double *dk_out,
                     double *dv_out, double *dlog_gate, double *dlambda);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float uni(void) { /* xorshift64*, uniform in [0, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (float)((rng * 2685821657736338717ull) >> 40) / (float)(1 << 24);
}
static float *arr(size_t n, float lo, float hi) {
  float *a = malloc(n * sizeof(float) + 1);
  for (size_t i = 0; i < n; i++) a[i] = lo + (hi - lo) * uni();
  return a;
}

static int failures = 0;
static void expect(int got, int want, const char *what) {
  if (got != want) {
    fprintf(stderr, "%s: returned %d, expected %d\n", what, got, want);
    failures++;
  }
}

static void run_shape(int B, int T, int H, int dk, int dv, int L, int rule) {
  const size_t rows = (size_t)B * T * H;
  float *q = arr(rows * dk, -0.5f, 0.5f), *k = arr(rows * dk, -0.5f, 0.5f), *v = arr(rows * dv, -1.f, 1.f);
  float *g = arr(rows, -0.1f, -0.001f), *lam = arr(rows * L, 0.2f, 2.f), *beta = arr(rows, 0.f, 1.f);
  float *dO = arr(rows * dv, -1.f, 1.f);
  double *o = calloc(rows * dv, sizeof(double)), *o2 = calloc(rows * dv, sizeof(double));
  double *st = calloc((size_t)B * H * L * dk * dv, sizeof(double));
  double *st2 = calloc((size_t)B * H * L * dk * dv, sizeof(double));
  const float *b = rule ? beta : NULL;
  int32_t heads[2] = {B - 1, H - 1};
  expect(llref_fwd_direct(B, T, H, dk, dv, L, rule, q, k, v, g, lam, b, 0, NULL, 0, T, o), 0, "fwd_direct");
  expect(llref_fwd_direct(B, T, H, dk, dv, L, rule, q, k, v, g, lam, b, 1, heads, T / 2, T, o), 0,
         "fwd_direct (one head, half the tokens)");
  expect(llref_fwd_recurrent(B, T, H, dk, dv, L, rule, q, k, v, g, lam, b, 0, NULL, o2, st), 0, "fwd_recurrent");
  expect(llref_state_direct(B, T, H, dk, dv, L, rule, k, v, g, b, 0, NULL, st2), 0, "state_direct");
  double maxd = 0.0;
  for (size_t i = 0; i < rows * dv; i++) maxd = fmax(maxd, fabs(o[i] - o2[i]));
  if (!(maxd < 1e-9)) {
    fprintf(stderr, "direct and recurrent forms differ by %g (B%d T%d H%d dk%d dv%d L%d rule %d)\n", maxd, B, T, H,
            dk, dv, L, rule);
    failures++;
  }
  /* one decode step after the prefix, inputs of the first token reused */
  double *od = calloc((size_t)B * H * dv, sizeof(double));
  if (T + 1 < (1LL << (L - 1)))
    expect(llref_decode_step(B, H, dk, dv, L, rule, T, q, k, v, g, lam, b, od, st), 0, "decode_step");
  if (rule == 0) {
    double *gq = calloc(rows * dk, sizeof(double)), *gk = calloc(rows * dk, sizeof(double));
    double *gv = calloc(rows * dv, sizeof(double)), *gg = calloc(rows, sizeof(double));
    double *gl = calloc(rows * L, sizeof(double));
    expect(llref_bwd_direct(B, T, H, dk, dv, L, q, k, v, g, lam, dO, gq, gk, gv, gg, gl), 0, "bwd_direct");
    free(gq), free(gk), free(gv), free(gg), free(gl);
  }
  free(q), free(k), free(v), free(g), free(lam), free(beta), free(dO), free(o), free(o2), free(st), free(st2),
      free(od);
}

int main(void) {
  if (llref_threads() < 1) failures++;
  int32_t row[70];
  llref_levels_row(69, row);
  for (int s = 0; s <= 69; s++) expect(row[s], llref_level(69, s), "levels_row");

  run_shape(1, 1, 1, 4, 4, 2, 0);     /* one token */
  run_shape(2, 37, 3, 8, 8, 7, 0);    /* ragged length */
  run_shape(1, 64, 2, 16, 16, 8, 0);  /* a power of two, one level spare */
  run_shape(2, 29, 2, 8, 12, 6, 0);   /* dk != dv */
  run_shape(1, 33, 2, 8, 8, 7, 1);    /* Gated DeltaNet */
  run_shape(1, 20, 1, 6, 5, 6, 1);    /* Gated DeltaNet, dk != dv */

  /* level-weight MLP, including no rows */
  float *d = arr(7 * 5, -1.f, 1.f), *w1 = arr(5 * 10, -1.f, 1.f), *w2 = arr(10 * 5, -1.f, 1.f);
  float *bias = arr(5, 0.f, 1.f);
  double *lam = calloc(7 * 5, sizeof(double));
  expect(llref_lambda_mlp(7, 5, 10, d, w1, w2, bias, lam), 0, "lambda_mlp");
  expect(llref_lambda_mlp(0, 5, 10, NULL, NULL, NULL, NULL, NULL), 0, "lambda_mlp (no rows)");
  /* curvature-conditioned query */
  float *q = arr(2 * 9 * 3 * 4, -1.f, 1.f), *k = arr(2 * 9 * 3 * 4, -1.f, 1.f), *w = arr(3 * 4, -1.f, 1.f);
  float *bb = arr(3, -1.f, 1.f);
  double *qc = calloc(2 * 9 * 3 * 4, sizeof(double));
  expect(llref_ccq_query(2, 9, 3, 4, q, k, w, bb, qc), 0, "ccq_query");

  /* rejected arguments: too few levels, a NULL input, an out-of-range head */
  int32_t bad_head[2] = {5, 0};
  double *o = calloc(64 * 4, sizeof(double));
  float *x = arr(64 * 4, 0.f, 1.f), *gg = arr(64, -0.1f, 0.f), *ll = arr(64 * 8, 0.f, 1.f);
  if (llref_fwd_direct(1, 64, 1, 4, 4, 3, 0, x, x, x, gg, ll, NULL, 0, NULL, 0, 64, o) == 0) failures++;
  if (llref_fwd_direct(1, 64, 1, 4, 4, 8, 0, x, NULL, x, gg, ll, NULL, 0, NULL, 0, 64, o) == 0) failures++;
  if (llref_fwd_recurrent(1, 64, 1, 4, 4, 8, 0, x, x, x, gg, ll, NULL, 1, bad_head, o, NULL) == 0) failures++;
  free(d), free(w1), free(w2), free(bias), free(lam), free(q), free(k), free(w), free(bb), free(qc), free(o), free(x),
      free(gg), free(ll);
  if (failures) fprintf(stderr, "%d failures\n", failures);
  else printf("oracle driver: all calls returned as expected\n");
  return failures ? 1 : 0;
}
