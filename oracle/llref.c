/*
 * llref.c -- CPU oracle for the log-linear (Fenwick-tree) attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this library: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the HIP
 * library under fenwick_tree_linear_amd/.
 *
 * Source of the method: "Log-Linear Attention" (gist.science explainer page of
 * arXiv 2506.04761), technical summary section 2 ("Proposed method"):
 *   - 2.1: the prefix is partitioned by a Fenwick tree into buckets, each with
 *     its own hidden state S_t^(l); recent tokens fine, distant tokens coarse;
 *   - 2.2: o_t = sum_{l=0}^{L-1} lambda_t^(l) q_t^T S_t^(l), and the prefix
 *     [0,t) is split into at most L = O(log T) disjoint buckets by the Fenwick
 *     decomposition;
 *   - 2.3: a recurrent form with O(log T) state for decoding;
 *   - section 3: applied to Mamba-2 and Gated DeltaNet with their structure kept.
 *
 * The level weights may come from the adaptive-decay MLP of "Adaptive memory
 * decay for log-linear attention" (section "Method"): llref_lambda_mlp.
 *
 * Readings taken where the page is silent:
 *   - tokens are 0-based; bucket level 0 is the token itself; a bucket of level
 *     l >= 1 holds 2^(l-1) tokens;
 *   - Mamba-2 write: S_t = a_t S_{t-1} + k_t v_t^T, so source s reaches position
 *     t with weight prod_{r=s+1}^{t} a_r (the token's own gate does not touch its
 *     own write), given here as log a_r;
 *   - Gated DeltaNet write: S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T;
 *     the hierarchical level weights act on the read only, the pseudo-values
 *     u_t = b_t (v_t - a_t S_{t-1}^T k_t) being exactly those of plain GDN;
 *   - no normaliser, no 1/sqrt(d) inside the operator.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 *
 * Layouts (row-major, host memory, inputs given as fp32, arithmetic in fp64):
 *   q, k        [B,T,H,dk]      v       [B,T,H,dv]
 *   log_gate    [B,T,H]         beta    [B,T,H]       lambda [B,T,H,L]
 *   o           [B,T,H,dv] (double)
 *   state       [B,H,L,dk,dv] (double) -- the true per-level states, level 0
 *               unused between tokens.
 * rule: 0 = Mamba-2 scalar-gated write, 1 = Gated DeltaNet write.
 * Return value: 0 on success, a negative code for inconsistent arguments.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LLREF_OK 0
#define LLREF_EARG -1
#define LLREF_ELEVELS -2
#define LLREF_ENOMEM -3

/* threads an OpenMP region of this library uses */
int llref_threads(void) { return omp_get_max_threads(); }

/* floor(log2(x)) for x >= 1 */
static int floor_log2(int64_t x) {
  int r = 0;
  while (x > 1) {
    x >>= 1;
    r++;
  }
  return r;
}

/*
 * Level of source token s as seen from position t (section 2.2, Fenwick-tree
 * partition of the prefix).  The prefix [0,t) is peeled from its right end:
 * the last bucket has the size of the lowest set bit of t, then the next, and
 * so on.  A bucket of size 2^j gets level j+1; the token itself gets level 0.
 * Returns -1 for s outside [0,t].
 */
int llref_level(int64_t t, int64_t s) {
  if (s < 0 || s > t) return -1;
  if (s == t) return 0;
  int64_t end = t; /* the buckets found so far cover [end, t) */
  while (end > 0) {
    int64_t size = end & (-end);
    if (s >= end - size) return floor_log2(size) + 1;
    end -= size;
  }
  return -1;
}

/* out[s] = llref_level(t, s) for s = 0..t */
void llref_levels_row(int64_t t, int32_t *out) {
  for (int64_t s = 0; s <= t; s++) out[s] = llref_level(t, s);
}

/* number of trailing zero bits of x > 0 */
static int trailing_zeros(int64_t x) {
  int n = 0;
  while ((x & 1) == 0) {
    x >>= 1;
    n++;
  }
  return n;
}

static double dot_f(const float *x, const float *y, int n) {
  double acc = 0.0;
  for (int i = 0; i < n; i++) acc += (double)x[i] * (double)y[i];
  return acc;
}

typedef struct {
  int B, T, H, dk, dv, L;
} dims_t;

static size_t ix_tok(const dims_t *d, int b, int64_t t, int h) {
  return ((size_t)b * d->T + (size_t)t) * d->H + (size_t)h;
}

/* largest position t whose whole prefix fits in levels 0..L-1 */
static int levels_cover(int64_t T, int L) {
  if (L < 1 || L > 62) return 0;
  return T <= ((int64_t)1 << (L - 1));
}

/*
 * Gated DeltaNet pseudo-values of one head, from their definition:
 *   u_t = beta_t ( v_t - sum_{s<t} prod_{r=s+1}^{t} a_r (k_t . k_s) u_s ).
 * u is [T, dv] in double.
 */
static void gdn_pseudo_values(const dims_t *d, int b, int h, const float *k,
                              const float *v, const float *log_gate,
                              const float *beta, int64_t T, double *u) {
  for (int64_t t = 0; t < T; t++) {
    const float *kt = k + ix_tok(d, b, t, h) * d->dk;
    const float *vt = v + ix_tok(d, b, t, h) * d->dv;
    double *ut = u + (size_t)t * d->dv;
    for (int j = 0; j < d->dv; j++) ut[j] = vt[j];
    double logw = log_gate[ix_tok(d, b, t, h)]; /* sum_{r=s+1}^{t} log a_r for s = t-1 */
    for (int64_t s = t - 1; s >= 0; s--) {
      const float *ks = k + ix_tok(d, b, s, h) * d->dk;
      double w = exp(logw) * dot_f(kt, ks, d->dk);
      const double *us = u + (size_t)s * d->dv;
      for (int j = 0; j < d->dv; j++) ut[j] -= w * us[j];
      logw += log_gate[ix_tok(d, b, s, h)];
    }
    double bt = beta[ix_tok(d, b, t, h)];
    for (int j = 0; j < d->dv; j++) ut[j] *= bt;
  }
}

/*
 * Direct O(T^2) evaluation of the masked form (sections 2.2 and 2.3):
 *   o_t = sum_{s<=t} lambda_t^(lev(t,s)) prod_{r=s+1}^{t} a_r (q_t . k_s) w_s
 * with w_s = v_s (Mamba-2) or the GDN pseudo-value u_s.
 *
 * Only heads listed in `heads` (pairs b,h; NULL = every head) and positions
 * t in [t_lo, t_hi) are written to o.
 */
int llref_fwd_direct(int B, int T, int H, int dk, int dv, int L, int rule,
                     const float *q, const float *k, const float *v,
                     const float *log_gate, const float *lambda,
                     const float *beta, int nheads, const int32_t *heads,
                     int64_t t_lo, int64_t t_hi, double *o) {
  dims_t d = {B, T, H, dk, dv, L};
  if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1) return LLREF_EARG;
  if (!q || !k || !v || !log_gate || !lambda || !o) return LLREF_EARG;
  if (rule != 0 && rule != 1) return LLREF_EARG;
  if (rule == 1 && !beta) return LLREF_EARG;
  if (t_lo < 0 || t_hi > T || t_lo > t_hi) return LLREF_EARG;
  if (!levels_cover(t_hi, L)) return LLREF_ELEVELS;
  int n = heads ? nheads : B * H;
  int bad = 0;

#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int i = 0; i < n; i++) {
    int b = heads ? heads[2 * i] : i / H;
    int h = heads ? heads[2 * i + 1] : i % H;
    if (b < 0 || b >= B || h < 0 || h >= H) {
      bad |= 1;
      continue;
    }
    double *u = NULL;
    if (rule == 1) {
      u = (double *)malloc(sizeof(double) * (size_t)(t_hi > 0 ? t_hi : 1) * dv);
      if (!u) {
        bad |= 2;
        continue;
      }
      gdn_pseudo_values(&d, b, h, k, v, log_gate, beta, t_hi, u);
    }
    for (int64_t t = t_lo; t < t_hi; t++) {
      const float *qt = q + ix_tok(&d, b, t, h) * dk;
      const float *lam = lambda + ix_tok(&d, b, t, h) * L;
      double *ot = o + ix_tok(&d, b, t, h) * dv;
      for (int j = 0; j < dv; j++) ot[j] = 0.0;
      double logw = 0.0; /* sum_{r=s+1}^{t} log a_r */
      for (int64_t s = t; s >= 0; s--) {
        int lev = llref_level(t, s);
        const float *ks = k + ix_tok(&d, b, s, h) * dk;
        double w = (double)lam[lev] * exp(logw) * dot_f(qt, ks, dk);
        if (rule == 0) {
          const float *vs = v + ix_tok(&d, b, s, h) * dv;
          for (int j = 0; j < dv; j++) ot[j] += w * (double)vs[j];
        } else {
          const double *us = u + (size_t)s * dv;
          for (int j = 0; j < dv; j++) ot[j] += w * us[j];
        }
        logw += log_gate[ix_tok(&d, b, s, h)];
      }
    }
    free(u);
  }
  if (bad & 2) return LLREF_ENOMEM;
  if (bad) return LLREF_EARG;
  return LLREF_OK;
}

/*
 * Per-level states of the prefix [0,T) from their definition (section 2.2):
 * level l >= 1 of the Fenwick partition of [0,T) is the sum over its bucket of
 *   prod_{r=s+1}^{T-1} a_r k_s w_s^T,
 * i.e. decayed through the last token T-1.  Empty levels and level 0 are zero.
 * state is [B,H,L,dk,dv]; heads as in llref_fwd_direct.
 */
int llref_state_direct(int B, int T, int H, int dk, int dv, int L, int rule,
                       const float *k, const float *v, const float *log_gate,
                       const float *beta, int nheads, const int32_t *heads,
                       double *state) {
  dims_t d = {B, T, H, dk, dv, L};
  if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return LLREF_EARG;
  if (!k || !v || !log_gate || !state) return LLREF_EARG;
  if (rule != 0 && rule != 1) return LLREF_EARG;
  if (rule == 1 && !beta) return LLREF_EARG;
  /* the prefix [0,T) needs a bucket of level floor(log2 T)+1 */
  if (L < 2 || L > 62 || (T > 0 && floor_log2(T) + 1 > L - 1)) return LLREF_ELEVELS;
  int n = heads ? nheads : B * H;
  size_t per_level = (size_t)dk * dv;
  int bad = 0;

#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int i = 0; i < n; i++) {
    int b = heads ? heads[2 * i] : i / H;
    int h = heads ? heads[2 * i + 1] : i % H;
    if (b < 0 || b >= B || h < 0 || h >= H) {
      bad |= 1;
      continue;
    }
    double *st = state + ((size_t)b * H + h) * L * per_level;
    memset(st, 0, sizeof(double) * L * per_level);
    double *u = NULL;
    if (rule == 1 && T > 0) {
      u = (double *)malloc(sizeof(double) * (size_t)T * dv);
      if (!u) {
        bad |= 2;
        continue;
      }
      gdn_pseudo_values(&d, b, h, k, v, log_gate, beta, T, u);
    }
    double logw = 0.0; /* sum_{r=s+1}^{T-1} log a_r */
    for (int64_t s = T - 1; s >= 0; s--) {
      /* the bucket of s in the partition of [0,T): same peeling as llref_level */
      int lev = llref_level(T, s);
      double *S = st + (size_t)lev * per_level;
      double wgt = exp(logw);
      const float *ks = k + ix_tok(&d, b, s, h) * dk;
      for (int a = 0; a < dk; a++) {
        double ka = wgt * (double)ks[a];
        if (rule == 0) {
          const float *vs = v + ix_tok(&d, b, s, h) * dv;
          for (int j = 0; j < dv; j++) S[(size_t)a * dv + j] += ka * (double)vs[j];
        } else {
          const double *us = u + (size_t)s * dv;
          for (int j = 0; j < dv; j++) S[(size_t)a * dv + j] += ka * us[j];
        }
      }
      logw += log_gate[ix_tok(&d, b, s, h)];
    }
    free(u);
  }
  if (bad & 2) return LLREF_ENOMEM;
  if (bad) return LLREF_EARG;
  return LLREF_OK;
}

/*
 * One token of the recurrent form (section 2.3) on the true per-level states
 * S[0..L-1] of one head (S[0] empty on entry):
 *   1. every stored level decays by a_t;
 *   2. level 0 receives the token's own write k_t w_t^T (GDN: w_t = u_t with
 *      u_t = beta_t (v_t - (sum_l S[l])^T k_t), the sum taken after step 1);
 *   3. o_t = sum_l lambda_t^(l) S[l]^T q_t;
 *   4. the buckets of levels 0..c, c = ctz(t+1), are exactly the trailing part
 *      of the partition that becomes one bucket of level c+1 for [0,t+1):
 *      S[c+1] = sum_{l<=c} S[l], S[0..c] = 0.
 * Step 4 is skipped (merge == 0) only after the last token of a prefill whose
 * state is not exported.
 */
static void recurrent_token(int dk, int dv, int L, int rule, int64_t t,
                            const float *qt, const float *kt, const float *vt,
                            double log_a, const float *lam, double bt,
                            double *S, double *ot, double *scratch, int merge) {
  size_t per_level = (size_t)dk * dv;
  double a = exp(log_a);
  for (int l = 1; l < L; l++)
    for (size_t e = 0; e < per_level; e++) S[l * per_level + e] *= a;

  double *w = scratch; /* [dv] value written at level 0 */
  if (rule == 0) {
    for (int j = 0; j < dv; j++) w[j] = vt[j];
  } else {
    for (int j = 0; j < dv; j++) {
      double acc = 0.0;
      for (int l = 1; l < L; l++)
        for (int i = 0; i < dk; i++)
          acc += S[l * per_level + (size_t)i * dv + j] * (double)kt[i];
      w[j] = bt * ((double)vt[j] - acc);
    }
  }
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) S[(size_t)i * dv + j] = (double)kt[i] * w[j];

  if (ot) {
    for (int j = 0; j < dv; j++) {
      double acc = 0.0;
      for (int l = 0; l < L; l++) {
        double r = 0.0;
        for (int i = 0; i < dk; i++) r += S[l * per_level + (size_t)i * dv + j] * (double)qt[i];
        acc += (double)lam[l] * r;
      }
      ot[j] = acc;
    }
  }

  if (merge) {
    int c = trailing_zeros(t + 1);
    double *dst = S + (size_t)(c + 1) * per_level;
    for (size_t e = 0; e < per_level; e++) dst[e] = 0.0;
    for (int l = 0; l <= c; l++) {
      for (size_t e = 0; e < per_level; e++) dst[e] += S[l * per_level + e];
      for (size_t e = 0; e < per_level; e++) S[l * per_level + e] = 0.0;
    }
  }
}

/*
 * Recurrent O(T log T) form (section 2.3), independent of the direct form: it
 * never computes a level map, only the merge rule.  o (nullable) receives every
 * output row; state_out (nullable) receives the per-level states of [0,T)
 * decayed through token T-1.  heads as in llref_fwd_direct.
 */
int llref_fwd_recurrent(int B, int T, int H, int dk, int dv, int L, int rule,
                        const float *q, const float *k, const float *v,
                        const float *log_gate, const float *lambda,
                        const float *beta, int nheads, const int32_t *heads,
                        double *o, double *state_out) {
  dims_t d = {B, T, H, dk, dv, L};
  if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1) return LLREF_EARG;
  if (!k || !v || !log_gate) return LLREF_EARG;
  if (o && (!q || !lambda)) return LLREF_EARG;
  if (rule != 0 && rule != 1) return LLREF_EARG;
  if (rule == 1 && !beta) return LLREF_EARG;
  if (!levels_cover(T, L)) return LLREF_ELEVELS;
  if (state_out && T >= ((int64_t)1 << (L - 1))) return LLREF_ELEVELS;
  int n = heads ? nheads : B * H;
  size_t per_level = (size_t)dk * dv;
  int bad = 0;

#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int i = 0; i < n; i++) {
    int b = heads ? heads[2 * i] : i / H;
    int h = heads ? heads[2 * i + 1] : i % H;
    if (b < 0 || b >= B || h < 0 || h >= H) {
      bad |= 1;
      continue;
    }
    double *S = (double *)calloc((size_t)L * per_level, sizeof(double));
    double *scratch = (double *)malloc(sizeof(double) * dv);
    if (!S || !scratch) {
      free(S);
      free(scratch);
      bad |= 2;
      continue;
    }
    for (int64_t t = 0; t < T; t++) {
      size_t tok = ix_tok(&d, b, t, h);
      int merge = (t + 1 < T) || (state_out != NULL);
      recurrent_token(dk, dv, L, rule, t, q ? q + tok * dk : NULL, k + tok * dk,
                      v + tok * dv, log_gate[tok], lambda ? lambda + tok * L : NULL,
                      beta ? beta[tok] : 0.0, S, o ? o + tok * dv : NULL, scratch,
                      merge);
    }
    if (state_out)
      memcpy(state_out + ((size_t)b * H + h) * L * per_level, S,
             sizeof(double) * L * per_level);
    free(S);
    free(scratch);
  }
  if (bad & 2) return LLREF_ENOMEM;
  if (bad) return LLREF_EARG;
  return LLREF_OK;
}

/*
 * One decode step at position pos for every head (section 2.3).  state holds
 * the true per-level states of [0,pos) ([B,H,L,dk,dv], level 0 empty) and is
 * updated in place to those of [0,pos+1).  Per-token inputs drop the T axis:
 * q,k [B,H,dk], v [B,H,dv], log_gate/beta [B,H], lambda [B,H,L]; o [B,H,dv].
 * The state of [0,pos+1) must fit: pos + 1 < 2^(L-1).
 */
int llref_decode_step(int B, int H, int dk, int dv, int L, int rule, int64_t pos,
                      const float *q, const float *k, const float *v,
                      const float *log_gate, const float *lambda,
                      const float *beta, double *o, double *state) {
  if (B < 1 || H < 1 || dk < 1 || dv < 1 || pos < 0) return LLREF_EARG;
  if (!q || !k || !v || !log_gate || !lambda || !o || !state) return LLREF_EARG;
  if (rule != 0 && rule != 1) return LLREF_EARG;
  if (rule == 1 && !beta) return LLREF_EARG;
  if (L < 2 || L > 62 || pos + 1 >= ((int64_t)1 << (L - 1))) return LLREF_ELEVELS;
  size_t per_level = (size_t)dk * dv;
  int bad = 0;

#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int i = 0; i < B * H; i++) {
    double *scratch = (double *)malloc(sizeof(double) * dv);
    if (!scratch) {
      bad |= 2;
      continue;
    }
    recurrent_token(dk, dv, L, rule, pos, q + (size_t)i * dk, k + (size_t)i * dk,
                    v + (size_t)i * dv, log_gate[i], lambda + (size_t)i * L,
                    beta ? beta[i] : 0.0, state + (size_t)i * L * per_level,
                    o + (size_t)i * dv, scratch, 1);
    free(scratch);
  }
  if (bad) return LLREF_ENOMEM;
  return LLREF_OK;
}

/*
 * The level weights from the adaptive-decay MLP ("Adaptive memory decay for
 * log-linear attention", section "Method", LambdaMLPSoftplus): for every token
 * and head, with d the baseline's per-level representation,
 *   h = d W1            (d [L], W1 [L][hidden])
 *   z = h W2 + b        (W2 [hidden][L], b [L])
 *   lambda = softplus(z) = log(1 + e^z)
 * in that order, layer by layer, in double precision.  softplus is evaluated
 * as max(z, 0) + log1p(e^-|z|), which is log(1 + e^z) without overflow.
 * d and lambda are [rows][L] (rows = B*T*H, or B*H for one decode step).
 */
int llref_lambda_mlp(int64_t rows, int L, int hidden, const float *d, const float *w1,
                     const float *w2, const float *bias, double *lambda) {
  if (rows < 0 || L < 1 || hidden < 1) return LLREF_EARG;
  if (rows > 0 && (!d || !w1 || !w2 || !bias || !lambda)) return LLREF_EARG;
  int bad = 0;

#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    double *h = (double *)malloc(sizeof(double) * hidden);
    if (!h) {
      bad |= 2;
      continue;
    }
    const float *dr = d + r * L;
    for (int j = 0; j < hidden; j++) {
      double acc = 0.0;
      for (int m = 0; m < L; m++) acc += (double)dr[m] * (double)w1[(size_t)m * hidden + j];
      h[j] = acc;
    }
    for (int l = 0; l < L; l++) {
      double z = (double)bias[l];
      for (int j = 0; j < hidden; j++) z += h[j] * (double)w2[(size_t)j * L + l];
      lambda[r * L + l] = (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
    }
    free(h);
  }
  if (bad) return LLREF_ENOMEM;
  return LLREF_OK;
}

/*
 * The curvature-conditioned query ("Don't read everything: curvature-
 * conditioned query for linear attention", section 2, "Mechanism"): before the
 * read, each query is contracted along the directions where the keys seen so
 * far are dense,
 *   mu_t    = (1/(t+1)) sum_{j<=t} k_j                      (running key mean)
 *   Sigma_t = (1/(t+1)) sum_{j<=t} k_j k_j^T - mu_t mu_t^T    (running key covariance)
 *   gamma_t = sigmoid(w_h . q_t + b_h)                         (query-conditioned gate)
 *   q_clean = q_t - gamma_t Sigma_t q_t
 * per token t and head h.  Readings taken where the page is silent: the
 * running covariance is the plain (population) covariance of keys 0..t, with
 * no decay; the gate has one weight vector and bias per head.  The running
 * sums are kept in double precision and Sigma_t is formed token by token.
 * q, k: [B][T][H][dk]; w: [H][dk]; b: [H]; q_clean: [B][T][H][dk].
 */
int llref_ccq_query(int B, int T, int H, int dk, const float *q, const float *k, const float *w,
                    const float *b, double *q_clean) {
  if (B < 1 || T < 0 || H < 1 || dk < 1) return LLREF_EARG;
  if (T > 0 && (!q || !k || !w || !b || !q_clean)) return LLREF_EARG;
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int bh = 0; bh < B * H; bh++) {
    const int bb = bh / H, h = bh % H;
    double *ksum = (double *)calloc((size_t)dk, sizeof(double));
    double *kk = (double *)calloc((size_t)dk * dk, sizeof(double));
    double *sig = (double *)malloc(sizeof(double) * dk * dk);
    if (!ksum || !kk || !sig) {
      bad |= 2;
      free(ksum);
      free(kk);
      free(sig);
      continue;
    }
    for (int t = 0; t < T; t++) {
      const size_t row = ((size_t)bb * T + t) * H + h;
      const float *kt = k + row * dk, *qt = q + row * dk;
      for (int i = 0; i < dk; i++) {
        ksum[i] += kt[i];
        for (int j = 0; j < dk; j++) kk[(size_t)i * dk + j] += (double)kt[i] * kt[j];
      }
      const double n = (double)(t + 1);
      for (int i = 0; i < dk; i++)
        for (int j = 0; j < dk; j++) sig[(size_t)i * dk + j] = kk[(size_t)i * dk + j] / n - (ksum[i] / n) * (ksum[j] / n);
      double z = b[h];
      for (int i = 0; i < dk; i++) z += (double)w[(size_t)h * dk + i] * qt[i];
      const double gamma = 1.0 / (1.0 + exp(-z));
      for (int i = 0; i < dk; i++) {
        double sq = 0.0;
        for (int j = 0; j < dk; j++) sq += sig[(size_t)i * dk + j] * qt[j];
        q_clean[row * dk + i] = qt[i] - gamma * sq;
      }
    }
    free(ksum);
    free(kk);
    free(sig);
  }
  if (bad) return LLREF_ENOMEM;
  return LLREF_OK;
}

/*
 * Gradients of the Mamba-2 log-linear read (the masked form of sections 2.2
 * and 2.3) for a loss whose gradient with respect to o is dO, from the
 * definition term by term.  With, for each pair s <= t,
 *   w  = prod_{r=s+1}^{t} a_r,   lam = lambda_t^(lev(t,s)),
 *   P  = q_t . k_s,              A   = dO_t . v_s,
 * the pair contributes lam w P v_s to o_t, hence
 *   dq_t += lam w A k_s,  dk_s += lam w A q_t,  dv_s += lam w P dO_t,
 *   dlambda_t^(lev) += w P A,
 * and, for s < t, lam w P A to dG_t and minus that to dG_s, where
 * G_t = sum_{r<=t} log a_r (w = e^{G_t - G_s}); then
 *   dlog_gate_r = sum_{t >= r} dG_t.
 * Inputs as llref_fwd_direct (Mamba-2 write); outputs in double, same
 * layouts: dq, dk [B][T][H][dk], dv [B][T][H][dv], dlog_gate [B][T][H],
 * dlambda [B][T][H][L].
 */
int llref_bwd_direct(int B, int T, int H, int dk, int dv, int L, const float *q, const float *k,
                     const float *v, const float *log_gate, const float *lambda, const float *dO,
                     double *dq, double *dk_out, double *dv_out, double *dlog_gate, double *dlambda) {
  if (B < 1 || T < 1 || H < 1 || dk < 1 || dv < 1) return LLREF_EARG;
  if (!q || !k || !v || !log_gate || !lambda || !dO) return LLREF_EARG;
  if (!dq || !dk_out || !dv_out || !dlog_gate || !dlambda) return LLREF_EARG;
  if (!levels_cover(T, L)) return LLREF_ELEVELS;
  const dims_t d = {B, T, H, dk, dv, L};
  memset(dq, 0, sizeof(double) * (size_t)B * T * H * dk);
  memset(dk_out, 0, sizeof(double) * (size_t)B * T * H * dk);
  memset(dv_out, 0, sizeof(double) * (size_t)B * T * H * dv);
  memset(dlambda, 0, sizeof(double) * (size_t)B * T * H * L);
  int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
  for (int bh = 0; bh < B * H; bh++) {
    const int b = bh / H, h = bh % H;
    double *dG = (double *)calloc((size_t)T, sizeof(double));
    if (!dG) {
      bad |= 2;
      continue;
    }
    for (int64_t t = 0; t < T; t++) {
      const size_t it = ix_tok(&d, b, t, h);
      const float *qt = q + it * dk, *dOt = dO + it * dv;
      double logw = 0.0; /* log w: the log-gates of tokens s+1..t */
      for (int64_t s = t; s >= 0; s--) {
        const size_t is = ix_tok(&d, b, s, h);
        const float *ks = k + is * dk, *vs = v + is * dv;
        const int lev = llref_level(t, s);
        const double w = exp(logw), lam = lambda[it * L + lev];
        const double P = dot_f(qt, ks, dk), A = dot_f(dOt, vs, dv);
        for (int i = 0; i < dk; i++) {
          dq[it * dk + i] += lam * w * A * ks[i];
          dk_out[is * dk + i] += lam * w * A * qt[i];
        }
        for (int j = 0; j < dv; j++) dv_out[is * dv + j] += lam * w * P * dOt[j];
        dlambda[it * L + lev] += w * P * A;
        if (s < t) {
          dG[t] += lam * w * P * A;
          dG[s] -= lam * w * P * A;
        }
        logw += log_gate[is];
      }
    }
    double acc = 0.0;
    for (int64_t r = T - 1; r >= 0; r--) {
      acc += dG[r];
      dlog_gate[ix_tok(&d, b, r, h)] = acc;
    }
    free(dG);
  }
  if (bad) return LLREF_ENOMEM;
  return LLREF_OK;
}
