/*
 * ssm_oracle.c -- float64 CPU oracle for the selective state-space scan VJP.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header, table or helper with the
 * HIP kernels.
 *
 * Everything is float64, single pass, no blocking beyond what the definitions
 * themselves state, and reductions run in a fixed (ascending) order so results
 * are reproducible run to run.  Work is split over independent (batch, head)
 * tasks with OpenMP; per-head partials of dB/dC are summed after the join in
 * ascending head order.
 *
 * Sources (the method pages):
 *  [P1] burn-mamba, "combined_backward.rs" (Mamba-3 double-SSD recompute backward):
 *       CombinedGrads, k3_ssd_chunk_state_extended, combined_backward -- the
 *       K1..K4 recompute, the reverse per-chunk loop (BLUE, ORANGE, K4 step) and
 *       the batched K3/K2/K1 backwards.
 *  [P2] K3 notes, section "反向传播推导" (backward derivation of the KDA gated
 *       delta rule): the forward F1..F6, the warning box on the two paths into
 *       the gated state's gradient, and the grouping of value heads under qk
 *       heads.  The backward here is derived from F1..F6 (see orc_kda_bwd).
 *  [P3] llama.cpp PR "S1-31: SSM_SCAN_BACK -- Mamba has a backward": the reverse
 *       recurrence with the non-zero final-state seed, store-all states, the
 *       Mamba-2 (per-head decay) and Mamba-1 (per-state decay) branches, and the
 *       five mutations of its verification table.
 *
 * Readings taken where the pages are silent:
 *  - dt is the raw pre-softplus value; delta = softplus(dt) (P3: "drop the
 *    softplus derivative" is a defect).  softplus(z) = log1p(exp(z)), z > 20 -> z.
 *  - the input is scaled by delta (P1: "(pre-scaled) input v"): v = x * delta.
 *  - y_t reads the state after the step-t update (P3: "s_{t-1} where s_t belongs
 *    in dC" is a defect; P1's triu(1) mask keeps the diagonal).
 *  - heads map to groups in contiguous blocks: g = h / (H/G).
 *  - a chunked run whose length is not a multiple of the chunk length ends with
 *    one shorter chunk (the chunked form is an exact re-association of the
 *    sequential recurrence, so a shorter last chunk is the same computation).
 *
 * Mutation switches: every backward takes `mutation`; 0 is the method.  A
 * non-zero value plants one named defect so the tests can show the
 * finite-difference check catches it (P3's verification table).  They exist
 * only for that test.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

/* mutation ids (mirrored in oracle/__init__.py) */
enum {
  MUT_NONE = 0,
  /* P3's table */
  MUT_DROP_DA_PATH = 1,      /* drop the dA term of d(delta) */
  MUT_ZERO_SEED = 2,         /* seed dS with zeros instead of ds_final */
  MUT_DROP_Y_TO_DS = 3,      /* drop y's own contribution dS += C (x) dy */
  MUT_PREV_STATE_IN_DC = 4,  /* use s_{t-1} where s_t belongs in dC */
  MUT_DROP_SOFTPLUS = 5,     /* drop sigma(dt), the softplus derivative */
  /* chunked form (P1) */
  MUT_DROP_BLUE_DA = 11,     /* drop BLUE's d_cumA term */
  MUT_DROP_ORANGE_DA = 12,   /* drop ORANGE's d_cumA term */
  MUT_DROP_K3_DA = 13,       /* drop K3's d_cumA terms */
  MUT_DROP_K4_DA = 14,       /* drop K4's d_da_chunk_end term */
  MUT_PREFIX_K1 = 15,        /* prefix instead of suffix sum in the K1 backward */
  MUT_STRICT_MASK = 16,      /* triu(0) mask: drop the diagonal of the causal mask */
  MUT_NO_M_REDUCE = 17,      /* forget the mimo_rank reduction of d_cumA (keep m=0) */
  /* KDA (P2) */
  MUT_DROP_KDR = 21,         /* drop the residual path -beta k u^T from the gated state's gradient */
  MUT_WRONG_GVA = 22         /* map value head hv to qk head hv % H instead of hv / G */
};

static double softplus(double z) { return z > 20.0 ? z : log1p(exp(z)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* ------------------------------------------------------------------------- */
/* O1: Mamba sequential scan (P3), Mamba-2 per-head decay or Mamba-1 per-state */
/*                                                                           */
/* x[b,T,H,P] dt[b,T,H] A[H] (per_state=0) or A[H,N] (per_state=1)           */
/* B,C[b,T,G,N] s0[b,H,P,N] (NULL = zeros) -> y[b,T,H,P], s_final[b,H,P,N]    */
/* ------------------------------------------------------------------------- */

#define IX4(a, b_, c, d, B_, C_, D_) ((((i64)(a) * (B_) + (b_)) * (C_) + (c)) * (D_) + (d))

static double decay_coef(const double* A, int per_state, i64 h, i64 n, i64 N) {
  return per_state ? A[h * N + n] : A[h];
}

int orc_mamba_seq_fwd(i64 b, i64 T, i64 H, i64 P, i64 N, i64 G, int per_state,
                      const double* x, const double* dt, const double* A,
                      const double* B, const double* C, const double* s0,
                      double* y, double* s_final, int nthreads) {
  if (b < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
  const i64 hpg = H / G;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * H; ++task) {
    const i64 bi = task / H, h = task % H, g = h / hpg;
    double* s = (double*)malloc(sizeof(double) * P * N);
    for (i64 e = 0; e < P * N; ++e) s[e] = s0 ? s0[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 t = 0; t < T; ++t) {
      const double d = softplus(dt[(bi * T + t) * H + h]);
      const double* Bt = B + IX4(bi, t, g, 0, T, G, N);
      const double* Ct = C + IX4(bi, t, g, 0, T, G, N);
      const double* xt = x + IX4(bi, t, h, 0, T, H, P);
      for (i64 p = 0; p < P; ++p) {
        double acc = 0.0;
        for (i64 n = 0; n < N; ++n) {
          const double a = exp(d * decay_coef(A, per_state, h, n, N));
          s[p * N + n] = a * s[p * N + n] + d * xt[p] * Bt[n];
          acc += Ct[n] * s[p * N + n];
        }
        y[IX4(bi, t, h, p, T, H, P)] = acc;
      }
    }
    for (i64 e = 0; e < P * N; ++e) s_final[IX4(bi, h, 0, 0, H, P, N) + e] = s[e];
    free(s);
  }
  return 0;
}

/* Store-all reverse recurrence (P3: seeded with ds_final at t = T, walking t
 * from T-1 down to 0, all T+1 states recomputed and kept). */
/* dA (optional, NULL = not computed): the gradient of the decay coefficients,
 * [H] (per head) or [H,N] (per state).  a_t = exp(delta_t A) gives
 * d s_t / d A = delta_t a_t s_{t-1} elementwise, so
 * dA[h,n] = sum_{b,t} delta_t a_t[n] sum_p dS_t[p,n] s_{t-1}[p,n]
 * (summed over n as well for a per-head A), with dS_t the gradient of s_t. */
int orc_mamba_seq_bwd(i64 b, i64 T, i64 H, i64 P, i64 N, i64 G, int per_state,
                      const double* x, const double* dt, const double* A,
                      const double* B, const double* C, const double* s0,
                      const double* dy, const double* ds_final,
                      double* dx, double* d_dt, double* dB, double* dC, double* d_s0, double* dA,
                      int mutation, int nthreads) {
  if (b < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
  const i64 hpg = H / G;
  /* per-head partials of dB and dC, summed over the group after the join */
  double* dBh = (double*)calloc((size_t)(b * T * H * N) + 1, sizeof(double));
  double* dCh = (double*)calloc((size_t)(b * T * H * N) + 1, sizeof(double));
  /* per-(batch, head) partials of dA, summed over the batch after the join */
  double* dAb = (double*)calloc((size_t)(b * H * N) + 1, sizeof(double));
  if (!dBh || !dCh || !dAb) { free(dBh); free(dCh); free(dAb); return 2; }
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * H; ++task) {
    const i64 bi = task / H, h = task % H, g = h / hpg;
    const i64 PN = P * N;
    double* S = (double*)malloc(sizeof(double) * (size_t)((T + 1) * PN)); /* S[t+1] = s_t, S[0] = s0 */
    double* dS = (double*)malloc(sizeof(double) * (size_t)PN);
    if (!S || !dS) { fail = 1; free(S); free(dS); continue; }
    /* forward, store all */
    for (i64 e = 0; e < PN; ++e) S[e] = s0 ? s0[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 t = 0; t < T; ++t) {
      const double d = softplus(dt[(bi * T + t) * H + h]);
      const double* Bt = B + IX4(bi, t, g, 0, T, G, N);
      const double* xt = x + IX4(bi, t, h, 0, T, H, P);
      const double* sp = S + t * PN;
      double* sn = S + (t + 1) * PN;
      for (i64 p = 0; p < P; ++p)
        for (i64 n = 0; n < N; ++n) {
          const double a = exp(d * decay_coef(A, per_state, h, n, N));
          sn[p * N + n] = a * sp[p * N + n] + d * xt[p] * Bt[n];
        }
    }
    /* reverse recurrence, seeded with the final-state gradient */
    for (i64 e = 0; e < PN; ++e)
      dS[e] = (ds_final && mutation != MUT_ZERO_SEED) ? ds_final[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 t = T - 1; t >= 0; --t) {
      const double zt = dt[(bi * T + t) * H + h];
      const double d = softplus(zt);
      const double* Bt = B + IX4(bi, t, g, 0, T, G, N);
      const double* Ct = C + IX4(bi, t, g, 0, T, G, N);
      const double* xt = x + IX4(bi, t, h, 0, T, H, P);
      const double* dyt = dy + IX4(bi, t, h, 0, T, H, P);
      const double* s_t = S + (t + 1) * PN;   /* state after step t */
      const double* s_prev = S + t * PN;      /* state before step t */
      /* y_t = C_t . s_t contributes dy_t (x) C_t to the state gradient */
      if (mutation != MUT_DROP_Y_TO_DS)
        for (i64 p = 0; p < P; ++p)
          for (i64 n = 0; n < N; ++n) dS[p * N + n] += dyt[p] * Ct[n];
      /* dC_t (this head's share): sum_p dy_t[p] s_t[p,n] */
      const double* s_for_dc = (mutation == MUT_PREV_STATE_IN_DC) ? s_prev : s_t;
      for (i64 n = 0; n < N; ++n) {
        double acc = 0.0;
        for (i64 p = 0; p < P; ++p) acc += dyt[p] * s_for_dc[p * N + n];
        dCh[IX4(bi, t, h, n, T, H, N)] = acc;
      }
      /* dx_t[p] = delta * sum_n dS[p,n] B_t[n] */
      for (i64 p = 0; p < P; ++p) {
        double acc = 0.0;
        for (i64 n = 0; n < N; ++n) acc += dS[p * N + n] * Bt[n];
        dx[IX4(bi, t, h, p, T, H, P)] = d * acc;
      }
      /* dB_t (this head's share): delta * sum_p dS[p,n] x_t[p] */
      for (i64 n = 0; n < N; ++n) {
        double acc = 0.0;
        for (i64 p = 0; p < P; ++p) acc += dS[p * N + n] * xt[p];
        dBh[IX4(bi, t, h, n, T, H, N)] = d * acc;
      }
      /* d(delta): input path x B plus the decay path A a s_{t-1} */
      double ddelta = 0.0;
      for (i64 p = 0; p < P; ++p)
        for (i64 n = 0; n < N; ++n) {
          const double An = decay_coef(A, per_state, h, n, N);
          const double a = exp(d * An);
          double term = xt[p] * Bt[n];
          if (mutation != MUT_DROP_DA_PATH) term += An * a * s_prev[p * N + n];
          ddelta += dS[p * N + n] * term;
          /* dA: d s_t / d A = delta a s_{t-1} */
          dAb[(bi * H + h) * N + n] += dS[p * N + n] * d * a * s_prev[p * N + n];
        }
      d_dt[(bi * T + t) * H + h] = (mutation == MUT_DROP_SOFTPLUS) ? ddelta : ddelta * sigmoid(zt);
      /* carry the gradient to s_{t-1} */
      for (i64 p = 0; p < P; ++p)
        for (i64 n = 0; n < N; ++n)
          dS[p * N + n] *= exp(d * decay_coef(A, per_state, h, n, N));
    }
    for (i64 e = 0; e < PN; ++e) d_s0[IX4(bi, h, 0, 0, H, P, N) + e] = dS[e];
    free(S);
    free(dS);
  }
  /* group reduction in ascending head order */
  for (i64 bi = 0; bi < b; ++bi)
    for (i64 t = 0; t < T; ++t)
      for (i64 g = 0; g < G; ++g)
        for (i64 n = 0; n < N; ++n) {
          double sb = 0.0, sc = 0.0;
          for (i64 hh = g * hpg; hh < (g + 1) * hpg; ++hh) {
            sb += dBh[IX4(bi, t, hh, n, T, H, N)];
            sc += dCh[IX4(bi, t, hh, n, T, H, N)];
          }
          dB[IX4(bi, t, g, n, T, G, N)] = sb;
          dC[IX4(bi, t, g, n, T, G, N)] = sc;
        }
  /* dA: sum over the batch (and over n for a per-head A), ascending */
  if (dA) {
    for (i64 h = 0; h < H; ++h)
      for (i64 n = 0; n < (per_state ? N : 1); ++n) {
        double acc = 0.0;
        for (i64 bi = 0; bi < b; ++bi)
          for (i64 nn = (per_state ? n : 0); nn < (per_state ? n + 1 : N); ++nn) acc += dAb[(bi * H + h) * N + nn];
        dA[per_state ? h * N + n : h] = acc;
      }
  }
  free(dBh);
  free(dCh);
  free(dAb);
  return fail ? 2 : 0;
}

/* ------------------------------------------------------------------------- */
/* RAW rank-M sequential form: the recurrence that P1's chunked kernels       */
/* re-associate.  s_t = exp(da_t) s_{t-1} + sum_m v[t,m] (x) B[t,m];          */
/* y[t,m] = C[t,m] . s_t.                                                     */
/* v[b,T,M,H,P] da[b,T,H] B,C[b,T,M,G,N] s0[b,H,P,N]                          */
/* ------------------------------------------------------------------------- */

#define IX5(a, b_, c, d, e, B_, C_, D_, E_) (((((i64)(a) * (B_) + (b_)) * (C_) + (c)) * (D_) + (d)) * (E_) + (e))

int orc_raw_seq_fwd(i64 b, i64 T, i64 M, i64 H, i64 P, i64 N, i64 G,
                    const double* v, const double* da, const double* B, const double* C,
                    const double* s0, double* y, double* s_final, int nthreads) {
  if (b < 0 || T < 0 || M <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
  const i64 hpg = H / G;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * H; ++task) {
    const i64 bi = task / H, h = task % H, g = h / hpg;
    double* s = (double*)malloc(sizeof(double) * P * N);
    for (i64 e = 0; e < P * N; ++e) s[e] = s0 ? s0[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 t = 0; t < T; ++t) {
      const double a = exp(da[(bi * T + t) * H + h]);
      for (i64 e = 0; e < P * N; ++e) s[e] *= a;
      for (i64 m = 0; m < M; ++m) {
        const double* vt = v + IX5(bi, t, m, h, 0, T, M, H, P);
        const double* Bt = B + IX5(bi, t, m, g, 0, T, M, G, N);
        for (i64 p = 0; p < P; ++p)
          for (i64 n = 0; n < N; ++n) s[p * N + n] += vt[p] * Bt[n];
      }
      for (i64 m = 0; m < M; ++m) {
        const double* Ct = C + IX5(bi, t, m, g, 0, T, M, G, N);
        for (i64 p = 0; p < P; ++p) {
          double acc = 0.0;
          for (i64 n = 0; n < N; ++n) acc += Ct[n] * s[p * N + n];
          y[IX5(bi, t, m, h, p, T, M, H, P)] = acc;
        }
      }
    }
    for (i64 e = 0; e < P * N; ++e) s_final[IX4(bi, h, 0, 0, H, P, N) + e] = s[e];
    free(s);
  }
  return 0;
}

int orc_raw_seq_bwd(i64 b, i64 T, i64 M, i64 H, i64 P, i64 N, i64 G,
                    const double* v, const double* da, const double* B, const double* C,
                    const double* s0, const double* dy, const double* ds_final,
                    double* dv, double* d_da, double* dB, double* dC, double* d_s0,
                    int nthreads) {
  if (b < 0 || T < 0 || M <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
  const i64 hpg = H / G;
  const i64 nBC = b * T * M * H * N;
  double* dBh = (double*)calloc((size_t)nBC + 1, sizeof(double));
  double* dCh = (double*)calloc((size_t)nBC + 1, sizeof(double));
  if (!dBh || !dCh) { free(dBh); free(dCh); return 2; }
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * H; ++task) {
    const i64 bi = task / H, h = task % H, g = h / hpg;
    const i64 PN = P * N;
    double* S = (double*)malloc(sizeof(double) * (size_t)((T + 1) * PN));
    double* dS = (double*)malloc(sizeof(double) * (size_t)PN);
    if (!S || !dS) { fail = 1; free(S); free(dS); continue; }
    for (i64 e = 0; e < PN; ++e) S[e] = s0 ? s0[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 t = 0; t < T; ++t) {
      const double a = exp(da[(bi * T + t) * H + h]);
      double* sn = S + (t + 1) * PN;
      for (i64 e = 0; e < PN; ++e) sn[e] = a * S[t * PN + e];
      for (i64 m = 0; m < M; ++m) {
        const double* vt = v + IX5(bi, t, m, h, 0, T, M, H, P);
        const double* Bt = B + IX5(bi, t, m, g, 0, T, M, G, N);
        for (i64 p = 0; p < P; ++p)
          for (i64 n = 0; n < N; ++n) sn[p * N + n] += vt[p] * Bt[n];
      }
    }
    for (i64 e = 0; e < PN; ++e) dS[e] = ds_final ? ds_final[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 t = T - 1; t >= 0; --t) {
      const double a = exp(da[(bi * T + t) * H + h]);
      const double* s_t = S + (t + 1) * PN;
      const double* s_prev = S + t * PN;
      for (i64 m = 0; m < M; ++m) {
        const double* Ct = C + IX5(bi, t, m, g, 0, T, M, G, N);
        const double* dyt = dy + IX5(bi, t, m, h, 0, T, M, H, P);
        for (i64 p = 0; p < P; ++p)
          for (i64 n = 0; n < N; ++n) dS[p * N + n] += dyt[p] * Ct[n];
        for (i64 n = 0; n < N; ++n) {
          double acc = 0.0;
          for (i64 p = 0; p < P; ++p) acc += dyt[p] * s_t[p * N + n];
          dCh[IX5(bi, t, m, h, n, T, M, H, N)] = acc;
        }
      }
      for (i64 m = 0; m < M; ++m) {
        const double* Bt = B + IX5(bi, t, m, g, 0, T, M, G, N);
        const double* vt = v + IX5(bi, t, m, h, 0, T, M, H, P);
        for (i64 p = 0; p < P; ++p) {
          double acc = 0.0;
          for (i64 n = 0; n < N; ++n) acc += dS[p * N + n] * Bt[n];
          dv[IX5(bi, t, m, h, p, T, M, H, P)] = acc;
        }
        for (i64 n = 0; n < N; ++n) {
          double acc = 0.0;
          for (i64 p = 0; p < P; ++p) acc += dS[p * N + n] * vt[p];
          dBh[IX5(bi, t, m, h, n, T, M, H, N)] = acc;
        }
      }
      double acc = 0.0;
      for (i64 e = 0; e < PN; ++e) acc += dS[e] * a * s_prev[e];
      d_da[(bi * T + t) * H + h] = acc;
      for (i64 e = 0; e < PN; ++e) dS[e] *= a;
    }
    for (i64 e = 0; e < PN; ++e) d_s0[IX4(bi, h, 0, 0, H, P, N) + e] = dS[e];
    free(S);
    free(dS);
  }
  for (i64 bi = 0; bi < b; ++bi)
    for (i64 t = 0; t < T; ++t)
      for (i64 m = 0; m < M; ++m)
        for (i64 g = 0; g < G; ++g)
          for (i64 n = 0; n < N; ++n) {
            double sb = 0.0, sc = 0.0;
            for (i64 hh = g * hpg; hh < (g + 1) * hpg; ++hh) {
              sb += dBh[IX5(bi, t, m, hh, n, T, M, H, N)];
              sc += dCh[IX5(bi, t, m, hh, n, T, M, H, N)];
            }
            dB[IX5(bi, t, m, g, n, T, M, G, N)] = sb;
            dC[IX5(bi, t, m, g, n, T, M, G, N)] = sc;
          }
  free(dBh);
  free(dCh);
  return fail ? 2 : 0;
}

/* ------------------------------------------------------------------------- */
/* O2: chunked SSD form (P1).  Same RAW inputs/layouts as above plus chunk    */
/* length L.  Forward: K1 cumsum, K2 CB, K3 intra-chunk state, K4 state       */
/* passing, K5 output = BLUE (inter-chunk) + ORANGE (intra-chunk).            */
/* ------------------------------------------------------------------------- */

/* Per-(batch, head) view of the RAW inputs with the group's B/C. */
typedef struct {
  i64 T, M, P, N, L, nc;
  const double *v, *da, *B, *C; /* strided views resolved through accessors */
  i64 bi, h, g, H, G;
} chunk_task;

static double tv(const chunk_task* k, i64 t, i64 m, i64 p) { return k->v[IX5(k->bi, t, m, k->h, p, k->T, k->M, k->H, k->P)]; }
static double tB(const chunk_task* k, i64 t, i64 m, i64 n) { return k->B[IX5(k->bi, t, m, k->g, n, k->T, k->M, k->G, k->N)]; }
static double tC(const chunk_task* k, i64 t, i64 m, i64 n) { return k->C[IX5(k->bi, t, m, k->g, n, k->T, k->M, k->G, k->N)]; }
static double tda(const chunk_task* k, i64 t) { return k->da[(k->bi * k->T + t) * k->H + k->h]; }
static i64 chunk_lo(const chunk_task* k, i64 c) { return c * k->L; }
static i64 chunk_hi(const chunk_task* k, i64 c) { i64 e = (c + 1) * k->L; return e < k->T ? e : k->T; }

/* K1: inclusive cumsum of da within each chunk, and the chunk-end value. */
static void k1_cumsum(const chunk_task* k, double* cumA, double* end) {
  for (i64 c = 0; c < k->nc; ++c) {
    double acc = 0.0;
    for (i64 t = chunk_lo(k, c); t < chunk_hi(k, c); ++t) { acc += tda(k, t); cumA[t] = acc; }
    end[c] = acc;
  }
}

/* K3 (extended) + K4: intra-chunk states from zero and the chunk-input states
 * S[c] (S[0] = s0, S[nc] = final). */
static void k3_k4_forward(const chunk_task* k, const double* cumA, const double* end,
                          const double* s0h, double* S) {
  const i64 PN = k->P * k->N;
  for (i64 e = 0; e < PN; ++e) S[e] = s0h ? s0h[e] : 0.0;
  for (i64 c = 0; c < k->nc; ++c) {
    double* Sc = S + c * PN;
    double* Sn = S + (c + 1) * PN;
    const double dec = exp(end[c]);
    for (i64 e = 0; e < PN; ++e) Sn[e] = dec * Sc[e];
    for (i64 t = chunk_lo(k, c); t < chunk_hi(k, c); ++t) {
      const double w = exp(end[c] - cumA[t]);
      for (i64 m = 0; m < k->M; ++m)
        for (i64 p = 0; p < k->P; ++p)
          for (i64 n = 0; n < k->N; ++n) Sn[p * k->N + n] += w * tv(k, t, m, p) * tB(k, t, m, n);
    }
  }
}

int orc_ssd_chunk_fwd(i64 b, i64 T, i64 M, i64 H, i64 P, i64 N, i64 G, i64 L,
                      const double* v, const double* da, const double* B, const double* C,
                      const double* s0, double* y, double* s_final, int nthreads) {
  if (b < 0 || T < 0 || M <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G || L <= 0) return 1;
  const i64 hpg = H / G, nc = (T + L - 1) / L;
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * H; ++task) {
    chunk_task k = {T, M, P, N, L, nc, v, da, B, C, task / H, task % H, (task % H) / hpg, H, G};
    const i64 PN = P * N;
    double* cumA = (double*)malloc(sizeof(double) * (size_t)(T + 1));
    double* end = (double*)malloc(sizeof(double) * (size_t)(nc + 1));
    double* S = (double*)malloc(sizeof(double) * (size_t)((nc + 1) * PN));
    if (!cumA || !end || !S) { fail = 1; free(cumA); free(end); free(S); continue; }
    k1_cumsum(&k, cumA, end);
    k3_k4_forward(&k, cumA, end, s0 ? s0 + IX4(k.bi, k.h, 0, 0, H, P, N) : NULL, S);
    for (i64 c = 0; c < nc; ++c) {
      const double* Sc = S + c * PN;
      for (i64 t = chunk_lo(&k, c); t < chunk_hi(&k, c); ++t)
        for (i64 m = 0; m < M; ++m)
          for (i64 p = 0; p < P; ++p) {
            /* BLUE: exp(cumA_t) C[t,m] . S_c[p,:] */
            double blue = 0.0;
            for (i64 n = 0; n < N; ++n) blue += tC(&k, t, m, n) * Sc[p * N + n];
            blue *= exp(cumA[t]);
            /* ORANGE: causal (CB . decay) v within the chunk */
            double orange = 0.0;
            for (i64 s = chunk_lo(&k, c); s <= t; ++s) {
              const double dec = exp(cumA[t] - cumA[s]);
              for (i64 mm = 0; mm < M; ++mm) {
                double cb = 0.0;
                for (i64 n = 0; n < N; ++n) cb += tC(&k, t, m, n) * tB(&k, s, mm, n);
                orange += cb * dec * tv(&k, s, mm, p);
              }
            }
            y[IX5(k.bi, t, m, k.h, p, T, M, H, P)] = blue + orange;
          }
    }
    for (i64 e = 0; e < PN; ++e) s_final[IX4(k.bi, k.h, 0, 0, H, P, N) + e] = S[nc * PN + e];
    free(cumA);
    free(end);
    free(S);
  }
  return fail ? 2 : 0;
}

/* The chunked backward, following P1's combined_backward step by step:
 * recompute K1..K4; reverse per-chunk loop with BLUE, ORANGE and the K4 step;
 * then the K3, K2 and K1 backwards over all chunks; then the combine. */
int orc_ssd_chunk_bwd(i64 b, i64 T, i64 M, i64 H, i64 P, i64 N, i64 G, i64 L,
                      const double* v, const double* da, const double* B, const double* C,
                      const double* s0, const double* dy, const double* ds_final,
                      double* dv, double* d_da, double* dB, double* dC, double* d_s0,
                      int mutation, int nthreads) {
  if (b < 0 || T < 0 || M <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G || L <= 0) return 1;
  const i64 hpg = H / G, nc = (T + L - 1) / L;
  const i64 nBC = b * T * M * H * N;
  double* dBh = (double*)calloc((size_t)nBC + 1, sizeof(double));
  double* dCh = (double*)calloc((size_t)nBC + 1, sizeof(double));
  if (!dBh || !dCh) { free(dBh); free(dCh); return 2; }
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * H; ++task) {
    chunk_task k = {T, M, P, N, L, nc, v, da, B, C, task / H, task % H, (task % H) / hpg, H, G};
    const i64 PN = P * N, bi = k.bi, h = k.h;
    double* cumA = (double*)malloc(sizeof(double) * (size_t)(T + 1));
    double* end = (double*)malloc(sizeof(double) * (size_t)(nc + 1));
    double* S = (double*)malloc(sizeof(double) * (size_t)((nc + 1) * PN));
    double* dintra = (double*)malloc(sizeof(double) * (size_t)(nc * PN + 1));
    double* dS = (double*)malloc(sizeof(double) * (size_t)PN);
    double* dstate_blue = (double*)malloc(sizeof(double) * (size_t)PN);
    double* dcumA = (double*)calloc((size_t)(T + 1), sizeof(double));          /* summed over m */
    double* dend = (double*)calloc((size_t)(nc + 1), sizeof(double));
    double* dvacc = (double*)calloc((size_t)(T * M * P + 1), sizeof(double));  /* [t][m][p] */
    double* dBacc = (double*)calloc((size_t)(T * M * N + 1), sizeof(double));  /* [t][m][n] */
    double* dCacc = (double*)calloc((size_t)(T * M * N + 1), sizeof(double));
    double* dcb = (double*)calloc((size_t)(L * M * L * M + 1), sizeof(double)); /* one chunk at a time */
    double* dcb_all = (double*)calloc((size_t)(nc * L * M * L * M + 1), sizeof(double));
    double* dcum_m = (double*)calloc((size_t)(M + 1), sizeof(double));
    if (!cumA || !end || !S || !dintra || !dS || !dstate_blue || !dcumA || !dend || !dvacc ||
        !dBacc || !dCacc || !dcb || !dcb_all || !dcum_m) {
      fail = 1;
      goto done;
    }
    /* ---- recompute forward intermediates: K1, K3, K4 (K2 is formed on the fly) ---- */
    k1_cumsum(&k, cumA, end);
    k3_k4_forward(&k, cumA, end, s0 ? s0 + IX4(bi, h, 0, 0, H, P, N) : NULL, S);

    /* ---- reverse per-chunk loop: BLUE + ORANGE + K4 step ---- */
    for (i64 e = 0; e < PN; ++e)
      dS[e] = ds_final ? ds_final[IX4(bi, h, 0, 0, H, P, N) + e] : 0.0;
    for (i64 c = nc - 1; c >= 0; --c) {
      const i64 lo = chunk_lo(&k, c), hi = chunk_hi(&k, c), Lc = hi - lo;
      const double* Sc = S + c * PN;
      /* BLUE backward: blue[t,m,p] = exp(cumA_t) sum_n C[t,m,n] S_c[p,n] */
      for (i64 e = 0; e < PN; ++e) dstate_blue[e] = 0.0;
      for (i64 t = lo; t < hi; ++t) {
        const double ea = exp(cumA[t]);
        for (i64 m = 0; m < M; ++m) dcum_m[m] = 0.0;
        for (i64 m = 0; m < M; ++m) {
          /* d_ch = dy * exp(cumA) */
          for (i64 p = 0; p < P; ++p) {
            const double dch = dy[IX5(bi, t, m, h, p, T, M, H, P)] * ea;
            for (i64 n = 0; n < N; ++n) dstate_blue[p * N + n] += tC(&k, t, m, n) * dch;
          }
          for (i64 n = 0; n < N; ++n) {
            double acc = 0.0;
            for (i64 p = 0; p < P; ++p) acc += dy[IX5(bi, t, m, h, p, T, M, H, P)] * ea * Sc[p * N + n];
            dCacc[(t * M + m) * N + n] += acc;
          }
          /* d_da (BLUE) = sum_p dy * ch * exp(cumA), ch = C . S^T */
          double acc = 0.0;
          for (i64 p = 0; p < P; ++p) {
            double ch = 0.0;
            for (i64 n = 0; n < N; ++n) ch += tC(&k, t, m, n) * Sc[p * N + n];
            acc += dy[IX5(bi, t, m, h, p, T, M, H, P)] * ch * ea;
          }
          dcum_m[m] = acc;
        }
        if (mutation != MUT_DROP_BLUE_DA) {
          /* reduce the fused l*m copies back to l */
          if (mutation == MUT_NO_M_REDUCE) dcumA[t] += dcum_m[0];
          else for (i64 m = 0; m < M; ++m) dcumA[t] += dcum_m[m];
        }
      }
      /* ORANGE backward over fused rows (t,m) x (s,mm), masked iff s > t */
      for (i64 e = 0; e < Lc * M * Lc * M; ++e) dcb[e] = 0.0;
      for (i64 t = lo; t < hi; ++t)
        for (i64 m = 0; m < M; ++m)
          for (i64 s = lo; s < hi; ++s)
            for (i64 mm = 0; mm < M; ++mm) {
              const int masked = (mutation == MUT_STRICT_MASK) ? (s >= t) : (s > t);
              const double decay = masked ? 0.0 : exp(cumA[t] - cumA[s]);
              double cb = 0.0;
              for (i64 n = 0; n < N; ++n) cb += tC(&k, t, m, n) * tB(&k, s, mm, n);
              double dw = 0.0;
              for (i64 p = 0; p < P; ++p) dw += dy[IX5(bi, t, m, h, p, T, M, H, P)] * tv(&k, s, mm, p);
              /* d_v_orange = w^T d_y */
              const double w = cb * decay;
              for (i64 p = 0; p < P; ++p)
                dvacc[(s * M + mm) * P + p] += w * dy[IX5(bi, t, m, h, p, T, M, H, P)];
              /* d_cb = d_w * decay ; d_diff = d_w * cb * decay */
              dcb[(((t - lo) * M + m) * Lc + (s - lo)) * M + mm] = dw * decay;
              const double ddiff = dw * cb * decay;
              if (mutation != MUT_DROP_ORANGE_DA) {
                /* diff = cumA_target - cumA_source */
                if (mutation != MUT_NO_M_REDUCE || m == 0) dcumA[t] += ddiff;
                if (mutation != MUT_NO_M_REDUCE || mm == 0) dcumA[s] -= ddiff;
              }
            }
      memcpy(dcb_all + c * L * M * L * M, dcb, sizeof(double) * (size_t)(Lc * M * Lc * M));
      /* K4 backward step: s_{c+1} = exp(end_c) s_c + intra_c */
      memcpy(dintra + c * PN, dS, sizeof(double) * (size_t)PN);
      const double dec = exp(end[c]);
      double dend_c = 0.0;
      for (i64 e = 0; e < PN; ++e) dend_c += dS[e] * Sc[e] * dec;
      dend[c] = dend_c;
      for (i64 e = 0; e < PN; ++e) dS[e] = dec * dS[e] + dstate_blue[e];
    }
    for (i64 e = 0; e < PN; ++e) d_s0[IX4(bi, h, 0, 0, H, P, N) + e] = dS[e];

    /* ---- K3 backward: intra = sum_t exp(end - cumA_t) v[t] (x) B[t] ---- */
    for (i64 c = 0; c < nc; ++c) {
      const i64 lo = chunk_lo(&k, c), hi = chunk_hi(&k, c);
      const double* di = dintra + c * PN;
      double qsum = 0.0;
      for (i64 t = lo; t < hi; ++t) {
        const double decay = exp(end[c] - cumA[t]);
        for (i64 m = 0; m < M; ++m) {
          double ddecay = 0.0;
          for (i64 p = 0; p < P; ++p) {
            double ddv = 0.0; /* d_decayed_v = d_intra . B^T */
            for (i64 n = 0; n < N; ++n) ddv += di[p * N + n] * tB(&k, t, m, n);
            ddecay += ddv * tv(&k, t, m, p);
            dvacc[(t * M + m) * P + p] += ddv * decay;
          }
          for (i64 n = 0; n < N; ++n) { /* d_b_k3 = decayed_v^T . d_intra */
            double acc = 0.0;
            for (i64 p = 0; p < P; ++p) acc += decay * tv(&k, t, m, p) * di[p * N + n];
            dBacc[(t * M + m) * N + n] += acc;
          }
          const double q = ddecay * decay;
          if (mutation != MUT_DROP_K3_DA) {
            if (mutation != MUT_NO_M_REDUCE || m == 0) dcumA[t] -= q;
            qsum += q;
          }
        }
      }
      if (hi > lo) {
        dcumA[hi - 1] += qsum;                                     /* d cumA_last (K3) */
        if (mutation != MUT_DROP_K4_DA) dcumA[hi - 1] += dend[c];  /* d da_chunk_end (K4) */
      }
    }
    /* ---- K2 backward: CB = C . B^T ---- */
    for (i64 c = 0; c < nc; ++c) {
      const i64 lo = chunk_lo(&k, c), hi = chunk_hi(&k, c), Lc = hi - lo;
      const double* dcbc = dcb_all + c * L * M * L * M;
      for (i64 t = lo; t < hi; ++t)
        for (i64 m = 0; m < M; ++m)
          for (i64 s = lo; s < hi; ++s)
            for (i64 mm = 0; mm < M; ++mm) {
              const double g_ = dcbc[(((t - lo) * M + m) * Lc + (s - lo)) * M + mm];
              if (g_ == 0.0) continue;
              for (i64 n = 0; n < N; ++n) {
                dCacc[(t * M + m) * N + n] += g_ * tB(&k, s, mm, n);
                dBacc[(s * M + mm) * N + n] += g_ * tC(&k, t, m, n);
              }
            }
    }
    /* ---- K1 backward: d_da[t] = sum_{t' >= t in the chunk} d_cumA[t'] ---- */
    for (i64 c = 0; c < nc; ++c) {
      const i64 lo = chunk_lo(&k, c), hi = chunk_hi(&k, c);
      if (mutation == MUT_PREFIX_K1) {
        double acc = 0.0;
        for (i64 t = lo; t < hi; ++t) { acc += dcumA[t]; d_da[(bi * T + t) * H + h] = acc; }
      } else {
        double acc = 0.0;
        for (i64 t = hi - 1; t >= lo; --t) { acc += dcumA[t]; d_da[(bi * T + t) * H + h] = acc; }
      }
    }
    /* ---- combine ---- */
    for (i64 t = 0; t < T; ++t)
      for (i64 m = 0; m < M; ++m) {
        for (i64 p = 0; p < P; ++p) dv[IX5(bi, t, m, h, p, T, M, H, P)] = dvacc[(t * M + m) * P + p];
        for (i64 n = 0; n < N; ++n) {
          dBh[IX5(bi, t, m, h, n, T, M, H, N)] = dBacc[(t * M + m) * N + n];
          dCh[IX5(bi, t, m, h, n, T, M, H, N)] = dCacc[(t * M + m) * N + n];
        }
      }
  done:
    free(cumA); free(end); free(S); free(dintra); free(dS); free(dstate_blue); free(dcumA);
    free(dend); free(dvacc); free(dBacc); free(dCacc); free(dcb); free(dcb_all); free(dcum_m);
  }
  for (i64 bi = 0; bi < b; ++bi)
    for (i64 t = 0; t < T; ++t)
      for (i64 m = 0; m < M; ++m)
        for (i64 g = 0; g < G; ++g)
          for (i64 n = 0; n < N; ++n) {
            double sb = 0.0, sc = 0.0;
            for (i64 hh = g * hpg; hh < (g + 1) * hpg; ++hh) {
              sb += dBh[IX5(bi, t, m, hh, n, T, M, H, N)];
              sc += dCh[IX5(bi, t, m, hh, n, T, M, H, N)];
            }
            dB[IX5(bi, t, m, g, n, T, M, G, N)] = sb;
            dC[IX5(bi, t, m, g, n, T, M, G, N)] = sc;
          }
  free(dBh);
  free(dCh);
  return fail ? 2 : 0;
}

/* Mamba-2 input form on top of the chunked backward (M = 1):
 * delta = softplus(dt), v = x delta, da = delta A_h; then the chain rule back
 * to x and dt: dx = dv delta, d(delta) = sum_p dv x + d_da A_h,
 * d_dt = d(delta) sigma(dt). */
int orc_ssd_mamba2_bwd(i64 b, i64 T, i64 H, i64 P, i64 N, i64 G, i64 L,
                       const double* x, const double* dt, const double* A,
                       const double* B, const double* C, const double* s0,
                       const double* dy, const double* ds_final,
                       double* dx, double* d_dt, double* dB, double* dC, double* d_s0,
                       int mutation, int nthreads) {
  if (b < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G || L <= 0) return 1;
  const i64 nx = b * T * H * P, nh = b * T * H;
  double* v = (double*)malloc(sizeof(double) * (size_t)(nx + 1));
  double* dv = (double*)malloc(sizeof(double) * (size_t)(nx + 1));
  double* da = (double*)malloc(sizeof(double) * (size_t)(nh + 1));
  double* dda = (double*)malloc(sizeof(double) * (size_t)(nh + 1));
  if (!v || !dv || !da || !dda) { free(v); free(dv); free(da); free(dda); return 2; }
  for (i64 i = 0; i < nh; ++i) {
    const i64 h = i % H;
    const double d = softplus(dt[i]);
    da[i] = d * A[h];
    for (i64 p = 0; p < P; ++p) v[i * P + p] = x[i * P + p] * d;
  }
  const int inner_mut = (mutation == MUT_ZERO_SEED || mutation == MUT_DROP_SOFTPLUS ||
                         mutation == MUT_DROP_DA_PATH) ? MUT_NONE : mutation;
  int rc = orc_ssd_chunk_bwd(b, T, 1, H, P, N, G, L, v, da, B, C, s0, dy,
                             mutation == MUT_ZERO_SEED ? NULL : ds_final,
                             dv, dda, dB, dC, d_s0, inner_mut, nthreads);
  if (rc == 0) {
    for (i64 i = 0; i < nh; ++i) {
      const i64 h = i % H;
      const double d = softplus(dt[i]);
      double ddelta = (mutation == MUT_DROP_DA_PATH) ? 0.0 : dda[i] * A[h];
      for (i64 p = 0; p < P; ++p) {
        dx[i * P + p] = dv[i * P + p] * d;
        ddelta += dv[i * P + p] * x[i * P + p];
      }
      d_dt[i] = (mutation == MUT_DROP_SOFTPLUS) ? ddelta : ddelta * sigmoid(dt[i]);
    }
  }
  free(v); free(dv); free(da); free(dda);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* O3: KDA gated delta rule (P2).  q,k[b,T,H,K] v[b,T,HV,V] beta[b,T,HV]      */
/* g[b,T,HV,K] (log gate) S0[b,HV,K,V] (NULL = zeros).  Value head hv reads   */
/* qk head hv / (HV/H) (P2's view(B,T,H,G,K)).  q is used as scale * q.       */
/* ------------------------------------------------------------------------- */

static i64 kda_qk_head(i64 hv, i64 H, i64 HV, int mutation) {
  const i64 grp = HV / H;
  return mutation == MUT_WRONG_GVA ? hv % H : hv / grp;
}

int orc_kda_fwd(i64 b, i64 T, i64 H, i64 HV, i64 K, i64 V, double scale,
                const double* q, const double* k, const double* v, const double* beta,
                const double* g, const double* S0, double* o, double* S_final, int nthreads) {
  if (b < 0 || T < 0 || H <= 0 || HV <= 0 || HV % H || K <= 0 || V <= 0) return 1;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * HV; ++task) {
    const i64 bi = task / HV, hv = task % HV, h = kda_qk_head(hv, H, HV, MUT_NONE);
    double* S = (double*)malloc(sizeof(double) * (size_t)(K * V));
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    for (i64 e = 0; e < K * V; ++e) S[e] = S0 ? S0[IX4(bi, hv, 0, 0, HV, K, V) + e] : 0.0;
    for (i64 t = 0; t < T; ++t) {
      const double* qt = q + IX4(bi, t, h, 0, T, H, K);
      const double* kt = k + IX4(bi, t, h, 0, T, H, K);
      const double* vt = v + IX4(bi, t, hv, 0, T, HV, V);
      const double* gt = g + IX4(bi, t, hv, 0, T, HV, K);
      const double bt = beta[(bi * T + t) * HV + hv];
      /* F1 S_dec = exp(g) (.) S ; F2 p = k^T S_dec ; F3 r = v - p */
      for (i64 kk = 0; kk < K; ++kk) {
        const double eg = exp(gt[kk]);
        for (i64 vv = 0; vv < V; ++vv) S[kk * V + vv] *= eg;
      }
      for (i64 vv = 0; vv < V; ++vv) {
        double p = 0.0;
        for (i64 kk = 0; kk < K; ++kk) p += kt[kk] * S[kk * V + vv];
        r[vv] = vt[vv] - p;
      }
      /* F4 a = beta k ; F5 S = S_dec + a (x) r ; F6 o = (scale q)^T S */
      for (i64 kk = 0; kk < K; ++kk)
        for (i64 vv = 0; vv < V; ++vv) S[kk * V + vv] += bt * kt[kk] * r[vv];
      for (i64 vv = 0; vv < V; ++vv) {
        double acc = 0.0;
        for (i64 kk = 0; kk < K; ++kk) acc += scale * qt[kk] * S[kk * V + vv];
        o[IX4(bi, t, hv, vv, T, HV, V)] = acc;
      }
    }
    for (i64 e = 0; e < K * V; ++e) S_final[IX4(bi, hv, 0, 0, HV, K, V) + e] = S[e];
    free(S);
    free(r);
  }
  return 0;
}

/* Backward of the KDA gated delta rule, derived here from the forward
 * equations F1..F6 of the notes ([P2]) by writing one step as a linear map of
 * the previous state.  Per value head, with Q = scale * q_t and the gated state
 * X = diag(exp(g_t)) S_{t-1}:
 *     S_t = X + beta_t k_t (v_t - X^T k_t)^T
 *         = (I - beta_t k_t k_t^T) X + beta_t k_t v_t^T,        o_t = S_t^T Q.
 * J = <d_o, o> + <dS_final, S_{T-1}> is differentiated in reverse time.  Let
 * Sbar be dJ/dS_t from the later steps and the seed.  The readout adds its own
 * part and gives q's gradient:
 *     Sbar' = Sbar + Q d_o_t^T,     qbar_t = scale * S_t d_o_t.
 * With the residual r = v_t - X^T k_t and one vector u = Sbar'^T k_t (a value
 * per state column), the write contributes
 *     vbar_t = beta_t u,    betabar_t = u . r,
 *     kbar_t = beta_t (Sbar' r - X u),
 *     Xbar   = Sbar' - beta_t k_t u^T
 * (the second term of Xbar is the path through the residual that the notes'
 * warning box insists on), and the gate
 *     gbar_t[i] = sum_j Xbar[i,j] X[i,j],      Sbar_{t-1} = diag(exp(g_t)) Xbar.
 * After step 0, Sbar is dJ/dS0.  q and k are shared by the HV/H value heads of
 * a qk head (the notes' view of the value heads as groups of a qk head), so
 * their gradients are the sums of the per-value-head ones, added in ascending
 * value-head order.  States of every step are kept (store-all).
 * dS_final NULL = zeros; dS0 NULL = not written. */
int orc_kda_bwd(i64 b, i64 T, i64 H, i64 HV, i64 K, i64 V, double scale,
                const double* q, const double* k, const double* v, const double* beta,
                const double* g, const double* S0, const double* d_o, const double* dS_final,
                double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dS0,
                int mutation, int nthreads) {
  if (b < 0 || T < 0 || H <= 0 || HV <= 0 || HV % H || K <= 0 || V <= 0) return 1;
  /* per-value-head gradients of q and k, summed over each group afterwards */
  double* qbar = (double*)calloc((size_t)(b * T * HV * K) + 1, sizeof(double));
  double* kbar = (double*)calloc((size_t)(b * T * HV * K) + 1, sizeof(double));
  if (!qbar || !kbar) { free(qbar); free(kbar); return 2; }
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (i64 task = 0; task < b * HV; ++task) {
    const i64 bi = task / HV, hv = task % HV, h = kda_qk_head(hv, H, HV, mutation);
    const i64 KV = K * V;
    double* hist = (double*)malloc(sizeof(double) * (size_t)((T + 1) * KV)); /* hist[t] = S_{t-1} */
    double* Sbar = (double*)malloc(sizeof(double) * (size_t)KV);
    double* X = (double*)malloc(sizeof(double) * (size_t)KV);
    double* resid = (double*)malloc(sizeof(double) * (size_t)V);
    double* u = (double*)malloc(sizeof(double) * (size_t)V);
    double* gate = (double*)malloc(sizeof(double) * (size_t)K);
    if (!hist || !Sbar || !X || !resid || !u || !gate) { fail = 1; goto next_task; }

    /* forward pass keeping every state */
    for (i64 e = 0; e < KV; ++e) hist[e] = S0 ? S0[IX4(bi, hv, 0, 0, HV, K, V) + e] : 0.0;
    for (i64 t = 0; t < T; ++t) {
      const double* kt = k + IX4(bi, t, h, 0, T, H, K);
      const double* vt = v + IX4(bi, t, hv, 0, T, HV, V);
      const double* gt = g + IX4(bi, t, hv, 0, T, HV, K);
      const double bt = beta[(bi * T + t) * HV + hv];
      const double* prev = hist + t * KV;
      double* cur = hist + (t + 1) * KV;
      for (i64 i = 0; i < K; ++i) {
        const double e = exp(gt[i]);
        for (i64 j = 0; j < V; ++j) cur[i * V + j] = e * prev[i * V + j];
      }
      for (i64 j = 0; j < V; ++j) {
        double kx = 0.0;
        for (i64 i = 0; i < K; ++i) kx += kt[i] * cur[i * V + j];
        resid[j] = vt[j] - kx;
      }
      for (i64 i = 0; i < K; ++i)
        for (i64 j = 0; j < V; ++j) cur[i * V + j] += bt * kt[i] * resid[j];
    }

    /* reverse pass */
    for (i64 e = 0; e < KV; ++e) Sbar[e] = dS_final ? dS_final[IX4(bi, hv, 0, 0, HV, K, V) + e] : 0.0;
    for (i64 t = T - 1; t >= 0; --t) {
      const double* qt = q + IX4(bi, t, h, 0, T, H, K);
      const double* kt = k + IX4(bi, t, h, 0, T, H, K);
      const double* vt = v + IX4(bi, t, hv, 0, T, HV, V);
      const double* gt = g + IX4(bi, t, hv, 0, T, HV, K);
      const double* obar = d_o + IX4(bi, t, hv, 0, T, HV, V);
      const double bt = beta[(bi * T + t) * HV + hv];
      const double* Sprev = hist + t * KV;       /* S_{t-1} */
      const double* St = hist + (t + 1) * KV;    /* S_t */
      double* qb = qbar + IX4(bi, t, hv, 0, T, HV, K);
      double* kb = kbar + IX4(bi, t, hv, 0, T, HV, K);

      /* readout o_t = S_t^T Q */
      for (i64 i = 0; i < K; ++i) {
        double so = 0.0;
        for (i64 j = 0; j < V; ++j) so += St[i * V + j] * obar[j];
        qb[i] = scale * so;
        for (i64 j = 0; j < V; ++j) Sbar[i * V + j] += scale * qt[i] * obar[j];
      }
      /* the gated state and the residual of this step, recomputed from S_{t-1} */
      for (i64 i = 0; i < K; ++i) {
        gate[i] = exp(gt[i]);
        for (i64 j = 0; j < V; ++j) X[i * V + j] = gate[i] * Sprev[i * V + j];
      }
      for (i64 j = 0; j < V; ++j) {
        double kx = 0.0, ks = 0.0;
        for (i64 i = 0; i < K; ++i) {
          kx += kt[i] * X[i * V + j];
          ks += kt[i] * Sbar[i * V + j];
        }
        resid[j] = vt[j] - kx;
        u[j] = ks;
      }
      /* the write S_t = X + beta k (v - X^T k)^T */
      double bb = 0.0;
      for (i64 j = 0; j < V; ++j) {
        dv[IX4(bi, t, hv, j, T, HV, V)] = bt * u[j];
        bb += u[j] * resid[j];
      }
      dbeta[(bi * T + t) * HV + hv] = bb;
      for (i64 i = 0; i < K; ++i) {
        double sr = 0.0, xu = 0.0;
        for (i64 j = 0; j < V; ++j) {
          sr += Sbar[i * V + j] * resid[j];
          xu += X[i * V + j] * u[j];
        }
        kb[i] = bt * (sr - xu);
      }
      if (mutation != MUT_DROP_KDR)
        for (i64 i = 0; i < K; ++i)
          for (i64 j = 0; j < V; ++j) Sbar[i * V + j] -= bt * kt[i] * u[j];
      /* the gate X = diag(exp(g)) S_{t-1} */
      for (i64 i = 0; i < K; ++i) {
        double gx = 0.0;
        for (i64 j = 0; j < V; ++j) gx += Sbar[i * V + j] * X[i * V + j];
        dg[IX4(bi, t, hv, i, T, HV, K)] = gx;
        for (i64 j = 0; j < V; ++j) Sbar[i * V + j] *= gate[i];
      }
    }
    if (dS0)
      for (i64 e = 0; e < KV; ++e) dS0[IX4(bi, hv, 0, 0, HV, K, V) + e] = Sbar[e];
  next_task:
    free(hist); free(Sbar); free(X); free(resid); free(u); free(gate);
  }
  /* q and k are read by every value head of their group: sum the per-value-head
   * gradients, ascending value head */
  for (i64 bi = 0; bi < b; ++bi)
    for (i64 t = 0; t < T; ++t)
      for (i64 h = 0; h < H; ++h)
        for (i64 i = 0; i < K; ++i) {
          double sq = 0.0, sk = 0.0;
          for (i64 hv = 0; hv < HV; ++hv) {
            if (kda_qk_head(hv, H, HV, mutation) != h) continue;
            sq += qbar[IX4(bi, t, hv, i, T, HV, K)];
            sk += kbar[IX4(bi, t, hv, i, T, HV, K)];
          }
          dq[IX4(bi, t, h, i, T, H, K)] = sq;
          dk[IX4(bi, t, h, i, T, H, K)] = sk;
        }
  free(qbar);
  free(kbar);
  return fail ? 2 : 0;
}
