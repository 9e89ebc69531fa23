/* Runs every function of the float64 oracle (test infrastructure) at small
 * shapes and at the edge cases (T = 0, an empty batch, NULL initial states and
 * seeds, ragged chunks, groups, rank > 1, every mutation code) for the
 * sanitizer build, and checks return codes and that outputs are finite.
 * Exit status = number of failed checks. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef int64_t i64;
int orc_mamba_seq_fwd(i64, i64, i64, i64, i64, i64, int, const double*, const double*, const double*,
                      const double*, const double*, const double*, double*, double*, int);
int orc_mamba_seq_bwd(i64, i64, i64, i64, i64, i64, int, const double*, const double*, const double*,
                      const double*, const double*, const double*, const double*, const double*, double*, double*,
                      double*, double*, double*, double*, int, int);
int orc_raw_seq_fwd(i64, i64, i64, i64, i64, i64, i64, const double*, const double*, const double*, const double*,
                    const double*, double*, double*, int);
int orc_raw_seq_bwd(i64, i64, i64, i64, i64, i64, i64, const double*, const double*, const double*, const double*,
                    const double*, const double*, const double*, double*, double*, double*, double*, double*, int);
int orc_ssd_chunk_fwd(i64, i64, i64, i64, i64, i64, i64, i64, const double*, const double*, const double*,
                      const double*, const double*, double*, double*, int);
int orc_ssd_chunk_bwd(i64, i64, i64, i64, i64, i64, i64, i64, const double*, const double*, const double*,
                      const double*, const double*, const double*, const double*, double*, double*, double*, double*,
                      double*, int, int);
int orc_ssd_mamba2_bwd(i64, i64, i64, i64, i64, i64, i64, const double*, const double*, const double*, const double*,
                       const double*, const double*, const double*, const double*, double*, double*, double*,
                       double*, double*, int, int);
int orc_kda_fwd(i64, i64, i64, i64, i64, i64, double, const double*, const double*, const double*, const double*,
                const double*, const double*, double*, double*, int);
int orc_kda_bwd(i64, i64, i64, i64, i64, i64, double, const double*, const double*, const double*, const double*,
                const double*, const double*, const double*, const double*, double*, double*, double*, double*,
                double*, double*, int, int);

static int failures = 0;
static unsigned long long rng = 12345;
static double uni(void) { /* in [-1, 1) */
  rng = rng * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
/* exactly n doubles (malloc(0) avoided), so out-of-bounds accesses are caught */
static double* vec(i64 n, double lo, double hi) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (i64 i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uni() + 1.0);
  return p;
}
static double* out(i64 n) { return vec(n, 0.0, 0.0); }
static void finite(const double* p, i64 n, const char* what) {
  for (i64 i = 0; i < n; ++i)
    if (!isfinite(p[i])) {
      fprintf(stderr, "%s: non-finite at %lld\n", what, (long long)i);
      ++failures;
      return;
    }
}
static void rc(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s returned %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static void mamba(i64 b, i64 T, i64 H, i64 P, i64 N, i64 G, int per_state, int null_states, i64 L) {
  const i64 nx = b * T * H * P, nh = b * T * H, nbc = b * T * G * N, ns = b * H * P * N, na = per_state ? H * N : H;
  double *x = vec(nx, -1, 1), *dt = vec(nh, -3, 0), *A = vec(na, -2, -0.1), *B = vec(nbc, -1, 1), *C = vec(nbc, -1, 1);
  double *s0 = null_states ? NULL : vec(ns, -1, 1), *dy = vec(nx, -1, 1), *dsf = null_states ? NULL : vec(ns, -1, 1);
  double *y = out(nx), *sf = out(ns), *dx = out(nx), *ddt = out(nh), *dB = out(nbc), *dC = out(nbc), *ds0 = out(ns);
  double* dA = out(na);
  rc(orc_mamba_seq_fwd(b, T, H, P, N, G, per_state, x, dt, A, B, C, s0, y, sf, 2), 0, "mamba_seq_fwd");
  finite(y, nx, "y");
  finite(sf, ns, "s_final");
  for (int mut = 0; mut <= 5; ++mut) {
    rc(orc_mamba_seq_bwd(b, T, H, P, N, G, per_state, x, dt, A, B, C, s0, dy, dsf, dx, ddt, dB, dC, ds0, dA, mut, 2),
       0, "mamba_seq_bwd");
    finite(dx, nx, "dx");
    finite(ddt, nh, "d_dt");
    finite(dB, nbc, "dB");
    finite(dC, nbc, "dC");
    finite(ds0, ns, "d_s0");
    finite(dA, na, "dA");
  }
  if (!per_state) {
    const int muts[] = {0, 1, 2, 5, 11, 12, 13, 14, 15, 16};
    for (unsigned m = 0; m < sizeof(muts) / sizeof(muts[0]); ++m) {
      rc(orc_ssd_mamba2_bwd(b, T, H, P, N, G, L, x, dt, A, B, C, s0, dy, dsf, dx, ddt, dB, dC, ds0, muts[m], 2), 0,
         "ssd_mamba2_bwd");
      finite(dx, nx, "dx (chunked)");
      finite(ddt, nh, "d_dt (chunked)");
    }
  }
  /* H = 3 heads in 2 groups is refused before anything is read */
  rc(orc_mamba_seq_bwd(b, T, 3, P, N, 2, per_state, x, dt, A, B, C, s0, dy, dsf, dx, ddt, dB, dC, ds0, dA, 0, 2), 1,
     "mamba_seq_bwd (H % G)");
  free(x); free(dt); free(A); free(B); free(C); free(s0); free(dy); free(dsf);
  free(y); free(sf); free(dx); free(ddt); free(dB); free(dC); free(ds0); free(dA);
}

static void raw(i64 b, i64 T, i64 M, i64 H, i64 P, i64 N, i64 G, i64 L, int null_states) {
  const i64 nv = b * T * M * H * P, nh = b * T * H, nbc = b * T * M * G * N, ns = b * H * P * N;
  double *v = vec(nv, -1, 1), *da = vec(nh, -1, 0), *B = vec(nbc, -1, 1), *C = vec(nbc, -1, 1);
  double *s0 = null_states ? NULL : vec(ns, -1, 1), *dy = vec(nv, -1, 1), *dsf = null_states ? NULL : vec(ns, -1, 1);
  double *y = out(nv), *sf = out(ns), *dv = out(nv), *dda = out(nh), *dB = out(nbc), *dC = out(nbc), *ds0 = out(ns);
  rc(orc_raw_seq_fwd(b, T, M, H, P, N, G, v, da, B, C, s0, y, sf, 2), 0, "raw_seq_fwd");
  finite(y, nv, "y (raw)");
  rc(orc_ssd_chunk_fwd(b, T, M, H, P, N, G, L, v, da, B, C, s0, y, sf, 2), 0, "ssd_chunk_fwd");
  finite(y, nv, "y (chunked)");
  rc(orc_raw_seq_bwd(b, T, M, H, P, N, G, v, da, B, C, s0, dy, dsf, dv, dda, dB, dC, ds0, 2), 0, "raw_seq_bwd");
  finite(dv, nv, "dv");
  const int muts[] = {0, 11, 12, 13, 14, 15, 16, 17};
  for (unsigned m = 0; m < sizeof(muts) / sizeof(muts[0]); ++m) {
    rc(orc_ssd_chunk_bwd(b, T, M, H, P, N, G, L, v, da, B, C, s0, dy, dsf, dv, dda, dB, dC, ds0, muts[m], 2), 0,
       "ssd_chunk_bwd");
    finite(dv, nv, "dv (chunked)");
    finite(dda, nh, "d_da (chunked)");
    finite(dB, nbc, "dB (chunked)");
    finite(ds0, ns, "d_s0 (chunked)");
  }
  free(v); free(da); free(B); free(C); free(s0); free(dy); free(dsf);
  free(y); free(sf); free(dv); free(dda); free(dB); free(dC); free(ds0);
}

static void kda(i64 b, i64 T, i64 H, i64 HV, i64 K, i64 V, int null_states) {
  const i64 nq = b * T * H * K, nvv = b * T * HV * V, ng = b * T * HV * K, nb = b * T * HV, ns = b * HV * K * V;
  double *q = vec(nq, -1, 1), *k = vec(nq, -0.5, 0.5), *v = vec(nvv, -1, 1), *beta = vec(nb, 0, 1);
  double *g = vec(ng, -1, 0), *S0 = null_states ? NULL : vec(ns, -1, 1), *dO = vec(nvv, -1, 1);
  double *dSf = null_states ? NULL : vec(ns, -1, 1);
  double *o = out(nvv), *Sf = out(ns), *dq = out(nq), *dk = out(nq), *dv = out(nvv), *dg = out(ng), *db = out(nb);
  double* dS0 = out(ns);
  rc(orc_kda_fwd(b, T, H, HV, K, V, 0.5, q, k, v, beta, g, S0, o, Sf, 2), 0, "kda_fwd");
  finite(o, nvv, "o");
  const int muts[] = {0, 21, 22};
  for (unsigned m = 0; m < 3; ++m) {
    rc(orc_kda_bwd(b, T, H, HV, K, V, 0.5, q, k, v, beta, g, S0, dO, dSf, dq, dk, dv, dg, db,
                   null_states ? NULL : dS0, muts[m], 2),
       0, "kda_bwd");
    finite(dq, nq, "dq");
    finite(dk, nq, "dk");
    finite(dv, nvv, "dv (kda)");
    finite(dg, ng, "dg");
    finite(db, nb, "dbeta");
  }
  /* 3 value heads over 2 qk heads is refused before anything is read */
  rc(orc_kda_bwd(b, T, 2, 3, K, V, 0.5, q, k, v, beta, g, S0, dO, dSf, dq, dk, dv, dg, db, dS0, 0, 2), 1,
     "kda_bwd (HV % H)");
  free(q); free(k); free(v); free(beta); free(g); free(S0); free(dO); free(dSf);
  free(o); free(Sf); free(dq); free(dk); free(dv); free(dg); free(db); free(dS0);
}

int main(void) {
  mamba(2, 9, 4, 3, 5, 2, 0, 0, 4);
  mamba(1, 7, 3, 2, 4, 1, 1, 1, 3);
  mamba(1, 0, 2, 2, 3, 1, 0, 0, 4); /* T = 0 */
  mamba(0, 5, 2, 2, 3, 1, 0, 0, 2); /* empty batch */
  mamba(1, 6, 2, 2, 3, 2, 0, 1, 6); /* one chunk, NULL states */
  raw(1, 7, 3, 2, 2, 3, 1, 3, 0);
  raw(2, 5, 2, 4, 2, 2, 2, 2, 1);
  raw(1, 4, 1, 2, 3, 2, 2, 1, 0);
  raw(1, 0, 2, 2, 2, 2, 1, 2, 0);
  kda(1, 6, 1, 2, 4, 3, 0);
  kda(2, 5, 2, 4, 3, 2, 1);
  kda(1, 0, 1, 1, 2, 2, 0);
  printf("oracle checks: %d failure(s)\n", failures);
  return failures;
}
