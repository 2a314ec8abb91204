/* Runs every entry point of the fp64 oracle (oracle/ssm_oracle.c) on small
 * seeded inputs, with and without each optional argument, several groups,
 * both input weights, empty sizes and the documented error returns, so that
 * an AddressSanitizer / UndefinedBehaviorSanitizer build of the oracle sees
 * every indexing path. Exits 0 when every call returns what it should and
 * every output is finite; the sanitizers abort the run on any memory or UB
 * error. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_scan_f64(int64_t, int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                    const double *, const double *, const double *, const double *,
                    const double *, const double *, const double *, int, double *, double *, int);
int oracle_state_update_f64(int64_t, int64_t, int64_t, int64_t, double *, const double *,
                            const double *, const double *, const double *, const double *,
                            const double *, const double *, const double *, int, double *, int);
int oracle_conv1d_silu_f64(int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                           const double *, const double *, double *, double *, int);
int oracle_conv1d_update_f64(int64_t, int64_t, int64_t, double *, const double *, const double *,
                             const double *, double *, int);
int oracle_scan_bwd_f64(int64_t, int64_t, int64_t, int64_t, int64_t, const double *,
                        const double *, const double *, const double *, const double *,
                        const double *, const double *, const double *, const double *,
                        const double *, const double *, double *, double *, double *, double *,
                        double *, double *, double *, double *, double *, int);
int oracle_ssd_f64(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double *,
                   const double *, const double *, const double *, const double *,
                   const double *, const double *, const double *, double *, double *, int);

static uint64_t rng = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(int64_t n, double scale) { /* exactly n doubles (ASan sees any overrun) */
  double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = scale * urand();
  return p;
}
static double *zeros(int64_t n) { return (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }
static int fails = 0;
static void expect(int got, int want, const char *what) {
  if (got != want) { fprintf(stderr, "%s: returned %d, expected %d\n", what, got, want); ++fails; }
}
static void finite(const double *p, int64_t n, const char *what) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) { fprintf(stderr, "%s: non-finite at %lld\n", what, (long long)i); ++fails; return; }
}

static void scan_case(int64_t b, int64_t L, int64_t d, int64_t N, int64_t G, int opt, int zoh) {
  double *x = arr(b * L * d, 1), *dl = arr(b * L * d, 0.5), *A = arr(d * N, 1);
  for (int64_t i = 0; i < d * N; ++i) A[i] = -1.0 - fabs(A[i]) * (double)(i % N + 1);
  double *B = arr(b * L * G * N, 1), *C = arr(b * L * G * N, 1), *D = arr(d, 1), *z = arr(b * L * d, 1);
  double *bias = arr(d, 1), *h0 = arr(b * d * N, 1), *out = zeros(b * L * d), *last = zeros(b * d * N);
  expect(oracle_scan_f64(b, L, d, N, G, x, dl, A, B, C, opt ? D : 0, opt ? z : 0, opt ? bias : 0,
                         opt ? h0 : 0, zoh, out, last, 2), 0, "scan");
  finite(out, b * L * d, "scan out");
  finite(last, b * d * N, "scan last");
  /* one token through the update (its own (batch, dim) and (batch, G, N)
     token arrays), from the scan's last state */
  double *st = zeros(b * d * N), *y1 = zeros(b * d);
  double *tx = arr(b * d, 1), *td = arr(b * d, 0.5), *tz = arr(b * d, 1);
  double *tB = arr(b * G * N, 1), *tC = arr(b * G * N, 1);
  for (int64_t i = 0; i < b * d * N; ++i) st[i] = last[i];
  expect(oracle_state_update_f64(b, d, N, G, st, tx, td, A, tB, tC, opt ? D : 0, opt ? tz : 0,
                                 opt ? bias : 0, zoh, y1, 2), 0, "state_update");
  finite(st, b * d * N, "update state");
  finite(y1, b * d, "update out");
  free(tx); free(td); free(tz); free(tB); free(tC);
  if (!zoh) {
    double *dout = arr(b * L * d, 1), *dlast = arr(b * d * N, 1);
    double *dx = zeros(b * L * d), *ddl = zeros(b * L * d), *dA = zeros(d * N);
    double *dB = zeros(b * L * G * N), *dC = zeros(b * L * G * N), *dD = zeros(d);
    double *dz = zeros(b * L * d), *db = zeros(d), *dh0 = zeros(b * d * N);
    expect(oracle_scan_bwd_f64(b, L, d, N, G, x, dl, A, B, C, opt ? D : 0, opt ? z : 0,
                               opt ? bias : 0, opt ? h0 : 0, dout, opt ? dlast : 0, dx, ddl, dA,
                               dB, dC, opt ? dD : 0, opt ? dz : 0, opt ? db : 0, opt ? dh0 : 0, 2),
           0, "scan_bwd");
    finite(dx, b * L * d, "bwd dx");
    finite(dA, d * N, "bwd dA");
    finite(dB, b * L * G * N, "bwd dB");
    free(dout); free(dlast); free(dx); free(ddl); free(dA); free(dB); free(dC); free(dD);
    free(dz); free(db); free(dh0);
  }
  free(x); free(dl); free(A); free(B); free(C); free(D); free(z); free(bias); free(h0);
  free(out); free(last); free(st); free(y1);
}

static void ssd_case(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int opt) {
  double *x = arr(b * L * H * P, 1), *dt = arr(b * L * H, 0.5), *A = arr(H, 1);
  for (int64_t i = 0; i < H; ++i) A[i] = -1.0 - fabs(A[i]);
  double *B = arr(b * L * G * N, 1), *C = arr(b * L * G * N, 1), *D = arr(H, 1), *bias = arr(H, 1);
  double *h0 = arr(b * H * N * P, 1), *out = zeros(b * L * H * P), *last = zeros(b * H * N * P);
  expect(oracle_ssd_f64(b, L, H, P, N, G, x, dt, A, B, C, opt ? D : 0, opt ? bias : 0,
                        opt ? h0 : 0, out, last, 2), 0, "ssd");
  finite(out, b * L * H * P, "ssd out");
  free(x); free(dt); free(A); free(B); free(C); free(D); free(bias); free(h0); free(out); free(last);
}

static void conv_case(int64_t b, int64_t L, int64_t d, int64_t W, int opt) {
  double *xin = arr(b * L * d, 1), *w = arr(d * W, 1), *bias = arr(d, 1);
  double *sin = arr(b * d * (W - 1), 1), *out = zeros(b * L * d), *sout = zeros(b * d * (W - 1));
  expect(oracle_conv1d_silu_f64(b, L, d, W, xin, w, opt ? bias : 0, opt ? sin : 0, out,
                                opt ? sout : 0, 2), 0, "conv1d");
  finite(out, b * L * d, "conv out");
  double *st = arr(b * d * (W - 1), 1), *y = zeros(b * d), *tok = arr(b * d, 1);
  expect(oracle_conv1d_update_f64(b, d, W, st, tok, w, opt ? bias : 0, y, 2), 0, "conv update");
  finite(y, b * d, "conv update out");
  free(xin); free(w); free(bias); free(sin); free(out); free(sout); free(st); free(y); free(tok);
}

int main(void) {
  for (int opt = 0; opt < 2; ++opt) {
    scan_case(2, 37, 6, 16, 1, opt, 0);
    scan_case(1, 19, 8, 4, 2, opt, 0);
    scan_case(3, 5, 9, 1, 3, opt, 0);
    scan_case(2, 11, 4, 16, 2, opt, 1);      /* exact zero-order hold */
    scan_case(2, 0, 5, 16, 1, opt, 0);       /* empty sequence */
    ssd_case(2, 9, 4, 8, 6, 2, opt);
    ssd_case(1, 1, 2, 3, 5, 1, opt);
    conv_case(2, 13, 7, 4, opt);
    conv_case(1, 3, 5, 1, opt);
    conv_case(1, 0, 3, 3, opt);
  }
  /* documented error returns */
  double one[64] = {0};
  expect(oracle_scan_f64(1, 1, 3, 16, 2, one, one, one, one, one, 0, 0, 0, 0, 0, one, 0, 1), -1,
         "groups not dividing dim");
  expect(oracle_scan_f64(1, 1, 1, 1, 1, one, one, one, one, one, 0, 0, 0, 0, 1, one, 0, 1), -2,
         "zoh with A = 0");
  expect(oracle_scan_f64(1, 1, 1, 1, 1, 0, one, one, one, one, 0, 0, 0, 0, 0, one, 0, 1), -1,
         "x missing");
  expect(oracle_ssd_f64(1, 1, 3, 2, 2, 2, one, one, one, one, one, 0, 0, 0, one, 0, 1), -1,
         "heads not dividing into groups");
  if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
  printf("oracle driver: every case ran clean\n");
  return 0;
}
