/*
 * Drives every function of the fp64 oracle (oracle/ssm_oracle.c) on tiny
 * shapes for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py): every array is allocated at exactly the size
 * the function's contract states, so any read or write outside it, and any
 * undefined arithmetic, stops the run.  Also checks a few identities so the
 * calls are not optimised away: W = T literal sum equals the reverse
 * recurrence, and the windowed identity equals the literal sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_project(int64_t T, int64_t P, int64_t M, const double *x, const double *W, const double *bias,
                 double *out);
void orc_forward(int64_t T, int64_t nc, int64_t N, const double *delta, const double *b, const double *c,
                 const double *x, const double *alpha, double *y, int64_t C, double *h_ckpt);
int orc_layer_grad(int64_t T, int64_t nc, int64_t N, int64_t W, int mode, const double *delta, const double *b,
                   const double *c, const double *x, const double *g, const double *alpha, double *y,
                   double *dDelta, double *dxdir, double *dalpha, double *dbias, double *db, double *dc);
void orc_weight_grad(int64_t T, int64_t P, int64_t M, const double *dY, const double *x, double *dW);
void orc_input_grad(int64_t T, int64_t P, int64_t M, const double *dY, const double *W, double *dx);
void orc_cast_input(int64_t n, const double *r, int to_bf16, double *out);
void orc_rmsnorm(int64_t T, int64_t P, const double *r, const double *gamma, double eps, double *out,
                 double *rinv);
void orc_rmsnorm_vjp(int64_t T, int64_t P, const double *r, const double *gamma, double eps, const double *d,
                     double *dr, double *dgamma);
int orc_num_threads(void);

static uint64_t rng = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(size_t n) {
  double *p = (double *)malloc(n * sizeof(double));
  if (!p) exit(3);
  for (size_t i = 0; i < n; i++) p[i] = rnd();
  return p;
}
static double maxdiff(const double *a, const double *b, size_t n) {
  double m = 0.0;
  for (size_t i = 0; i < n; i++) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

int main(void) {
  const int64_t T = 37, P = 5, N = 3, M = P + 2 * N;
  double *x = arr(T * P), *W = arr(M * P), *bias = arr(P), *g = arr(T * P), *alpha = arr(P * N);
  for (int64_t i = 0; i < P * N; i++) alpha[i] = fabs(alpha[i]) + 0.5;
  double *pr = arr(T * M);
  orc_project(T, P, M, x, W, NULL, pr);
  double *delta = arr(T * P), *b = arr(T * N), *c = arr(T * N);
  orc_project(T, P, P, x, W, bias, delta);
  orc_project(T, P, N, x, W + P * P, NULL, b);
  orc_project(T, P, N, x, W + (P + N) * P, NULL, c);
  const int64_t C = 8, K = (T + C - 1) / C;
  double *y = arr(T * P), *hck = arr(K * P * N);
  orc_forward(T, P, N, delta, b, c, x, alpha, y, C, hck);
  orc_forward(T, P, N, delta, b, c, x, alpha, y, 0, NULL);
  double *out[3][7];
  const int64_t Ws[3] = {T, 5, 1};
  for (int w = 0; w < 3; w++) {
    double *res[3];
    for (int mode = 0; mode < 3; mode++) {
      if (mode == 0 && Ws[w] < T) continue;
      double *yy = arr(T * P), *dD = arr(T * P), *dxd = arr(T * P), *dal = arr(P * N), *dbi = arr(P);
      double *db = arr(T * N), *dc = arr(T * N);
      if (orc_layer_grad(T, P, N, Ws[w], mode, delta, b, c, x, g, alpha, yy, dD, dxd, dal, dbi, db, dc) != 0)
        return 4;
      out[w][0] = yy; out[w][1] = dD; out[w][2] = dxd; out[w][3] = dal; out[w][4] = dbi; out[w][5] = db;
      out[w][6] = dc;
      res[mode] = dD;
      (void)res;
      if (mode == 2) {
        /* literal double sum against the O(T P N) form of the same window */
        const int other = Ws[w] < T ? 1 : 0;
        double *yy2 = arr(T * P), *dD2 = arr(T * P), *dxd2 = arr(T * P), *dal2 = arr(P * N), *dbi2 = arr(P);
        double *db2 = arr(T * N), *dc2 = arr(T * N);
        if (orc_layer_grad(T, P, N, Ws[w], other, delta, b, c, x, g, alpha, yy2, dD2, dxd2, dal2, dbi2, db2,
                           dc2) != 0)
          return 5;
        if (maxdiff(dD, dD2, T * P) > 1e-9 || maxdiff(db, db2, T * N) > 1e-9) return 6;
        free(yy2); free(dD2); free(dxd2); free(dal2); free(dbi2); free(db2); free(dc2);
      }
    }
  }
  /* bad mode and window are refused */
  if (orc_layer_grad(T, P, N, 0, 1, delta, b, c, x, g, alpha, y, y, y, alpha, bias, b, c) == 0) return 7;
  if (orc_layer_grad(T, P, N, 5, 0, delta, b, c, x, g, alpha, y, y, y, alpha, bias, b, c) == 0) return 8;
  double *dW = arr(P * P), *dx = arr(T * P);
  orc_weight_grad(T, P, P, out[0][1], x, dW);
  orc_input_grad(T, P, P, out[0][1], W, dx);
  double *cast = arr(T * P);
  orc_cast_input(T * P, x, 1, cast);
  orc_cast_input(T * P, x, 0, cast);
  double *gam = arr(P), *nrm = arr(T * P), *rinv = arr(T), *dr = arr(T * P), *dgam = arr(P);
  orc_rmsnorm(T, P, x, gam, 1e-5, nrm, rinv);
  orc_rmsnorm_vjp(T, P, x, gam, 1e-5, g, dr, dgam);
  printf("oracle sanitizer run OK (%d threads)\n", orc_num_threads());
  return 0;
}
