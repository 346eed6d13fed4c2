/*
 * ssm_oracle.c -- plain fp64 CPU reference of the selective-SSM gradient path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or helper with the GPU library; the two never call each other.
 *
 * Sources (page titles as cited throughout):
 *   [AS] Pith review of "Adjoint sharding for very long context training of
 *        state space models" (arXiv 2501.00692).
 *        - "Assumptions", Section 3.1: h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t.
 *        - "What carries the argument": adjoint state
 *          lambda_{t,tau} = C_t A_t ... A_{tau+1}; Proposition 1 (adjoint method
 *          for recurrences, lambda_{i-1} = lambda_i df/dh_{i-1}).
 *        - "Core claim": Proposition 2 (gradient of l_t as a sum over i <= t of
 *          vjp^{A_i}, vjp^{B_i} terms plus vjp^{C_t}); truncated adjoint
 *          sharding keeps only the last T-bar states of that sum.
 *        - "Circularity Check", Eq. 8: the recurrence substituted into
 *          Proposition 1.
 *   The selective parameterisation (a = exp(-softplus(Delta) alpha),
 *   Delta = W_delta x + bias, b = W_B x, c = W_C x, diagonal state per
 *   channel) is the problem statement this library is written for.
 *
 * Conventions: t, i in [0,T) tokens, p in [0,P) channels, n in [0,N) states.
 * Inputs are double (the f32 / bf16 storage values widen exactly); every
 * computation and every output is double.  h_{-1} = 0.  The loss is
 * L = sum_t <g_t, y_t>, so dl_t/dy_t = g_t.
 *
 * Parity pins: every function here is checked in tests/ against finite
 * differences of the forward, torch float64 autograd, closed forms
 * (alpha = 0 cumulative sums, window = 1, geometric decay) and the literal
 * Proposition 2 double sum; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(d) = log(1 + e^d), written without overflow. */
static double softplus(double d) { return (d > 0.0 ? d : 0.0) + log1p(exp(-fabs(d))); }

/* d softplus / d Delta = logistic sigmoid. */
static double sigmoid(double d) {
    if (d >= 0.0) return 1.0 / (1.0 + exp(-d));
    double e = exp(d);
    return e / (1.0 + e);
}

static int nthreads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int thread_id(void) {
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

int orc_num_threads(void) { return nthreads(); }

/*
 * Projections of the selective layer: out[t][m] = sum_q W[m][q] x[t][q] + bias[m].
 * Used for Delta = W_delta x + bias, b = W_B x, c = W_C x (bias NULL for b, c).
 */
void orc_project(int64_t T, int64_t P, int64_t M, const double *x, const double *W,
                 const double *bias, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const double *xt = x + t * P;
        for (int64_t m = 0; m < M; m++) {
            const double *wm = W + m * P;
            double acc = 0.0;
            for (int64_t q = 0; q < P; q++) acc += wm[q] * xt[q];
            out[t * M + m] = acc + (bias ? bias[m] : 0.0);
        }
    }
}

/*
 * Forward recurrence for a set of channels given column-wise ([T][nc] arrays):
 *   s_t = softplus(Delta_t), a_t[n] = exp(-s_t alpha[n]),
 *   h_t[n] = a_t[n] h_{t-1}[n] + b_t[n] x_t,  y_t = sum_n c_t[n] h_t[n].
 * If h_ck is not NULL it receives h_{kC-1} for k = 0..ceil(T/C)-1 as
 * [nck][nc][N] (entry 0 is the zero initial state).
 */
void orc_forward(int64_t T, int64_t nc, int64_t N, const double *delta, const double *b,
                 const double *c, const double *x, const double *alpha, double *y,
                 int64_t C, double *h_ck) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nc; j++) {
        double *h = (double *)calloc((size_t)N, sizeof(double));
        for (int64_t t = 0; t < T; t++) {
            if (h_ck && C > 0 && t % C == 0)
                for (int64_t n = 0; n < N; n++) h_ck[((t / C) * nc + j) * N + n] = h[n];
            double s = softplus(delta[t * nc + j]);
            double xv = x[t * nc + j];
            double acc = 0.0;
            for (int64_t n = 0; n < N; n++) {
                double a = exp(-s * alpha[j * N + n]);
                h[n] = a * h[n] + b[t * N + n] * xv;
                acc += c[t * N + n] * h[n];
            }
            y[t * nc + j] = acc;
        }
        free(h);
    }
}

/* Which adjoint accumulation produces mu_i = sum over the window of
 * (dl_t/dy_t) lambda_{t,i}. */
enum { ORC_BPTT = 0, ORC_WINDOW_IDENTITY = 1, ORC_LITERAL = 2 };

/*
 * Gradient of one layer for a set of channels (columns of [T][nc] arrays).
 *
 * mu_i[n] is the adjoint-weighted sum that multiplies the local Jacobians of
 * token i.  With window W (pairs 0 <= t - i < W):
 *   mu_i = sum_{t=i}^{min(T, i+W)-1} g_t c_t[n] prod_{j=i+1}^{t} a_j[n].
 * Three ways to get it (all exact in real arithmetic):
 *   ORC_LITERAL : the Proposition 2 double sum itself -- for every t, walk the
 *                 adjoint state lambda_{t,i} back from lambda_{t,t} = C_t,
 *                 multiplying by A_i each step, for the last W tokens.
 *                 Cost O(T W N).
 *   ORC_BPTT    : Proposition 1's backward recurrence with df/dh = diag(a):
 *                 M_{T} = 0, M_i = g_i c_i + a_{i+1} M_{i+1}.  Accepted
 *                 only for W >= T (returns -1 otherwise).
 *   ORC_WINDOW_IDENTITY : M as above, then
 *                 mu_i = M_i - exp(-alpha (S_{i+W} - S_i)) M_{i+W}
 *                 with S the prefix sums of s (mu_i = M_i when i+W >= T).
 *
 * Local VJPs (the vjp^{A_i}, vjp^{B_i}, vjp^{C_t} terms of Proposition 2,
 * with the chain rule through a = exp(-s alpha), s = softplus(Delta)):
 *   da_i     = mu_i h_{i-1}
 *   dDelta_i = sigmoid(Delta_i) * sum_n da_i[n] (-alpha[n] a_i[n])
 *   dalpha[n] = sum_i da_i[n] (-s_i a_i[n])
 *   dbias    = sum_i dDelta_i
 *   dxdir_i  = sum_n mu_i[n] b_i[n]                (direct B_i x_i term)
 *   db_i[n] += mu_i[n] x_i                         (summed over channels)
 *   dc_t[n] += g_t h_t[n]                          (summed over channels; no
 *                                                   time sum, so no window)
 *
 * Outputs: y, dDelta, dxdir [T][nc]; dalpha [nc][N]; dbias [nc];
 * db, dc [T][N] receive the sums over the given channels (overwritten).
 * Returns 0, or -1 for a bad mode / allocation failure.
 */
int orc_layer_grad(int64_t T, int64_t nc, int64_t N, int64_t W, int mode,
                   const double *delta, const double *b, const double *c,
                   const double *x, const double *g, const double *alpha,
                   double *y, double *dDelta, double *dxdir, double *dalpha,
                   double *dbias, double *db, double *dc) {
    if (mode != ORC_BPTT && mode != ORC_WINDOW_IDENTITY && mode != ORC_LITERAL) return -1;
    if (W < 1) return -1;
    if (mode == ORC_BPTT && W < T) return -1; /* BPTT is the full sum only */
    const int nt = nthreads();
    const size_t TN = (size_t)T * (size_t)N;
    double *db_part = (double *)calloc((size_t)nt * TN, sizeof(double));
    double *dc_part = (double *)calloc((size_t)nt * TN, sizeof(double));
    if (!db_part || !dc_part) {
        free(db_part);
        free(dc_part);
        return -1;
    }
    int fail = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nc; j++) {
        const int tid = thread_id();
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        double *S = (double *)malloc(sizeof(double) * (size_t)(T + 1));
        double *a = (double *)malloc(sizeof(double) * TN);
        double *h = (double *)malloc(sizeof(double) * TN);
        double *mu = (double *)malloc(sizeof(double) * TN);
        double *lam = (double *)malloc(sizeof(double) * (size_t)N);
        double *M = (double *)malloc(sizeof(double) * TN);
        if (!s || !S || !a || !h || !mu || !lam || !M) {
#pragma omp atomic write
            fail = 1;
        } else {
            double *mydb = db_part + (size_t)tid * TN;
            double *mydc = dc_part + (size_t)tid * TN;
            const double *al = alpha + j * N;
            /* forward: s, a, h, y (Section 3.1 recurrence) */
            S[0] = 0.0;
            for (int64_t t = 0; t < T; t++) {
                double d = delta[t * nc + j];
                s[t] = softplus(d);
                S[t + 1] = S[t] + s[t];
                double xv = x[t * nc + j];
                double acc = 0.0;
                for (int64_t n = 0; n < N; n++) {
                    double at = exp(-s[t] * al[n]);
                    double hp = t > 0 ? h[(t - 1) * N + n] : 0.0;
                    a[t * N + n] = at;
                    h[t * N + n] = at * hp + b[t * N + n] * xv;
                    acc += c[t * N + n] * h[t * N + n];
                }
                y[t * nc + j] = acc;
            }
            /* adjoint-weighted sums mu */
            if (mode == ORC_LITERAL) {
                memset(mu, 0, sizeof(double) * TN);
                for (int64_t t = 0; t < T; t++) {
                    double gt = g[t * nc + j];
                    for (int64_t n = 0; n < N; n++) lam[n] = c[t * N + n]; /* lambda_{t,t} = C_t */
                    int64_t lo = t - W + 1;
                    if (lo < 0) lo = 0;
                    for (int64_t i = t; i >= lo; i--) {
                        for (int64_t n = 0; n < N; n++) {
                            mu[i * N + n] += gt * lam[n];
                            lam[n] *= a[i * N + n]; /* lambda_{t,i-1} = lambda_{t,i} A_i */
                        }
                    }
                }
            } else {
                /* Proposition 1: reverse recurrence for the full sums */
                for (int64_t i = T - 1; i >= 0; i--) {
                    double gi = g[i * nc + j];
                    for (int64_t n = 0; n < N; n++) {
                        double nxt = (i + 1 < T) ? a[(i + 1) * N + n] * M[(i + 1) * N + n] : 0.0;
                        M[i * N + n] = gi * c[i * N + n] + nxt;
                    }
                }
                for (int64_t i = 0; i < T; i++) {
                    for (int64_t n = 0; n < N; n++) {
                        double v = M[i * N + n];
                        if (mode == ORC_WINDOW_IDENTITY && i + W < T) {
                            double decay = exp(-al[n] * (S[i + W + 1] - S[i + 1]));
                            v -= decay * M[(i + W) * N + n];
                        }
                        mu[i * N + n] = v;
                    }
                }
            }
            /* local VJPs */
            double dbias_acc = 0.0;
            for (int64_t n = 0; n < N; n++) dalpha[j * N + n] = 0.0;
            for (int64_t i = 0; i < T; i++) {
                double xv = x[i * nc + j];
                double gi = g[i * nc + j];
                double ds = 0.0, dxd = 0.0;
                for (int64_t n = 0; n < N; n++) {
                    double m = mu[i * N + n];
                    double hprev = i > 0 ? h[(i - 1) * N + n] : 0.0;
                    double da = m * hprev;
                    ds += da * (-al[n] * a[i * N + n]);
                    dalpha[j * N + n] += da * (-s[i] * a[i * N + n]);
                    dxd += m * b[i * N + n];
                    mydb[i * N + n] += m * xv;
                    mydc[i * N + n] += gi * h[i * N + n];
                }
                double dd = ds * sigmoid(delta[i * nc + j]);
                dDelta[i * nc + j] = dd;
                dxdir[i * nc + j] = dxd;
                dbias_acc += dd;
            }
            dbias[j] = dbias_acc;
        }
        free(s);
        free(S);
        free(a);
        free(h);
        free(mu);
        free(lam);
        free(M);
    }
    if (!fail) {
        memset(db, 0, sizeof(double) * TN);
        memset(dc, 0, sizeof(double) * TN);
        for (int k = 0; k < nt; k++) {
            const double *pb = db_part + (size_t)k * TN, *pc = dc_part + (size_t)k * TN;
            for (size_t e = 0; e < TN; e++) {
                db[e] += pb[e];
                dc[e] += pc[e];
            }
        }
    }
    free(db_part);
    free(dc_part);
    return fail ? -1 : 0;
}

/*
 * Sum over tokens of outer products (the time sum of Proposition 2's VJPs for
 * a linear projection): dW[m][q] = sum_t dY[t][m] x[t][q].
 */
void orc_weight_grad(int64_t T, int64_t P, int64_t M, const double *dY, const double *x,
                     double *dW) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        double *row = dW + m * P;
        for (int64_t q = 0; q < P; q++) row[q] = 0.0;
        for (int64_t t = 0; t < T; t++) {
            double v = dY[t * M + m];
            const double *xt = x + t * P;
            for (int64_t q = 0; q < P; q++) row[q] += v * xt[q];
        }
    }
}

/* Input cotangent through a projection: dx[t][q] += sum_m dY[t][m] W[m][q]. */
void orc_input_grad(int64_t T, int64_t P, int64_t M, const double *dY, const double *W,
                    double *dx) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        double *row = dx + t * P;
        for (int64_t m = 0; m < M; m++) {
            double v = dY[t * M + m];
            const double *wm = W + m * P;
            for (int64_t q = 0; q < P; q++) row[q] += v * wm[q];
        }
    }
}

/*
 * Storage cast of the residual stream for a layer input: double -> float32
 * (round to nearest) -> bfloat16 (round to nearest, ties to even) when
 * to_bf16 is set.  Written independently of any other rounding helper.
 */
void orc_cast_input(int64_t n, const double *r, int to_bf16, double *out) {
    for (int64_t e = 0; e < n; e++) {
        float f = (float)r[e];
        if (to_bf16) {
            uint32_t u;
            memcpy(&u, &f, 4);
            if ((u & 0x7F800000u) != 0x7F800000u) { /* finite */
                uint32_t keep = u >> 16;
                uint32_t rest = u & 0xFFFFu;
                if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
                u = keep << 16;
            } else {
                u &= 0xFFFF0000u;
            }
            memcpy(&f, &u, 4);
        }
        out[e] = (double)f;
    }
}

/*
 * Normalised layer input of the residual stack.  The pages name a normalised
 * input (x-hat, y-hat^{k-1} in the review's Algorithm 1) without defining the
 * norm; the reading taken is RMS normalisation with a per-channel scale:
 *   rinv_t = 1 / sqrt(mean_p r[t][p]^2 + eps),  out[t][p] = gamma[p] r[t][p] rinv_t.
 * Plain loops over rows in double precision.
 */
void orc_rmsnorm(int64_t T, int64_t P, const double *r, const double *gamma, double eps, double *out,
                 double *rinv) {
    for (int64_t t = 0; t < T; t++) {
        const double *row = r + t * P;
        double ss = 0.0;
        for (int64_t p = 0; p < P; p++) ss += row[p] * row[p];
        const double ri = 1.0 / sqrt(ss / (double)P + eps);
        rinv[t] = ri;
        for (int64_t p = 0; p < P; p++) out[t * P + p] = gamma[p] * row[p] * ri;
    }
}

/*
 * Vector-Jacobian product of orc_rmsnorm for the cotangent dout of its
 * output: with xh = r rinv and u = gamma * dout,
 *   dr[t][p] = rinv_t (u[p] - xh[p] mean_q(u[q] xh[q])),   dgamma[p] = sum_t dout[t][p] xh[t][p].
 * (The derivative of rinv_t with respect to r[t][p] is -rinv_t^3 r[t][p] / P.)
 */
void orc_rmsnorm_vjp(int64_t T, int64_t P, const double *r, const double *gamma, double eps,
                     const double *dout, double *dr, double *dgamma) {
    for (int64_t p = 0; p < P; p++) dgamma[p] = 0.0;
    for (int64_t t = 0; t < T; t++) {
        const double *row = r + t * P;
        const double *d = dout + t * P;
        double ss = 0.0;
        for (int64_t p = 0; p < P; p++) ss += row[p] * row[p];
        const double ri = 1.0 / sqrt(ss / (double)P + eps);
        double dot = 0.0;
        for (int64_t p = 0; p < P; p++) dot += gamma[p] * d[p] * row[p] * ri;
        const double m = dot / (double)P;
        for (int64_t p = 0; p < P; p++) {
            const double xh = row[p] * ri;
            dr[t * P + p] = ri * (gamma[p] * d[p] - xh * m);
            dgamma[p] += d[p] * xh;
        }
    }
}
