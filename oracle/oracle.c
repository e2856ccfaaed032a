/*
 * oracle.c -- plain, slow, sequential fp64 reference for the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP path (selective_state_space_chunked_amd/csrc); the only
 * thing both sides consume is the seeded input arrays from synth/.
 *
 * Every routine is the defining recurrence written out as a loop over time,
 * one independent sequence at a time, in double precision, with libm's exp /
 * cos / sin (no fast-math).  Inputs arrive as doubles holding exactly the
 * float32 / bfloat16 values the GPU consumes.
 *
 * The problem (the pages do not print it as one formula; the readings below
 * are the plainest ones the pages support):
 *   h_t = A_t h_{t-1} + b_t,  y_t = C_t . h_t,  t = 0..L-1,  h_{-1} = h0.
 *   - diagonal real, selective (lpnh.cn "S3M" page, section 1.1: step size
 *     delta = softplus(proj x) and a = exp(delta*A) with A < 0); the input
 *     term uses the Euler form b_t = delta_t * x_t * B_t.
 *   - diagonal real, dense: a_t and b_t given directly.
 *   - diagonal complex with shared controls (SPARC page, abstract: two
 *     input-dependent scalars, retention r_t and phase phi_t, steer every
 *     complex mode, each with its own baseline rate lambda_m and frequency
 *     theta_m): a_{t,m} = exp(r_t ln(lambda_m) + i phi_t theta_m),
 *     b_t = u_t, y_t = Re sum_m c_m h_{t,m}.
 *   - PD (Flash PD-SSM page, "Neuer Selektionsmechanismus"): at every step
 *     the argmax over K scores picks one column-one-hot matrix P from a
 *     dictionary; A_t = P diag(d_t), so h_t[i] = b_t[i] +
 *     sum_{j : pi_t(j) = i} d_t[j] h_{t-1}[j].
 * Gradients are those of the scalar loss  sum_t <gy_t, y_t> + <gh_last, h_{L-1}>
 * (the PGF page's "exact analytical derivatives"), by the adjoint recurrence
 * lambda_t = C_t gy_t + A_{t+1}^T lambda_{t+1}.  Complex gradients use the
 * real-pair convention g = dL/dRe + i dL/dIm.
 *
 * Pins that tie this file to the mathematics rather than to itself live in
 * tests/test_oracle_pins.py (brute-force sums, closed forms, dense-matrix
 * routes, finite differences, a DFA simulation).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef long long i64;

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

int orc_threads(void) { return nthreads(); }
/* Thread count of the following calls (timing of a single core); n < 1 leaves it unchanged. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Selective real scan, general form: the discretisation of the input term    */
/* and the shape of B_t, C_t are parameters.                                  */
/*   disc 0 (Euler): b_t[n] = delta_t x_t B_t[n]                              */
/*   disc 1 (zero-order hold, S3M page section 1.1):                          */
/*        b_t[n] = (exp(delta_t A[d,n]) - 1) / A[d,n] x_t B_t[n],             */
/*        delta_t x_t B_t[n] where A[d,n] = 0 (the limit)                     */
/*   perd 0: Bm, C (B,L,N) shared by the channels; perd 1: (B,D,L,N), one     */
/*        B_t, C_t per channel.                                               */
/* a_t[n] = exp(delta_t A[d,n]) either way.  Layouts otherwise as above.      */
/* ------------------------------------------------------------------------- */
static double sel_coef(int disc, double dl, double Av) {
    if (disc == 0 || Av == 0.0) return dl;
    return expm1(dl * Av) / Av;
}
/* d coef / d A: the derivative of expm1(delta A) / A, delta^2 / 2 at A = 0,
 * and the series delta^2 (1/2 + z/3 + z^2/8 + z^3/30) for |z| = |delta A| < 1e-3
 * (the closed form cancels there); 0 for the Euler term. */
static double sel_coef_dA(int disc, double dl, double Av) {
    if (disc == 0) return 0.0;
    double z = dl * Av;
    if (fabs(z) < 1e-3) return dl * dl * (0.5 + z * (1.0 / 3.0 + z * (0.125 + z / 30.0)));
    return (dl * exp(z) * Av - expm1(z)) / (Av * Av);
}
static i64 bc_index(int perd, i64 D, i64 L, i64 N, i64 bi, i64 di, i64 t, i64 n) {
    return perd ? ((bi * D + di) * L + t) * N + n : (bi * L + t) * N + n;
}

void orc_sel_fwd(int disc, int perd, i64 B, i64 D, i64 L, i64 N,
                 const double* delta, const double* x, const double* A, const double* Bm,
                 const double* C, const double* h0, double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * D; ++s) {
            i64 bi = s / D, di = s % D;
            for (i64 n = 0; n < N; ++n) h[n] = h0 ? h0[s * N + n] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                double dl = delta[s * L + t], xv = x[s * L + t], acc = 0.0;
                for (i64 n = 0; n < N; ++n) {
                    double Av = A[di * N + n];
                    i64 o = bc_index(perd, D, L, N, bi, di, t, n);
                    h[n] = exp(dl * Av) * h[n] + sel_coef(disc, dl, Av) * xv * Bm[o];
                    acc += C[o] * h[n];
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 n = 0; n < N; ++n) hlast[s * N + n] = h[n];
        }
        free(h);
    }
}

/* Gradients of sum <gy, y> + <ghlast, h_last>.  gBm, gC: (B,L,N) sums over the
 * channels (perd 0, per-thread partials added in thread order) or (B,D,L,N)
 * (perd 1).  With b_t = coef x_t B_t and a_t = exp(delta_t A):
 *   gdelta_t = sum_n [lambda_t h_{t-1} a_t A + lambda_t x_t B_t d coef/d delta],
 *              d coef/d delta = 1 (Euler), a_t (ZOH);
 *   gx_t = sum_n lambda_t coef B_t;   gB_t[n] (+)= lambda_t coef x_t;
 *   gA[d,n] += lambda_t (h_{t-1} a_t delta_t + x_t B_t d coef/d A). */
void orc_sel_bwd(int disc, int perd, i64 B, i64 D, i64 L, i64 N,
                 const double* delta, const double* x, const double* A, const double* Bm,
                 const double* C, const double* h0, const double* gy, const double* ghlast,
                 double* gdelta, double* gx, double* gA, double* gBm, double* gC, double* gh0) {
    int T = nthreads();
    double* pB = perd ? NULL : (double*)calloc((size_t)T * L * N, sizeof(double));
    double* pC = perd ? NULL : (double*)calloc((size_t)T * L * N, sizeof(double));
    double* pA = (double*)calloc((size_t)T * D * N, sizeof(double));
    for (i64 bi = 0; bi < B; ++bi) {
        #pragma omp parallel
        {
            int tid = thread_id();
            double* hist = (double*)malloc(sizeof(double) * (L + 1) * N);
            double* lam = (double*)malloc(sizeof(double) * N);
            double* myA = pA + (size_t)tid * D * N;
            #pragma omp for schedule(static)
            for (i64 di = 0; di < D; ++di) {
                i64 s = bi * D + di;
                for (i64 n = 0; n < N; ++n) hist[n] = h0 ? h0[s * N + n] : 0.0;
                for (i64 t = 0; t < L; ++t) {
                    double dl = delta[s * L + t], xv = x[s * L + t];
                    for (i64 n = 0; n < N; ++n) {
                        double Av = A[di * N + n];
                        i64 o = bc_index(perd, D, L, N, bi, di, t, n);
                        hist[(t + 1) * N + n] = exp(dl * Av) * hist[t * N + n] + sel_coef(disc, dl, Av) * xv * Bm[o];
                    }
                }
                for (i64 n = 0; n < N; ++n) lam[n] = ghlast ? ghlast[s * N + n] : 0.0;
                for (i64 t = L - 1; t >= 0; --t) {
                    double g = gy[s * L + t], dl = delta[s * L + t], xv = x[s * L + t];
                    double dsum = 0.0, xsum = 0.0;
                    for (i64 n = 0; n < N; ++n) {
                        double Av = A[di * N + n];
                        double at = exp(dl * Av), coef = sel_coef(disc, dl, Av);
                        i64 o = bc_index(perd, D, L, N, bi, di, t, n);
                        double ht = hist[(t + 1) * N + n], hp = hist[t * N + n], bm = Bm[o];
                        lam[n] += C[o] * g;
                        double dcoef_dl = disc == 0 ? 1.0 : at;
                        dsum += lam[n] * hp * at * Av + lam[n] * xv * bm * dcoef_dl;
                        xsum += lam[n] * coef * bm;
                        if (perd) {
                            if (gBm) gBm[o] = lam[n] * coef * xv;
                            if (gC) gC[o] = g * ht;
                        } else {
                            pB[(size_t)tid * L * N + t * N + n] += lam[n] * coef * xv;
                            pC[(size_t)tid * L * N + t * N + n] += g * ht;
                        }
                        myA[di * N + n] += lam[n] * (hp * at * dl + xv * bm * sel_coef_dA(disc, dl, Av));
                        lam[n] *= at;
                    }
                    if (gdelta) gdelta[s * L + t] = dsum;
                    if (gx) gx[s * L + t] = xsum;
                }
                if (gh0) for (i64 n = 0; n < N; ++n) gh0[s * N + n] = lam[n];
            }
            free(hist);
            free(lam);
        }
        if (!perd)
            for (i64 o = 0; o < L * N; ++o) {
                double sb = 0.0, sc = 0.0;
                for (int k = 0; k < T; ++k) {
                    sb += pB[(size_t)k * L * N + o];
                    sc += pC[(size_t)k * L * N + o];
                    pB[(size_t)k * L * N + o] = 0.0;
                    pC[(size_t)k * L * N + o] = 0.0;
                }
                if (gBm) gBm[bi * L * N + o] = sb;
                if (gC) gC[bi * L * N + o] = sc;
            }
    }
    if (gA)
        for (i64 o = 0; o < D * N; ++o) {
            double sa = 0.0;
            for (int k = 0; k < T; ++k) sa += pA[(size_t)k * D * N + o];
            gA[o] = sa;
        }
    free(pB);
    free(pC);
    free(pA);
}

/* ------------------------------------------------------------------------- */
/* Diagonal real scan.                                                        */
/* mode 0 = selective: a_t[n] = exp(delta[b,d,t] * A[d,n]),                    */
/*                     b_t[n] = delta[b,d,t] * x[b,d,t] * Bm[b,t,n]            */
/* mode 1 = dense:     a_t[n] = a[b,d,t,n], b_t[n] = b[b,d,t,n]               */
/* Layouts: delta, x, y, gy (B,D,L); A (D,N); Bm, C (B,L,N); a, b (B,D,L,N);  */
/* h0, hlast (B,D,N).                                                         */
/* ------------------------------------------------------------------------- */
/* Selective scan with a scalar transition per head (the S3M page's chunked   */
/* matrix form applies to it, section 4.1): head h owns channels              */
/* d = h*P .. h*P+P-1 and one state matrix of P x N; per step                 */
/*   a_t = exp(delta[b,h,t] * A[h])          (one number per head and step)   */
/*   h_t[p,n] = a_t h_{t-1}[p,n] + delta[b,h,t] x[b,d,t] B[b,t,n]             */
/*   y[b,d,t] = sum_n C[b,t,n] h_t[p,n]                                       */
/* Layouts: delta (B,H,L); x, y, gy (B,D,L); A (H); Bm, C (B,L,N);            */
/* h0, hlast (B,D,N) with d = h*P + p.                                        */
/* ------------------------------------------------------------------------- */
void orc_head_fwd(i64 B, i64 H, i64 P, i64 L, i64 N, const double* delta, const double* x, const double* A,
                  const double* Bm, const double* C, const double* h0, double* y, double* hlast) {
    const i64 D = H * P;
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * D; ++s) {
            i64 bi = s / D, di = s % D, hi = di / P;
            for (i64 n = 0; n < N; ++n) h[n] = h0 ? h0[s * N + n] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                double dl = delta[(bi * H + hi) * L + t];
                double at = exp(dl * A[hi]), u = dl * x[s * L + t], acc = 0.0;
                for (i64 n = 0; n < N; ++n) {
                    h[n] = at * h[n] + u * Bm[(bi * L + t) * N + n];
                    acc += C[(bi * L + t) * N + n] * h[n];
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 n = 0; n < N; ++n) hlast[s * N + n] = h[n];
        }
        free(h);
    }
}

/* Gradients of sum <gy,y> + <ghlast,h_last>:
 *   gdelta[b,h,t] = sum_{p,n} lambda_t (h_{t-1} a_t A[h] + x B_t),  gx = delta sum_n lambda B,
 *   gA[h] = sum_{b,p,t,n} lambda h_{t-1} a_t delta,  gB, gC (B,L,N) sums over every channel;
 * sums over channels and batch rows in per-thread partials added in thread order. */
void orc_head_bwd(i64 B, i64 H, i64 P, i64 L, i64 N, const double* delta, const double* x, const double* A,
                  const double* Bm, const double* C, const double* h0, const double* gy, const double* ghlast,
                  double* gdelta, double* gx, double* gA, double* gBm, double* gC, double* gh0) {
    const i64 D = H * P;
    int T = nthreads();
    double* pB = (double*)calloc((size_t)T * L * N, sizeof(double));
    double* pC = (double*)calloc((size_t)T * L * N, sizeof(double));
    double* pA = (double*)calloc((size_t)T * H, sizeof(double));
    double* pD = (double*)calloc((size_t)T * H * L, sizeof(double));
    for (i64 bi = 0; bi < B; ++bi) {
        #pragma omp parallel
        {
            int tid = thread_id();
            double* hist = (double*)malloc(sizeof(double) * (L + 1) * N);
            double* lam = (double*)malloc(sizeof(double) * N);
            #pragma omp for schedule(static)
            for (i64 di = 0; di < D; ++di) {
                i64 s = bi * D + di, hi = di / P;
                const double* dl = delta + (bi * H + hi) * L;
                for (i64 n = 0; n < N; ++n) hist[n] = h0 ? h0[s * N + n] : 0.0;
                for (i64 t = 0; t < L; ++t) {
                    double at = exp(dl[t] * A[hi]), u = dl[t] * x[s * L + t];
                    for (i64 n = 0; n < N; ++n)
                        hist[(t + 1) * N + n] = at * hist[t * N + n] + u * Bm[(bi * L + t) * N + n];
                }
                for (i64 n = 0; n < N; ++n) lam[n] = ghlast ? ghlast[s * N + n] : 0.0;
                for (i64 t = L - 1; t >= 0; --t) {
                    double g = gy[s * L + t], at = exp(dl[t] * A[hi]), xv = x[s * L + t];
                    double dsum = 0.0, xsum = 0.0, asum = 0.0;
                    for (i64 n = 0; n < N; ++n) {
                        i64 o = (bi * L + t) * N + n;
                        lam[n] += C[o] * g;
                        pC[(size_t)tid * L * N + t * N + n] += g * hist[(t + 1) * N + n];
                        pB[(size_t)tid * L * N + t * N + n] += lam[n] * dl[t] * xv;
                        double q = lam[n] * hist[t * N + n] * at;   /* lambda h_{t-1} a_t */
                        dsum += q * A[hi] + lam[n] * xv * Bm[o];
                        xsum += lam[n] * Bm[o];
                        asum += q * dl[t];
                        lam[n] *= at;
                    }
                    pD[((size_t)tid * H + hi) * L + t] += dsum;
                    pA[(size_t)tid * H + hi] += asum;
                    if (gx) gx[s * L + t] = dl[t] * xsum;
                }
                if (gh0) for (i64 n = 0; n < N; ++n) gh0[s * N + n] = lam[n];
            }
            free(hist);
            free(lam);
        }
        for (i64 o = 0; o < L * N; ++o) {
            double sb = 0.0, sc = 0.0;
            for (int k = 0; k < T; ++k) {
                sb += pB[(size_t)k * L * N + o];
                sc += pC[(size_t)k * L * N + o];
                pB[(size_t)k * L * N + o] = 0.0;
                pC[(size_t)k * L * N + o] = 0.0;
            }
            if (gBm) gBm[bi * L * N + o] = sb;
            if (gC) gC[bi * L * N + o] = sc;
        }
        for (i64 o = 0; o < H * L; ++o) {
            double sd = 0.0;
            for (int k = 0; k < T; ++k) {
                sd += pD[(size_t)k * H * L + o];
                pD[(size_t)k * H * L + o] = 0.0;
            }
            if (gdelta) gdelta[bi * H * L + o] = sd;
        }
    }
    if (gA)
        for (i64 hh = 0; hh < H; ++hh) {
            double sa = 0.0;
            for (int k = 0; k < T; ++k) sa += pA[(size_t)k * H + hh];
            gA[hh] = sa;
        }
    free(pB);
    free(pC);
    free(pA);
    free(pD);
}

/* ------------------------------------------------------------------------- */
static void real_terms(int mode, i64 D, i64 L, i64 N, i64 bi, i64 di, i64 t,
                       const double* delta, const double* x, const double* A,
                       const double* Bm, const double* a, const double* b,
                       i64 n, double* at, double* bt) {
    if (mode == 0) {
        double dl = delta[(bi * D + di) * L + t];
        *at = exp(dl * A[di * N + n]);
        *bt = dl * x[(bi * D + di) * L + t] * Bm[(bi * L + t) * N + n];
    } else {
        i64 o = ((bi * D + di) * L + t) * N + n;
        *at = a[o];
        *bt = b[o];
    }
}

void orc_real_fwd(int mode, i64 B, i64 D, i64 L, i64 N,
                  const double* delta, const double* x, const double* A, const double* Bm,
                  const double* a, const double* b, const double* C, const double* h0,
                  double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * D; ++s) {
            i64 bi = s / D, di = s % D;
            for (i64 n = 0; n < N; ++n) h[n] = h0 ? h0[s * N + n] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                double acc = 0.0;
                for (i64 n = 0; n < N; ++n) {
                    double at, bt;
                    real_terms(mode, D, L, N, bi, di, t, delta, x, A, Bm, a, b, n, &at, &bt);
                    h[n] = at * h[n] + bt;
                    acc += C[(bi * L + t) * N + n] * h[n];
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 n = 0; n < N; ++n) hlast[s * N + n] = h[n];
        }
        free(h);
    }
}

/* Backward of the real scan.  Any output pointer may be NULL (not wanted).
 * Selective: gdelta, gx (B,D,L); gA (D,N); gBm (B,L,N).
 * Dense:     ga, gb (B,D,L,N).
 * Both:      gC (B,L,N); gh0 (B,D,N).
 * Cross-sequence sums (gA over b and t, gBm and gC over d) are accumulated in
 * per-thread partial arrays and added in thread order. */
void orc_real_bwd(int mode, i64 B, i64 D, i64 L, i64 N,
                  const double* delta, const double* x, const double* A, const double* Bm,
                  const double* a, const double* b, const double* C, const double* h0,
                  const double* gy, const double* ghlast,
                  double* gdelta, double* gx, double* gA, double* gBm,
                  double* ga, double* gb, double* gC, double* gh0) {
    int T = nthreads();
    double* pB = (double*)calloc((size_t)T * L * N, sizeof(double));
    double* pC = (double*)calloc((size_t)T * L * N, sizeof(double));
    double* pA = (double*)calloc((size_t)T * D * N, sizeof(double));
    for (i64 bi = 0; bi < B; ++bi) {
        #pragma omp parallel
        {
            int tid = thread_id();
            double* hist = (double*)malloc(sizeof(double) * (L + 1) * N); /* h_{-1..L-1} */
            double* lam = (double*)malloc(sizeof(double) * N);
            double* myB = pB + (size_t)tid * L * N;
            double* myC = pC + (size_t)tid * L * N;
            double* myA = pA + (size_t)tid * D * N;
            #pragma omp for schedule(static)
            for (i64 di = 0; di < D; ++di) {
                i64 s = bi * D + di;
                /* forward, keeping the whole state history */
                for (i64 n = 0; n < N; ++n) hist[n] = h0 ? h0[s * N + n] : 0.0;
                for (i64 t = 0; t < L; ++t)
                    for (i64 n = 0; n < N; ++n) {
                        double at, bt;
                        real_terms(mode, D, L, N, bi, di, t, delta, x, A, Bm, a, b, n, &at, &bt);
                        hist[(t + 1) * N + n] = at * hist[t * N + n] + bt;
                    }
                /* reverse (adjoint) sweep */
                for (i64 n = 0; n < N; ++n) lam[n] = ghlast ? ghlast[s * N + n] : 0.0;
                for (i64 t = L - 1; t >= 0; --t) {
                    double g = gy[s * L + t];
                    double dsum = 0.0, xsum = 0.0;
                    for (i64 n = 0; n < N; ++n) {
                        double at, bt;
                        real_terms(mode, D, L, N, bi, di, t, delta, x, A, Bm, a, b, n, &at, &bt);
                        double ht = hist[(t + 1) * N + n], hp = hist[t * N + n];
                        lam[n] += C[(bi * L + t) * N + n] * g;
                        myC[t * N + n] += g * ht;
                        double gat = lam[n] * hp; /* dL/da_t */
                        if (mode == 0) {
                            double dl = delta[s * L + t], xv = x[s * L + t];
                            double bm = Bm[(bi * L + t) * N + n];
                            dsum += gat * at * A[di * N + n] + lam[n] * xv * bm;
                            xsum += lam[n] * bm;
                            myB[t * N + n] += lam[n] * dl * xv;
                            myA[di * N + n] += gat * at * dl;
                        } else {
                            i64 o = (s * L + t) * N + n;
                            if (ga) ga[o] = gat;
                            if (gb) gb[o] = lam[n];
                        }
                        lam[n] *= at;
                    }
                    if (mode == 0) {
                        if (gdelta) gdelta[s * L + t] = dsum;
                        if (gx) gx[s * L + t] = delta[s * L + t] * xsum;
                    }
                }
                if (gh0) for (i64 n = 0; n < N; ++n) gh0[s * N + n] = lam[n];
            }
            free(hist);
            free(lam);
        }
        /* fixed-order sum of the per-thread partials for this batch row */
        for (i64 o = 0; o < L * N; ++o) {
            double sb = 0.0, sc = 0.0;
            for (int k = 0; k < T; ++k) {
                sb += pB[(size_t)k * L * N + o];
                sc += pC[(size_t)k * L * N + o];
                pB[(size_t)k * L * N + o] = 0.0;
                pC[(size_t)k * L * N + o] = 0.0;
            }
            if (gBm && mode == 0) gBm[bi * L * N + o] = sb;
            if (gC) gC[bi * L * N + o] = sc;
        }
    }
    if (gA && mode == 0)
        for (i64 o = 0; o < D * N; ++o) {
            double sa = 0.0;
            for (int k = 0; k < T; ++k) sa += pA[(size_t)k * D * N + o];
            gA[o] = sa;
        }
    free(pB);
    free(pC);
    free(pA);
}

/* Sensitivity of one output to every input of the selective real scan
 * (PGF page, abstract: impulse-response sensitivity):
 *   s[b,d,t] = d y[b,d,t_out] / d x[b,d,t]
 *            = delta_t * sum_n Bm[b,t,n] * mu_t[n],  t <= t_out,  0 after,
 * with mu_{t_out} = C[b,t_out,:] and mu_{t-1} = a_t * mu_t (reverse costate). */
void orc_impulse_sens(i64 B, i64 D, i64 L, i64 N, i64 t_out,
                      const double* delta, const double* A, const double* Bm,
                      const double* C, double* s_out) {
    #pragma omp parallel
    {
        double* mu = (double*)malloc(sizeof(double) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * D; ++s) {
            i64 bi = s / D, di = s % D;
            for (i64 t = t_out + 1; t < L; ++t) s_out[s * L + t] = 0.0;
            for (i64 n = 0; n < N; ++n) mu[n] = C[(bi * L + t_out) * N + n];
            for (i64 t = t_out; t >= 0; --t) {
                double dl = delta[s * L + t], acc = 0.0;
                for (i64 n = 0; n < N; ++n) acc += Bm[(bi * L + t) * N + n] * mu[n];
                s_out[s * L + t] = dl * acc;
                for (i64 n = 0; n < N; ++n) mu[n] *= exp(dl * A[di * N + n]);
            }
        }
        free(mu);
    }
}

/* Sensitivity of one output to the step sizes as well (PGF page, abstract:
 * sensitivities of the SSM dynamics), for the selective real scan:
 *   s_x[b,d,t]     = d y[b,d,t_out] / d x[b,d,t]     = mu_t . (delta_t Bm_t),
 *   s_delta[b,d,t] = d y[b,d,t_out] / d delta[b,d,t] = mu_t . (A a_t h_{t-1} + x_t Bm_t),
 * t <= t_out (0 after), with mu_{t_out} = C[b,t_out,:], mu_{t-1} = a_t mu_t and
 * h_t the forward states (h_{-1} = h0).  Either output may be NULL. */
void orc_output_sens(i64 B, i64 D, i64 L, i64 N, i64 t_out,
                     const double* delta, const double* x, const double* A, const double* Bm,
                     const double* C, const double* h0, double* s_x, double* s_delta) {
    #pragma omp parallel
    {
        double* mu = (double*)malloc(sizeof(double) * N);
        double* hist = (double*)malloc(sizeof(double) * (t_out + 2) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * D; ++s) {
            i64 bi = s / D, di = s % D;
            for (i64 n = 0; n < N; ++n) hist[n] = h0 ? h0[s * N + n] : 0.0;
            for (i64 t = 0; t <= t_out; ++t) {
                double dl = delta[s * L + t], xv = x[s * L + t];
                for (i64 n = 0; n < N; ++n)
                    hist[(t + 1) * N + n] = exp(dl * A[di * N + n]) * hist[t * N + n] +
                                            dl * xv * Bm[(bi * L + t) * N + n];
            }
            for (i64 t = t_out + 1; t < L; ++t) {
                if (s_x) s_x[s * L + t] = 0.0;
                if (s_delta) s_delta[s * L + t] = 0.0;
            }
            for (i64 n = 0; n < N; ++n) mu[n] = C[(bi * L + t_out) * N + n];
            for (i64 t = t_out; t >= 0; --t) {
                double dl = delta[s * L + t], xv = x[s * L + t], gx = 0.0, gd = 0.0;
                for (i64 n = 0; n < N; ++n) {
                    double An = A[di * N + n], a = exp(dl * An), bt = Bm[(bi * L + t) * N + n];
                    gx += mu[n] * dl * bt;
                    gd += mu[n] * (An * a * hist[t * N + n] + xv * bt);
                }
                if (s_x) s_x[s * L + t] = gx;
                if (s_delta) s_delta[s * L + t] = gd;
                for (i64 n = 0; n < N; ++n) mu[n] *= exp(dl * A[di * N + n]);
            }
        }
        free(mu);
        free(hist);
    }
}

/* ------------------------------------------------------------------------- */
/* Complex diagonal scan with shared controls.  Complex arrays are            */
/* interleaved (re, im).  r, phi, y, gy (B,H,L); lam, theta (H,M);            */
/* u (B,H,L,M); c (H,M); h0, hlast (B,H,M).                                   */
/* ------------------------------------------------------------------------- */
static void cplx_a(double r, double phi, double lam, double theta, double* are, double* aim) {
    double mag = exp(r * log(lam));
    double ang = phi * theta;
    *are = mag * cos(ang);
    *aim = mag * sin(ang);
}

void orc_complex_fwd(i64 B, i64 H, i64 L, i64 M,
                     const double* r, const double* phi, const double* lam, const double* theta,
                     const double* u, const double* c, const double* h0,
                     double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * 2 * M);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 m = 0; m < 2 * M; ++m) h[m] = h0 ? h0[s * 2 * M + m] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                double acc = 0.0;
                for (i64 m = 0; m < M; ++m) {
                    double are, aim;
                    cplx_a(r[s * L + t], phi[s * L + t], lam[hi * M + m], theta[hi * M + m], &are, &aim);
                    const double* ut = u + ((s * L + t) * M + m) * 2;
                    double hre = are * h[2 * m] - aim * h[2 * m + 1] + ut[0];
                    double him = are * h[2 * m + 1] + aim * h[2 * m] + ut[1];
                    h[2 * m] = hre;
                    h[2 * m + 1] = him;
                    acc += c[(hi * M + m) * 2] * hre - c[(hi * M + m) * 2 + 1] * him;
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 m = 0; m < 2 * M; ++m) hlast[s * 2 * M + m] = h[m];
        }
        free(h);
    }
}

/* Complex diagonal scan with the transitions given (SPARC page, abstract:
 * the diagonal affine recurrence h_t = a_t * h_{t-1} + u_t per complex mode,
 * here with a_t an input instead of the shared-control form):
 *   h_t[m] = a_t[m] h_{t-1}[m] + u_t[m],  y_t = Re sum_m c_m h_t[m].
 * a, u (B,H,L,M) complex; c (H,M) complex; h0 (B,H,M) complex or NULL;
 * y (B,H,L); hlast (B,H,M) complex or NULL.  Complex arrays are (re, im). */
void orc_complex_dense_fwd(i64 B, i64 H, i64 L, i64 M, const double* a, const double* u, const double* c,
                           const double* h0, double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * 2 * M);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 m = 0; m < 2 * M; ++m) h[m] = h0 ? h0[s * 2 * M + m] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                double acc = 0.0;
                for (i64 m = 0; m < M; ++m) {
                    const double* at = a + ((s * L + t) * M + m) * 2;
                    const double* ut = u + ((s * L + t) * M + m) * 2;
                    double hre = at[0] * h[2 * m] - at[1] * h[2 * m + 1] + ut[0];
                    double him = at[0] * h[2 * m + 1] + at[1] * h[2 * m] + ut[1];
                    h[2 * m] = hre;
                    h[2 * m + 1] = him;
                    acc += c[(hi * M + m) * 2] * hre - c[(hi * M + m) * 2 + 1] * him;
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 m = 0; m < 2 * M; ++m) hlast[s * 2 * M + m] = h[m];
        }
        free(h);
    }
}

/* Backward of the given-transition complex scan for Loss = sum_t gy_t y_t +
 * Re <gh_last, h_{L-1}> (real-pair inner product).  With the adjoint
 * mu_t = gy_t conj(c) + conj(a_{t+1}) mu_{t+1} (mu_L = gh_last):
 *   gu_t = mu_t,  ga_t = mu_t conj(h_{t-1}),  gc = sum_t gy_t conj(h_t),  gh0 = conj(a_0) mu_0.
 * Outputs (any may be NULL): ga, gu (B,H,L,M) complex; gc (H,M) complex;
 * gh0 (B,H,M) complex. */
void orc_complex_dense_bwd(i64 B, i64 H, i64 L, i64 M, const double* a, const double* u, const double* c,
                           const double* h0, const double* gy, const double* ghlast,
                           double* ga, double* gu, double* gc, double* gh0) {
    int T = nthreads();
    double* pc = (double*)calloc((size_t)T * H * M * 2, sizeof(double));
    #pragma omp parallel
    {
        int tid = thread_id();
        double* hist = (double*)malloc(sizeof(double) * (L + 1) * 2 * M);
        double* mu = (double*)malloc(sizeof(double) * 2 * M);
        double* myc = pc + (size_t)tid * H * M * 2;
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 m = 0; m < 2 * M; ++m) hist[m] = h0 ? h0[s * 2 * M + m] : 0.0;
            for (i64 t = 0; t < L; ++t)
                for (i64 m = 0; m < M; ++m) {
                    const double* at = a + ((s * L + t) * M + m) * 2;
                    const double* hp = hist + t * 2 * M + 2 * m;
                    const double* ut = u + ((s * L + t) * M + m) * 2;
                    hist[(t + 1) * 2 * M + 2 * m] = at[0] * hp[0] - at[1] * hp[1] + ut[0];
                    hist[(t + 1) * 2 * M + 2 * m + 1] = at[0] * hp[1] + at[1] * hp[0] + ut[1];
                }
            for (i64 m = 0; m < 2 * M; ++m) mu[m] = ghlast ? ghlast[s * 2 * M + m] : 0.0;
            for (i64 t = L - 1; t >= 0; --t) {
                double g = gy[s * L + t];
                for (i64 m = 0; m < M; ++m) {
                    mu[2 * m] += g * c[(hi * M + m) * 2];
                    mu[2 * m + 1] += -g * c[(hi * M + m) * 2 + 1];
                    const double* ht = hist + (t + 1) * 2 * M + 2 * m;
                    const double* hp = hist + t * 2 * M + 2 * m;
                    myc[(hi * M + m) * 2] += g * ht[0];
                    myc[(hi * M + m) * 2 + 1] += -g * ht[1];
                    const i64 o = ((s * L + t) * M + m) * 2;
                    if (gu) { gu[o] = mu[2 * m]; gu[o + 1] = mu[2 * m + 1]; }
                    if (ga) {
                        ga[o] = mu[2 * m] * hp[0] + mu[2 * m + 1] * hp[1];
                        ga[o + 1] = mu[2 * m + 1] * hp[0] - mu[2 * m] * hp[1];
                    }
                    const double* at = a + o;
                    double mre = at[0] * mu[2 * m] + at[1] * mu[2 * m + 1];
                    double mim = at[0] * mu[2 * m + 1] - at[1] * mu[2 * m];
                    mu[2 * m] = mre;
                    mu[2 * m + 1] = mim;
                }
            }
            if (gh0) for (i64 m = 0; m < 2 * M; ++m) gh0[s * 2 * M + m] = mu[m];
        }
        free(hist);
        free(mu);
    }
    if (gc)
        for (i64 o = 0; o < H * M * 2; ++o) {
            double v = 0.0;
            for (int k = 0; k < T; ++k) v += pc[(size_t)k * H * M * 2 + o];
            gc[o] = v;
        }
    free(pc);
}

/* Backward of the complex scan.  Outputs (any may be NULL):
 * gu (B,H,L,M) complex; gr, gphi (B,H,L); glam, gtheta (H,M); gc (H,M) complex;
 * gh0 (B,H,M) complex. */
void orc_complex_bwd(i64 B, i64 H, i64 L, i64 M,
                     const double* r, const double* phi, const double* lam, const double* theta,
                     const double* u, const double* c, const double* h0,
                     const double* gy, const double* ghlast,
                     double* gu, double* gr, double* gphi, double* glam, double* gtheta,
                     double* gc, double* gh0) {
    int T = nthreads();
    double* pl = (double*)calloc((size_t)T * H * M, sizeof(double));
    double* pt = (double*)calloc((size_t)T * H * M, sizeof(double));
    double* pc = (double*)calloc((size_t)T * H * M * 2, sizeof(double));
    #pragma omp parallel
    {
        int tid = thread_id();
        double* hist = (double*)malloc(sizeof(double) * (L + 1) * 2 * M);
        double* mu = (double*)malloc(sizeof(double) * 2 * M);
        double* myl = pl + (size_t)tid * H * M;
        double* myt = pt + (size_t)tid * H * M;
        double* myc = pc + (size_t)tid * H * M * 2;
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 m = 0; m < 2 * M; ++m) hist[m] = h0 ? h0[s * 2 * M + m] : 0.0;
            for (i64 t = 0; t < L; ++t)
                for (i64 m = 0; m < M; ++m) {
                    double are, aim;
                    cplx_a(r[s * L + t], phi[s * L + t], lam[hi * M + m], theta[hi * M + m], &are, &aim);
                    const double* hp = hist + t * 2 * M + 2 * m;
                    const double* ut = u + ((s * L + t) * M + m) * 2;
                    hist[(t + 1) * 2 * M + 2 * m] = are * hp[0] - aim * hp[1] + ut[0];
                    hist[(t + 1) * 2 * M + 2 * m + 1] = are * hp[1] + aim * hp[0] + ut[1];
                }
            for (i64 m = 0; m < 2 * M; ++m) mu[m] = ghlast ? ghlast[s * 2 * M + m] : 0.0;
            for (i64 t = L - 1; t >= 0; --t) {
                double g = gy[s * L + t], sr = 0.0, sp = 0.0;
                for (i64 m = 0; m < M; ++m) {
                    double cre = c[(hi * M + m) * 2], cim = c[(hi * M + m) * 2 + 1];
                    /* mu += gy * conj(c) */
                    mu[2 * m] += g * cre;
                    mu[2 * m + 1] += -g * cim;
                    const double* ht = hist + (t + 1) * 2 * M + 2 * m;
                    const double* hp = hist + t * 2 * M + 2 * m;
                    /* gc += gy * conj(h_t) */
                    myc[(hi * M + m) * 2] += g * ht[0];
                    myc[(hi * M + m) * 2 + 1] += -g * ht[1];
                    if (gu) {
                        gu[((s * L + t) * M + m) * 2] = mu[2 * m];
                        gu[((s * L + t) * M + m) * 2 + 1] = mu[2 * m + 1];
                    }
                    /* g_a = mu * conj(h_{t-1}) */
                    double gare = mu[2 * m] * hp[0] + mu[2 * m + 1] * hp[1];
                    double gaim = mu[2 * m + 1] * hp[0] - mu[2 * m] * hp[1];
                    double are, aim;
                    cplx_a(r[s * L + t], phi[s * L + t], lam[hi * M + m], theta[hi * M + m], &are, &aim);
                    /* g_z = conj(a) * g_a */
                    double gzre = are * gare + aim * gaim;
                    double gzim = are * gaim - aim * gare;
                    double lnl = log(lam[hi * M + m]);
                    sr += gzre * lnl;
                    sp += gzim * theta[hi * M + m];
                    myl[hi * M + m] += gzre * r[s * L + t];
                    myt[hi * M + m] += gzim * phi[s * L + t];
                    /* mu <- conj(a) * mu */
                    double mre = are * mu[2 * m] + aim * mu[2 * m + 1];
                    double mim = are * mu[2 * m + 1] - aim * mu[2 * m];
                    mu[2 * m] = mre;
                    mu[2 * m + 1] = mim;
                }
                if (gr) gr[s * L + t] = sr;
                if (gphi) gphi[s * L + t] = sp;
            }
            if (gh0) for (i64 m = 0; m < 2 * M; ++m) gh0[s * 2 * M + m] = mu[m];
        }
        free(hist);
        free(mu);
    }
    for (i64 o = 0; o < H * M; ++o) {
        double sl = 0.0, st = 0.0, scr = 0.0, sci = 0.0;
        for (int k = 0; k < T; ++k) {
            sl += pl[(size_t)k * H * M + o];
            st += pt[(size_t)k * H * M + o];
            scr += pc[((size_t)k * H * M + o) * 2];
            sci += pc[((size_t)k * H * M + o) * 2 + 1];
        }
        /* d/d lambda = (d/d ln lambda) / lambda */
        if (glam) glam[o] = sl / lam[o];
        if (gtheta) gtheta[o] = st;
        if (gc) { gc[o * 2] = scr; gc[o * 2 + 1] = sci; }
    }
    free(pl);
    free(pt);
    free(pc);
}

/* Forward-mode (real-time recurrent) gradient of the complex scan with respect
 * to the per-mode parameters lambda and theta (SPARC page, abstract: the
 * structured recurrence admits exact real-time recurrent learning).  The
 * sensitivities of the state are carried alongside it:
 *   a_t = exp(r_t ln lambda + i phi_t theta),  da/dlambda = a r_t / lambda,
 *   da/dtheta = i phi_t a,
 *   sl_t = a_t sl_{t-1} + (r_t / lambda) a_t h_{t-1},
 *   st_t = a_t st_{t-1} + i phi_t a_t h_{t-1},     sl_{-1} = st_{-1} = 0,
 * and the gradient of  sum_t gy_t y_t + <ghlast, h_{L-1}>  (real-pair inner
 * product) accumulates online:
 *   glam += gy_t Re(c sl_t),  gtheta += gy_t Re(c st_t),
 * plus  Re(conj(ghlast) sl_{L-1})  and the same for st at the end.
 * y (B,H,L) and ghlast (B,H,M complex) may be NULL; glam, gtheta are (H,M). */
void orc_complex_rtrl(i64 B, i64 H, i64 L, i64 M,
                      const double* r, const double* phi, const double* lam, const double* theta,
                      const double* u, const double* c, const double* h0,
                      const double* gy, const double* ghlast,
                      double* y, double* glam, double* gtheta) {
    int T = nthreads();
    double* pl = (double*)calloc((size_t)T * H * M, sizeof(double));
    double* pt = (double*)calloc((size_t)T * H * M, sizeof(double));
    #pragma omp parallel
    {
        int tid = thread_id();
        double* st = (double*)malloc(sizeof(double) * 6 * M);   /* per mode: h, sl, st (re, im) */
        double* myl = pl + (size_t)tid * H * M;
        double* myt = pt + (size_t)tid * H * M;
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 m = 0; m < M; ++m) {
                st[6 * m] = h0 ? h0[(s * M + m) * 2] : 0.0;
                st[6 * m + 1] = h0 ? h0[(s * M + m) * 2 + 1] : 0.0;
                for (int k = 2; k < 6; ++k) st[6 * m + k] = 0.0;
            }
            for (i64 t = 0; t < L; ++t) {
                double acc = 0.0, g = gy[s * L + t], rt = r[s * L + t], pht = phi[s * L + t];
                for (i64 m = 0; m < M; ++m) {
                    double lm = lam[hi * M + m], are, aim;
                    cplx_a(rt, pht, lm, theta[hi * M + m], &are, &aim);
                    double* q = st + 6 * m;
                    /* a h_{t-1} */
                    double ahre = are * q[0] - aim * q[1], ahim = are * q[1] + aim * q[0];
                    /* a sl, a st */
                    double aslre = are * q[2] - aim * q[3], aslim = are * q[3] + aim * q[2];
                    double astre = are * q[4] - aim * q[5], astim = are * q[5] + aim * q[4];
                    const double* ut = u + ((s * L + t) * M + m) * 2;
                    q[0] = ahre + ut[0];
                    q[1] = ahim + ut[1];
                    q[2] = aslre + (rt / lm) * ahre;
                    q[3] = aslim + (rt / lm) * ahim;
                    q[4] = astre - pht * ahim;
                    q[5] = astim + pht * ahre;
                    double cre = c[(hi * M + m) * 2], cim = c[(hi * M + m) * 2 + 1];
                    acc += cre * q[0] - cim * q[1];
                    myl[hi * M + m] += g * (cre * q[2] - cim * q[3]);
                    myt[hi * M + m] += g * (cre * q[4] - cim * q[5]);
                }
                if (y) y[s * L + t] = acc;
            }
            if (ghlast)
                for (i64 m = 0; m < M; ++m) {
                    const double* gl = ghlast + (s * M + m) * 2;
                    const double* q = st + 6 * m;
                    myl[hi * M + m] += gl[0] * q[2] + gl[1] * q[3];
                    myt[hi * M + m] += gl[0] * q[4] + gl[1] * q[5];
                }
        }
        free(st);
    }
    for (i64 o = 0; o < H * M; ++o) {
        double sl = 0.0, stt = 0.0;
        for (int k = 0; k < T; ++k) {
            sl += pl[(size_t)k * H * M + o];
            stt += pt[(size_t)k * H * M + o];
        }
        glam[o] = sl;
        gtheta[o] = stt;
    }
    free(pl);
    free(pt);
}

/* ------------------------------------------------------------------------- */
/* PD scan.  logits (B,H,L,K); sel (B,H,L) int32; dict (H,K,N) int32 (row of  */
/* the one in each column); d, b, C (B,H,L,N); y, gy (B,H,L); h0 (B,H,N).     */
/* ------------------------------------------------------------------------- */
static int argmax_first(const double* v, i64 K) {
    int best = 0;
    for (i64 k = 1; k < K; ++k)
        if (v[k] > v[best]) best = (int)k;
    return best;
}

void orc_pd_select(i64 B, i64 H, i64 L, i64 K, const double* logits, int32_t* sel) {
    #pragma omp parallel for schedule(static)
    for (i64 o = 0; o < B * H * L; ++o) sel[o] = argmax_first(logits + o * K, K);
}

void orc_pd_fwd(i64 B, i64 H, i64 L, i64 N, i64 K, const int32_t* sel, const int32_t* dict,
                const double* d, const double* b, const double* C, const double* h0,
                double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * N);
        double* hn = (double*)malloc(sizeof(double) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 i = 0; i < N; ++i) h[i] = h0 ? h0[s * N + i] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                const int32_t* pi = dict + ((i64)hi * K + sel[s * L + t]) * N;
                const double* dt = d + (s * L + t) * N;
                const double* bt = b + (s * L + t) * N;
                for (i64 i = 0; i < N; ++i) hn[i] = bt[i];
                for (i64 j = 0; j < N; ++j) hn[pi[j]] += dt[j] * h[j]; /* ascending j */
                double acc = 0.0;
                for (i64 i = 0; i < N; ++i) {
                    h[i] = hn[i];
                    acc += C[(s * L + t) * N + i] * h[i];
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 i = 0; i < N; ++i) hlast[s * N + i] = h[i];
        }
        free(h);
        free(hn);
    }
}

/* Second, independent PD route: the transition as a dense N x N matrix
 * A_t[i][j] = d_t[j] if pi_t(j) == i else 0, applied by a dense mat-vec. */
void orc_pd_dense_fwd(i64 B, i64 H, i64 L, i64 N, i64 K, const int32_t* sel, const int32_t* dict,
                      const double* d, const double* b, const double* C, const double* h0,
                      double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * N);
        double* hn = (double*)malloc(sizeof(double) * N);
        double* At = (double*)malloc(sizeof(double) * N * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 i = 0; i < N; ++i) h[i] = h0 ? h0[s * N + i] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                const int32_t* pi = dict + ((i64)hi * K + sel[s * L + t]) * N;
                for (i64 i = 0; i < N; ++i)
                    for (i64 j = 0; j < N; ++j)
                        At[i * N + j] = (pi[j] == i) ? d[(s * L + t) * N + j] : 0.0;
                double acc = 0.0;
                for (i64 i = 0; i < N; ++i) {
                    double v = b[(s * L + t) * N + i];
                    for (i64 j = 0; j < N; ++j) v += At[i * N + j] * h[j];
                    hn[i] = v;
                }
                for (i64 i = 0; i < N; ++i) {
                    h[i] = hn[i];
                    acc += C[(s * L + t) * N + i] * h[i];
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 i = 0; i < N; ++i) hlast[s * N + i] = h[i];
        }
        free(h);
        free(hn);
        free(At);
    }
}

/* Backward of the PD scan with the selection held fixed (the argmax has zero
 * derivative almost everywhere; surrogate selection gradients are not part of
 * this routine).  Outputs (any may be NULL): gd, gb, gC (B,H,L,N); gh0 (B,H,N). */
void orc_pd_bwd(i64 B, i64 H, i64 L, i64 N, i64 K, const int32_t* sel, const int32_t* dict,
                const double* d, const double* b, const double* C, const double* h0,
                const double* gy, const double* ghlast,
                double* gd, double* gb, double* gC, double* gh0) {
    #pragma omp parallel
    {
        double* hist = (double*)malloc(sizeof(double) * (L + 1) * N);
        double* lam = (double*)malloc(sizeof(double) * N);
        double* ln = (double*)malloc(sizeof(double) * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 i = 0; i < N; ++i) hist[i] = h0 ? h0[s * N + i] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                const int32_t* pi = dict + ((i64)hi * K + sel[s * L + t]) * N;
                double* hn = hist + (t + 1) * N;
                const double* hp = hist + t * N;
                for (i64 i = 0; i < N; ++i) hn[i] = b[(s * L + t) * N + i];
                for (i64 j = 0; j < N; ++j) hn[pi[j]] += d[(s * L + t) * N + j] * hp[j];
            }
            for (i64 i = 0; i < N; ++i) lam[i] = ghlast ? ghlast[s * N + i] : 0.0;
            for (i64 t = L - 1; t >= 0; --t) {
                const int32_t* pi = dict + ((i64)hi * K + sel[s * L + t]) * N;
                double g = gy[s * L + t];
                for (i64 i = 0; i < N; ++i) {
                    lam[i] += C[(s * L + t) * N + i] * g;
                    if (gb) gb[(s * L + t) * N + i] = lam[i];
                    if (gC) gC[(s * L + t) * N + i] = g * hist[(t + 1) * N + i];
                }
                /* lambda_{t-1}[j] (before adding its own readout) = d_t[j] lambda_t[pi_t(j)] */
                for (i64 j = 0; j < N; ++j) {
                    double lp = lam[pi[j]];
                    if (gd) gd[(s * L + t) * N + j] = lp * hist[t * N + j];
                    ln[j] = d[(s * L + t) * N + j] * lp;
                }
                for (i64 j = 0; j < N; ++j) lam[j] = ln[j];
            }
            if (gh0) for (i64 i = 0; i < N; ++i) gh0[s * N + i] = lam[i];
        }
        free(hist);
        free(lam);
        free(ln);
    }
}

/* Straight-through surrogate gradient of the PD selection (Flash PD-SSM page,
 * "Gradientenpropagation": hard argmax in the forward pass, a tempered softmax
 * in its place for the backward pass).  Reading: the transition is a mixture
 * A_t(w) = sum_k w_{t,k} P_k diag(d_t) whose weights are one-hot at the
 * selected entry in the forward pass and softmax(logits_t / tau) for the
 * backward pass, every other gradient flowing through the hard forward.  With
 * lambda_t = dLoss/dh_t (the hard-forward adjoint, lambda_t = C_t gy_t +
 * A_{t+1}^T lambda_{t+1}):
 *   gw[t,k]      = dLoss/dw_{t,k} = sum_j lambda_t[pi_k(j)] d_t[j] h_{t-1}[j],
 *   glogits[t,k] = (1/tau) s_k (gw[t,k] - sum_i s_i gw[t,i]),  s = softmax(logits_t / tau).
 * gw, glogits (B,H,L,K); either may be NULL. */
void orc_pd_ste(i64 B, i64 H, i64 L, i64 N, i64 K, const double* logits, const int32_t* sel,
                const int32_t* dict, const double* d, const double* b, const double* C,
                const double* h0, const double* gy, const double* ghlast, double tau,
                double* gw, double* glogits) {
    #pragma omp parallel
    {
        double* hist = (double*)malloc(sizeof(double) * (L + 1) * N);
        double* lam = (double*)malloc(sizeof(double) * N);
        double* ln = (double*)malloc(sizeof(double) * N);
        double* g = (double*)malloc(sizeof(double) * K);
        double* sm = (double*)malloc(sizeof(double) * K);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 i = 0; i < N; ++i) hist[i] = h0 ? h0[s * N + i] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                const int32_t* pi = dict + ((i64)hi * K + sel[s * L + t]) * N;
                double* hn = hist + (t + 1) * N;
                const double* hp = hist + t * N;
                for (i64 i = 0; i < N; ++i) hn[i] = b[(s * L + t) * N + i];
                for (i64 j = 0; j < N; ++j) hn[pi[j]] += d[(s * L + t) * N + j] * hp[j];
            }
            for (i64 i = 0; i < N; ++i) lam[i] = ghlast ? ghlast[s * N + i] : 0.0;
            for (i64 t = L - 1; t >= 0; --t) {
                const int32_t* pi = dict + ((i64)hi * K + sel[s * L + t]) * N;
                const double* dt = d + (s * L + t) * N;
                const double* hp = hist + t * N;
                for (i64 i = 0; i < N; ++i) lam[i] += C[(s * L + t) * N + i] * gy[s * L + t];
                /* lam now holds lambda_t */
                for (i64 k = 0; k < K; ++k) {
                    const int32_t* pk = dict + ((i64)hi * K + k) * N;
                    double acc = 0.0;
                    for (i64 j = 0; j < N; ++j) acc += lam[pk[j]] * dt[j] * hp[j];
                    g[k] = acc;
                }
                const double* x = logits + (s * L + t) * K;
                double mx = x[0];
                for (i64 k = 1; k < K; ++k) mx = x[k] > mx ? x[k] : mx;
                double z = 0.0;
                for (i64 k = 0; k < K; ++k) {
                    sm[k] = exp((x[k] - mx) / tau);
                    z += sm[k];
                }
                double dot = 0.0;
                for (i64 k = 0; k < K; ++k) {
                    sm[k] /= z;
                    dot += sm[k] * g[k];
                }
                for (i64 k = 0; k < K; ++k) {
                    if (gw) gw[(s * L + t) * K + k] = g[k];
                    if (glogits) glogits[(s * L + t) * K + k] = sm[k] * (g[k] - dot) / tau;
                }
                for (i64 j = 0; j < N; ++j) ln[j] = dt[j] * lam[pi[j]];
                for (i64 j = 0; j < N; ++j) lam[j] = ln[j];
            }
        }
        free(hist);
        free(lam);
        free(ln);
        free(g);
        free(sm);
    }
}

/* The mixture forward of the reading above, as dense N x N matrices:
 * A_t = sum_k w[t,k] P_k diag(d_t), P_k[i][j] = 1 if dict[h,k,j] == i.
 * w (B,H,L,K).  With w one-hot at sel it is the PD forward; its derivative in
 * w at that point is gw above. */
void orc_pd_mix_fwd(i64 B, i64 H, i64 L, i64 N, i64 K, const double* w, const int32_t* dict,
                    const double* d, const double* b, const double* C, const double* h0,
                    double* y, double* hlast) {
    #pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * N);
        double* hn = (double*)malloc(sizeof(double) * N);
        double* At = (double*)malloc(sizeof(double) * N * N);
        #pragma omp for schedule(static)
        for (i64 s = 0; s < B * H; ++s) {
            i64 hi = s % H;
            for (i64 i = 0; i < N; ++i) h[i] = h0 ? h0[s * N + i] : 0.0;
            for (i64 t = 0; t < L; ++t) {
                for (i64 e = 0; e < N * N; ++e) At[e] = 0.0;
                for (i64 k = 0; k < K; ++k) {
                    const int32_t* pk = dict + ((i64)hi * K + k) * N;
                    const double wk = w[(s * L + t) * K + k];
                    for (i64 j = 0; j < N; ++j) At[pk[j] * N + j] += wk * d[(s * L + t) * N + j];
                }
                double acc = 0.0;
                for (i64 i = 0; i < N; ++i) {
                    double v = b[(s * L + t) * N + i];
                    for (i64 j = 0; j < N; ++j) v += At[i * N + j] * h[j];
                    hn[i] = v;
                }
                for (i64 i = 0; i < N; ++i) {
                    h[i] = hn[i];
                    acc += C[(s * L + t) * N + i] * h[i];
                }
                y[s * L + t] = acc;
            }
            if (hlast) for (i64 i = 0; i < N; ++i) hlast[s * N + i] = h[i];
        }
        free(h);
        free(hn);
        free(At);
    }
}
