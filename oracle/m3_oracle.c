/*
 * Plain sequential fp64 reference ("oracle") for the Mamba-3 SSM mixer core.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes is the plain definition of the method, one token at a time,
 * in the physical (un-rotated) state frame, for every (batch, head) chain:
 *
 *   BCNorm + bias   B_t[r] = Braw_t[r] / sqrt(mean_n Braw_t[r,n]^2 + eps) * wB + B_bias[h,r]
 *                   (same for C)       -- Mamba-3 paper, §3.4 "BC / QK normalization"
 *                                         and "B, C bias" (bias added after the norm)
 *   coefficients    alpha_t = exp(dt_t A_t)
 *                   beta_t  = (1 - lam_t) dt_t exp(dt_t A_t)
 *                   gamma_t = lam_t dt_t           -- §3.1.1, Proposition 1
 *   rotation        R_t = block rotation by angles dt_t * theta_t[i], acting on the
 *                   coordinate pairs (i, i + N/2) of the state, i.e. the stacked
 *                   [real; imaginary] halves    -- §3.2.1, Proposition 2
 *   update          H_t = R_t (alpha_t H_{t-1} + beta_t sum_r B_{t-1}[r] X_{t-1}[r]^T)
 *                         + gamma_t sum_r B_t[r] X_t[r]^T          (N x P)
 *                   -- the real form of the exponential-trapezoidal complex SSM,
 *                      App. B.3 (proof of Proposition 4, eq. 25), with the rank-R
 *                      state input of App. C (MIMO), all ranks sharing alpha, beta,
 *                      gamma and R_t
 *   output          y_t[r, p] = sum_n C_t[r, n] H_t[n, p]    -- App. C, Y_t = H_t^T C_t
 *
 * Boundary: H_{-1} = h0 (or zero). The beta term at t = 0 uses the caller's
 * previous token (Braw_prev, x_prev) when both are given and is absent otherwise,
 * as in the unrolled form of §3.1.3 which starts from h_0 = gamma_0 B_0 x_0.
 *
 * Layouts (row-major, float32 inputs upcast exactly to double):
 *   x [b,L,H,R,P]  Braw,Craw [b,L,G,R,N]  dt,A,lam [b,L,H]  theta [b,L,G,N/2]
 *   B_bias,C_bias [H,R,N]  B_normw,C_normw [N] (NULL = ones)
 *   h0 [b,H,P,N] (NULL = zero)  x_prev [b,H,R,P]  Braw_prev [b,G,R,N] (NULL = none)
 *   y [b,L,H,R,P] (double)      h_final [b,H,P,N] (double, may be NULL)
 * Head h belongs to group h / (H/G).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* RMS-normalise one length-N row, scale by the optional gain, add the bias. */
static void norm_bias(const float *raw, const float *gain, const float *bias,
                      long N, double eps, double *out)
{
    double ms = 0.0;
    for (long n = 0; n < N; ++n) {
        double v = (double)raw[n];
        ms += v * v;
    }
    ms /= (double)N;
    double inv = 1.0 / sqrt(ms + eps);
    for (long n = 0; n < N; ++n) {
        double g = gain ? (double)gain[n] : 1.0;
        out[n] = (double)raw[n] * inv * g + (double)bias[n];
    }
}

int m3o_scan(long b, long L, long H, long G, long P, long N, long R, double eps,
             const float *x, const float *Braw, const float *Craw,
             const float *dt, const float *A, const float *lam, const float *theta,
             const float *B_bias, const float *C_bias,
             const float *B_normw, const float *C_normw,
             const float *h0, const float *x_prev, const float *Braw_prev,
             double *y, double *h_final, int nthreads)
{
    if (b < 0 || L < 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || R <= 0)
        return -1;
    if (N % 2 != 0 || H % G != 0)
        return -1;
    const long half = N / 2;
    const long hpg = H / G;
    const long nchains = b * H;
    int bad = 0;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long chain = 0; chain < nchains; ++chain) {
        const long bi = chain / H, hi = chain % H, g = hi / hpg;
        double *Hs = malloc(sizeof(double) * (size_t)(N * P));   /* state H[n][p] */
        double *U = malloc(sizeof(double) * (size_t)(N * P));
        double *Bn = malloc(sizeof(double) * (size_t)(R * N));   /* current B_t[r][n] */
        double *Cn = malloc(sizeof(double) * (size_t)(R * N));
        double *Bp = malloc(sizeof(double) * (size_t)(R * N));   /* previous B_{t-1} */
        double *xp = malloc(sizeof(double) * (size_t)(R * P));   /* previous x_{t-1} */
        double *cs = malloc(sizeof(double) * (size_t)(2 * half));
        if (!Hs || !U || !Bn || !Cn || !Bp || !xp || !cs) {
            bad = 1;
            free(Hs); free(U); free(Bn); free(Cn); free(Bp); free(xp); free(cs);
            continue;
        }
        /* initial state, stored [P][N] by the caller */
        for (long n = 0; n < N; ++n)
            for (long p = 0; p < P; ++p)
                Hs[n * P + p] = h0 ? (double)h0[((bi * H + hi) * P + p) * N + n] : 0.0;
        int has_prev = (x_prev != NULL && Braw_prev != NULL);
        if (has_prev) {
            for (long r = 0; r < R; ++r) {
                norm_bias(Braw_prev + ((bi * G + g) * R + r) * N, B_normw,
                          B_bias + (hi * R + r) * N, N, eps, Bp + r * N);
                for (long p = 0; p < P; ++p)
                    xp[r * P + p] = (double)x_prev[((bi * H + hi) * R + r) * P + p];
            }
        }

        for (long t = 0; t < L; ++t) {
            const long tok = bi * L + t;
            for (long r = 0; r < R; ++r) {
                norm_bias(Braw + ((tok * G + g) * R + r) * N, B_normw,
                          B_bias + (hi * R + r) * N, N, eps, Bn + r * N);
                norm_bias(Craw + ((tok * G + g) * R + r) * N, C_normw,
                          C_bias + (hi * R + r) * N, N, eps, Cn + r * N);
            }
            const double d = (double)dt[tok * H + hi];
            const double a = (double)A[tok * H + hi];
            const double l = (double)lam[tok * H + hi];
            const double alpha = exp(d * a);
            const double beta = (1.0 - l) * d * alpha;
            const double gamma = l * d;
            const float *xt = x + (tok * H + hi) * R * P;

            /* U = alpha H + beta sum_r B_{t-1}[r] x_{t-1}[r]^T */
            for (long n = 0; n < N; ++n)
                for (long p = 0; p < P; ++p) {
                    double v = alpha * Hs[n * P + p];
                    if (has_prev) {
                        double s = 0.0;
                        for (long r = 0; r < R; ++r)
                            s += Bp[r * N + n] * xp[r * P + p];
                        v += beta * s;
                    }
                    U[n * P + p] = v;
                }
            /* H = R_t U : rotate each pair (i, i + N/2) by dt * theta[i] */
            for (long i = 0; i < half; ++i) {
                double phi = d * (double)theta[(tok * G + g) * half + i];
                cs[2 * i] = cos(phi);
                cs[2 * i + 1] = sin(phi);
            }
            for (long i = 0; i < half; ++i) {
                const double c = cs[2 * i], s = cs[2 * i + 1];
                for (long p = 0; p < P; ++p) {
                    double u = U[i * P + p], v = U[(i + half) * P + p];
                    Hs[i * P + p] = c * u - s * v;
                    Hs[(i + half) * P + p] = s * u + c * v;
                }
            }
            /* H += gamma sum_r B_t[r] x_t[r]^T */
            for (long n = 0; n < N; ++n)
                for (long p = 0; p < P; ++p) {
                    double s = 0.0;
                    for (long r = 0; r < R; ++r)
                        s += Bn[r * N + n] * (double)xt[r * P + p];
                    Hs[n * P + p] += gamma * s;
                }
            /* y_t[r, p] = sum_n C_t[r, n] H[n, p] */
            double *yt = y + (tok * H + hi) * R * P;
            for (long r = 0; r < R; ++r)
                for (long p = 0; p < P; ++p) {
                    double s = 0.0;
                    for (long n = 0; n < N; ++n)
                        s += Cn[r * N + n] * Hs[n * P + p];
                    yt[r * P + p] = s;
                }
            /* this token becomes the previous one */
            memcpy(Bp, Bn, sizeof(double) * (size_t)(R * N));
            for (long r = 0; r < R; ++r)
                for (long p = 0; p < P; ++p)
                    xp[r * P + p] = (double)xt[r * P + p];
            has_prev = 1;
        }
        if (h_final)
            for (long p = 0; p < P; ++p)
                for (long n = 0; n < N; ++n)
                    h_final[((bi * H + hi) * P + p) * N + n] = Hs[n * P + p];
        free(Hs); free(U); free(Bn); free(Cn); free(Bp); free(xp); free(cs);
    }
    return bad ? -2 : 0;
}

int m3o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
