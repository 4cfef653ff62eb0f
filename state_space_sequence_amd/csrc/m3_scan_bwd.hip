// Backward of the chunked-scan prefill of the Mamba-3 SSM core (gfx950, fp32).
//
// The forward (see the fp32 prefill kernel) works in the rotated frame of the
// Mamba-3 paper's §3.2.2 (Proposition 4): B_bar = R(-Phi) B, C_bar = R(-Phi) C,
// and per chunk of tokens
//   y_rho  = e^{cs_t} C_bar_rho^T S_in + sum_{sigma: s <= t} m(t,s) (C_bar_rho . B_bar_sigma) x_sigma
//   S_out  = e^{cs_end} S_in + sum_sigma E_s B_bar_sigma x_sigma^T,   E_s = e^{cs_end - cs_s} w_s
// with rows rho = (t, r), m(t,s) = e^{cs_t - cs_s} w_s (s < t), gamma_t (s = t)
// (the §3.1.3 eq. 7 mask with the trapezoid's beta folded into the weights
// w_s = lam_s dt_s + (1 - lam_{s+1}) dt_{s+1}), cs the chunk-local cumulative
// dt A, and h_final = R(Phi_end) S_final. The pages give no backward; this file
// is the adjoint of exactly those expressions, term by term.
//
// Kernels:
//  1. bwd_chain_kernel, one workgroup per (batch, head) chain:
//     a forward sweep stores every chunk's starting state (and angle carry) in
//     the workspace; a reverse sweep carries dS (the adjoint of the state) back
//     through the chunks and produces, per row, dx (final), the per-head dB and dC
//     in the physical frame, and per token the gradients of cs (summed into the
//     decay increments), w, gamma and the rotation angles (their suffix sum over
//     the sequence gives d(dt theta)); at the start, dh0 and the previous token's
//     fold.
//  2. bwd_group_kernel, one workgroup per (batch, token, group): sums dB, dC and
//     d theta over the heads of the group and takes BCNorm's backward (the norm
//     factor and gain are shared by those heads), leaving per-row gain terms.
//  3. column sums (bias and gain gradients over all tokens), two levels, fixed
//     order, so every result is deterministic.
//  4. bwd_token_kernel: dt, A, lam from the per-token gradients of the decay
//     increments, of w (whose look-ahead half belongs to the next token) and of
//     gamma, plus the angle term of dt.
// The backward uses its own chunk (32 / R tokens) to keep every tile in LDS.
#include "m3_internal.h"

namespace m3i {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsB = 32;  // rows (token, rank) per backward chunk
constexpr float kInv2Pi = 0.15915494309189535f;

struct BwdDims {
    int N, P, R, half, Cb, T, nch, npb;
    int64_t slot;  // floats per checkpoint slot: N*P state + N/2 angle carry
};

__host__ __device__ inline BwdDims bwd_dims(int64_t L, int64_t N, int64_t P, int64_t R) {
    BwdDims d;
    d.N = (int)N;
    d.P = (int)P;
    d.R = (int)R;
    d.half = (int)(N / 2);
    d.Cb = kRowsB / (int)R > 0 ? kRowsB / (int)R : 1;
    d.T = d.Cb * (int)R;
    d.nch = (int)((L + d.Cb - 1) / d.Cb);
    d.npb = (int)((P + 7) / 8);
    d.slot = N * P + N / 2;
    return d;
}

// floats of the aliased region (state copy in the forward sweep; scores, mask
// and per-token angle tables in the reverse sweep)
__host__ __device__ inline int alias_floats(const BwdDims &d) {
    const int a = d.N * d.P;
    const int b = 2 * d.T * d.T + 2 * d.Cb * d.Cb + 2 * d.Cb * d.half;
    return a > b ? a : b;
}

__host__ __device__ inline size_t chain_smem_floats(const BwdDims &d) {
    return (size_t)d.N * d.P           // dS
           + alias_floats(d)           // U
           + 3 * (size_t)d.T * d.N     // B_bar, C_bar, dCoff
           + 2 * (size_t)d.T * d.P     // X, dY
           + (size_t)d.Cb * d.half     // Phi
           + (size_t)d.T * d.npb       // Q partials
           + 8 * (size_t)d.Cb          // token scalars
           + 2 * (size_t)d.T           // 1/rms of B, C rows
           + 2 * (size_t)d.half        // angle carry, reverse angle-gradient carry
           + kThreads + 4;             // reduction scratch
}

struct BwdArgs {
    ScanArgs f;
    const void *dy;
    const float *dh_final;
    float *dx, *dh0, *dx_prev;
    // workspace
    float *chk;   // [b*H][nch+1][slot]
    float *gB;    // [b,L,H,R,N] per-head dB (physical frame)
    float *gC;    // [b,L,H,R,N]
    float *gth;   // [b,L,H,N/2] per-head d theta
    float *tok;   // [b,L,H,4]   d(dt A), dw, dgamma, dt's angle term
    float *gBp;   // [b,H,R,N]   previous token's dB (per head)
    float *fold;  // [b,H]       gradient of the fold factor (1 - lam_0) dt_0
};

template <bool BF16>
__global__ __launch_bounds__(kThreads) void bwd_chain_kernel(BwdArgs ba) {
    const ScanArgs &a = ba.f;
    const BwdDims dm = bwd_dims(a.L, a.N, a.P, a.R);
    const int N = dm.N, P = dm.P, R = dm.R, half = dm.half, Cb = dm.Cb, T = dm.T, nch = dm.nch, npb = dm.npb;
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int64_t g = hi / (a.H / a.G);
    const int64_t L = a.L, H = a.H, G = a.G;

    extern __shared__ float sm[];
    float *dS = sm;                          // [N][P] adjoint of the carried state
    float *U = dS + N * P;                   // aliased region
    float *Bb = U + alias_floats(dm);        // [T][N] rotated B
    float *Cc = Bb + T * N;                  // [T][N] rotated C
    float *dCo = Cc + T * N;                 // [T][N] dC_bar from the carried-state output term
    float *Xs = dCo + T * N;                 // [T][P]
    float *dYs = Xs + T * P;                 // [T][P]
    float *Phi = dYs + T * P;                // [Cb][half] cumulative angle, revolutions
    float *Qp = Phi + Cb * half;             // [T][npb]
    float *lcs = Qp + T * npb;               // [Cb] chunk-local cumulative dt A
    float *wgt = lcs + Cb;                   // [Cb] folded weight w
    float *gam = wgt + Cb;                   // [Cb]
    float *dtv = gam + Cb;                   // [Cb]
    float *dcs = dtv + Cb;                   // [Cb] gradient of cs
    float *dwv = dcs + Cb;                   // [Cb]
    float *dgv = dwv + Cb;                   // [Cb]
    float *dthv = dgv + Cb;                  // [Cb] angle term of d dt
    float *rsB = dthv + Cb;                  // [T]
    float *rsC = rsB + T;                    // [T]
    float *carry = rsC + T;                  // [half] angle before the chunk, revolutions
    float *rcar = carry + half;              // [half] suffix sum of d Phi after the chunk (radians)
    float *red = rcar + half;                // [kThreads] reduction scratch
    float *misc = red + kThreads;            // [4]
    // reverse-sweep views of U
    float *Sc = U;                           // [T][T] C_bar . B_bar
    float *dP = Sc + T * T;                  // [T][T] dy . x
    float *Mk = dP + T * T;                  // [Cb][Cb] mask m(t, s)
    float *dMk = Mk + Cb * Cb;               // [Cb][Cb] gradient of the mask entry
    float *offp = dMk + Cb * Cb;             // [Cb][half] partial d cs from the output term
    float *dPh = offp + Cb * half;           // [Cb][half] d Phi (radians), then theta * suffix

    float *chk = ba.chk + bh * (int64_t)(nch + 1) * dm.slot;
    const float *wB = a.B_normw, *wC = a.C_normw;

    // ---- per-chunk helpers ---------------------------------------------------
    auto token_scalars = [&](int64_t c0, int nv) {
        if (tid == 0) {
            float run = 0.f;
            for (int t = 0; t < Cb; ++t) {
                if (t < nv) {
                    const int64_t o = (bi * L + c0 + t) * H + hi;
                    const float d = a.dt[o], lm = a.lam[o];
                    run += d * a.A[o];
                    const float look = (c0 + t + 1 < L) ? (1.0f - a.lam[o + H]) * a.dt[o + H] : 0.f;
                    lcs[t] = run;
                    gam[t] = lm * d;
                    wgt[t] = lm * d + look;
                    dtv[t] = d;
                } else {
                    lcs[t] = run;
                    gam[t] = 0.f;
                    wgt[t] = 0.f;
                    dtv[t] = 0.f;
                }
            }
        }
    };
    auto angles = [&](int64_t c0, int nv) {  // needs carry
        for (int i = tid; i < half; i += kThreads) {
            float ph = carry[i];
            for (int t = 0; t < nv; ++t) {
                const int64_t tok = bi * L + c0 + t;
                ph += a.dt[tok * H + hi] * a.theta[(tok * G + g) * half + i] * kInv2Pi;
                Phi[t * half + i] = ph;
            }
        }
    };
    auto row_norms = [&](int64_t c0, int nv, bool withC) {
        for (int rho = tid; rho < T; rho += kThreads) {
            const int t = rho / R, r = rho % R;
            float sb = 0.f, sc = 0.f;
            if (t < nv) {
                const int64_t row = (((bi * L + c0 + t) * G + g) * R + r) * N;
                for (int n = 0; n < N; ++n) {
                    const float vb = ld_io<BF16>(a.Braw, row + n);
                    sb += vb * vb;
                    if (withC) {
                        const float vc = ld_io<BF16>(a.Craw, row + n);
                        sc += vc * vc;
                    }
                }
            }
            rsB[rho] = 1.0f / sqrtf(sb / (float)N + a.eps);
            rsC[rho] = 1.0f / sqrtf(sc / (float)N + a.eps);
        }
    };
    // rotated, normalised, biased rows of B (and C) and the rows of x (and dy)
    auto rows = [&](int64_t c0, int nv, bool withC) {
        for (int e = tid; e < T * half; e += kThreads) {
            const int rho = e / half, i = e % half;
            const int t = rho / R, r = rho % R;
            float bl = 0.f, bhv = 0.f, cl = 0.f, chv = 0.f;
            if (t < nv) {
                const int64_t row = (((bi * L + c0 + t) * G + g) * R + r) * N;
                const float *bb = a.B_bias + (hi * R + r) * N;
                float sn, cs;
                sincospif(2.f * Phi[t * half + i], &sn, &cs);
                const float B0 = ld_io<BF16>(a.Braw, row + i) * rsB[rho] * (wB ? wB[i] : 1.f) + bb[i];
                const float B1 =
                    ld_io<BF16>(a.Braw, row + i + half) * rsB[rho] * (wB ? wB[i + half] : 1.f) + bb[i + half];
                bl = cs * B0 + sn * B1;
                bhv = -sn * B0 + cs * B1;
                if (withC) {
                    const float *cb = a.C_bias + (hi * R + r) * N;
                    const float C0 = ld_io<BF16>(a.Craw, row + i) * rsC[rho] * (wC ? wC[i] : 1.f) + cb[i];
                    const float C1 =
                        ld_io<BF16>(a.Craw, row + i + half) * rsC[rho] * (wC ? wC[i + half] : 1.f) + cb[i + half];
                    cl = cs * C0 + sn * C1;
                    chv = -sn * C0 + cs * C1;
                }
            }
            Bb[rho * N + i] = bl;
            Bb[rho * N + i + half] = bhv;
            if (withC) {
                Cc[rho * N + i] = cl;
                Cc[rho * N + i + half] = chv;
            }
        }
        for (int e = tid; e < T * P; e += kThreads) {
            const int rho = e / P, p = e % P;
            const int t = rho / R, r = rho % R;
            const int64_t o = (((bi * L + c0 + t) * H + hi) * R + r) * P + p;
            Xs[e] = (t < nv) ? ld_io<BF16>(a.x, o) : 0.f;
            if (withC) dYs[e] = (t < nv) ? ld_io<BF16>(ba.dy, o) : 0.f;
        }
    };

    // ---- initial state: h0 (physical = rotated frame before token 0) + fold
    float *S = U;  // forward-sweep state lives in the aliased region
    for (int e = tid; e < N * P; e += kThreads) {
        const int n = e / P, p = e % P;
        S[e] = a.h0 ? a.h0[(bh * P + p) * N + n] : 0.f;
    }
    for (int i = tid; i < half; i += kThreads) carry[i] = 0.f;
    const float fold_f = (a.has_prev && L > 0) ? (1.0f - a.lam[bi * L * H + hi]) * a.dt[bi * L * H + hi] : 0.f;
    // previous token's normalised, biased B rows ([R][N], in the dCo region) and x rows ([R][P], in Xs)
    auto prev_rows = [&]() {
        for (int r = tid; r < R; r += kThreads) {
            const int64_t row = ((bi * G + g) * R + r) * N;
            float ss = 0.f;
            for (int n = 0; n < N; ++n) {
                const float v = ld_io<BF16>(a.Braw_prev, row + n);
                ss += v * v;
            }
            rsB[r] = 1.0f / sqrtf(ss / (float)N + a.eps);
        }
        __syncthreads();
        for (int e = tid; e < R * N; e += kThreads) {
            const int r = e / N, n = e % N;
            dCo[e] = ld_io<BF16>(a.Braw_prev, ((bi * G + g) * R + r) * N + n) * rsB[r] * (wB ? wB[n] : 1.f) +
                     a.B_bias[(hi * R + r) * N + n];
        }
        for (int e = tid; e < R * P; e += kThreads) Xs[e] = ld_io<BF16>(a.x_prev, ((bi * H + hi) * R) * P + e);
        __syncthreads();
    };
    if (a.has_prev && L > 0) {
        prev_rows();
        for (int e = tid; e < N * P; e += kThreads) {
            const int n = e / P, p = e % P;
            float acc = 0.f;
            for (int r = 0; r < R; ++r) acc += dCo[r * N + n] * Xs[r * P + p];
            S[e] += fold_f * acc;
        }
    }
    __syncthreads();

    // ---- forward sweep: checkpoint every chunk's starting state and angle
    for (int k = 0; k < nch; ++k) {
        const int64_t c0 = (int64_t)k * Cb;
        const int nv = (int)((L - c0) < Cb ? (L - c0) : Cb);
        float *slot = chk + (int64_t)k * dm.slot;
        for (int e = tid; e < N * P; e += kThreads) slot[e] = S[e];
        for (int i = tid; i < half; i += kThreads) slot[N * P + i] = carry[i];
        token_scalars(c0, nv);
        angles(c0, nv);
        row_norms(c0, nv, false);
        __syncthreads();
        rows(c0, nv, false);
        __syncthreads();
        const float cse = lcs[nv - 1];
        const float dec = expf(cse);
        for (int e = tid; e < N * P; e += kThreads) {
            const int n = e / P, p = e % P;
            float acc = 0.f;
            for (int sg = 0; sg < T; ++sg) {
                const int s = sg / R;
                acc += Bb[sg * N + n] * (expf(cse - lcs[s]) * wgt[s]) * Xs[sg * P + p];
            }
            S[e] = dec * S[e] + acc;
        }
        for (int i = tid; i < half; i += kThreads) carry[i] = __builtin_amdgcn_fractf(Phi[(nv - 1) * half + i]);
        __syncthreads();
    }
    {
        float *slot = chk + (int64_t)nch * dm.slot;
        for (int e = tid; e < N * P; e += kThreads) slot[e] = S[e];
        for (int i = tid; i < half; i += kThreads) slot[N * P + i] = carry[i];
    }

    // ---- reverse sweep: dS = R(-Phi_end) dh_final; angle gradient of h_final
    for (int e = tid; e < half * P; e += kThreads) {
        const int i = e / P, p = e % P;
        float dlo = 0.f, dhi = 0.f;
        if (ba.dh_final) {
            float sn, cs;
            sincospif(2.f * carry[i], &sn, &cs);
            const float hl = ba.dh_final[(bh * P + p) * N + i], hh = ba.dh_final[(bh * P + p) * N + i + half];
            dlo = cs * hl + sn * hh;
            dhi = -sn * hl + cs * hh;
        }
        dS[i * P + p] = dlo;
        dS[(i + half) * P + p] = dhi;
    }
    // d Phi_end[i] = sum_p (-dh_lo h_hi + dh_hi h_lo) with h = h_final = R(Phi_end) S_final:
    // one thread per channel pair, fixed order
    for (int i = tid; i < half; i += kThreads) {
        float rg = 0.f;
        if (ba.dh_final) {
            float sn, cs;
            sincospif(2.f * carry[i], &sn, &cs);
            for (int p = 0; p < P; ++p) {
                const float hl = ba.dh_final[(bh * P + p) * N + i], hh = ba.dh_final[(bh * P + p) * N + i + half];
                const float su = S[i * P + p], sv = S[(i + half) * P + p];
                rg += -hl * (sn * su + cs * sv) + hh * (cs * su - sn * sv);
            }
        }
        rcar[i] = rg;
    }
    __syncthreads();

    for (int k = nch - 1; k >= 0; --k) {
        const int64_t c0 = (int64_t)k * Cb;
        const int nv = (int)((L - c0) < Cb ? (L - c0) : Cb);
        const float *slot = chk + (int64_t)k * dm.slot;
        const float *slot1 = chk + (int64_t)(k + 1) * dm.slot;
        for (int i = tid; i < half; i += kThreads) carry[i] = slot[N * P + i];
        token_scalars(c0, nv);
        row_norms(c0, nv, true);
        __syncthreads();
        angles(c0, nv);
        __syncthreads();
        rows(c0, nv, true);
        for (int e = tid; e < N * P; e += kThreads) U[e] = slot[e];
        __syncthreads();

        const float cse = lcs[nv - 1];
        // P2: dC_bar from the carried-state output term; <S_out, dS> partials
        for (int e = tid; e < T * N; e += kThreads) {
            const int rho = e / N, n = e % N;
            const int t = rho / R;
            float acc = 0.f;
            if (t < nv) {
                for (int p = 0; p < P; ++p) acc += U[n * P + p] * dYs[rho * P + p];
                acc *= expf(lcs[t]);
            }
            dCo[e] = acc;
        }
        {
            float part = 0.f;
            for (int e = tid; e < N * P; e += kThreads) part += slot1[e] * dS[e];
            red[tid] = part;
        }
        __syncthreads();
        // P3: scores and dy . x (U is free now)
        for (int e = tid; e < T * T; e += kThreads) {
            const int rho = e / T, sg = e % T;
            const int t = rho / R, s = sg / R;
            float sc = 0.f, dp = 0.f;
            if (s <= t && t < nv) {
                for (int n = 0; n < N; ++n) sc += Cc[rho * N + n] * Bb[sg * N + n];
                for (int p = 0; p < P; ++p) dp += dYs[rho * P + p] * Xs[sg * P + p];
            }
            Sc[e] = sc;
            dP[e] = dp;
        }
        if (tid == 0) {
            float sod = 0.f;
            for (int j = 0; j < kThreads; ++j) sod += red[j];
            misc[0] = sod;
        }
        __syncthreads();
        // P4: mask entries and their gradients per token pair
        for (int e = tid; e < Cb * Cb; e += kThreads) {
            const int t = e / Cb, s = e % Cb;
            float m = 0.f, dmv = 0.f;
            if (s <= t && t < nv) {
                m = (s == t) ? gam[t] : expf(lcs[t] - lcs[s]) * wgt[s];
                for (int r = 0; r < R; ++r)
                    for (int r2 = 0; r2 < R; ++r2) {
                        const int idx = (t * R + r) * T + s * R + r2;
                        dmv += dP[idx] * Sc[idx];
                    }
            }
            Mk[e] = m;
            dMk[e] = dmv;
        }
        __syncthreads();
        // P5: dx rows (items (sigma, block of 8 p)) and per (token, pair) items
        const int nD = T * npb;
        for (int e = tid; e < nD + Cb * half; e += kThreads) {
            if (e < nD) {
                const int sg = e / npb, pb = e % npb;
                const int s = sg / R;
                if (s >= nv) {
                    Qp[sg * npb + pb] = 0.f;
                    continue;
                }
                const float Es = expf(cse - lcs[s]) * wgt[s];
                float q = 0.f;
                const int p1 = (8 * pb + 8 < P) ? 8 * pb + 8 : P;
                for (int p = 8 * pb; p < p1; ++p) {
                    float intra = 0.f;
                    for (int rho = s * R; rho < nv * R; ++rho) intra += Mk[(rho / R) * Cb + s] * Sc[rho * T + sg] * dYs[rho * P + p];
                    float st = 0.f;
                    for (int n = 0; n < N; ++n) st += dS[n * P + p] * Bb[sg * N + n];
                    q += Xs[sg * P + p] * st;
                    ba.dx[(((bi * L + c0 + s) * H + hi) * R + sg % R) * P + p] = intra + Es * st;
                }
                Qp[sg * npb + pb] = q;
            } else {
                const int e2 = e - nD;
                const int t = e2 / half, i = e2 % half;
                float dphi = 0.f, off = 0.f;
                if (t < nv) {
                    const float Et = expf(cse - lcs[t]) * wgt[t];
                    float sn, cs;
                    sincospif(2.f * Phi[t * half + i], &sn, &cs);
                    for (int r = 0; r < R; ++r) {
                        const int rho = t * R + r;
                        float dcl = dCo[rho * N + i], dch = dCo[rho * N + i + half];
                        off += Cc[rho * N + i] * dcl + Cc[rho * N + i + half] * dch;
                        for (int sg = 0; sg < (t + 1) * R; ++sg) {
                            const float f = Mk[t * Cb + sg / R] * dP[rho * T + sg];
                            dcl += f * Bb[sg * N + i];
                            dch += f * Bb[sg * N + i + half];
                        }
                        float dbl = 0.f, dbh = 0.f;
                        for (int r2 = t * R; r2 < nv * R; ++r2) {
                            const float f = Mk[(r2 / R) * Cb + t] * dP[r2 * T + rho];
                            dbl += f * Cc[r2 * N + i];
                            dbh += f * Cc[r2 * N + i + half];
                        }
                        float sl = 0.f, sh = 0.f;
                        for (int p = 0; p < P; ++p) {
                            sl += dS[i * P + p] * Xs[rho * P + p];
                            sh += dS[(i + half) * P + p] * Xs[rho * P + p];
                        }
                        dbl += Et * sl;
                        dbh += Et * sh;
                        dphi += dbl * Bb[rho * N + i + half] - dbh * Bb[rho * N + i] + dcl * Cc[rho * N + i + half] -
                                dch * Cc[rho * N + i];
                        // back to the physical frame: d B = R(Phi) d B_bar
                        const int64_t o = (((bi * L + c0 + t) * H + hi) * R + r) * N;
                        ba.gB[o + i] = cs * dbl - sn * dbh;
                        ba.gB[o + i + half] = sn * dbl + cs * dbh;
                        ba.gC[o + i] = cs * dcl - sn * dch;
                        ba.gC[o + i + half] = sn * dcl + cs * dch;
                    }
                }
                offp[t * half + i] = off;
                dPh[t * half + i] = dphi;
            }
        }
        __syncthreads();
        // P6: per-token scalar gradients; suffix sums of d Phi per channel
        for (int j = tid; j < Cb + half; j += kThreads) {
            if (j < Cb) {
                const int t = j;
                float dc = 0.f, dw = 0.f, dg = 0.f;
                if (t < nv) {
                    float Qt = 0.f;
                    for (int r = 0; r < R; ++r)
                        for (int pb = 0; pb < npb; ++pb) Qt += Qp[(t * R + r) * npb + pb];
                    for (int i = 0; i < half; ++i) dc += offp[t * half + i];
                    for (int s = 0; s < t; ++s) dc += dMk[t * Cb + s] * Mk[t * Cb + s];
                    for (int t2 = t + 1; t2 < nv; ++t2) {
                        dc -= dMk[t2 * Cb + t] * Mk[t2 * Cb + t];
                        dw += dMk[t2 * Cb + t] * expf(lcs[t2] - lcs[t]);
                    }
                    const float Et = expf(cse - lcs[t]);
                    dc -= Et * wgt[t] * Qt;
                    dw += Et * Qt;
                    if (t == nv - 1) dc += misc[0];
                    dg = dMk[t * Cb + t];
                }
                dcs[t] = dc;
                dwv[t] = dw;
                dgv[t] = dg;
            } else {
                const int i = j - Cb;
                float rc = rcar[i];
                for (int t = nv - 1; t >= 0; --t) {
                    rc += dPh[t * half + i];
                    const int64_t tok = bi * L + c0 + t;
                    ba.gth[(tok * H + hi) * half + i] = dtv[t] * rc;
                    dPh[t * half + i] = a.theta[(tok * G + g) * half + i] * rc;
                }
                rcar[i] = rc;
            }
        }
        __syncthreads();
        // P7: token records (suffix sums of d cs give d(dt A)); dS back to the chunk start
        for (int t = tid; t < nv; t += kThreads) {
            float da = 0.f;
            for (int t2 = t; t2 < nv; ++t2) da += dcs[t2];
            float dth = 0.f;
            for (int i = 0; i < half; ++i) dth += dPh[t * half + i];
            float *rec = ba.tok + ((bi * L + c0 + t) * H + hi) * 4;
            rec[0] = da;
            rec[1] = dwv[t];
            rec[2] = dgv[t];
            rec[3] = dth;
        }
        const float dec = expf(cse);
        for (int e = tid; e < N * P; e += kThreads) {
            const int n = e / P, p = e % P;
            float acc = 0.f;
            for (int rho = 0; rho < nv * R; ++rho) acc += expf(lcs[rho / R]) * Cc[rho * N + n] * dYs[rho * P + p];
            dS[e] = dec * dS[e] + acc;
        }
        __syncthreads();
    }

    // ---- chain start: dh0 and the previous token's fold
    if (ba.dh0) {
        for (int e = tid; e < N * P; e += kThreads) {
            const int p = e / N, n = e % N;
            ba.dh0[(bh * P + p) * N + n] = dS[n * P + p];
        }
    }
    if (a.has_prev && L > 0) {
        prev_rows();  // dCo <- B_{-1} rows, Xs <- x_{-1} rows
        for (int e = tid; e < R * N; e += kThreads) {
            const int r = e / N, n = e % N;
            float acc = 0.f;
            for (int p = 0; p < P; ++p) acc += dS[n * P + p] * Xs[r * P + p];
            ba.gBp[(bh * R + r) * N + n] = fold_f * acc;
        }
        for (int e = tid; e < R * P; e += kThreads) {
            const int r = e / P, p = e % P;
            float acc = 0.f;
            for (int n = 0; n < N; ++n) acc += dS[n * P + p] * dCo[r * N + n];
            ba.dx_prev[(bh * R + r) * P + p] = fold_f * acc;
        }
        // d f = <dS, sum_r B_{-1}[r] x_{-1}[r]^T>
        float part = 0.f;
        for (int e = tid; e < N * P; e += kThreads) {
            const int n = e / P, p = e % P;
            float v = 0.f;
            for (int r = 0; r < R; ++r) v += dCo[r * N + n] * Xs[r * P + p];
            part += dS[e] * v;
        }
        red[tid] = part;
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
            for (int j = 0; j < kThreads; ++j) s += red[j];
            ba.fold[bh] = s;
        }
    }
}

// Sum the per-head dB / dC / d theta of a token over the heads of its group and
// take BCNorm's backward: with v = Braw rs w + bias, rs = (mean Braw^2 + eps)^-1/2,
//   dBraw = rs w dv - Braw rs^3 / N sum_n (Braw w dv).
// Also writes, per row, Braw rs dv (the gain's gradient terms, summed later).
// One workgroup per (row block): rows are (batch, token, group) for the
// sequence, or (batch, group) for the previous token (prev = true).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void bwd_group_kernel(BwdArgs ba, bool prev, float *gWB, float *gWC,
                                                             float *dBraw_out, float *dCraw_out) {
    const ScanArgs &a = ba.f;
    const int N = (int)a.N, R = (int)a.R, half = N / 2;
    const int64_t H = a.H, G = a.G, hpg = H / G;
    const int64_t row = blockIdx.x;  // (b, t, g) or (b, g)
    const int tid = threadIdx.x;
    __shared__ float red[2][kThreads];
    __shared__ float tot[2];
    const int64_t g = row % G;
    const int64_t bt = row / G;  // b * L + t, or b
    for (int r = 0; r < R; ++r) {
        // one pass per rank row: N channels over the threads
        const int64_t rawrow = (row * R + r) * N;
        float ssb = 0.f, ssc = 0.f;
        for (int n = tid; n < N; n += kThreads) {
            const float vb = ld_io<BF16>(prev ? a.Braw_prev : a.Braw, rawrow + n);
            ssb += vb * vb;
            if (!prev) {
                const float vc = ld_io<BF16>(a.Craw, rawrow + n);
                ssc += vc * vc;
            }
        }
        red[0][tid] = ssb;
        red[1][tid] = ssc;
        __syncthreads();
        if (tid == 0) {
            float s0 = 0.f, s1 = 0.f;
            for (int j = 0; j < kThreads; ++j) {
                s0 += red[0][j];
                s1 += red[1][j];
            }
            tot[0] = 1.0f / sqrtf(s0 / (float)N + a.eps);
            tot[1] = 1.0f / sqrtf(s1 / (float)N + a.eps);
        }
        __syncthreads();
        const float rsb = tot[0], rsc = tot[1];
        float db_keep[4] = {0.f, 0.f, 0.f, 0.f}, dc_keep[4] = {0.f, 0.f, 0.f, 0.f};  // N <= 4 * kThreads / 2
        float pb = 0.f, pc = 0.f;
        int kk = 0;
        for (int n = tid; n < N; n += kThreads, ++kk) {
            float sb = 0.f, sc = 0.f;
            for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
                if (prev) {
                    sb += ba.gBp[((bt * H + h) * R + r) * N + n];
                } else {
                    const int64_t o = ((bt * H + h) * R + r) * N + n;
                    sb += ba.gB[o];
                    sc += ba.gC[o];
                }
            }
            db_keep[kk] = sb;
            dc_keep[kk] = sc;
            const float wbn = a.B_normw ? a.B_normw[n] : 1.f, wcn = a.C_normw ? a.C_normw[n] : 1.f;
            const float vb = ld_io<BF16>(prev ? a.Braw_prev : a.Braw, rawrow + n);
            pb += vb * wbn * sb;
            if (!prev) pc += ld_io<BF16>(a.Craw, rawrow + n) * wcn * sc;
        }
        __syncthreads();
        red[0][tid] = pb;
        red[1][tid] = pc;
        __syncthreads();
        if (tid == 0) {
            float s0 = 0.f, s1 = 0.f;
            for (int j = 0; j < kThreads; ++j) {
                s0 += red[0][j];
                s1 += red[1][j];
            }
            tot[0] = s0;
            tot[1] = s1;
        }
        __syncthreads();
        kk = 0;
        for (int n = tid; n < N; n += kThreads, ++kk) {
            const float wbn = a.B_normw ? a.B_normw[n] : 1.f, wcn = a.C_normw ? a.C_normw[n] : 1.f;
            const float vb = ld_io<BF16>(prev ? a.Braw_prev : a.Braw, rawrow + n);
            dBraw_out[rawrow + n] = rsb * wbn * db_keep[kk] - vb * rsb * rsb * rsb / (float)N * tot[0];
            gWB[rawrow + n] = vb * rsb * db_keep[kk];
            if (!prev) {
                const float vc = ld_io<BF16>(a.Craw, rawrow + n);
                dCraw_out[rawrow + n] = rsc * wcn * dc_keep[kk] - vc * rsc * rsc * rsc / (float)N * tot[1];
                gWC[rawrow + n] = vc * rsc * dc_keep[kk];
            }
        }
        __syncthreads();
    }
    (void)half;
}

// d theta[b,t,g,i] = sum over the heads of group g of the per-head terms
__global__ __launch_bounds__(kThreads) void bwd_theta_kernel(BwdArgs ba, float *dtheta) {
    const ScanArgs &a = ba.f;
    const int64_t half = a.N / 2, H = a.H, G = a.G, hpg = H / G;
    const int64_t total = a.b * a.L * G * half;
    for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < total; e += (int64_t)gridDim.x * kThreads) {
        const int64_t i = e % half, g = (e / half) % G, bt = e / (half * G);
        float s = 0.f;
        for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) s += ba.gth[(bt * H + h) * half + i];
        dtheta[e] = s;
    }
}

// Column sums, level 1: out[split][c] = sum of rows [split*rows_per, ...) of column c
// of a row-major [rows][cols] array (rows given as two segments: src and an optional
// second array src2 of rows2 rows appended after it).
__global__ __launch_bounds__(kThreads) void colsum_partial_kernel(const float *src, int64_t rows, const float *src2,
                                                                  int64_t rows2, int64_t cols, int64_t rows_per,
                                                                  float *out) {
    const int64_t c = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    const int64_t split = blockIdx.y;
    if (c >= cols) return;
    const int64_t r0 = split * rows_per, r1 = (r0 + rows_per < rows + rows2) ? r0 + rows_per : rows + rows2;
    float s = 0.f;
    for (int64_t r = r0; r < r1; ++r) s += (r < rows) ? src[r * cols + c] : src2[(r - rows) * cols + c];
    out[split * cols + c] = s;
}

// level 2: dst[c] = sum over splits
__global__ __launch_bounds__(kThreads) void colsum_final_kernel(const float *part, int64_t nsplit, int64_t cols,
                                                                float *dst) {
    const int64_t c = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (c >= cols) return;
    float s = 0.f;
    for (int64_t k = 0; k < nsplit; ++k) s += part[k * cols + c];
    dst[c] = s;
}

// dt, A, lam per (batch, token, head) from the token records:
//   d(dt A) = da:        dA = dt da, ddt += A da
//   w_t = lam_t dt_t + (1 - lam_{t+1}) dt_{t+1}:  the second half belongs to token t+1
//   gamma_t = lam_t dt_t
//   Phi: ddt += the angle term; the fold factor (1 - lam_0) dt_0 acts at t = 0.
__global__ __launch_bounds__(kThreads) void bwd_token_kernel(BwdArgs ba, float *ddt, float *dA, float *dlam) {
    const ScanArgs &a = ba.f;
    const int64_t total = a.b * a.L * a.H;
    for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < total; e += (int64_t)gridDim.x * kThreads) {
        const int64_t h = e % a.H, bt = e / a.H, t = bt % a.L, bi = bt / a.L;
        const float *rec = ba.tok + e * 4;
        const float d = a.dt[e], lm = a.lam[e], av = a.A[e];
        const float da = rec[0], dw = rec[1], dg = rec[2], dth = rec[3];
        float dprev;  // gradient of the factor (1 - lam_t) dt_t
        if (t > 0)
            dprev = ba.tok[(e - a.H) * 4 + 1];
        else
            dprev = (a.has_prev) ? ba.fold[bi * a.H + h] : 0.f;
        dA[e] = d * da;
        ddt[e] = av * da + lm * (dw + dg) + (1.0f - lm) * dprev + dth;
        dlam[e] = d * (dw + dg) - d * dprev;
    }
}

}  // namespace

size_t scan_bwd_workspace_bytes(const ScanArgs &a, int64_t *nsplit_out) {
    const BwdDims d = bwd_dims(a.L, a.N, a.P, a.R);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t chains = a.b * a.H;
    const int64_t rowsBC = a.b * a.L * a.G * a.R;  // raw B / C rows
    const int64_t rows_prev = a.b * a.G * a.R;
    const int64_t cols_max = (a.H * a.R * a.N > a.N) ? a.H * a.R * a.N : a.N;
    const int64_t nsplit = 64;
    if (nsplit_out) *nsplit_out = nsplit;
    size_t s = 0;
    s += al(sizeof(float) * chains * (d.nch + 1) * d.slot);      // checkpoints
    s += 2 * al(sizeof(float) * a.b * a.L * a.H * a.R * a.N);    // gB, gC
    s += al(sizeof(float) * a.b * a.L * a.H * (a.N / 2));        // gth
    s += al(sizeof(float) * a.b * a.L * a.H * 4);                // tok
    s += al(sizeof(float) * chains * a.R * a.N);                 // gBp
    s += al(sizeof(float) * chains);                             // fold
    s += 2 * al(sizeof(float) * (rowsBC + rows_prev) * a.N);     // gWB, gWC
    s += al(sizeof(float) * nsplit * cols_max);                  // column-sum partials
    return s;
}

hipError_t launch_scan_bwd(const ScanArgs &a, const BwdIO &io, void *ws, hipStream_t st) {
    if (a.b * a.H == 0) return hipSuccess;
    const BwdDims d = bwd_dims(a.L, a.N, a.P, a.R);
    int64_t nsplit = 0;
    scan_bwd_workspace_bytes(a, &nsplit);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t chains = a.b * a.H;
    const int64_t rowsBC = a.b * a.L * a.G * a.R;
    const int64_t rows_prev = a.b * a.G * a.R;
    char *p = static_cast<char *>(ws);
    BwdArgs ba{};
    ba.f = a;
    ba.dy = io.dy;
    ba.dh_final = io.dh_final;
    ba.dx = io.dx;
    ba.dh0 = io.dh0;
    ba.dx_prev = io.dx_prev;
    ba.chk = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * chains * (d.nch + 1) * d.slot);
    ba.gB = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * a.b * a.L * a.H * a.R * a.N);
    ba.gC = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * a.b * a.L * a.H * a.R * a.N);
    ba.gth = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * a.b * a.L * a.H * (a.N / 2));
    ba.tok = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * a.b * a.L * a.H * 4);
    ba.gBp = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * chains * a.R * a.N);
    ba.fold = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * chains);
    float *gWB = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * (rowsBC + rows_prev) * a.N);
    float *gWC = reinterpret_cast<float *>(p);
    p += al(sizeof(float) * (rowsBC + rows_prev) * a.N);
    float *part = reinterpret_cast<float *>(p);

    hipError_t e;
    const size_t smem = sizeof(float) * chain_smem_floats(d);
    const void *fn = a.bf16 ? (const void *)bwd_chain_kernel<true> : (const void *)bwd_chain_kernel<false>;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    if (a.bf16)
        hipLaunchKernelGGL(bwd_chain_kernel<true>, dim3((unsigned)chains), dim3(kThreads), smem, st, ba);
    else
        hipLaunchKernelGGL(bwd_chain_kernel<false>, dim3((unsigned)chains), dim3(kThreads), smem, st, ba);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const unsigned nrow = (unsigned)(a.b * a.L * a.G);
    if (nrow > 0) {
        if (a.bf16)
            hipLaunchKernelGGL(bwd_group_kernel<true>, dim3(nrow), dim3(kThreads), 0, st, ba, false, gWB, gWC, io.dBraw,
                               io.dCraw);
        else
            hipLaunchKernelGGL(bwd_group_kernel<false>, dim3(nrow), dim3(kThreads), 0, st, ba, false, gWB, gWC,
                               io.dBraw, io.dCraw);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    float *gWBp = gWB + rowsBC * a.N;
    if (a.has_prev && a.L > 0) {
        const unsigned np = (unsigned)(a.b * a.G);
        if (a.bf16)
            hipLaunchKernelGGL(bwd_group_kernel<true>, dim3(np), dim3(kThreads), 0, st, ba, true, gWBp, nullptr,
                               io.dBraw_prev, nullptr);
        else
            hipLaunchKernelGGL(bwd_group_kernel<false>, dim3(np), dim3(kThreads), 0, st, ba, true, gWBp, nullptr,
                               io.dBraw_prev, nullptr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        const int64_t tot = a.b * a.L * a.G * (a.N / 2);
        const unsigned nb = (unsigned)((tot + kThreads - 1) / kThreads < 65536 ? (tot + kThreads - 1) / kThreads : 65536);
        if (tot > 0) {
            hipLaunchKernelGGL(bwd_theta_kernel, dim3(nb), dim3(kThreads), 0, st, ba, io.dtheta);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    // column sums: biases over (b, t) rows (plus the previous token's rows), gains over every raw row
    auto colsum = [&](const float *src, int64_t rows, const float *src2, int64_t rows2, int64_t cols,
                      float *dst) -> hipError_t {
        const int64_t tr = rows + rows2;
        const int64_t rows_per = (tr + nsplit - 1) / nsplit > 0 ? (tr + nsplit - 1) / nsplit : 1;
        const int64_t ns = (tr + rows_per - 1) / rows_per > 0 ? (tr + rows_per - 1) / rows_per : 1;
        const unsigned cb = (unsigned)((cols + kThreads - 1) / kThreads);
        hipLaunchKernelGGL(colsum_partial_kernel, dim3(cb, (unsigned)ns), dim3(kThreads), 0, st, src, rows, src2,
                           rows2, cols, rows_per, part);
        hipError_t e2 = hipGetLastError();
        if (e2 != hipSuccess) return e2;
        hipLaunchKernelGGL(colsum_final_kernel, dim3(cb), dim3(kThreads), 0, st, part, ns, cols, dst);
        return hipGetLastError();
    };
    const int64_t cols_bias = a.H * a.R * a.N;
    const bool prev = a.has_prev && a.L > 0;
    if ((e = colsum(ba.gB, a.b * a.L, prev ? ba.gBp : nullptr, prev ? a.b : 0, cols_bias, io.dB_bias)) != hipSuccess)
        return e;
    if ((e = colsum(ba.gC, a.b * a.L, nullptr, 0, cols_bias, io.dC_bias)) != hipSuccess) return e;
    if (io.dB_normw &&
        (e = colsum(gWB, rowsBC, prev ? gWBp : nullptr, prev ? rows_prev : 0, a.N, io.dB_normw)) != hipSuccess)
        return e;
    if (io.dC_normw && (e = colsum(gWC, rowsBC, nullptr, 0, a.N, io.dC_normw)) != hipSuccess) return e;
    {
        const int64_t tot = a.b * a.L * a.H;
        const unsigned nb = (unsigned)((tot + kThreads - 1) / kThreads < 65536 ? (tot + kThreads - 1) / kThreads : 65536);
        if (tot > 0) {
            hipLaunchKernelGGL(bwd_token_kernel, dim3(nb), dim3(kThreads), 0, st, ba, io.ddt, io.dA, io.dlam);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

size_t scan_bwd_smem_bytes(const ScanArgs &a) {
    return sizeof(float) * chain_smem_floats(bwd_dims(a.L, a.N, a.P, a.R));
}

}  // namespace m3i
