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
constexpr int kChainThreads = 512;  // chain kernel: 8 waves, one workgroup per CU (LDS-bound)
constexpr int kRowsB = 32;  // rows (token, rank) per backward chunk
constexpr float kInv2Pi = 0.15915494309189535f;

typedef float f4 __attribute__((ext_vector_type(4)));

// x / d for a runtime divisor by one multiply-high: with m = floor(2^32 / d) + 1,
// floor(x m / 2^32) = floor(x / d) whenever x < 2^16 and d < 2^16 (the error term
// x (m d - 2^32) / (d 2^32) stays below 1/d). Every item index here is below 2^16.
struct FDiv {
    uint32_t d;
    uint64_t m;
    __device__ explicit FDiv(uint32_t dd) : d(dd), m((1ull << 32) / dd + 1) {}
    __device__ int q(int x) const { return (int)(((uint64_t)(uint32_t)x * m) >> 32); }
};
__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ float dot4(f4 a, f4 b, float c) {
    return __builtin_fmaf(a[3], b[3], __builtin_fmaf(a[2], b[2], __builtin_fmaf(a[1], b[1], __builtin_fmaf(a[0], b[0], c))));
}

struct BwdDims {
    int N, P, R, half, Cb, T, nch, npb;
    int NS, PS, HS;  // padded LDS row strides (one extra float: strided walks hit distinct banks)
    int64_t slot;    // floats per checkpoint slot: N*P state + N/2 angle carry
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
    d.npb = (int)(P / 4);  // dx items: 4 columns each (P % 4 == 0)
    d.NS = d.N + 4;  // rows stay 16-byte aligned for vector reads and shift by 4 banks
    d.PS = d.P + 4;
    d.HS = d.half + 1;
    d.slot = N * P + N / 2;
    return d;
}

// floats of the aliased region (the state in the forward sweep; scores, mask and
// per-token angle tables in the reverse sweep)
__host__ __device__ inline int alias_floats(const BwdDims &d) {
    const int a = d.N * d.PS;
    const int b = 2 * d.T * d.T + 2 * d.Cb * d.Cb + 2 * d.Cb * d.HS;
    return ((a > b ? a : b) + 3) / 4 * 4;  // keeps the tiles after it 16-byte aligned
}

__host__ __device__ inline size_t chain_smem_floats(const BwdDims &d) {
    return (size_t)d.N * d.PS          // dS
           + alias_floats(d)           // U
           + 3 * (size_t)d.T * d.NS    // B_bar, C_bar, dCoff
           + 2 * (size_t)d.T * d.PS    // X, dY
           + 2 * (size_t)d.Cb * d.half // Phi, theta
           + (size_t)d.T * d.npb       // Q partials
           + 14 * (size_t)(d.Cb + 1)   // token scalars
           + 2 * (size_t)d.T           // 1/rms of B, C rows
           + 2 * (size_t)d.half        // angle carry, reverse angle-gradient carry
           + kChainThreads + 4;        // reduction scratch
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
    float *bpart; // [b,H][2][R][2][N] matrix-core chain kernel: per-chain bias sums (row tile, rank, B / C)
    // Rows of gB, gC and gth: token t of batch b is row b * Lb + t - tbase (Lb = L, tbase = 0
    // in one pass; the window's tokens under the low-memory schedule).
    int64_t Lb, tbase;
    // Low-memory schedule (matrix-core chain kernel only; wchunks = 0: one pass). chk then
    // holds a checkpoint every wchunks chunks plus the final state ([b*H][nwin+1][slot]).
    // A launch with win < 0 runs the forward sweep only; a launch with win = w recomputes
    // the states of window w's chunks into chkw ([b*H][wchunks+1][slot]) from its
    // checkpoint and runs the reverse sweep over them, carrying dS, the angle-gradient
    // carry and the bias sums to the next window (win - 1) through rst.
    int wchunks, win;
    float *chkw;
    float *rst;   // [b*H][N*P + N/2 + 4*512]
};

// NF, PF: N and P fixed at compile time (0: taken from the arguments)
template <bool BF16, int R, int NF, int PF>
__global__ __launch_bounds__(kChainThreads) void bwd_chain_kernel(BwdArgs ba) {
    const ScanArgs &a = ba.f;
    const BwdDims dm = bwd_dims(a.L, NF ? NF : a.N, PF ? PF : a.P, R);
    constexpr int Cb = kRowsB / R, T = Cb * R;  // tokens and rows per chunk (compile-time)
    const int N = NF ? NF : dm.N, P = PF ? PF : dm.P, half = N / 2, nch = dm.nch, npb = P / 4;
    const int NS = N + 4, PS = P + 4, HS = half + 1;
    constexpr int NT = kChainThreads;
    const FDiv fN((uint32_t)N), fP((uint32_t)P), fH((uint32_t)half), fP4((uint32_t)(P / 4));
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int64_t g = hi / (a.H / a.G);
    const int64_t L = a.L, H = a.H, G = a.G;

    extern __shared__ float sm[];
    float *dS = sm;                          // [N][PS] adjoint of the carried state
    float *U = dS + N * PS;                  // aliased region
    float *Bb = U + alias_floats(dm);        // [T][NS] rotated B (raw rows first)
    float *Cc = Bb + T * NS;                 // [T][NS] rotated C
    float *dCo = Cc + T * NS;                // [T][NS] dC_bar from the carried-state output term
    float *Xs = dCo + T * NS;                // [T][PS]
    float *dYs = Xs + T * PS;                // [T][PS]
    float *Phi = dYs + T * PS;               // [Cb][half] angle increments, then cumulative angle (revolutions)
    float *thv = Phi + Cb * half;            // [Cb][half] theta of the chunk's tokens
    float *Qp = thv + Cb * half;             // [T][npb]
    float *dtv = Qp + T * npb;               // [Cb+1] dt (the extra one: the token after the chunk)
    float *lamv = dtv + (Cb + 1);            // [Cb+1] lam
    float *Av = lamv + (Cb + 1);             // [Cb+1] A
    float *lcs = Av + (Cb + 1);              // [Cb+1] chunk-local cumulative dt A
    float *wgt = lcs + (Cb + 1);             // [Cb+1] folded weight w
    float *gam = wgt + (Cb + 1);             // [Cb+1]
    float *ecs = gam + (Cb + 1);             // [Cb+1] e^{cs_t}
    float *Ew = ecs + (Cb + 1);              // [Cb+1] e^{cs_end - cs_t} w_t
    float *Ee = Ew + (Cb + 1);               // [Cb+1] e^{cs_end - cs_t}
    float *dcs = Ee + (Cb + 1);              // [Cb+1] gradient of cs
    float *dwv = dcs + (Cb + 1);             // [Cb+1]
    float *dgv = dwv + (Cb + 1);             // [Cb+1]
    float *dthv = dgv + (Cb + 1);            // [Cb+1] (spare)
    float *sp2 = dthv + (Cb + 1);            // [Cb+1] (spare)
    float *rsB = sp2 + (Cb + 1);             // [T]
    float *rsC = rsB + T;                    // [T]
    float *carry = rsC + T;                  // [half] angle before the chunk, revolutions
    float *rcar = carry + half;              // [half] suffix sum of d Phi after the chunk (radians)
    float *red = rcar + half;                // [NT] reduction scratch
    float *misc = red + NT;                  // [4]
    // reverse-sweep views of U
    float *Sc = U;                           // [T][T] C_bar . B_bar
    float *dP = Sc + T * T;                  // [T][T] dy . x
    float *Mk = dP + T * T;                  // [Cb][Cb] mask m(t, s)
    float *dMk = Mk + Cb * Cb;               // [Cb][Cb] gradient of the mask entry
    float *offp = dMk + Cb * Cb;             // [Cb][HS] partial d cs from the output term
    float *dPh = offp + Cb * HS;             // [Cb][HS] d Phi (radians), then theta * suffix
    (void)dthv;
    (void)sp2;

    float *chk = ba.chk + bh * (int64_t)(nch + 1) * dm.slot;
    const float *wB = a.B_normw, *wC = a.C_normw;

    // ---- per-chunk staging (every global load in parallel, every serial walk in LDS)
    // phase 1: token scalars (and the one after the chunk), raw B / C rows, x / dy rows,
    // angle increments
    auto stage_loads = [&](int64_t c0, int nv, bool withC) {
        for (int t = tid; t <= Cb; t += NT) {
            float d = 0.f, lm = 0.f, av = 0.f;
            if (t <= nv && c0 + t < L) {
                const int64_t o = (bi * L + c0 + t) * H + hi;
                d = a.dt[o];
                lm = a.lam[o];
                av = a.A[o];
            }
            dtv[t] = d;
            lamv[t] = lm;
            Av[t] = av;
        }
        for (int e = tid; e < T * N; e += NT) {
            const int rho = fN.q(e), n = e - rho * N;
            const int t = rho / R, r = rho % R;
            float vb = 0.f, vc = 0.f;
            if (t < nv) {
                const int64_t row = (((bi * L + c0 + t) * G + g) * R + r) * N;
                vb = ld_io<BF16>(a.Braw, row + n);
                if (withC) vc = ld_io<BF16>(a.Craw, row + n);
            }
            Bb[rho * NS + n] = vb;
            if (withC) Cc[rho * NS + n] = vc;
        }
        for (int e = tid; e < T * P; e += NT) {
            const int rho = fP.q(e), p = e - rho * P;
            const int t = rho / R, r = rho % R;
            const int64_t o = (((bi * L + c0 + t) * H + hi) * R + r) * P + p;
            Xs[rho * PS + p] = (t < nv) ? ld_io<BF16>(a.x, o) : 0.f;
            if (withC) dYs[rho * PS + p] = (t < nv) ? ld_io<BF16>(ba.dy, o) : 0.f;
        }
        for (int e = tid; e < Cb * half; e += NT) {
            const int t = fH.q(e), i = e - t * half;
            float v = 0.f, th = 0.f;
            if (t < nv) {
                const int64_t tok = bi * L + c0 + t;
                th = a.theta[(tok * G + g) * half + i];
                v = a.dt[tok * H + hi] * th * kInv2Pi;
            }
            Phi[e] = v;
            thv[e] = th;
        }
    };
    // phase 2: prefix sums (decay: one thread; angles: one thread per channel), row norms
    // (groups of 8 lanes per row)
    auto stage_scans = [&](int64_t c0, int nv, bool withC) {
        if (tid == 0) {
            float run = 0.f;
            for (int t = 0; t < Cb; ++t) {
                if (t < nv) {
                    run += dtv[t] * Av[t];
                    const float look = (c0 + t + 1 < L) ? (1.0f - lamv[t + 1]) * dtv[t + 1] : 0.f;
                    lcs[t] = run;
                    gam[t] = lamv[t] * dtv[t];
                    wgt[t] = lamv[t] * dtv[t] + look;
                } else {
                    lcs[t] = run;
                    gam[t] = 0.f;
                    wgt[t] = 0.f;
                }
            }
        }
        for (int i = tid - 64; i >= 0 && i < half; i += NT) {  // threads 64.. : angle prefix
            float ph = carry[i];
            for (int t = 0; t < nv; ++t) {
                ph += Phi[t * half + i];
                Phi[t * half + i] = ph;
            }
        }
        const int nrow = withC ? 2 * T : T;
        for (int grp = tid / 8; grp < nrow; grp += NT / 8) {  // the 8 lanes of a group run together
            const int lane8 = tid % 8;
            const bool isC = grp >= T;
            const int rho = isC ? grp - T : grp;
            const float *row = (isC ? Cc : Bb) + rho * NS;
            float ss = 0.f;
            for (int n = lane8; n < N; n += 8) ss += row[n] * row[n];
            ss = group_sum<8>(ss);
            if (lane8 == 0) (isC ? rsC : rsB)[rho] = 1.0f / sqrtf(ss / (float)N + a.eps);
        }
    };
    // phase 3: exponentials of the decay; normalise, bias and rotate B / C in place
    auto stage_rows = [&](int nv, bool withC) {
        const float cse = lcs[nv - 1];
        for (int t = tid; t < Cb; t += NT) {
            ecs[t] = expf(lcs[t]);
            Ee[t] = (t < nv) ? expf(cse - lcs[t]) : 0.f;
            Ew[t] = Ee[t] * wgt[t];
        }
        for (int e = tid; e < T * half; e += NT) {
            const int rho = fH.q(e), i = e - rho * half;
            const int t = rho / R, r = rho % R;
            float bl = 0.f, bhv = 0.f, cl = 0.f, chv = 0.f;
            if (t < nv) {
                const float *bb = a.B_bias + (hi * R + r) * N;
                float sn, cs;
                sincospif(2.f * Phi[t * half + i], &sn, &cs);
                const float B0 = Bb[rho * NS + i] * rsB[rho] * (wB ? wB[i] : 1.f) + bb[i];
                const float B1 = Bb[rho * NS + i + half] * rsB[rho] * (wB ? wB[i + half] : 1.f) + bb[i + half];
                bl = cs * B0 + sn * B1;
                bhv = -sn * B0 + cs * B1;
                if (withC) {
                    const float *cb = a.C_bias + (hi * R + r) * N;
                    const float C0 = Cc[rho * NS + i] * rsC[rho] * (wC ? wC[i] : 1.f) + cb[i];
                    const float C1 = Cc[rho * NS + i + half] * rsC[rho] * (wC ? wC[i + half] : 1.f) + cb[i + half];
                    cl = cs * C0 + sn * C1;
                    chv = -sn * C0 + cs * C1;
                }
            }
            Bb[rho * NS + i] = bl;
            Bb[rho * NS + i + half] = bhv;
            if (withC) {
                Cc[rho * NS + i] = cl;
                Cc[rho * NS + i + half] = chv;
            }
        }
    };
    auto stage_chunk = [&](int64_t c0, int nv, bool withC) {
        stage_loads(c0, nv, withC);
        __syncthreads();
        stage_scans(c0, nv, withC);
        __syncthreads();
        stage_rows(nv, withC);
        __syncthreads();
    };

    // ---- initial state: h0 (physical = rotated frame before token 0) + fold
    float *S = U;  // forward-sweep state lives in the aliased region, [N][PS]
    for (int e = tid; e < N * P; e += NT) {
        const int n = e / P, p = e % P;
        S[n * PS + p] = a.h0 ? a.h0[(bh * P + p) * N + n] : 0.f;
    }
    for (int i = tid; i < half; i += NT) carry[i] = 0.f;
    const float fold_f = (a.has_prev && L > 0) ? (1.0f - a.lam[bi * L * H + hi]) * a.dt[bi * L * H + hi] : 0.f;
    // previous token's normalised, biased B rows ([R][NS], in dCo) and x rows ([R][PS], in Xs)
    auto prev_rows = [&]() {
        for (int e = tid; e < R * N; e += NT) {
            const int r = e / N, n = e % N;
            dCo[r * NS + n] = ld_io<BF16>(a.Braw_prev, ((bi * G + g) * R + r) * N + n);
        }
        for (int e = tid; e < R * P; e += NT) {
            const int r = e / P, p = e % P;
            Xs[r * PS + p] = ld_io<BF16>(a.x_prev, ((bi * H + hi) * R + r) * P + p);
        }
        __syncthreads();
        for (int grp = tid / 8; grp < R; grp += NT / 8) {
            const int lane8 = tid % 8;
            float ss = 0.f;
            for (int n = lane8; n < N; n += 8) ss += dCo[grp * NS + n] * dCo[grp * NS + n];
            ss = group_sum<8>(ss);
            if (lane8 == 0) rsB[grp] = 1.0f / sqrtf(ss / (float)N + a.eps);
        }
        __syncthreads();
        for (int e = tid; e < R * N; e += NT) {
            const int r = e / N, n = e % N;
            dCo[r * NS + n] = dCo[r * NS + n] * rsB[r] * (wB ? wB[n] : 1.f) + a.B_bias[(hi * R + r) * N + n];
        }
        __syncthreads();
    };
    if (a.has_prev && L > 0) {
        __syncthreads();
        prev_rows();
        for (int e = tid; e < N * P; e += NT) {
            const int n = e / P, p = e % P;
            float acc = 0.f;
            for (int r = 0; r < R; ++r) acc += dCo[r * NS + n] * Xs[r * PS + p];
            S[n * PS + p] += fold_f * acc;
        }
    }
    __syncthreads();

    // ---- forward sweep: checkpoint every chunk's starting state and angle
    for (int k = 0; k < nch; ++k) {
        const int64_t c0 = (int64_t)k * Cb;
        const int nv = (int)((L - c0) < Cb ? (L - c0) : Cb);
        float *slot = chk + (int64_t)k * dm.slot;
        for (int e = tid; e < N * P; e += NT) {
            const int n = fP.q(e);
            slot[e] = S[n * PS + e - n * P];
        }
        for (int i = tid; i < half; i += NT) slot[N * P + i] = carry[i];
        stage_chunk(c0, nv, false);
        const float dec = expf(lcs[nv - 1]);
        for (int e = tid; e < N * (P / 4); e += NT) {
            const int n = fP4.q(e), p = 4 * (e - n * (P / 4));
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int sg = 0; sg < nv * R; ++sg) acc += (Bb[sg * NS + n] * Ew[sg / R]) * ld4(&Xs[sg * PS + p]);
            *reinterpret_cast<f4 *>(&S[n * PS + p]) = dec * ld4(&S[n * PS + p]) + acc;
        }
        for (int i = tid; i < half; i += NT) carry[i] = __builtin_amdgcn_fractf(Phi[(nv - 1) * half + i]);
        __syncthreads();
    }
    {
        float *slot = chk + (int64_t)nch * dm.slot;
        for (int e = tid; e < N * P; e += NT) slot[e] = S[(e / P) * PS + e % P];
        for (int i = tid; i < half; i += NT) slot[N * P + i] = carry[i];
    }

    // ---- reverse sweep: dS = R(-Phi_end) dh_final
    for (int e = tid; e < half * P; e += NT) {
        const int i = e / P, p = e % P;
        float dlo = 0.f, dhi = 0.f;
        if (ba.dh_final) {
            float sn, cs;
            sincospif(2.f * carry[i], &sn, &cs);
            const float hl = ba.dh_final[(bh * P + p) * N + i], hh = ba.dh_final[(bh * P + p) * N + i + half];
            dlo = cs * hl + sn * hh;
            dhi = -sn * hl + cs * hh;
        }
        dS[i * PS + p] = dlo;
        dS[(i + half) * PS + p] = dhi;
    }
    // d Phi_end[i] = sum_p (-dh_lo h_hi + dh_hi h_lo) with h = h_final = R(Phi_end) S_final:
    // one thread per channel pair, fixed order
    for (int i = tid; i < half; i += NT) {
        float rg = 0.f;
        if (ba.dh_final) {
            float sn, cs;
            sincospif(2.f * carry[i], &sn, &cs);
            for (int p = 0; p < P; ++p) {
                const float hl = ba.dh_final[(bh * P + p) * N + i], hh = ba.dh_final[(bh * P + p) * N + i + half];
                const float su = S[i * PS + p], sv = S[(i + half) * PS + p];
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
        for (int i = tid; i < half; i += NT) carry[i] = slot[N * P + i];
        for (int e = tid; e < N * P; e += NT) {
            const int n = fP.q(e);
            U[n * PS + e - n * P] = slot[e];
        }
        stage_chunk(c0, nv, true);
        const float cse = lcs[nv - 1];

        // P2: dC_bar from the carried-state output term; <S_out, dS> partials
        for (int e = tid; e < T * N; e += NT) {
            const int rho = fN.q(e), n = e - rho * N;
            const int t = rho / R;
            float acc = 0.f;
            if (t < nv) {
                for (int p = 0; p < P; p += 4) acc = dot4(ld4(&U[n * PS + p]), ld4(&dYs[rho * PS + p]), acc);
                acc *= ecs[t];
            }
            dCo[rho * NS + n] = acc;
        }
        {
            float part = 0.f;
            for (int e = tid; e < N * P; e += NT) {
                const int n = fP.q(e);
                part += slot1[e] * dS[n * PS + e - n * P];
            }
            red[tid] = part;
        }
        __syncthreads();
        // P3: scores and dy . x (U is free now)
        for (int e = tid; e < T * T; e += NT) {
            const int rho = e / T, sg = e % T;
            const int t = rho / R, s = sg / R;
            float sc = 0.f, dp = 0.f;
            if (s <= t && t < nv) {
                for (int n = 0; n < N; n += 4) sc = dot4(ld4(&Cc[rho * NS + n]), ld4(&Bb[sg * NS + n]), sc);
                for (int p = 0; p < P; p += 4) dp = dot4(ld4(&dYs[rho * PS + p]), ld4(&Xs[sg * PS + p]), dp);
            }
            Sc[e] = sc;
            dP[e] = dp;
        }
        if (tid == 0) {
            float sod = 0.f;
            for (int j = 0; j < NT; ++j) sod += red[j];
            misc[0] = sod;
        }
        __syncthreads();
        // P4: mask entries and their gradients per token pair
        for (int e = tid; e < Cb * Cb; e += NT) {
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
        // fold the mask into the tiles: Sc <- m o Sc (= P), dP <- m o dP (= d S_bar)
        for (int e = tid; e < T * T; e += NT) {
            const float m = Mk[(e / T / R) * Cb + (e % T) / R];
            Sc[e] *= m;
            dP[e] *= m;
        }
        __syncthreads();
        // P5: dx rows (items (sigma, block of 8 p)) and per (token, pair) items
        const int nD = T * npb;
        for (int e = tid; e < nD + Cb * half; e += NT) {
            if (e < nD) {
                const int sg = fP4.q(e), pb = e - sg * npb;  // npb = P / 4
                const int s = sg / R;
                if (s >= nv) {
                    Qp[sg * npb + pb] = 0.f;
                    continue;
                }
                const float Es = Ew[s];
                const int p0 = 4 * pb;  // 4 columns per item
                f4 intra = {0.f, 0.f, 0.f, 0.f}, st = {0.f, 0.f, 0.f, 0.f};
                for (int rho = s * R; rho < nv * R; ++rho)
                    intra += Sc[rho * T + sg] * ld4(&dYs[rho * PS + p0]);
                for (int n = 0; n < N; ++n) st += Bb[sg * NS + n] * ld4(&dS[n * PS + p0]);
                const f4 xv = ld4(&Xs[sg * PS + p0]);
                Qp[sg * npb + pb] = dot4(xv, st, 0.f);
                float *dxo = ba.dx + (((bi * L + c0 + s) * H + hi) * R + sg % R) * P + p0;
                const f4 dxv = intra + Es * st;
                dxo[0] = dxv[0];
                dxo[1] = dxv[1];
                dxo[2] = dxv[2];
                dxo[3] = dxv[3];
            } else {
                const int e2 = e - nD;
                const int t = fH.q(e2), i = e2 - t * half;
                float dphi = 0.f, off = 0.f;
                if (t < nv) {
                    const float Et = Ew[t];
                    float sn, cs;
                    sincospif(2.f * Phi[t * half + i], &sn, &cs);
                    for (int r = 0; r < R; ++r) {
                        const int rho = t * R + r;
                        float dcl = dCo[rho * NS + i], dch = dCo[rho * NS + i + half];
                        off += Cc[rho * NS + i] * dcl + Cc[rho * NS + i + half] * dch;
                        for (int sg = 0; sg < (t + 1) * R; ++sg) {
                            const float f = dP[rho * T + sg];
                            dcl += f * Bb[sg * NS + i];
                            dch += f * Bb[sg * NS + i + half];
                        }
                        float dbl = 0.f, dbh = 0.f;
                        for (int r2 = t * R; r2 < nv * R; ++r2) {
                            const float f = dP[r2 * T + rho];
                            dbl += f * Cc[r2 * NS + i];
                            dbh += f * Cc[r2 * NS + i + half];
                        }
                        float sl = 0.f, sh = 0.f;
                        for (int p = 0; p < P; p += 4) {
                            const f4 xv = ld4(&Xs[rho * PS + p]);
                            sl = dot4(ld4(&dS[i * PS + p]), xv, sl);
                            sh = dot4(ld4(&dS[(i + half) * PS + p]), xv, sh);
                        }
                        dbl += Et * sl;
                        dbh += Et * sh;
                        dphi += dbl * Bb[rho * NS + i + half] - dbh * Bb[rho * NS + i] +
                                dcl * Cc[rho * NS + i + half] - dch * Cc[rho * NS + i];
                        // back to the physical frame: d B = R(Phi) d B_bar
                        const int64_t o = (((bi * L + c0 + t) * H + hi) * R + r) * N;
                        ba.gB[o + i] = cs * dbl - sn * dbh;
                        ba.gB[o + i + half] = sn * dbl + cs * dbh;
                        ba.gC[o + i] = cs * dcl - sn * dch;
                        ba.gC[o + i + half] = sn * dcl + cs * dch;
                    }
                }
                offp[t * HS + i] = off;
                dPh[t * HS + i] = dphi;
            }
        }
        __syncthreads();
        // P6: per-token scalar gradients; suffix sums of d Phi per channel
        for (int j = tid; j < Cb + half; j += NT) {
            if (j < Cb) {
                const int t = j;
                float dc = 0.f, dw = 0.f, dg = 0.f;
                if (t < nv) {
                    float Qt = 0.f;
                    for (int r = 0; r < R; ++r)
                        for (int pb = 0; pb < npb; ++pb) Qt += Qp[(t * R + r) * npb + pb];
                    for (int i = 0; i < half; ++i) dc += offp[t * HS + i];
                    for (int s = 0; s < t; ++s) dc += dMk[t * Cb + s] * Mk[t * Cb + s];
                    for (int t2 = t + 1; t2 < nv; ++t2) {
                        dc -= dMk[t2 * Cb + t] * Mk[t2 * Cb + t];
                        dw += dMk[t2 * Cb + t] * expf(lcs[t2] - lcs[t]);
                    }
                    dc -= Ew[t] * Qt;
                    dw += Ee[t] * Qt;
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
                    rc += dPh[t * HS + i];
                    const int64_t tok = bi * L + c0 + t;
                    ba.gth[(tok * H + hi) * half + i] = dtv[t] * rc;
                    dPh[t * HS + i] = thv[t * half + i] * rc;
                }
                rcar[i] = rc;
            }
        }
        __syncthreads();
        // P7: token records (suffix sums of d cs give d(dt A)); dS back to the chunk start
        for (int t = tid; t < nv; t += NT) {
            float da = 0.f;
            for (int t2 = t; t2 < nv; ++t2) da += dcs[t2];
            float dth = 0.f;
            for (int i = 0; i < half; ++i) dth += dPh[t * HS + i];
            float *rec = ba.tok + ((bi * L + c0 + t) * H + hi) * 4;
            rec[0] = da;
            rec[1] = dwv[t];
            rec[2] = dgv[t];
            rec[3] = dth;
        }
        const float dec = expf(cse);
        for (int e = tid; e < N * (P / 4); e += NT) {
            const int n = fP4.q(e), p = 4 * (e - n * (P / 4));
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int rho = 0; rho < nv * R; ++rho) acc += (ecs[rho / R] * Cc[rho * NS + n]) * ld4(&dYs[rho * PS + p]);
            *reinterpret_cast<f4 *>(&dS[n * PS + p]) = dec * ld4(&dS[n * PS + p]) + acc;
        }
        __syncthreads();
    }

    // ---- chain start: dh0 and the previous token's fold
    if (ba.dh0) {
        for (int e = tid; e < N * P; e += NT) {
            const int p = e / N, n = e % N;
            ba.dh0[(bh * P + p) * N + n] = dS[n * PS + p];
        }
    }
    if (a.has_prev && L > 0) {
        prev_rows();  // dCo <- B_{-1} rows, Xs <- x_{-1} rows
        for (int e = tid; e < R * N; e += NT) {
            const int r = e / N, n = e % N;
            float acc = 0.f;
            for (int p = 0; p < P; ++p) acc += dS[n * PS + p] * Xs[r * PS + p];
            ba.gBp[(bh * R + r) * N + n] = fold_f * acc;
        }
        for (int e = tid; e < R * P; e += NT) {
            const int r = e / P, p = e % P;
            float acc = 0.f;
            for (int n = 0; n < N; ++n) acc += dS[n * PS + p] * dCo[r * NS + n];
            ba.dx_prev[(bh * R + r) * P + p] = fold_f * acc;
        }
        // d f = <dS, sum_r B_{-1}[r] x_{-1}[r]^T>
        float part = 0.f;
        for (int e = tid; e < N * P; e += NT) {
            const int n = e / P, p = e % P;
            float v = 0.f;
            for (int r = 0; r < R; ++r) v += dCo[r * NS + n] * Xs[r * PS + p];
            part += dS[n * PS + p] * v;
        }
        red[tid] = part;
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
            for (int j = 0; j < NT; ++j) s += red[j];
            ba.fold[bh] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core chain kernel for N = 128, P = 64 and R in {1, 2, 4} (32 rows per
// chunk): the same algebra as bwd_chain_kernel, every contraction on
// v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate, so the fp32 bar holds).
// Operand layout: lane l supplies A[i = l%16][k] and B[k][j = l%16]; in a
// 16-wide K block starting at k0, lane group g = l/16 takes k = k0 + 4g + j for
// the block's MFMA j, so a K-contiguous operand row is one 16-byte read and a
// strided one four 4-byte reads. The accumulator holds rows 4g..4g+3 of column
// l%16. The state S (forward sweep) and its adjoint dS (reverse sweep) live in
// accumulators: wave w owns rows n = 16w..16w+15 and all 64 columns p.
namespace mf {
constexpr int N = 128, P = 64, HALF = 64, T = 32;
constexpr int NS = N + 4, PS = P + 4, TS = T + 4;  // 16-byte aligned rows, shifted 4 banks each
constexpr int PHS = HALF + 1;  // per-token angle rows: scans walk lanes over tokens, so rows shift one bank
constexpr int NT = kChainThreads;

__device__ __forceinline__ f4 mfma4(f4 a, f4 b, f4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}
// four strided values at k0 + 4g + j, j = 0..3 (row stride in floats)
__device__ __forceinline__ f4 ld_str(const float *p, int stride) {
    return f4{p[0], p[stride], p[2 * stride], p[3 * stride]};
}
// sum over the 16 lanes of a DPP row; lane 15 of each row ends with the total. Every
// step is one DPP add: no contraction (a caller's product fused into the first step
// took it apart), and the total is formed by every lane (callers keep lane 15's inside
// a branch, into which the last add had been sunk as a move and a separate add).
__device__ __forceinline__ float row_sum16(float v) {
#pragma clang fp contract(off)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
    asm volatile("" : "+v"(v));
    return v;
}

// sine and cosine of an angle given in revolutions, by the hardware v_sin / v_cos
// (which take revolutions) after reducing to [0, 1)
__device__ __forceinline__ void sincos_rev(float x, float *sn, float *cs) {
    const float r = __builtin_amdgcn_fractf(x);
    *sn = __builtin_amdgcn_sinf(r);
    *cs = __builtin_amdgcn_cosf(r);
}

// a value the compiler cannot see through: lane-derived addresses computed from it
// inside the chunk loops are rebuilt each chunk instead of being hoisted and kept
// live (or spilled) across the loop
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int K>
__device__ __forceinline__ float shr(float v) {  // row_shr:K (lanes without a source in their row read 0)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + K, 0xf, 0xf, false));
}
// inclusive prefix sum over aligned groups of G lanes (G in {8, 16, 32}); ln = lane index.
// A row shift gives 0 to the lanes without a source in their 16-lane row, so groups of
// 16 or 32 need no mask and each step is one DPP add; groups of 8 mask the lanes whose
// source lies in the other half of the row. (No contraction: a caller's product fused
// into the first step would take that add apart.)
template <int G>
__device__ __forceinline__ float group_scan(float v, int ln) {
#pragma clang fp contract(off)
    static_assert(G == 8 || G == 16 || G == 32, "groups of 8, 16 or 32 lanes");
    if constexpr (G >= 16) {
        v += shr<1>(v);
        v += shr<2>(v);
        v += shr<4>(v);
        v += shr<8>(v);
    } else {
        const int q = ln & (G - 1);
        float s;
        s = shr<1>(v);
        v += (q >= 1) ? s : 0.f;
        s = shr<2>(v);
        v += (q >= 2) ? s : 0.f;
        s = shr<4>(v);
        v += (q >= 4) ? s : 0.f;
    }
    if constexpr (G >= 32)  // row_bcast:15 into rows 1 and 3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    return v;
}

__host__ __device__ constexpr size_t smem_floats() {
    return (size_t)N * PS            // dSl: dS (reverse) / S (forward set-up), [n][p]
           + 2 * (size_t)T * NS      // Bb, Cc
           + 2 * (size_t)T * PS      // Xs, dYs
           + 2 * (size_t)T * TS      // Sc, dP (mask folded in)
           + 2 * (size_t)T * PHS     // Phi, theta (at most 32 tokens)
           + (size_t)T * (HALF + 1)  // dPh
           + (size_t)T * T           // Mk, dMk (tokens <= 32: two [Cb][Cb] <= 32*32 halves)
           + (size_t)T * T
           + 8 * (size_t)T           // offq [T][4], Qp [T][4]
           + 13 * (size_t)(T + 1)    // token scalars
           + 8 * (size_t)T           // per-wave partial sums of theta * suffix, per token
           + 4 * 2 * (size_t)N + 2 * (size_t)N  // biases [2][R][N] (R <= 4) and gains [2][N]
           + 2 * (size_t)T           // 1/rms rows
           + 2 * (size_t)HALF        // carry, rcar
           + NT + 4
           + 4 * (size_t)NT          // per-lane bias sums [R][NT]
           + 4 * (size_t)T;          // BCNorm: sums of squares of half rows [2][T][2]
}
}  // namespace mf

template <bool BF16, int R>
__global__ __launch_bounds__(kChainThreads) void bwd_chain_mfma_kernel(BwdArgs ba) {
    using namespace mf;
    static_assert(R == 1 || R == 2 || R == 4, "32 rows per chunk");
    constexpr int Cb = T / R;
    const ScanArgs &a = ba.f;
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int lr = l & 15, lg = l >> 4;
    const int64_t bh = blockIdx.x;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int64_t g = hi / (a.H / a.G);
    const int64_t L = a.L, H = a.H, G = a.G;
    const int nch = (int)((L + Cb - 1) / Cb);
    const int64_t slotf = (int64_t)N * P + HALF;
    // chunks this launch sweeps: all of them in one pass, else window ba.win (the
    // forward-only launch, win < 0, sweeps all and keeps every wchunks-th state)
    const bool windowed = ba.wchunks > 0;
    const int nwin = windowed ? (nch + ba.wchunks - 1) / ba.wchunks : 1;
    const bool fwd_only = windowed && ba.win < 0;
    const int kc0 = (windowed && !fwd_only) ? ba.win * ba.wchunks : 0;
    const int kc1 = (windowed && !fwd_only) ? (kc0 + ba.wchunks < nch ? kc0 + ba.wchunks : nch) : nch;
    const bool last_win = !windowed || fwd_only || ba.win == nwin - 1;
    const bool first_win = !windowed || ba.win == 0;

    extern __shared__ float sm[];
    float *dSl = sm;                  // [N][PS]
    float *Bb = dSl + N * PS;         // [T][NS]
    float *Cc = Bb + T * NS;          // [T][NS]
    float *Xs = Cc + T * NS;          // [T][PS]
    float *dYs = Xs + T * PS;         // [T][PS]
    float *Sc = dYs + T * PS;         // [T][TS]
    float *dP = Sc + T * TS;          // [T][TS]
    float *Phi = dP + T * TS;         // [Cb][PHS]
    float *thv = Phi + T * PHS;       // [Cb][PHS]
    float *dPh = thv + T * PHS;       // [Cb][HALF + 1]
    float *Mk = dPh + T * (HALF + 1); // [Cb][Cb]
    float *dMk = Mk + T * T;          // [Cb][Cb]
    float *offq = dMk + T * T;        // [T][4]
    float *Qp = offq + 4 * T;         // [T][4]
    float *dtv = Qp + 4 * T;          // [Cb+1]
    float *lamv = dtv + (T + 1);
    float *Av = lamv + (T + 1);
    float *lcs = Av + (T + 1);
    float *wgt = lcs + (T + 1);
    float *gam = wgt + (T + 1);
    float *ecs = gam + (T + 1);
    float *Ew = ecs + (T + 1);
    float *Ee = Ew + (T + 1);
    float *dcs = Ee + (T + 1);
    float *dwv = dcs + (T + 1);
    float *dgv = dwv + (T + 1);
    float *dcr = dgv + (T + 1);       // [Cb+1] d cs: mask terms (row and column sums)
    float *dthp = dcr + (T + 1);      // [8][T] per-wave partial angle terms of dt
    float *rsB = dthp + 8 * T;        // [T]
    float *rsC = rsB + T;             // [T]
    float *carry = rsC + T;           // [HALF]
    float *rcar = carry + HALF;       // [HALF]
    float *red = rcar + HALF;         // [NT]
    float *misc = red + NT;           // [4]
    float *sbias = misc + 4;          // [2][R][N] B / C bias of this head
    float *sgain = sbias + 8 * N;     // [2][N] BCNorm gains (ones when absent)
    float *sbacc = sgain + 2 * N;     // [R][NT] this lane's bias sums over the chunks done so far
    float *qsq = sbacc + 4 * NT;      // [2][T][2] sums of squares of the half rows of B and C
#pragma unroll
    for (int r = 0; r < R; ++r) sbacc[r * NT + tid] = 0.f;

    // where the forward sweep stores the state before chunk k (k = kc1: after the last
    // chunk), and where the reverse sweep reads it; nullptr: not stored
    float *const chk = ba.chk + bh * (int64_t)((windowed ? nwin : nch) + 1) * slotf;
    float *const chkw = windowed ? ba.chkw + bh * (int64_t)(ba.wchunks + 1) * slotf : nullptr;
    auto fwd_slot = [&](int k) -> float * {
        if (!windowed) return chk + (int64_t)k * slotf;
        if (fwd_only) return (k == nch) ? chk + (int64_t)nwin * slotf
                                        : ((k % ba.wchunks == 0) ? chk + (int64_t)(k / ba.wchunks) * slotf : nullptr);
        return chkw + (int64_t)(k - kc0) * slotf;
    };
    auto rev_slot = [&](int k) -> const float * {
        return windowed ? chkw + (int64_t)(k - kc0) * slotf : chk + (int64_t)k * slotf;
    };
    for (int e = tid; e < 2 * R * N; e += NT) {
        const int which = e / (R * N), rem = e % (R * N);
        sbias[e] = (which == 0 ? a.B_bias : a.C_bias)[hi * R * N + rem];
    }
    for (int e = tid; e < 2 * N; e += NT) {
        const float *src = (e < N) ? a.B_normw : a.C_normw;
        sgain[e] = src ? src[e % N] : 1.f;
    }
    __syncthreads();

    // ---- staging (as in bwd_chain_kernel, with N, P fixed). Every global load of a chunk is
    // issued before any of them is stored to LDS, so the chunk waits for memory once.
    constexpr int KBC = T * N / NT, KXY = T * P / NT, KPH = (T * HALF + NT - 1) / NT;
    struct StageRegs {
        float vb[KBC], vc[KBC], vx[KXY], vy[KXY], vph[KPH], vth[KPH];
        float d, lm, av;
    };
    // loads of a chunk's inputs into registers (they can be in flight during other work)
    auto stage_issue = [&](int64_t c0, int nv, bool withC, StageRegs &sr) {
        {
            // token scalars of threads 0..Cb (clamped indices; zeroed past the chunk)
            const bool okt = tid <= Cb && tid <= nv && c0 + tid < L;
            int64_t tt = c0 + (tid <= Cb ? tid : Cb);
            tt = tt < L ? tt : L - 1;
            const int64_t o = (bi * L + tt) * H + hi;
            const float d = a.dt[o], lm = a.lam[o], av = a.A[o];
            sr.d = okt ? d : 0.f;
            sr.lm = okt ? lm : 0.f;
            sr.av = okt ? av : 0.f;
        }
        // The loads of a thread step through the chunk with a fixed token stride: row
        // rho = rho0 + (NT / N) kk, i.e. token t0 + (NT / N / R) kk, same rank (R divides NT / N).
        // Rows past the chunk's last token read that token's row instead (always in bounds)
        // and are zeroed afterwards: no branch around a load, so the loads stay in flight
        // together instead of each being waited for at the end of its own branch.
        {
            constexpr int DT = NT / N / R;
            const int rho0 = tid / N, n = tid % N, t0 = rho0 / R, r = rho0 % R;
            const int64_t rowb = ((bi * L + c0) * G + g) * R + r;  // row of token 0, rank r
#pragma unroll
            for (int kk = 0; kk < KBC; ++kk) {
                const int t = t0 + DT * kk;
                const bool v_ = t < nv;
                const int64_t o = (rowb + (int64_t)(v_ ? t : nv - 1) * G * R) * N + n;
                const float fb = ld_io<BF16>(a.Braw, o);
                const float fc = withC ? ld_io<BF16>(a.Craw, o) : 0.f;
                sr.vb[kk] = v_ ? fb : 0.f;
                sr.vc[kk] = v_ ? fc : 0.f;
            }
        }
        {
            constexpr int DT = NT / P / R;
            const int rho0 = tid / P, p = tid % P, t0 = rho0 / R, r = rho0 % R;
            const int64_t rowb = ((bi * L + c0) * H + hi) * R + r;
#pragma unroll
            for (int kk = 0; kk < KXY; ++kk) {
                const int t = t0 + DT * kk;
                const bool v_ = t < nv;
                const int64_t o = (rowb + (int64_t)(v_ ? t : nv - 1) * H * R) * P + p;
                const float fx = ld_io<BF16>(a.x, o);
                const float fy = withC ? ld_io<BF16>(ba.dy, o) : 0.f;
                sr.vx[kk] = v_ ? fx : 0.f;
                sr.vy[kk] = v_ ? fy : 0.f;
            }
        }
        {
            constexpr int DT = NT / HALF;
            const int t0 = tid / HALF, i = tid % HALF;
#pragma unroll
            for (int kk = 0; kk < KPH; ++kk) {
                const int t = t0 + DT * kk;
                const bool v_ = t < nv;
                const int64_t tok = bi * L + c0 + (v_ ? t : nv - 1);
                const float th = a.theta[(tok * G + g) * HALF + i];
                const float d = a.dt[tok * H + hi];
                sr.vth[kk] = v_ ? th : 0.f;
                sr.vph[kk] = v_ ? d : 0.f;  // dt of the token (the product is formed when stored)
            }
        }
    };
    // the registers into LDS
    auto stage_put = [&](int nv, const StageRegs &sr, bool withC) {
        if (tid <= Cb) {
            dtv[tid] = sr.d;
            lamv[tid] = sr.lm;
            Av[tid] = sr.av;
        }
        // BCNorm: a wave holds half of one row (N = 128) per kk, so a wave sum of
        // the squares is that half row's share
#pragma unroll
        for (int kk = 0; kk < KBC; ++kk) {
            const int e = tid + kk * NT;
            Bb[(e / N) * NS + e % N] = sr.vb[kk];
            Cc[(e / N) * NS + e % N] = sr.vc[kk];
            const float qb = wave_sum(sr.vb[kk] * sr.vb[kk]);
            const float qc = withC ? wave_sum(sr.vc[kk] * sr.vc[kk]) : 0.f;
            if ((tid & 63) == 0) {
                const int hr = 2 * (e / N) + (e % N) / 64;
                qsq[hr] = qb;
                qsq[2 * T + hr] = qc;
            }
        }
#pragma unroll
        for (int kk = 0; kk < KXY; ++kk) {
            const int e = tid + kk * NT;
            Xs[(e / P) * PS + e % P] = sr.vx[kk];
            dYs[(e / P) * PS + e % P] = sr.vy[kk];
        }
#pragma unroll
        for (int kk = 0; kk < KPH; ++kk) {
            const int e = tid + kk * NT;
            if (e < Cb * HALF) {
                const int eo = (e / HALF) * PHS + e % HALF;
                Phi[eo] = sr.vph[kk] * sr.vth[kk] * kInv2Pi;
                thv[eo] = sr.vth[kk];
            }
        }
    };
    // prefix scans, row norms, rotation (three barriers)
    auto stage_finish = [&](int64_t c0, int nv, bool withC) {
        __syncthreads();
        // decay prefix over the tokens (wave 0, lane t) and angle prefixes (every wave, two
        // channels per pass, lanes 32h + t): DPP scans instead of serial walks
        if (w == 0 && l < 32) {
            const int t = l;
            const bool v_ = t < nv;
            const float run = group_scan<32>(v_ ? dtv[t] * Av[t] : 0.f, l);
            if (t < Cb) {
                const float look = (v_ && c0 + t + 1 < L) ? (1.0f - lamv[t + 1]) * dtv[t + 1] : 0.f;
                lcs[t] = run;
                gam[t] = v_ ? lamv[t] * dtv[t] : 0.f;
                wgt[t] = v_ ? lamv[t] * dtv[t] + look : 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < HALF / 16; ++m) {
            const int i = 8 * w + 2 * m + (l >> 5), t = l & 31;
            float v = (t < nv) ? Phi[t * PHS + i] : 0.f;
            v = group_scan<32>(v, l) + carry[i];
            if (t < nv) Phi[t * PHS + i] = v;
        }
        if (tid < (withC ? 2 * T : T)) {
            const bool isC = tid >= T;
            const int rho = isC ? tid - T : tid;
            const float *q = qsq + (isC ? 2 * T : 0) + 2 * rho;
            (isC ? rsC : rsB)[rho] = 1.0f / sqrtf((q[0] + q[1]) / (float)N + a.eps);
        }
        __syncthreads();
        const float cse = lcs[nv - 1];
        for (int t = tid; t < Cb; t += NT) {
            ecs[t] = expf(lcs[t]);
            Ee[t] = (t < nv) ? expf(cse - lcs[t]) : 0.f;
            Ew[t] = Ee[t] * wgt[t];
        }
        for (int e = tid; e < T * HALF; e += NT) {
            const int rho = e / HALF, i = e % HALF;
            const int t = rho / R, r = rho % R;
            float bl = 0.f, bhv = 0.f, cl = 0.f, chv = 0.f;
            if (t < nv) {
                const float *bb = sbias + r * N;
                float sn, cs;
                sincos_rev(Phi[t * PHS + i], &sn, &cs);
                const float B0 = Bb[rho * NS + i] * rsB[rho] * sgain[i] + bb[i];
                const float B1 = Bb[rho * NS + i + HALF] * rsB[rho] * sgain[i + HALF] + bb[i + HALF];
                bl = cs * B0 + sn * B1;
                bhv = -sn * B0 + cs * B1;
                if (withC) {
                    const float *cb = sbias + (R + r) * N;
                    const float C0 = Cc[rho * NS + i] * rsC[rho] * sgain[N + i] + cb[i];
                    const float C1 = Cc[rho * NS + i + HALF] * rsC[rho] * sgain[N + i + HALF] + cb[i + HALF];
                    cl = cs * C0 + sn * C1;
                    chv = -sn * C0 + cs * C1;
                }
            }
            Bb[rho * NS + i] = bl;
            Bb[rho * NS + i + HALF] = bhv;
            Cc[rho * NS + i] = cl;
            Cc[rho * NS + i + HALF] = chv;
        }
        __syncthreads();
    };
    auto stage_chunk = [&](int64_t c0, int nv, bool withC) {
        StageRegs sr;
        stage_issue(c0, nv, withC, sr);
        stage_put(nv, sr, withC);
        stage_finish(c0, nv, withC);
    };

    // previous token's normalised, biased B rows ([R][NS] in Sc) and x rows ([R][PS] in dP)
    float *pB = Sc, *pX = dP;
    auto prev_rows = [&]() {
        for (int e = tid; e < R * N; e += NT) {
            const int r = e / N, n = e % N;
            pB[r * NS + n] = ld_io<BF16>(a.Braw_prev, ((bi * G + g) * R + r) * N + n);
        }
        for (int e = tid; e < R * P; e += NT) {
            const int r = e / P, p = e % P;
            pX[r * PS + p] = ld_io<BF16>(a.x_prev, ((bi * H + hi) * R + r) * P + p);
        }
        __syncthreads();
        for (int grp = tid / 8; grp < R; grp += NT / 8) {
            const int lane8 = tid % 8;
            float ss = 0.f;
            for (int n = lane8; n < N; n += 8) ss += pB[grp * NS + n] * pB[grp * NS + n];
            ss = group_sum<8>(ss);
            if (lane8 == 0) rsB[grp] = 1.0f / sqrtf(ss / (float)N + a.eps);
        }
        __syncthreads();
        for (int e = tid; e < R * N; e += NT) {
            const int r = e / N, n = e % N;
            pB[r * NS + n] = pB[r * NS + n] * rsB[r] * sgain[n] + sbias[r * N + n];
        }
        __syncthreads();
    };

    // ---- initial state into LDS, then into the accumulators (rows 16w + 4lg + jj, column 16pt + lr):
    // h0 with the previous token's fold, or a window's checkpoint
    const float fold_f = (a.has_prev && L > 0) ? (1.0f - a.lam[bi * L * H + hi]) * a.dt[bi * L * H + hi] : 0.f;
    if (windowed && !fwd_only) {
        const float *s0 = chk + (int64_t)ba.win * slotf;
        for (int e = tid; e < N * P; e += NT) dSl[(e / P) * PS + e % P] = s0[e];
        for (int i = tid; i < HALF; i += NT) carry[i] = s0[N * P + i];
    } else {
        for (int e = tid; e < N * P; e += NT) {
            const int p = e / N, n = e % N;  // coalesced over h0's n
            dSl[n * PS + p] = a.h0 ? a.h0[(bh * P + p) * N + n] : 0.f;
        }
        for (int i = tid; i < HALF; i += NT) carry[i] = 0.f;
        if (a.has_prev && L > 0) {
            __syncthreads();
            prev_rows();
            for (int e = tid; e < N * P; e += NT) {
                const int n = e / P, p = e % P;
                float acc = 0.f;
                for (int r = 0; r < R; ++r) acc += pB[r * NS + n] * pX[r * PS + p];
                dSl[n * PS + p] += fold_f * acc;
            }
        }
    }
    __syncthreads();
    f4 acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[pt][jj] = dSl[(16 * w + 4 * lg + jj) * PS + 16 * pt + lr];

    // ---- forward sweep (each chunk's inputs are loaded during the previous chunk)
    StageRegs fsr;
    if (kc0 < kc1) {
        const int64_t cf = (int64_t)kc0 * Cb;
        stage_issue(cf, (int)((L - cf) < Cb ? (L - cf) : Cb), false, fsr);
    }
    for (int k = kc0; k < kc1; ++k) {
        const int l = opaque(tid & 63), lr = l & 15, lg = l >> 4;
        const int64_t c0 = (int64_t)k * Cb;
        const int nv = (int)((L - c0) < Cb ? (L - c0) : Cb);
        float *slot = fwd_slot(k);
        stage_put(nv, fsr, false);
        if (k + 1 < kc1) {
            const int64_t c1 = c0 + Cb;
            stage_issue(c1, (int)((L - c1) < Cb ? (L - c1) : Cb), false, fsr);
        }
        if (slot) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) slot[(16 * w + 4 * lg + jj) * P + 16 * pt + lr] = acc[pt][jj];
            for (int i = tid; i < HALF; i += NT) slot[N * P + i] = carry[i];
        }
        stage_finish(c0, nv, false);
        // S <- e^{cs_end} S + sum_sigma (E B_bar)^T x: A[n][sigma] = E_s B_bar[sigma][n], B[sigma][p] = x
        const float dec = expf(lcs[nv - 1]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] *= dec;
#pragma unroll
        for (int k0 = 0; k0 < T; k0 += 16) {
            const int kk = k0 + 4 * lg;
            f4 av = ld_str(&Bb[kk * NS + 16 * w + lr], NS);
#pragma unroll
            for (int j = 0; j < 4; ++j) av[j] *= Ew[(kk + j) / R];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma4(av, ld_str(&Xs[kk * PS + 16 * pt + lr], PS), acc[pt]);
        }
        for (int i = tid; i < HALF; i += NT) carry[i] = __builtin_amdgcn_fractf(Phi[(nv - 1) * PHS + i]);
        __syncthreads();
    }
    {
        float *slot = fwd_slot(kc1);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                slot[(16 * w + 4 * lg + jj) * P + 16 * pt + lr] = acc[pt][jj];
                dSl[(16 * w + 4 * lg + jj) * PS + 16 * pt + lr] = acc[pt][jj];  // S_final (last window)
            }
        for (int i = tid; i < HALF; i += NT) slot[N * P + i] = carry[i];
    }
    __syncthreads();
    if (fwd_only) return;
    constexpr int64_t rstf = (int64_t)N * P + HALF + 4 * NT;  // dS, angle-gradient carry, bias sums
    if (!last_win) {
        // a later window's reverse sweep left dS, the angle-gradient carry and the bias sums
        const float *rs = ba.rst + bh * rstf;
        for (int e = tid; e < N * P; e += NT) dSl[(e / P) * PS + e % P] = rs[e];
        for (int i = tid; i < HALF; i += NT) rcar[i] = rs[N * P + i];
#pragma unroll
        for (int r = 0; r < R; ++r) sbacc[r * NT + tid] = rs[N * P + HALF + r * NT + tid];
    }
    // ---- d Phi_end[i] = sum_p (-dh_lo h_hi + dh_hi h_lo), h = R(Phi_end) S_final
    for (int i = tid; last_win && i < HALF; i += NT) {
        float rg = 0.f;
        if (ba.dh_final) {
            float sn, cs;
            sincos_rev(carry[i], &sn, &cs);
            for (int p = 0; p < P; ++p) {
                const float hl = ba.dh_final[(bh * P + p) * N + i], hh = ba.dh_final[(bh * P + p) * N + i + HALF];
                const float su = dSl[i * PS + p], sv = dSl[(i + HALF) * PS + p];
                rg += -hl * (sn * su + cs * sv) + hh * (cs * su - sn * sv);
            }
        }
        rcar[i] = rg;
    }
    __syncthreads();
    // dS = R(-Phi_end) dh_final
    for (int e = tid; last_win && e < HALF * P; e += NT) {
        const int p = e / HALF, i = e % HALF;
        float dlo = 0.f, dhi = 0.f;
        if (ba.dh_final) {
            float sn, cs;
            sincos_rev(carry[i], &sn, &cs);
            const float hl = ba.dh_final[(bh * P + p) * N + i], hh = ba.dh_final[(bh * P + p) * N + i + HALF];
            dlo = cs * hl + sn * hh;
            dhi = -sn * hl + cs * hh;
        }
        dSl[i * PS + p] = dlo;
        dSl[(i + HALF) * PS + p] = dhi;
    }
    __syncthreads();
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[pt][jj] = dSl[(16 * w + 4 * lg + jj) * PS + 16 * pt + lr];

    // wave roles for the [T][N] tiles: rows 16*rt.., columns 16*nt0.. and 16*(nt0+4).. (a rotation pair)
    const int rt = w >> 2, nt0 = w & 3;
    // S_out of the chunk being processed, in the fragment layout of (1): rows n = 16 (nt0 + 4q) + lr,
    // columns p = 16 kb + 4 lg + j. The first is S_final; after that, the previous chunk's S_in.
    f4 uprev[2][4];
    {
        const float *slotf_ = rev_slot(kc1);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                uprev[q][kb] = *reinterpret_cast<const f4 *>(&slotf_[(16 * (nt0 + 4 * q) + lr) * P + 16 * kb + 4 * lg]);
    }
    // (reverse chunks are staged in place: holding the next chunk's loads across
    // steps 6 and 7 cost 33-55 spilled registers and ran slower)
    StageRegs rsr;
    for (int k = kc1 - 1; k >= kc0; --k) {
        const int l = opaque(tid & 63), lr = l & 15, lg = l >> 4;
        const int64_t c0 = (int64_t)k * Cb;
        const int nv = (int)((L - c0) < Cb ? (L - c0) : Cb);
        const float *slot = rev_slot(k);
        // S_in fragments of (1), in flight during the staging
        f4 uin[2][4];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                uin[q][kb] = *reinterpret_cast<const f4 *>(&slot[(16 * (nt0 + 4 * q) + lr) * P + 16 * kb + 4 * lg]);
        // the chunk's starting angle carry: loaded with the staging loads below and
        // stored with them (a load-then-store here had cost its own memory round trip)
        const float carry_in = slot[N * P + (tid < HALF ? tid : 0)];
        // <S_out, dS>: S_out fragments in registers, dS in LDS (waves 4..7 hold the same fragments)
        {
            float part = 0.f;
            if (rt == 0) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
                        part = dot4(uprev[q][kb], ld4(&dSl[(16 * (nt0 + 4 * q) + lr) * PS + 16 * kb + 4 * lg]), part);
            }
            part = wave_sum(part);
            if (l == 0) red[w] = part;
        }
        stage_issue(c0, nv, true, rsr);
        stage_put(nv, rsr, true);
        if (tid < HALF) carry[tid] = carry_in;
        stage_finish(c0, nv, true);
        const float cse = lcs[nv - 1];

        // (1) dC_bar from the carried-state output term: e^{cs_t} sum_p dY[rho][p] S_in[n][p]
        f4 dC[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int nt = nt0 + 4 * q;
            f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) c = mfma4(ld4(&dYs[(16 * rt + lr) * PS + 16 * kb + 4 * lg]), uin[q][kb], c);
            (void)nt;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) c[jj] *= ecs[(16 * rt + 4 * lg + jj) / R];
            dC[q] = c;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) uprev[q][kb] = uin[q][kb];
        __builtin_amdgcn_sched_barrier(0);
        // off-term part of d cs: sum_n C_bar[rho][n] dCoff[rho][n], per row, this wave's 32 columns
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int rho = 16 * rt + 4 * lg + jj;
            float v = Cc[rho * NS + 16 * nt0 + lr] * dC[0][jj] + Cc[rho * NS + 16 * (nt0 + 4) + lr] * dC[1][jj];
            v = row_sum16(v);
            if (lr == 15) offq[rho * 4 + nt0] = v;
        }
        __builtin_amdgcn_sched_barrier(0);
        // (2) scores and dy . x on waves 0..5: tiles (0,0), (1,0), (1,1)
        if (w < 6) {
            const int tix = (w < 3) ? w : w - 3;
            const int ta = (tix == 0) ? 0 : 1, tb = (tix == 2) ? 1 : 0;
            f4 c = {0.f, 0.f, 0.f, 0.f};
            if (w < 3) {
#pragma unroll 2
                for (int k0 = 0; k0 < N; k0 += 16)
                    c = mfma4(ld4(&Cc[(16 * ta + lr) * NS + k0 + 4 * lg]), ld4(&Bb[(16 * tb + lr) * NS + k0 + 4 * lg]), c);
            } else {
#pragma unroll 2
                for (int k0 = 0; k0 < P; k0 += 16)
                    c = mfma4(ld4(&dYs[(16 * ta + lr) * PS + k0 + 4 * lg]), ld4(&Xs[(16 * tb + lr) * PS + k0 + 4 * lg]), c);
            }
            float *dst = (w < 3) ? Sc : dP;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dst[(16 * ta + 4 * lg + jj) * TS + 16 * tb + lr] = c[jj];
        } else {
            // the tile above the diagonal is zero
            for (int e = tid - 384; e < 256; e += 128) {
                const int rr = e / 16, cc = e % 16;
                Sc[rr * TS + 16 + cc] = 0.f;
                dP[rr * TS + 16 + cc] = 0.f;
            }
        }
        if (tid == 0) {
            float sod = 0.f;
            for (int j = 0; j < NT / 64; ++j) sod += red[j];
            misc[0] = sod;
        }
        __syncthreads();
        // (3) mask per token pair m(t,s) and its gradient dm = sum over the rank block of dP Sc;
        //     the gradient's sums go straight to the tokens (groups of Cb lanes hold one row, or
        //     one column): d cs_t += sum_{s<t} dm m - sum_{t2>t} dm(t2,t) m(t2,t),
        //     dw_t = sum_{t2>t} dm(t2,t) e^{cs_t2 - cs_t}, dgamma_t = dm(t,t)
        auto mask_at = [&](int t, int s, float &m, float &dmv) {
            m = 0.f;
            dmv = 0.f;
            if (s <= t && t < nv) {
                m = (s == t) ? gam[t] : expf(lcs[t] - lcs[s]) * wgt[s];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int r2 = 0; r2 < R; ++r2) {
                        const int idx = (t * R + r) * TS + s * R + r2;
                        dmv += dP[idx] * Sc[idx];
                    }
            }
        };
        for (int e = tid; e < Cb * Cb; e += NT) {  // rows: lane s of the group
            const int t = e / Cb, s = e % Cb;
            float m, dmv;
            mask_at(t, s, m, dmv);
            Mk[e] = m;
            dMk[e] = dmv;
            const float rs_ = group_sum<Cb>((s < t) ? dmv * m : 0.f);
            if (s == 0) dcr[t] = rs_;
            if (s == t) dgv[t] = dmv;
        }
        for (int e = tid; e < Cb * Cb; e += NT) {  // columns: lane t2 of the group
            const int t = e / Cb, t2 = e % Cb;
            float m, dmv;
            mask_at(t2, t, m, dmv);
            const bool after = t2 > t;
            const float cc = group_sum<Cb>(after ? -dmv * m : 0.f);
            const float cw = group_sum<Cb>(after ? dmv * expf(lcs[t2] - lcs[t]) : 0.f);
            if (t2 == 0) {
                dcs[t] = cc;
                dwv[t] = cw;
            }
        }
        __syncthreads();
        for (int e = tid; e < T * T; e += NT) {
            const int rho = e / T, sg = e % T;
            const float m = Mk[(rho / R) * Cb + sg / R];
            Sc[rho * TS + sg] *= m;
            dP[rho * TS + sg] *= m;
        }
        __syncthreads();
        // (4) dx tile (rows sigma 16*st.., columns 16*pt..): intra sum_rho MSc[rho][sigma] dY[rho][p]
        //     + E_sigma sum_n B_bar[sigma][n] dS[n][p]; Q_sigma partial = sum_p x[sigma][p] (state part)
        {
            const int st = w >> 2, pt = w & 3;
            f4 ci = {0.f, 0.f, 0.f, 0.f}, cs_ = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 16 * st; k0 < T; k0 += 16) {
                const int kk = k0 + 4 * lg;
                ci = mfma4(ld_str(&Sc[kk * TS + 16 * st + lr], TS), ld_str(&dYs[kk * PS + 16 * pt + lr], PS), ci);
            }
#pragma unroll 2
            for (int k0 = 0; k0 < N; k0 += 16) {
                const int kk = k0 + 4 * lg;
                cs_ = mfma4(ld4(&Bb[(16 * st + lr) * NS + kk]), ld_str(&dSl[kk * PS + 16 * pt + lr], PS), cs_);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int sg = 16 * st + 4 * lg + jj, s = sg / R;
                const float q = row_sum16(Xs[sg * PS + 16 * pt + lr] * cs_[jj]);
                if (lr == 15) Qp[sg * 4 + pt] = q;
                if (s < nv)
                    ba.dx[(((bi * L + c0 + s) * H + hi) * R + sg % R) * P + 16 * pt + lr] = ci[jj] + Ew[s] * cs_[jj];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (5) dC_bar += MdP B_bar, dB_bar = MdP^T C_bar + E_sigma x dS^T, for the column pair
        {
            f4 dB[2], dBs[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int nt = nt0 + 4 * q;
                f4 c = dC[q], b = {0.f, 0.f, 0.f, 0.f}, bs = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < 16 * (rt + 1); k0 += 16) {  // sigma <= rho
                    const int kk = k0 + 4 * lg;
                    c = mfma4(ld4(&dP[(16 * rt + lr) * TS + kk]), ld_str(&Bb[kk * NS + 16 * nt + lr], NS), c);
                }
                for (int k0 = 16 * rt; k0 < T; k0 += 16) {  // rho >= sigma
                    const int kk = k0 + 4 * lg;
                    b = mfma4(ld_str(&dP[kk * TS + 16 * rt + lr], TS), ld_str(&Cc[kk * NS + 16 * nt + lr], NS), b);
                }
#pragma unroll 2
                for (int k0 = 0; k0 < P; k0 += 16) {
                    const int kk = k0 + 4 * lg;
                    bs = mfma4(ld4(&Xs[(16 * rt + lr) * PS + kk]), ld4(&dSl[(16 * nt + lr) * PS + kk]), bs);
                }
                dC[q] = c;
                dB[q] = b;
                dBs[q] = bs;
            }
            const int i = 16 * nt0 + lr;  // channel of the pair (i, i + 64)
            float dphi_tok[4] = {0.f, 0.f, 0.f, 0.f};
            float bsum[R][4] = {};  // per rank (rho % R == jj % R): B lo, B hi, C lo, C hi
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rho = 16 * rt + 4 * lg + jj, t = rho / R, r = rho % R;
                const float E = Ew[t];
                const float dbl = dB[0][jj] + E * dBs[0][jj], dbh = dB[1][jj] + E * dBs[1][jj];
                const float dcl = dC[0][jj], dch = dC[1][jj];
                dphi_tok[jj] = dbl * Bb[rho * NS + i + HALF] - dbh * Bb[rho * NS + i] + dcl * Cc[rho * NS + i + HALF] -
                               dch * Cc[rho * NS + i];
                if (t < nv) {
                    float sn, cs;
                    sincos_rev(Phi[t * PHS + i], &sn, &cs);
                    const int64_t o = (((bi * ba.Lb + c0 + t - ba.tbase) * H + hi) * R + r) * N;
                    const float gbl = cs * dbl - sn * dbh, gbh = sn * dbl + cs * dbh;
                    const float gcl = cs * dcl - sn * dch, gch = sn * dcl + cs * dch;
                    ba.gB[o + i] = gbl;
                    ba.gB[o + i + HALF] = gbh;
                    ba.gC[o + i] = gcl;
                    ba.gC[o + i + HALF] = gch;
                    bsum[jj % R][0] += gbl;
                    bsum[jj % R][1] += gbh;
                    bsum[jj % R][2] += gcl;
                    bsum[jj % R][3] += gch;
                }
            }
            // bias sums: the four lane groups of the wave hold the same channels on
            // different rows; a reduce-scatter over them leaves component lg (B lo,
            // B hi, C lo, C hi) summed over the wave's 16 rows in lane group lg
            {
                const bool hi2 = (lg & 2) != 0, lo1 = (lg & 1) != 0;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float k0 = (hi2 ? bsum[r][2] : bsum[r][0]) + __shfl_xor(hi2 ? bsum[r][0] : bsum[r][2], 32);
                    const float k1 = (hi2 ? bsum[r][3] : bsum[r][1]) + __shfl_xor(hi2 ? bsum[r][1] : bsum[r][3], 32);
                    sbacc[r * NT + tid] += (lo1 ? k1 : k0) + __shfl_xor(lo1 ? k0 : k1, 16);
                }
            }
            // the lane's 4 rows are 4/R whole tokens: sum the ranks of each token
#pragma unroll
            for (int u = 0; u < 4 / R; ++u) {
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) v += dphi_tok[u * R + r];
                dPh[((16 * rt + 4 * lg) / R + u) * (HALF + 1) + i] = v;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (6) dS <- e^{cs_end} dS + sum_rho e^{cs_t} C_bar[rho]^T dY[rho] (accumulators; the LDS copy is
        //     still read above by other waves, so it is rewritten after the barrier)
        {
            const float dec = expf(cse);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc[pt] *= dec;
#pragma unroll
            for (int k0 = 0; k0 < T; k0 += 16) {
                const int kk = k0 + 4 * lg;
                const f4 av = ld_str(&Cc[kk * NS + 16 * w + lr], NS);
                f4 sc4;
#pragma unroll
                for (int j = 0; j < 4; ++j) sc4[j] = ecs[(kk + j) / R];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma4(av, ld_str(&dYs[kk * PS + 16 * pt + lr], PS) * sc4, acc[pt]);
            }
        }
        __syncthreads();
        // (7) token scalars, suffix sums of d Phi, and the new dS into LDS
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dSl[(16 * w + 4 * lg + jj) * PS + 16 * pt + lr] = acc[pt][jj];
        // angle gradients: per channel, the suffix over the chunk's tokens (lanes 32h + t) plus the
        // carry from later chunks; d theta = dt * suffix; the dt term sum_i theta * suffix per token
        {
            float dth_acc = 0.f;
#pragma unroll
            for (int m = 0; m < HALF / 16; ++m) {
                const int i = 8 * w + 2 * m + (l >> 5), t = l & 31;
                const bool v_ = t < nv;
                const float d = v_ ? dPh[t * (HALF + 1) + i] : 0.f;
                const float incl = group_scan<32>(d, l);
                const float tot = group_sum<32>(d);
                const float rc = rcar[i] + tot - incl + d;  // sum over tokens >= t
                if (v_) {
                    const int64_t tokp = bi * ba.Lb + c0 + t - ba.tbase;
                    ba.gth[(tokp * H + hi) * HALF + i] = dtv[t] * rc;
                    dth_acc += thv[t * PHS + i] * rc;
                }
                if (t == 0) rcar[i] += tot;
            }
            // lanes t and 32 + t hold different channels of the same token
            const float other = __shfl_xor(dth_acc, 32);
            if (l < 32) dthp[w * T + l] = dth_acc + other;
        }
        __syncthreads();
        // token scalars and records: wave 0, lane t; suffix sums of d cs in registers
        if (w == 0 && l < 32) {
            const int t = l;
            const bool v_ = t < nv;
            float dc = 0.f, dw = 0.f, dg = 0.f, dth = 0.f;
            if (v_) {
                float Qt = 0.f, off = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        Qt += Qp[(t * R + r) * 4 + q];
                        off += offq[(t * R + r) * 4 + q];
                    }
                dc = off + dcr[t] + dcs[t] - Ew[t] * Qt;
                if (t == nv - 1) dc += misc[0];
                dw = dwv[t] + Ee[t] * Qt;
                dg = dgv[t];
#pragma unroll
                for (int ww = 0; ww < 8; ++ww) dth += dthp[ww * T + t];
            }
            const float incl = group_scan<32>(dc, l);
            const float da = group_sum<32>(dc) - incl + dc;  // sum over tokens >= t
            if (v_) {
                float *rec = ba.tok + ((bi * L + c0 + t) * H + hi) * 4;
                rec[0] = da;
                rec[1] = dw;
                rec[2] = dg;
                rec[3] = dth;
            }
        }
    }

    if (!first_win) {
        // dS, the angle-gradient carry and the bias sums go to the previous window
        float *rs = ba.rst + bh * rstf;
        for (int e = tid; e < N * P; e += NT) rs[e] = dSl[(e / P) * PS + e % P];
        for (int i = tid; i < HALF; i += NT) rs[N * P + i] = rcar[i];
#pragma unroll
        for (int r = 0; r < R; ++r) rs[N * P + HALF + r * NT + tid] = sbacc[r * NT + tid];
        return;
    }
    // the chain's bias sums: lane group lg of wave w holds component lg of row tile
    // rt over channel 16 nt0 + lr (+ 64 for the high halves)
    {
        const int n = 16 * nt0 + lr + HALF * (lg & 1);
#pragma unroll
        for (int r = 0; r < R; ++r)
            ba.bpart[(((bh * 2 + rt) * R + r) * 2 + (lg >> 1)) * N + n] = sbacc[r * NT + tid];
    }

    // ---- chain start: dh0 and the previous token's fold (dS is in dSl)
    if (ba.dh0) {
        for (int e = tid; e < N * P; e += NT) {
            const int p = e / N, n = e % N;
            ba.dh0[(bh * P + p) * N + n] = dSl[n * PS + p];
        }
    }
    if (a.has_prev && L > 0) {
        prev_rows();
        for (int e = tid; e < R * N; e += NT) {
            const int r = e / N, n = e % N;
            float s = 0.f;
            for (int p = 0; p < P; ++p) s += dSl[n * PS + p] * pX[r * PS + p];
            ba.gBp[(bh * R + r) * N + n] = fold_f * s;
        }
        for (int e = tid; e < R * P; e += NT) {
            const int r = e / P, p = e % P;
            float s = 0.f;
            for (int n = 0; n < N; ++n) s += dSl[n * PS + p] * pB[r * NS + n];
            ba.dx_prev[(bh * R + r) * P + p] = fold_f * s;
        }
        float part = 0.f;
        for (int e = tid; e < N * P; e += NT) {
            const int n = e / P, p = e % P;
            float v = 0.f;
            for (int r = 0; r < R; ++r) v += pB[r * NS + n] * pX[r * PS + p];
            part += dSl[n * PS + p] * v;
        }
        red[tid] = part;
        __syncthreads();
        if (tid == 0) {
            float s = 0.f;
            for (int j = 0; j < NT; ++j) s += red[j];
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
// BCNorm's backward per raw row ((batch, token), group, rank), one wave per row and
// two adjacent channels per lane: dB and dC are first summed over the heads of the
// group (eight heads of loads in flight per lane), then
//   d Braw = rs w dB - Braw rs^3 / N * sum_n(Braw w dB),   rs = 1 / sqrt(mean(Braw^2) + eps)
// and the gain term Braw rs dB is kept per row for the column sums. The previous
// token's rows (prev) read the per-head fold rows instead and have no C part.
// Rows of the sequence are those of tokens tbase .. tbase + nt - 1 of every batch (all
// tokens in one pass, a window's under the low-memory schedule); the per-head rows are
// the window's (ba.Lb per batch), the raw rows and the outputs the sequence's.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void bwd_group_kernel(BwdArgs ba, bool prev, int64_t nrows, int64_t nt,
                                                             float *gWB, float *gWC, float *dBraw_out,
                                                             float *dCraw_out) {
    const ScanArgs &a = ba.f;
    const int N = (int)a.N;
    const int64_t R = a.R, H = a.H, G = a.G, hpg = H / G;
    const int64_t wrow = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wrow >= nrows) return;  // a whole wave; the kernel has no barrier
    const int l = threadIdx.x & 63;
    const int64_t r = wrow % R, bg = wrow / R, g = bg % G, btw = bg / G;
    // (batch, token) of the per-head rows and of the sequence
    const int64_t bt = prev ? btw : (btw / nt) * ba.Lb + btw % nt;
    const int64_t row = prev ? wrow : (((btw / nt) * a.L + ba.tbase + btw % nt) * G + g) * R + r;
    const int n = 2 * l;
    const bool on = n < N;  // N is even
    const int nc = on ? n : 0;
    const int64_t h0 = ((bt * H + g * hpg) * R + r) * N + nc, hstride = R * N;
    const float *pB = (prev ? ba.gBp : ba.gB) + h0;
    const float *pC = ba.gC + h0;
    float2 sb = {0.f, 0.f}, sc = {0.f, 0.f};
    int64_t h = 0;
    for (; h + 8 <= hpg; h += 8) {
        float2 vb[8], vc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            vb[k] = *reinterpret_cast<const float2 *>(pB + (h + k) * hstride);
            if (!prev) vc[k] = *reinterpret_cast<const float2 *>(pC + (h + k) * hstride);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            sb.x += vb[k].x;
            sb.y += vb[k].y;
            if (!prev) {
                sc.x += vc[k].x;
                sc.y += vc[k].y;
            }
        }
    }
    for (; h < hpg; ++h) {
        const float2 vb = *reinterpret_cast<const float2 *>(pB + h * hstride);
        sb.x += vb.x;
        sb.y += vb.y;
        if (!prev) {
            const float2 vc = *reinterpret_cast<const float2 *>(pC + h * hstride);
            sc.x += vc.x;
            sc.y += vc.y;
        }
    }
    const int64_t raw = row * N + nc;
    const void *Bsrc = prev ? a.Braw_prev : a.Braw;
    const float b0 = on ? ld_io<BF16>(Bsrc, raw) : 0.f, b1 = on ? ld_io<BF16>(Bsrc, raw + 1) : 0.f;
    const float wb0 = a.B_normw ? a.B_normw[nc] : 1.f, wb1 = a.B_normw ? a.B_normw[nc + 1] : 1.f;
    const float rsb = 1.0f / sqrtf(wave_sum(b0 * b0 + b1 * b1) / (float)N + a.eps);
    const float kb = wave_sum(b0 * wb0 * sb.x + b1 * wb1 * sb.y) * rsb * rsb * rsb / (float)N;
    float c0 = 0.f, c1 = 0.f, wc0 = 1.f, wc1 = 1.f, rsc = 0.f, kc = 0.f;
    if (!prev) {
        c0 = on ? ld_io<BF16>(a.Craw, raw) : 0.f;
        c1 = on ? ld_io<BF16>(a.Craw, raw + 1) : 0.f;
        wc0 = a.C_normw ? a.C_normw[nc] : 1.f;
        wc1 = a.C_normw ? a.C_normw[nc + 1] : 1.f;
        rsc = 1.0f / sqrtf(wave_sum(c0 * c0 + c1 * c1) / (float)N + a.eps);
        kc = wave_sum(c0 * wc0 * sc.x + c1 * wc1 * sc.y) * rsc * rsc * rsc / (float)N;
    }
    if (!on) return;
    *reinterpret_cast<float2 *>(dBraw_out + raw) = float2{rsb * wb0 * sb.x - b0 * kb, rsb * wb1 * sb.y - b1 * kb};
    *reinterpret_cast<float2 *>(gWB + raw) = float2{b0 * rsb * sb.x, b1 * rsb * sb.y};
    if (!prev) {
        *reinterpret_cast<float2 *>(dCraw_out + raw) = float2{rsc * wc0 * sc.x - c0 * kc, rsc * wc1 * sc.y - c1 * kc};
        *reinterpret_cast<float2 *>(gWC + raw) = float2{c0 * rsc * sc.x, c1 * rsc * sc.y};
    }
}

// d theta[b,t,g,i] = sum over the heads of group g of the per-head terms, for tokens
// tbase .. tbase + nt - 1 of every batch (per-head rows as in bwd_group_kernel)
__global__ __launch_bounds__(kThreads) void bwd_theta_kernel(BwdArgs ba, int64_t nt, float *dtheta) {
    const ScanArgs &a = ba.f;
    const int64_t half = a.N / 2, H = a.H, G = a.G, hpg = H / G;
    const int64_t total = a.b * nt * G * half;
    for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < total; e += (int64_t)gridDim.x * kThreads) {
        const int64_t i = e % half, g = (e / half) % G, btw = e / (half * G);
        const int64_t bt = (btw / nt) * ba.Lb + btw % nt;
        const int64_t out = ((((btw / nt) * a.L + ba.tbase + btw % nt) * G + g) * half) + i;
        const float *src = ba.gth + (bt * H + g * hpg) * half + i;
        float s = 0.f;
        int64_t h = 0;
        for (; h + 8 <= hpg; h += 8) {  // eight heads of loads in flight, summed in order
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = src[(h + k) * half];
#pragma unroll
            for (int k = 0; k < 8; ++k) s += v[k];
        }
        for (; h < hpg; ++h) s += src[h * half];
        dtheta[out] = s;
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

// Bias gradients from the matrix-core chain kernel's per-chain sums:
//   d bias[h][r][n] = sum over batches of both row tiles' sums (B and C), plus the
//   previous token's per-head rows for B; a fixed order, so the result is deterministic.
__global__ __launch_bounds__(kThreads) void bwd_bias_kernel(BwdArgs ba, bool prev, float *dB_bias, float *dC_bias) {
    const ScanArgs &a = ba.f;
    const int64_t R = a.R, N = a.N, H = a.H, cols = H * R * N;
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= 2 * cols) return;
    const int64_t arr = e / cols, c = e % cols;  // c = (h R + r) N + n
    const int64_t n = c % N, h = c / (R * N), r = (c / N) % R;
    float s = 0.f;
    for (int64_t b = 0; b < a.b; ++b) {
        for (int rt = 0; rt < 2; ++rt) s += ba.bpart[((((b * H + h) * 2 + rt) * R + r) * 2 + arr) * N + n];
        if (arr == 0 && prev) s += ba.gBp[c + b * cols];
    }
    (arr ? dC_bias : dB_bias)[c] = s;
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

template <int R, int NF, int PF>
hipError_t launch_chain_np(const BwdArgs &ba, int64_t chains, size_t smem, hipStream_t st) {
    const void *fn = ba.f.bf16 ? (const void *)bwd_chain_kernel<true, R, NF, PF>
                               : (const void *)bwd_chain_kernel<false, R, NF, PF>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    if (ba.f.bf16)
        hipLaunchKernelGGL((bwd_chain_kernel<true, R, NF, PF>), dim3((unsigned)chains), dim3(kChainThreads), smem,
                           st, ba);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<false, R, NF, PF>), dim3((unsigned)chains), dim3(kChainThreads), smem,
                           st, ba);
    return hipGetLastError();
}

template <int R>
hipError_t launch_chain_mfma(const BwdArgs &ba, int64_t chains, hipStream_t st) {
    const size_t smem = sizeof(float) * mf::smem_floats();
    const void *fn = ba.f.bf16 ? (const void *)bwd_chain_mfma_kernel<true, R> : (const void *)bwd_chain_mfma_kernel<false, R>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    if (ba.f.bf16)
        hipLaunchKernelGGL((bwd_chain_mfma_kernel<true, R>), dim3((unsigned)chains), dim3(kChainThreads), smem, st, ba);
    else
        hipLaunchKernelGGL((bwd_chain_mfma_kernel<false, R>), dim3((unsigned)chains), dim3(kChainThreads), smem, st, ba);
    return hipGetLastError();
}

// the 1.5B-scale head shape (N = 128, P = 64) runs on the matrix cores for R in {1, 2, 4}
inline bool chain_on_mfma(const ScanArgs &a) { return a.N == 128 && a.P == 64 && (a.R == 1 || a.R == 2 || a.R == 4); }

template <int R>
hipError_t launch_chain(const BwdArgs &ba, int64_t chains, size_t smem, hipStream_t st) {
    if (ba.f.N == 128 && ba.f.P == 64) {
        if constexpr (R == 1 || R == 2 || R == 4) {
            if (chain_on_mfma(ba.f)) return launch_chain_mfma<R>(ba, chains, st);
        }
        return launch_chain_np<R, 128, 64>(ba, chains, smem, st);
    }
    return launch_chain_np<R, 0, 0>(ba, chains, smem, st);
}

}  // namespace

// Workspace layout, in one pass or under the low-memory schedule (lowmem: the
// matrix-core chain shapes only). The window of the low-memory schedule, k chunks,
// minimises nch/k checkpoints plus k recomputed states plus k chunks of per-head
// partials: k = sqrt(nch S / (S + Pc)) with S the bytes of one checkpoint of every
// chain and Pc those of one chunk's partials.
struct BwdLayout {
    int wchunks = 0, nwin = 1;
    int64_t Lw = 0;  // tokens per batch of the per-head partial rows
    size_t chk = 0, chkw = 0, rst = 0, gB = 0, gC = 0, gth = 0, tok = 0, gBp = 0, fold = 0, bpart = 0, gWB = 0,
           gWC = 0, part = 0, total = 0;
    int64_t nsplit = 64;
};

static BwdLayout bwd_layout(const ScanArgs &a, bool lowmem, int windows) {
    const BwdDims d = bwd_dims(a.L, a.N, a.P, a.R);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t chains = a.b * a.H;
    const int64_t rowsBC = a.b * a.L * a.G * a.R;  // raw B / C rows
    const int64_t rows_prev = a.b * a.G * a.R;
    const int64_t cols_max = (a.H * a.R * a.N > a.N) ? a.H * a.R * a.N : a.N;
    BwdLayout y;
    y.Lw = a.L;
    int64_t nslots = d.nch + 1;
    if (lowmem && d.nch > 0) {
        const double S = 4.0 * chains * d.slot;
        const double Pc = 4.0 * a.b * d.Cb * a.H * (2.0 * a.R * a.N + a.N / 2);
        int64_t k = (int64_t)(sqrt((double)d.nch * S / (S + Pc)) + 0.5);
        if (windows > 0) k = (d.nch + windows - 1) / windows;  // the caller's window count
        k = k < 1 ? 1 : (k > d.nch ? d.nch : k);
        y.wchunks = (int)k;
        y.nwin = (int)((d.nch + k - 1) / k);
        y.Lw = k * d.Cb < a.L ? k * d.Cb : a.L;
        nslots = y.nwin + 1;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += al(bytes);
        return o;
    };
    y.chk = take(sizeof(float) * chains * nslots * d.slot);  // checkpoints
    if (y.wchunks > 0) {
        y.chkw = take(sizeof(float) * chains * (y.wchunks + 1) * d.slot);          // a window's states
        y.rst = take(sizeof(float) * chains * (a.N * a.P + a.N / 2 + 4 * kChainThreads));  // between windows
    }
    y.gB = take(sizeof(float) * a.b * y.Lw * a.H * a.R * a.N);
    y.gC = take(sizeof(float) * a.b * y.Lw * a.H * a.R * a.N);
    y.gth = take(sizeof(float) * a.b * y.Lw * a.H * (a.N / 2));
    y.tok = take(sizeof(float) * a.b * a.L * a.H * 4);
    y.gBp = take(sizeof(float) * chains * a.R * a.N);
    y.fold = take(sizeof(float) * chains);
    y.bpart = take(sizeof(float) * chains * 2 * a.R * 2 * a.N);
    y.gWB = take(sizeof(float) * (rowsBC + rows_prev) * a.N);
    y.gWC = take(sizeof(float) * (rowsBC + rows_prev) * a.N);
    y.part = take(sizeof(float) * y.nsplit * cols_max);  // column-sum partials
    y.total = off;
    return y;
}

bool scan_bwd_lowmem_ok(const ScanArgs &a) { return a.N == 128 && a.P == 64 && (a.R == 1 || a.R == 2 || a.R == 4); }

size_t scan_bwd_workspace_bytes(const ScanArgs &a, bool lowmem, int windows) {
    return bwd_layout(a, lowmem, windows).total;
}

int scan_bwd_windows(const ScanArgs &a, bool lowmem, int windows) { return bwd_layout(a, lowmem, windows).nwin; }

hipError_t launch_scan_bwd(const ScanArgs &a, const BwdIO &io, void *ws, bool lowmem, int windows, hipStream_t st) {
    if (a.b * a.H == 0) return hipSuccess;
    const BwdDims d = bwd_dims(a.L, a.N, a.P, a.R);
    const BwdLayout y = bwd_layout(a, lowmem, windows);
    const int64_t nsplit = y.nsplit;
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
    ba.chk = reinterpret_cast<float *>(p + y.chk);
    ba.chkw = y.wchunks > 0 ? reinterpret_cast<float *>(p + y.chkw) : nullptr;
    ba.rst = y.wchunks > 0 ? reinterpret_cast<float *>(p + y.rst) : nullptr;
    ba.gB = reinterpret_cast<float *>(p + y.gB);
    ba.gC = reinterpret_cast<float *>(p + y.gC);
    ba.gth = reinterpret_cast<float *>(p + y.gth);
    ba.tok = reinterpret_cast<float *>(p + y.tok);
    ba.gBp = reinterpret_cast<float *>(p + y.gBp);
    ba.fold = reinterpret_cast<float *>(p + y.fold);
    ba.bpart = reinterpret_cast<float *>(p + y.bpart);
    float *gWB = reinterpret_cast<float *>(p + y.gWB);
    float *gWC = reinterpret_cast<float *>(p + y.gWC);
    float *part = reinterpret_cast<float *>(p + y.part);
    ba.Lb = y.Lw;
    ba.tbase = 0;
    ba.wchunks = y.wchunks;
    ba.win = -1;

    hipError_t e;
    auto group = [&](bool prv, int64_t rows, int64_t nt, float *wb, float *wc, float *ob, float *oc) -> hipError_t {
        if (rows == 0) return hipSuccess;
        const unsigned nb = (unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64));
        if (a.bf16)
            hipLaunchKernelGGL(bwd_group_kernel<true>, dim3(nb), dim3(kThreads), 0, st, ba, prv, rows, nt, wb, wc,
                               ob, oc);
        else
            hipLaunchKernelGGL(bwd_group_kernel<false>, dim3(nb), dim3(kThreads), 0, st, ba, prv, rows, nt, wb, wc,
                               ob, oc);
        return hipGetLastError();
    };
    // the per-head sums of the tokens tbase .. tbase + nt - 1 (every batch)
    auto reduce_tokens = [&](int64_t nt) -> hipError_t {
        hipError_t e2 = group(false, a.b * nt * a.G * a.R, nt, gWB, gWC, io.dBraw, io.dCraw);
        if (e2 != hipSuccess) return e2;
        const int64_t tot = a.b * nt * a.G * (a.N / 2);
        const unsigned nb = (unsigned)((tot + kThreads - 1) / kThreads < 65536 ? (tot + kThreads - 1) / kThreads : 65536);
        if (tot > 0) {
            hipLaunchKernelGGL(bwd_theta_kernel, dim3(nb), dim3(kThreads), 0, st, ba, nt, io.dtheta);
            return hipGetLastError();
        }
        return hipSuccess;
    };
    if (y.wchunks == 0) {
        const size_t smem = sizeof(float) * chain_smem_floats(d);
        switch (a.R) {
            case 1: e = launch_chain<1>(ba, chains, smem, st); break;
            case 2: e = launch_chain<2>(ba, chains, smem, st); break;
            case 3: e = launch_chain<3>(ba, chains, smem, st); break;
            case 4: e = launch_chain<4>(ba, chains, smem, st); break;
            default: e = hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
        if ((e = reduce_tokens(a.L)) != hipSuccess) return e;
    } else {
        // low-memory schedule: the forward sweep keeps a checkpoint every wchunks chunks;
        // then, last window first, each window's states are recomputed, its reverse sweep
        // run and its per-head sums reduced before the next window reuses the buffers
        auto chain = [&]() -> hipError_t {
            switch (a.R) {
                case 1: return launch_chain_mfma<1>(ba, chains, st);
                case 2: return launch_chain_mfma<2>(ba, chains, st);
                case 4: return launch_chain_mfma<4>(ba, chains, st);
                default: return hipErrorInvalidValue;
            }
        };
        ba.win = -1;
        if ((e = chain()) != hipSuccess) return e;
        for (int wdx = y.nwin - 1; wdx >= 0; --wdx) {
            ba.win = wdx;
            ba.tbase = (int64_t)wdx * y.wchunks * d.Cb;
            const int64_t nt = a.L - ba.tbase < y.Lw ? a.L - ba.tbase : y.Lw;
            if ((e = chain()) != hipSuccess) return e;
            if ((e = reduce_tokens(nt)) != hipSuccess) return e;
        }
        ba.win = 0;
        ba.tbase = 0;
    }
    float *gWBp = gWB + rowsBC * a.N;
    if (a.has_prev && a.L > 0 && (e = group(true, rows_prev, 1, gWBp, nullptr, io.dBraw_prev, nullptr)) != hipSuccess)
        return e;
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
    if (chain_on_mfma(a)) {  // the chain kernel summed its own tokens
        const unsigned nb = (unsigned)((2 * cols_bias + kThreads - 1) / kThreads);
        hipLaunchKernelGGL(bwd_bias_kernel, dim3(nb), dim3(kThreads), 0, st, ba, prev, io.dB_bias, io.dC_bias);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        if ((e = colsum(ba.gB, a.b * a.L, prev ? ba.gBp : nullptr, prev ? a.b : 0, cols_bias, io.dB_bias)) !=
            hipSuccess)
            return e;
        if ((e = colsum(ba.gC, a.b * a.L, nullptr, 0, cols_bias, io.dC_bias)) != hipSuccess) return e;
    }
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
