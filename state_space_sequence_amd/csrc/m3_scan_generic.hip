// Chunked-scan prefill of the Mamba-3 SSM core in fp32 vector ALU (gfx950).
//
// This kernel handles every shape the C ABI accepts for the fp32 io path (and
// bf16 io when asked): any L (ragged last chunk), chunk * rank <= 64,
// N <= 128, P <= 128, N * P <= 8192. It evaluates the same chunked algorithm as
// the matrix-core kernel, in fp32 throughout, so it is also the exact-algebra
// check of that algorithm at fp32 tolerance.
//
// Algorithm (one workgroup per (batch, head) chain, chunks in sequence):
//  * rotated frame (§3.2.2, Proposition 4 / App. B.3): B_bar_t = R(-Phi_t) B_t,
//    C_bar_t = R(-Phi_t) C_t with Phi_t the cumulative angle sum_{s<=t} dt_s theta_s
//    measured from the first token; the state is carried in that frame and
//    rotated back by Phi_{L-1} at the end;
//  * the trapezoid's beta term is folded into the carried state: with
//    w_s = lam_s dt_s + (1 - lam_{s+1}) dt_{s+1} (and w = gamma at the last token)
//    the chunk mask is L[t,s] = exp(cs_t - cs_s) w_s (s < t), gamma_t (s = t),
//    which is the product form of the §3.1.3 mask (eq. 7) written out with
//    alpha_{s+1} gamma_s + beta_{s+1} = alpha_{s+1} w_s;
//  * chunk pieces (SSD chunked algorithm, §3.3): Y = (L o C_bar B_bar^T) X +
//    exp(cs_t) C_bar_t^T S, S <- exp(cs_end) S + sum_s exp(cs_end - cs_s) w_s B_bar_s X_s^T,
//    with cs the chunk-local cumulative log decay.
//  * MIMO rows are the flattened (token, rank) pairs; the mask depends on tokens.
//  * angles are carried in revolutions (turns): the running total is reduced
//    mod 1 at every chunk boundary (a whole turn changes no rotation), and each
//    chunk's prefix starts from that reduced carry, so an angle never grows
//    beyond a chunk's worth of increments and keeps its fp32 resolution over
//    any sequence length; sine and cosine take it through sincospif;
//  * output epilogue: the skip D[h] x_t (the D term of y = C h + D x) and the
//    grouped output RMSNorm of every (token, rank) row over its P channels; with
//    the norm the chunk's rows are staged in LDS until their mean square is known.
#include "m3_internal.h"

namespace m3i {

namespace {

constexpr int kThreads = 256;
constexpr float kInv2Pi = 0.15915494309189535f;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void scan_generic_kernel(ScanArgs a) {
    const int N = (int)a.N, P = (int)a.P, R = (int)a.R, C = (int)a.C;
    const int HALF = N / 2;
    const int T = C * R;  // rows per chunk
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int64_t g = hi / (a.H / a.G);
    const int64_t L = a.L;

    extern __shared__ float sm[];
    float *S = sm;                   // state [N][P] (rotated frame, folded)
    float *Bb = S + N * P;           // [T][N] rotated B
    float *Cb = Bb + T * N;          // [T][N] rotated C
    float *Xs = Cb + T * N;          // [T][P]
    float *Pm = Xs + T * P;          // [T][T] masked scores; Phi [C][HALF] aliases it
    const int pmsz = (T * T > C * HALF) ? T * T : C * HALF;
    float *lcs = Pm + pmsz;          // [C] chunk-local cumulative log decay
    float *wgt = lcs + C;            // [C] folded weight w
    float *gam = wgt + C;            // [C] gamma
    float *dtv = gam + C;            // [C] dt
    float *carry = dtv + C;          // [HALF] cumulative angle before this chunk, revolutions mod 1
    float *rsB = carry + HALF;       // [T] 1/rms of B rows
    float *rsC = rsB + T;            // [T]
    float *misc = rsC + T;           // [4]: exp(cs_end)
    float *Yb = misc + 4;            // [T][P] output rows before the norm (only with the norm)
    float *Phi = Pm;
    const float dsk = a.D ? a.D[hi] : 0.f;

    // ---- initial state (physical frame = rotated frame at position -1)
    for (int e = tid; e < N * P; e += kThreads) {
        const int n = e / P, p = e % P;
        S[e] = a.h0 ? a.h0[(bh * P + p) * N + n] : 0.f;
    }
    for (int i = tid; i < HALF; i += kThreads) carry[i] = 0.f;
    if (a.has_prev && L > 0) {
        // fold (1 - lam_0) dt_0 B_{-1} x_{-1}^T into the starting state
        for (int r = tid; r < R; r += kThreads) {
            const int64_t row = ((bi * a.G + g) * R + r) * N;
            float ss = 0.f;
            for (int n = 0; n < N; ++n) {
                const float v = ld_io<BF16>(a.Braw_prev, row + n);
                ss += v * v;
            }
            rsB[r] = 1.0f / sqrtf(ss / (float)N + a.eps);
        }
        __syncthreads();
        const float f = (1.0f - a.lam[bi * L * a.H + hi]) * a.dt[bi * L * a.H + hi];
        for (int e = tid; e < N * P; e += kThreads) {
            const int n = e / P, p = e % P;
            float acc = 0.f;
            for (int r = 0; r < R; ++r) {
                const float w = a.B_normw ? a.B_normw[n] : 1.f;
                const float bv = ld_io<BF16>(a.Braw_prev, ((bi * a.G + g) * R + r) * N + n) * rsB[r] * w +
                                 a.B_bias[(hi * R + r) * N + n];
                acc += bv * ld_io<BF16>(a.x_prev, ((bi * a.H + hi) * R + r) * P + p);
            }
            S[e] += f * acc;
        }
    }
    __syncthreads();

    for (int64_t c0 = 0; c0 < L; c0 += C) {
        const int nv = (int)((L - c0) < C ? (L - c0) : C);  // valid tokens in chunk
        // ---- per-token scalars (serial: chunks are at most 64 tokens)
        if (tid == 0) {
            float run = 0.f;
            for (int t = 0; t < C; ++t) {
                if (t < nv) {
                    const int64_t o = (bi * L + c0 + t) * a.H + hi;
                    const float d = a.dt[o], lm = a.lam[o];
                    run += d * a.A[o];
                    float look = 0.f;
                    if (c0 + t + 1 < L) {
                        const int64_t o1 = o + a.H;
                        look = (1.0f - a.lam[o1]) * a.dt[o1];
                    }
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
            misc[0] = expf(run);
        }
        // ---- cumulative angles per channel (serial over the chunk's tokens), in
        // revolutions from the reduced carry
        for (int i = tid; i < HALF; i += kThreads) {
            float ph = carry[i];
            for (int t = 0; t < nv; ++t) {
                const int64_t tok = bi * L + c0 + t;
                ph += a.dt[tok * a.H + hi] * a.theta[(tok * a.G + g) * HALF + i] * kInv2Pi;
                Phi[t * HALF + i] = ph;
            }
        }
        // ---- BCNorm factors per row
        for (int rho = tid; rho < T; rho += kThreads) {
            const int t = rho / R, r = rho % R;
            float sb = 0.f, sc = 0.f;
            if (t < nv) {
                const int64_t row = (((bi * L + c0 + t) * a.G + g) * R + r) * N;
                for (int n = 0; n < N; ++n) {
                    const float vb = ld_io<BF16>(a.Braw, row + n), vc = ld_io<BF16>(a.Craw, row + n);
                    sb += vb * vb;
                    sc += vc * vc;
                }
            }
            rsB[rho] = 1.0f / sqrtf(sb / (float)N + a.eps);
            rsC[rho] = 1.0f / sqrtf(sc / (float)N + a.eps);
        }
        __syncthreads();
        // ---- rotated, normalised, biased B and C; X
        for (int e = tid; e < T * HALF; e += kThreads) {
            const int rho = e / HALF, i = e % HALF;
            const int t = rho / R, r = rho % R;
            float bl = 0.f, bhv = 0.f, cl = 0.f, chv = 0.f;
            if (t < nv) {
                const int64_t row = (((bi * L + c0 + t) * a.G + g) * R + r) * N;
                const float *bb = a.B_bias + (hi * R + r) * N;
                const float *cb = a.C_bias + (hi * R + r) * N;
                const float wbl = a.B_normw ? a.B_normw[i] : 1.f, wbh = a.B_normw ? a.B_normw[i + HALF] : 1.f;
                const float wcl = a.C_normw ? a.C_normw[i] : 1.f, wch = a.C_normw ? a.C_normw[i + HALF] : 1.f;
                const float B0 = ld_io<BF16>(a.Braw, row + i) * rsB[rho] * wbl + bb[i];
                const float B1 = ld_io<BF16>(a.Braw, row + i + HALF) * rsB[rho] * wbh + bb[i + HALF];
                const float C0 = ld_io<BF16>(a.Craw, row + i) * rsC[rho] * wcl + cb[i];
                const float C1 = ld_io<BF16>(a.Craw, row + i + HALF) * rsC[rho] * wch + cb[i + HALF];
                float sn, cs;
                sincospif(2.0f * Phi[t * HALF + i], &sn, &cs);
                // R(-Phi): (u, v) -> (cos u + sin v, -sin u + cos v)
                bl = cs * B0 + sn * B1;
                bhv = -sn * B0 + cs * B1;
                cl = cs * C0 + sn * C1;
                chv = -sn * C0 + cs * C1;
            }
            Bb[rho * N + i] = bl;
            Bb[rho * N + i + HALF] = bhv;
            Cb[rho * N + i] = cl;
            Cb[rho * N + i + HALF] = chv;
        }
        for (int e = tid; e < T * P; e += kThreads) {
            const int rho = e / P, p = e % P;
            const int t = rho / R, r = rho % R;
            Xs[e] = (t < nv) ? ld_io<BF16>(a.x, (((bi * L + c0 + t) * a.H + hi) * R + r) * P + p) : 0.f;
        }
        __syncthreads();
        // carry the angle to the end of this chunk, reduced mod 1 revolution (Phi
        // no longer needed after the sync below)
        float newcarry = 0.f;
        if (tid < HALF) {
            const float e = (nv > 0) ? Phi[(nv - 1) * HALF + tid] : carry[tid];
            newcarry = e - floorf(e);
        }
        __syncthreads();
        if (tid < HALF) carry[tid] = newcarry;
        // ---- masked scores P[rho][sigma]
        for (int e = tid; e < T * T; e += kThreads) {
            const int rho = e / T, sg = e % T;
            const int t = rho / R, s = sg / R;
            float v = 0.f;
            if (s <= t) {
                float dot = 0.f;
                for (int n = 0; n < N; ++n) dot += Cb[rho * N + n] * Bb[sg * N + n];
                const float m = (s == t) ? gam[t] : expf(lcs[t] - lcs[s]) * wgt[s];
                v = m * dot;
            }
            Pm[e] = v;
        }
        __syncthreads();
        // ---- outputs
        for (int e = tid; e < T * P; e += kThreads) {
            const int rho = e / P, p = e % P;
            const int t = rho / R, r = rho % R;
            if (t >= nv) continue;
            float off = 0.f;
            for (int n = 0; n < N; ++n) off += Cb[rho * N + n] * S[n * P + p];
            float intra = 0.f;
            for (int sg = 0; sg < T; ++sg) intra += Pm[rho * T + sg] * Xs[sg * P + p];
            const float yv = expf(lcs[t]) * off + intra + dsk * Xs[e];
            if (a.onorm)
                Yb[e] = yv;
            else
                st_io<BF16>(a.y, (((bi * L + c0 + t) * a.H + hi) * R + r) * P + p, yv);
        }
        __syncthreads();
        if (a.onorm) {
            // one thread per row: mean square over P, in a fixed order
            for (int rho = tid; rho < T; rho += kThreads) {
                float ss = 0.f;
                for (int p = 0; p < P; ++p) ss += Yb[rho * P + p] * Yb[rho * P + p];
                rsB[rho] = 1.0f / sqrtf(ss / (float)P + a.eps);
            }
            __syncthreads();
            for (int e = tid; e < T * P; e += kThreads) {
                const int rho = e / P, p = e % P;
                const int t = rho / R, r = rho % R;
                if (t >= nv) continue;
                const float wn = a.out_normw ? a.out_normw[hi * P + p] : 1.f;
                st_io<BF16>(a.y, (((bi * L + c0 + t) * a.H + hi) * R + r) * P + p, Yb[e] * rsB[rho] * wn);
            }
            __syncthreads();
        }
        // ---- state update
        const float dec = misc[0];
        const float lend = lcs[C - 1];
        for (int e = tid; e < N * P; e += kThreads) {
            const int n = e / P, p = e % P;
            float acc = 0.f;
            for (int sg = 0; sg < T; ++sg) {
                const int s = sg / R;
                acc += Bb[sg * N + n] * (expf(lend - lcs[s]) * wgt[s]) * Xs[sg * P + p];
            }
            S[e] = dec * S[e] + acc;
        }
        __syncthreads();
    }

    // ---- final state back to the physical frame: h = R(Phi_{L-1}) h_tilde
    if (a.h_final) {
        for (int e = tid; e < HALF * P; e += kThreads) {
            const int i = e / P, p = e % P;
            float sn, cs;
            sincospif(2.0f * carry[i], &sn, &cs);
            const float u = S[i * P + p], v = S[(i + HALF) * P + p];
            a.h_final[(bh * P + p) * N + i] = cs * u - sn * v;
            a.h_final[(bh * P + p) * N + i + HALF] = sn * u + cs * v;
        }
    }
}

}  // namespace

size_t generic_smem_bytes(const ScanArgs &a) {
    const int64_t T = a.C * a.R;
    const int64_t pmsz = (T * T > a.C * (a.N / 2)) ? T * T : a.C * (a.N / 2);
    return sizeof(float) * (size_t)(a.N * a.P + 2 * T * a.N + T * a.P + pmsz + 4 * a.C + a.N / 2 + 2 * T + 4 +
                                    (a.onorm ? T * a.P : 0));
}

hipError_t launch_scan_generic(const ScanArgs &a, hipStream_t s) {
    if (a.b * a.H == 0) return hipSuccess;
    const size_t smem = generic_smem_bytes(a);
    dim3 grid((unsigned)(a.b * a.H)), block(kThreads);
    const void *fn = a.bf16 ? (const void *)scan_generic_kernel<true> : (const void *)scan_generic_kernel<false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    if (a.bf16)
        hipLaunchKernelGGL(scan_generic_kernel<true>, grid, block, smem, s, a);
    else
        hipLaunchKernelGGL(scan_generic_kernel<false>, grid, block, smem, s, a);
    return hipGetLastError();
}

}  // namespace m3i
