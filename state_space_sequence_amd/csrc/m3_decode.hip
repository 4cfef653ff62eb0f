// Fused single-token decode step of the Mamba-3 SSM core (gfx950).
//
// One step of the real-form exponential-trapezoidal recurrence (Mamba-3 paper,
// App. B.3 eq. 25) with the rank-R input/output of App. C:
//   H <- R_t (alpha H + beta sum_r B_prev[r] x_prev[r]^T) + gamma sum_r B[r] x[r]^T
//   y[r] = H^T C[r]
// B, C (current and previous token) get BCNorm + bias first (§3.4). R_t rotates
// the coordinate pairs (i, i + N/2) by dt * theta[i] (§3.2.1, Proposition 2).
//
// The step is bound by HBM: the fp32 state is read and written once (arithmetic
// intensity ~2.5 flop/byte for SISO, ~2.5 R for MIMO; §3.3 "decode arithmetic
// intensity"). One workgroup owns one (batch, head) state [P, N]. Each thread
// keeps one quad of state columns n..n+3 and the matching quad of the other
// half (n + N/2), so a rotation pair never leaves a thread; the per-column
// B, C, B_prev values of that quad stay in registers while the thread walks the
// rows p. Rows are streamed as 16-byte loads/stores: 64 lanes cover
// contiguous N/2-float half-rows. y for a row is reduced across the N/8 lanes
// that share it.
#include "m3_internal.h"

namespace m3i {

namespace {

constexpr int kThreads = 256;

template <bool BF16, int N, int R>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int HALF = N / 2;
    constexpr int NQ = N / 8;  // quads per half row; lanes that share one row p
    static_assert(NQ >= 2 && NQ <= 32 && (64 % NQ) == 0, "N must be 16..256");

    extern __shared__ float sm[];
    float *sB = sm;              // [R][N]   normalised B_t
    float *sC = sB + R * N;      // [R][N]   normalised C_t
    float *sBp = sC + R * N;     // [R][N]   normalised B_{t-1}
    float *sx = sBp + R * N;     // [R][P]
    float *sxp = sx + R * a.P;   // [R][P]
    float *scs = sxp + R * a.P;  // [HALF] cos
    float *ssn = scs + HALF;     // [HALF] sin
    float *srs = ssn + HALF;     // [3R]  1/rms per row

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t bi = bh / a.H, hi = bh % a.H;
    const int64_t g = hi / (a.H / a.G);
    const int P = (int)a.P;

    // ---- raw rows into LDS
    const int64_t rowBC = (bi * a.G + g) * R * N;
    for (int e = tid; e < R * N; e += kThreads) {
        sB[e] = ld_io<BF16>(a.Braw, rowBC + e);
        sC[e] = ld_io<BF16>(a.Craw, rowBC + e);
        sBp[e] = a.has_prev ? ld_io<BF16>(a.Braw_prev, rowBC + e) : 0.f;
    }
    const int64_t rowX = (bi * a.H + hi) * R * P;
    for (int e = tid; e < R * P; e += kThreads) {
        sx[e] = ld_io<BF16>(a.x, rowX + e);
        sxp[e] = a.has_prev ? ld_io<BF16>(a.x_prev, rowX + e) : 0.f;
    }
    const float d = a.dt[bh], Av = a.A[bh], lm = a.lam[bh];
    for (int i = tid; i < HALF; i += kThreads) {
        float s, c;
        sincosf(d * a.theta[(bi * a.G + g) * HALF + i], &s, &c);
        scs[i] = c;
        ssn[i] = s;
    }
    __syncthreads();

    // ---- BCNorm: one wave per row (B rows, C rows, B_prev rows)
    const int wave = tid / 64, lane = tid % 64;
    for (int k = wave; k < 3 * R; k += kThreads / 64) {
        const float *row = (k < R ? sB : (k < 2 * R ? sC : sBp)) + (k % R) * N;
        float ss = 0.f;
        for (int n = lane; n < N; n += 64) ss += row[n] * row[n];
        ss = wave_sum(ss);
        if (lane == 0) srs[k] = 1.0f / sqrtf(ss / (float)N + a.eps);
    }
    __syncthreads();

    const float alpha = expf(d * Av);
    const float beta = (1.0f - lm) * d * alpha;
    const float gamma = lm * d;

    // ---- this thread's column quad: n0..n0+3 and HALF+n0..HALF+n0+3
    const int q = tid % NQ;
    const int n0 = 4 * q;
    float bl[R][4], bh_[R][4], cl[R][4], ch[R][4], pl[R][4], ph[R][4];
    float cs[4], sn[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        cs[k] = scs[n0 + k];
        sn[k] = ssn[n0 + k];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float *bb = a.B_bias + (hi * R + r) * N;
        const float *cb = a.C_bias + (hi * R + r) * N;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int nl = n0 + k, nh = HALF + n0 + k;
            const float wbl = a.B_normw ? a.B_normw[nl] : 1.f, wbh = a.B_normw ? a.B_normw[nh] : 1.f;
            const float wcl = a.C_normw ? a.C_normw[nl] : 1.f, wch = a.C_normw ? a.C_normw[nh] : 1.f;
            bl[r][k] = sB[r * N + nl] * srs[r] * wbl + bb[nl];
            bh_[r][k] = sB[r * N + nh] * srs[r] * wbh + bb[nh];
            cl[r][k] = sC[r * N + nl] * srs[R + r] * wcl + cb[nl];
            ch[r][k] = sC[r * N + nh] * srs[R + r] * wch + cb[nh];
            pl[r][k] = sBp[r * N + nl] * srs[2 * R + r] * wbl + bb[nl];
            ph[r][k] = sBp[r * N + nh] * srs[2 * R + r] * wbh + bb[nh];
        }
    }
    const float betae = a.has_prev ? beta : 0.f;

    // ---- stream the state rows
    float *hbase = a.h + bh * (int64_t)P * N;
    const int64_t ybase = rowX;  // y has the x layout
    for (int e = tid; e < P * NQ; e += kThreads) {
        const int p = e / NQ;
        float4 *rowp = reinterpret_cast<float4 *>(hbase + (int64_t)p * N);
        float4 lo = rowp[q];
        float4 hi4 = rowp[NQ + q];
        float xv[R], xpv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            xv[r] = sx[r * P + p];
            xpv[r] = sxp[r * P + p];
        }
        float l[4] = {lo.x, lo.y, lo.z, lo.w};
        float h[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
        float yacc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) yacc[r] = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float u = alpha * l[k], v = alpha * h[k];
            float su = 0.f, sv = 0.f, gu = 0.f, gv = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                su += pl[r][k] * xpv[r];
                sv += ph[r][k] * xpv[r];
                gu += bl[r][k] * xv[r];
                gv += bh_[r][k] * xv[r];
            }
            u += betae * su;
            v += betae * sv;
            const float nu = cs[k] * u - sn[k] * v + gamma * gu;
            const float nv = sn[k] * u + cs[k] * v + gamma * gv;
            l[k] = nu;
            h[k] = nv;
#pragma unroll
            for (int r = 0; r < R; ++r) yacc[r] += cl[r][k] * nu + ch[r][k] * nv;
        }
        rowp[q] = make_float4(l[0], l[1], l[2], l[3]);
        rowp[NQ + q] = make_float4(h[0], h[1], h[2], h[3]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float v = yacc[r];
#pragma unroll
            for (int o = NQ / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
            yacc[r] = v;
        }
        if (q == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) st_io<BF16>(a.y, ybase + r * P + p, yacc[r]);
        }
    }
}

template <bool BF16, int N>
hipError_t launch_n(const DecodeArgs &a, hipStream_t s) {
    const size_t smem = sizeof(float) * (3 * a.R * N + 2 * a.R * a.P + N + 3 * a.R);
    dim3 grid((unsigned)(a.b * a.H)), block(kThreads);
    switch (a.R) {
#define M3_CASE_R(RR)                                                                     \
    case RR:                                                                             \
        hipLaunchKernelGGL((decode_kernel<BF16, N, RR>), grid, block, smem, s, a);      \
        break;
        M3_CASE_R(1)
        M3_CASE_R(2)
        M3_CASE_R(3)
        M3_CASE_R(4)
#undef M3_CASE_R
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_io(const DecodeArgs &a, hipStream_t s) {
    switch (a.N) {
        case 16: return launch_n<BF16, 16>(a, s);
        case 32: return launch_n<BF16, 32>(a, s);
        case 64: return launch_n<BF16, 64>(a, s);
        case 128: return launch_n<BF16, 128>(a, s);
        case 256: return launch_n<BF16, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    if (a.b * a.H == 0) return hipSuccess;
    return a.bf16 ? launch_io<true>(a, s) : launch_io<false>(a, s);
}

}  // namespace m3i
