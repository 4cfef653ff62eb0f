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
// owns V consecutive state columns n..n+V-1 of the first half and the matching
// columns of the second half (n + N/2), so a rotation pair never leaves a
// thread; the per-column B, C, B_prev coefficients of those columns stay in
// registers while the thread walks rows p. A wave covers contiguous half-rows,
// so every state access is a coalesced V*4-byte vector access. The thread's
// first batch of state rows is requested before the per-head set-up (BCNorm,
// sincos), so that set-up overlaps the HBM latency. y for a row is reduced over
// the N/(2V) lanes that share the row.
#include "m3_internal.h"

namespace m3i {

namespace {

constexpr int kThreads = 256;

template <int V>
struct VecT;
template <>
struct VecT<1> {
    typedef float type;
};
template <>
struct VecT<2> {
    typedef float2 type;
};
template <>
struct VecT<4> {
    typedef float4 type;
};

template <int V>
__device__ __forceinline__ void unpack(const typename VecT<V>::type &v, float *o) {
    if constexpr (V == 1) {
        o[0] = v;
    } else if constexpr (V == 2) {
        o[0] = v.x; o[1] = v.y;
    } else {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
}

template <int V>
__device__ __forceinline__ typename VecT<V>::type pack(const float *o) {
    if constexpr (V == 1)
        return o[0];
    else if constexpr (V == 2)
        return make_float2(o[0], o[1]);
    else
        return make_float4(o[0], o[1], o[2], o[3]);
}

template <bool BF16, int N, int R, int V>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int HALF = N / 2;
    constexpr int NQ = HALF / V;            // lanes that share one row p
    constexpr int ROWS = kThreads / NQ;     // rows covered per pass of the workgroup
    constexpr int KB = (V == 4) ? 4 : 8;    // passes whose state is held in registers at once
    static_assert(NQ >= 2 && NQ <= 64 && (64 % NQ) == 0, "unsupported N/V");
    typedef typename VecT<V>::type vec;

    extern __shared__ float sm[];
    float *sB = sm;              // [R][N]   raw, then normalised B_t
    float *sC = sB + R * N;      // [R][N]   C_t
    float *sBp = sC + R * N;     // [R][N]   B_{t-1}
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
    const int q = tid % NQ;
    const int n0 = V * q;
    const int prow = tid / NQ;
    const int passes = (P + ROWS - 1) / ROWS;
    float *hbase = a.h + bh * (int64_t)P * N;

    // ---- first batch of state rows: in flight during the set-up below
    vec lo[KB], hiv[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int p = prow + k * ROWS;
        if (k < passes && p < P) {
            lo[k] = *reinterpret_cast<const vec *>(hbase + (int64_t)p * N + n0);
            hiv[k] = *reinterpret_cast<const vec *>(hbase + (int64_t)p * N + HALF + n0);
        }
    }

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
    const float beta = a.has_prev ? (1.0f - lm) * d * alpha : 0.f;
    const float gamma = lm * d;

    // ---- this thread's columns: coefficients in registers
    float bl[R][V], bhc[R][V], cl[R][V], ch[R][V], pl[R][V], ph[R][V];
    float cs[V], sn[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        cs[k] = scs[n0 + k];
        sn[k] = ssn[n0 + k];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float *bb = a.B_bias + (hi * R + r) * N;
        const float *cb = a.C_bias + (hi * R + r) * N;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int nl = n0 + k, nh = HALF + n0 + k;
            const float wbl = a.B_normw ? a.B_normw[nl] : 1.f, wbh = a.B_normw ? a.B_normw[nh] : 1.f;
            const float wcl = a.C_normw ? a.C_normw[nl] : 1.f, wch = a.C_normw ? a.C_normw[nh] : 1.f;
            bl[r][k] = gamma * (sB[r * N + nl] * srs[r] * wbl + bb[nl]);
            bhc[r][k] = gamma * (sB[r * N + nh] * srs[r] * wbh + bb[nh]);
            cl[r][k] = sC[r * N + nl] * srs[R + r] * wcl + cb[nl];
            ch[r][k] = sC[r * N + nh] * srs[R + r] * wch + cb[nh];
            pl[r][k] = beta * (sBp[r * N + nl] * srs[2 * R + r] * wbl + bb[nl]);
            ph[r][k] = beta * (sBp[r * N + nh] * srs[2 * R + r] * wbh + bb[nh]);
        }
    }

    // ---- stream the state rows
    const int64_t ybase = rowX;  // y has the x layout
    for (int kb = 0; kb < passes; kb += KB) {
        if (kb > 0) {
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int p = prow + (kb + k) * ROWS;
                if (kb + k < passes && p < P) {
                    lo[k] = *reinterpret_cast<const vec *>(hbase + (int64_t)p * N + n0);
                    hiv[k] = *reinterpret_cast<const vec *>(hbase + (int64_t)p * N + HALF + n0);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int p = prow + (kb + k) * ROWS;
            // rows past P: the whole NQ-lane group is out together, so the
            // shuffles below stay inside active groups
            if (kb + k >= passes || p >= P) continue;
            float xv[R], xpv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                xv[r] = sx[r * P + p];
                xpv[r] = sxp[r * P + p];
            }
            float l[V], h[V];
            unpack<V>(lo[k], l);
            unpack<V>(hiv[k], h);
            float yacc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) yacc[r] = 0.f;
#pragma unroll
            for (int c = 0; c < V; ++c) {
                float u = alpha * l[c], v = alpha * h[c];
                float gu = 0.f, gv = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    u += pl[r][c] * xpv[r];
                    v += ph[r][c] * xpv[r];
                    gu += bl[r][c] * xv[r];
                    gv += bhc[r][c] * xv[r];
                }
                const float nu = cs[c] * u - sn[c] * v + gu;
                const float nv = sn[c] * u + cs[c] * v + gv;
                l[c] = nu;
                h[c] = nv;
#pragma unroll
                for (int r = 0; r < R; ++r) yacc[r] += cl[r][c] * nu + ch[r][c] * nv;
            }
            *reinterpret_cast<vec *>(hbase + (int64_t)p * N + n0) = pack<V>(l);
            *reinterpret_cast<vec *>(hbase + (int64_t)p * N + HALF + n0) = pack<V>(h);
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
}

template <bool BF16, int N>
hipError_t launch_n(const DecodeArgs &a, hipStream_t s) {
    const size_t smem = sizeof(float) * (3 * a.R * N + 2 * a.R * a.P + N + 3 * a.R);
    dim3 grid((unsigned)(a.b * a.H)), block(kThreads);
    switch (a.R) {
        case 1: hipLaunchKernelGGL((decode_kernel<BF16, N, 1, 4>), grid, block, smem, s, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<BF16, N, 2, 2>), grid, block, smem, s, a); break;
        case 3: hipLaunchKernelGGL((decode_kernel<BF16, N, 3, 2>), grid, block, smem, s, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<BF16, N, 4, 2>), grid, block, smem, s, a); break;
        default: return hipErrorInvalidValue;
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
