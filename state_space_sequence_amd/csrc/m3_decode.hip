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
// sincos), so that set-up overlaps the HBM latency. The per-column coefficients
// are formed once per workgroup in LDS. State rows are streamed with
// non-temporal accesses (read once, written once). y for a row is reduced over
// the N/(2V) lanes that share the row.
//
// With the fused rank projections (App. C) x and x_prev are X' [P] and the
// step writes O'[p] = sum_r W_O[p][r] y[r][p] SiLU(W_Z[p][r] Z'[p]) instead of y:
// X = W_X (.) X' is formed in LDS with x, and the gate factors
// W_O SiLU(W_Z Z') in a table, so each lane contracts its R partial sums with
// the gate before the one reduction over the row's lanes.
//
// Output epilogue: the skip D[h] x (the D term of y = C h + D x) starts the
// partial sums of each row's first lane. With the grouped output RMSNorm the output vectors
// (each rank row of y, or Y before the gate, or O' after it) are staged in LDS
// until their mean square over P is known, and written after one more barrier.
#include <type_traits>

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
    typedef float type __attribute__((ext_vector_type(2)));
};
template <>
struct VecT<4> {
    typedef float type __attribute__((ext_vector_type(4)));
};

template <int V>
__device__ __forceinline__ void unpack(const typename VecT<V>::type &v, float *o) {
    if constexpr (V == 1) {
        o[0] = v;
    } else {
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = v[k];
    }
}

template <int V>
__device__ __forceinline__ typename VecT<V>::type pack(const float *o) {
    if constexpr (V == 1) {
        return o[0];
    } else {
        typename VecT<V>::type v;
#pragma unroll
        for (int k = 0; k < V; ++k) v[k] = o[k];
        return v;
    }
}

// One reduce-scatter step at lane bit B over the first 2*HALF of vals: the lower
// lane of each pair keeps vals[0..HALF) plus the partner's, the upper lane keeps
// vals[HALF..2HALF) plus the partner's (stored back into vals[0..HALF)).
template <int B, int HALF, int R>
__device__ __forceinline__ void scatter_step(float (&vals)[R], int q) {
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        if constexpr (B >= 4) {
            float f, s;
            row_swap<B>(vals[i], vals[i + HALF], f, s);
            vals[i] = f + s;
        } else {
            const bool up = (q >> B) & 1;
            const float send = up ? vals[i] : vals[i + HALF];
            const float keep = up ? vals[i + HALF] : vals[i];
            vals[i] = keep + lane_partner<B>(send);
        }
    }
}

// sum over the low LB bits of the lane group
template <int LB>
__device__ __forceinline__ float tree_sum_low(float x) {
    if constexpr (LB >= 1) x += lane_partner<0>(x);
    if constexpr (LB >= 2) x += lane_partner<1>(x);
    if constexpr (LB >= 3) x += lane_partner<2>(x);
    if constexpr (LB >= 4) x += lane_partner<3>(x);
    if constexpr (LB >= 5) {
        float f, s;
        row_swap<4>(x, x, f, s);
        x = f + s;
    }
    static_assert(LB <= 5, "at most 32 lanes below the scatter bits");
    return x;
}

// Registers of V state columns: V floats for an fp32 state, V bf16 values packed
// in V/2 dwords for a bf16 state (arithmetic is fp32 either way).
template <bool BS, int V>
struct StateT {
    typedef typename VecT<V>::type type;
};
template <>
struct StateT<true, 4> {
    typedef unsigned int type __attribute__((ext_vector_type(2)));
};
template <>
struct StateT<true, 2> {
    typedef unsigned int type;
};

__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
    return __builtin_bit_cast(unsigned int, v);
}

template <bool BS, int V>
__device__ __forceinline__ void unpack_state(const typename StateT<BS, V>::type &v, float *o) {
    if constexpr (!BS) {
        unpack<V>(v, o);
    } else if constexpr (V == 2) {
        o[0] = __uint_as_float(v << 16);
        o[1] = __uint_as_float(v & 0xffff0000u);
    } else {
        static_assert(V == 4, "bf16 state: 2 or 4 columns per thread");
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            o[2 * k] = __uint_as_float(v[k] << 16);
            o[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
        }
    }
}

template <bool BS, int V>
__device__ __forceinline__ typename StateT<BS, V>::type pack_state(const float *o) {
    if constexpr (!BS) {
        return pack<V>(o);
    } else if constexpr (V == 2) {
        return pack_bf16x2(o[0], o[1]);
    } else {
        typename StateT<true, 4>::type v;
        v[0] = pack_bf16x2(o[0], o[1]);
        v[1] = pack_bf16x2(o[2], o[3]);
        return v;
    }
}

// io element i of a uniform base, and loads / stores at a 32-bit offset from it:
// with the base in scalar registers and an unsigned offset the compiler can use
// the scalar-base addressing form instead of a 64-bit vector add per access
template <bool BF16>
__device__ __forceinline__ const void *io_at(const void *p, int64_t i) {
    if constexpr (BF16)
        return static_cast<const uint16_t *>(p) + i;
    else
        return static_cast<const float *>(p) + i;
}
template <bool BF16>
__device__ __forceinline__ void *io_at(void *p, int64_t i) {
    if constexpr (BF16)
        return static_cast<uint16_t *>(p) + i;
    else
        return static_cast<float *>(p) + i;
}
template <bool BF16>
__device__ __forceinline__ float ld_io_u(const void *p, unsigned i) {
    if constexpr (BF16)
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else
        return static_cast<const float *>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void st_io_u(void *p, unsigned i, float v) {
    if constexpr (BF16)
        static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(v);
    else
        static_cast<float *>(p)[i] = v;
}

template <bool BF16, bool BS, int N, int R, int V, int KBATCH, bool ONORM>
__global__ __launch_bounds__(kThreads, (R == 1 ? 7 : 5)) void decode_kernel(DecodeArgs a) {
    constexpr int HALF = N / 2;
    constexpr int NQ = HALF / V;            // lanes that share one row p
    constexpr int ROWS = kThreads / NQ;     // rows covered per pass of the workgroup
    constexpr int KB = KBATCH;              // passes whose state is held in registers at once
    static_assert(NQ >= 2 && NQ <= 64 && (64 % NQ) == 0, "unsupported N/V");
    typedef typename VecT<V>::type vec;       // V floats (LDS coefficient reads)
    typedef typename StateT<BS, V>::type svec;  // V state values as stored
    typedef typename std::conditional<BS, __bf16, float>::type selem;

    extern __shared__ float sm[];
    // every array below starts on a 16-byte boundary (sizes are multiples of 4
    // floats) except the last two, which are only read as scalars
    float *sB = sm;              // [R][N]   gamma * normalised B_t (+ bias)
    float *sC = sB + R * N;      // [R][N]   normalised C_t (+ bias)
    float *sBp = sC + R * N;     // [R][N]   beta * normalised B_{t-1} (+ bias)
    float *scs = sBp + R * N;    // [HALF]   cos
    float *ssn = scs + HALF;     // [HALF]   sin
    float *sx = ssn + HALF;      // [P][R]
    float *sxp = sx + R * a.P;   // [P][R]
    float *sgt = sxp + R * a.P;  // [P][R]   fused: W_O SiLU(W_Z Z')
    float *sy = sgt + (a.fused ? R * a.P : 0);  // [R][P] output norm: rows before the norm
    float *srn = sy + R * a.P;   // [R]      output norm: 1/rms per row

    const int tid = threadIdx.x;
    // 32-bit index arithmetic (the launcher keeps b H below 2^31): a 64-bit
    // division by a run-time value is a long scalar sequence at the top of the kernel
    const unsigned bhu = blockIdx.x, Hu = (unsigned)a.H;
    const unsigned biu = bhu / Hu, hiu = bhu - biu * Hu;
    const int64_t bh = bhu, bi = biu, hi = hiu;
    const int64_t g = hiu / (unsigned)a.hpg;
    const int P = (int)a.P;
    const int q = tid % NQ;
    const int n0 = V * q;
    const int prow = tid / NQ;
    const int passes = (P + ROWS - 1) / ROWS;
    selem *hbase = static_cast<selem *>(a.h) + bh * (int64_t)P * N;

    // ---- first batch of state rows: in flight during the set-up below
    svec lo[KB], hiv[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int p = prow + k * ROWS;
        if (k < passes && p < P) {
            lo[k] = __builtin_nontemporal_load(reinterpret_cast<const svec *>(hbase + (int64_t)p * N + n0));
            hiv[k] = __builtin_nontemporal_load(reinterpret_cast<const svec *>(hbase + (int64_t)p * N + HALF + n0));
        }
    }

    // ---- set-up inputs: every global load is issued before the first LDS store,
    // from clamped indices and with optional inputs read through a valid stand-in
    // pointer (the value is masked afterwards), so that no load sits in a branch:
    // the compiler ends such a branch by waiting for its loads, and a load-then-
    // store loop per input had cost one memory round trip each.
    // raw row r of B, C and B_prev (and the head's bias rows) belongs to wave r
    // (R <= 4 waves), NE elements per lane, so BCNorm's sums are wave sums
    constexpr int NE = (N + 63) / 64;
    static_assert(R <= kThreads / 64, "one wave per rank row");
    const int wv = tid / 64, ln = tid % 64;
    const int rr = wv < R ? wv : 0;  // waves past R load row 0 and store nothing
    const int64_t rowBC = (bi * a.G + g) * R * N;
    const int64_t rowX = (bi * a.H + hi) * R * P;
    const int64_t rowP = (bi * a.H + hi) * P;
    const bool hp = a.has_prev;
    const void *srcBp = hp ? a.Braw_prev : a.Braw;
    const void *gB = io_at<BF16>(a.Braw, rowBC), *gC = io_at<BF16>(a.Craw, rowBC), *gBp = io_at<BF16>(srcBp, rowBC);
    const float *gbb = a.B_bias + hi * R * N, *gcb = a.C_bias + hi * R * N;
    const float *pwb = a.B_normw ? a.B_normw : a.B_bias, *pwc = a.C_normw ? a.C_normw : a.C_bias;
    float rB[NE], rC[NE], rBp[NE], rbb[NE], rcb[NE], rwb[NE], rwc[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        const unsigned n = ln + 64 * j < N ? ln + 64 * j : N - 1;
        const unsigned e = rr * N + n;
        rB[j] = ld_io_u<BF16>(gB, e);
        rC[j] = ld_io_u<BF16>(gC, e);
        rBp[j] = ld_io_u<BF16>(gBp, e);
        rbb[j] = gbb[e];
        rcb[j] = gcb[e];
        rwb[j] = pwb[n];
        rwc[j] = pwc[n];
    }
    const int ei = tid < HALF ? tid : HALF - 1;
    const float rth = a.theta[(bi * a.G + g) * HALF + ei];
    const float d = a.dt[bh], Av = a.A[bh], lm = a.lam[bh];
    // x and x_prev, first 2 * kThreads of the R P elements (with the fused
    // projections X', Z' [P] and the weights [P][R], element e = p R + r)
    const int EXN = R * P;
    const int ex0 = tid < EXN ? tid : EXN - 1, ex1 = tid + kThreads < EXN ? tid + kThreads : EXN - 1;
    const void *srcXp = hp ? a.x_prev : a.x;
    const void *gx = io_at<BF16>(a.x, a.fused ? rowP : rowX), *gxp = io_at<BF16>(srcXp, a.fused ? rowP : rowX);
    if (!a.fused) {
        // the tables are stored rank-minor, [p][r], so one row's ranks are
        // adjacent: thread element e of a table is x[r = e % R][p = e / R]
        float rx[2], rxp[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const unsigned e = k == 0 ? ex0 : ex1;
            const unsigned src = (e % R) * P + e / R;
            rx[k] = ld_io_u<BF16>(gx, src);
            rxp[k] = ld_io_u<BF16>(gxp, src);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = tid + k * kThreads;
            if (e < EXN) {
                sx[e] = rx[k];
                sxp[e] = hp ? rxp[k] : 0.f;
            }
        }
    } else {
        const void *gz = io_at<BF16>(a.z, rowP);
        const float *gwx = a.W_X + hi * R * P, *gwz = a.W_Z + hi * R * P, *gwo = a.W_O + hi * R * P;
        float rx[2], rxp[2], rz[2], rwx[2], rwz[2], rwo[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const unsigned e = k == 0 ? ex0 : ex1, pp = e / R;
            rx[k] = ld_io_u<BF16>(gx, pp);
            rxp[k] = ld_io_u<BF16>(gxp, pp);
            rz[k] = ld_io_u<BF16>(gz, pp);
            rwx[k] = gwx[e];
            rwz[k] = gwz[e];
            rwo[k] = gwo[e];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = tid + k * kThreads;
            if (e < EXN) {
                // W is [H][P][R]: e = p R + r is already the table order
                sx[e] = rwx[k] * rx[k];
                sxp[e] = hp ? rwx[k] * rxp[k] : 0.f;
                const float zz = rwz[k] * rz[k];
                sgt[e] = rwo[k] * (zz / (1.f + expf(-zz)));
            }
        }
    }

    // ---- BCNorm of the wave's rows: 1/rms from wave sums of the registers, then the
    // per-column coefficients sB = gamma B_t, sBp = beta B_{t-1}, sC = C_t (all
    // normalised, with gain and bias)
    const float alpha = expf(d * Av);
    const float beta = a.has_prev ? (1.0f - lm) * d * alpha : 0.f;
    const float gamma = lm * d;
    {
        float qb = 0.f, qc = 0.f, qp = 0.f;
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            const bool ok = ln + 64 * j < N;
            qb += ok ? rB[j] * rB[j] : 0.f;
            qc += ok ? rC[j] * rC[j] : 0.f;
            qp += ok ? rBp[j] * rBp[j] : 0.f;
        }
        const float rsb = __builtin_amdgcn_rsqf(wave_sum(qb) * (1.0f / (float)N) + a.eps);  // v_rsq_f32, ~1 ulp
        const float rsc = __builtin_amdgcn_rsqf(wave_sum(qc) * (1.0f / (float)N) + a.eps);
        const float rsp = __builtin_amdgcn_rsqf(wave_sum(qp) * (1.0f / (float)N) + a.eps);
        if (wv < R) {
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                const int n = ln + 64 * j;
                if (n < N) {
                    const float wb = a.B_normw ? rwb[j] : 1.f, wc = a.C_normw ? rwc[j] : 1.f;
                    sB[wv * N + n] = gamma * (rB[j] * rsb * wb + rbb[j]);
                    sC[wv * N + n] = rC[j] * rsc * wc + rcb[j];
                    sBp[wv * N + n] = hp ? beta * (rBp[j] * rsp * wb + rbb[j]) : 0.f;
                }
            }
        }
    }
    // x elements past the first 2 * kThreads (R P > 512: large heads only)
    for (int e = tid + 2 * kThreads; e < EXN; e += kThreads) {
        if (!a.fused) {
            const unsigned src = (e % R) * P + e / R;
            sx[e] = ld_io_u<BF16>(gx, src);
            sxp[e] = a.has_prev ? ld_io_u<BF16>(gxp, src) : 0.f;
        } else {
            const int pp = e / R;
            const float wx = a.W_X[hi * R * P + e];
            sx[e] = wx * ld_io<BF16>(a.x, rowP + pp);
            sxp[e] = a.has_prev ? wx * ld_io<BF16>(a.x_prev, rowP + pp) : 0.f;
            const float zz = a.W_Z[hi * R * P + e] * ld_io<BF16>(a.z, rowP + pp);
            sgt[e] = a.W_O[hi * R * P + e] * (zz / (1.f + expf(-zz)));
        }
    }
    if (tid < HALF) {
        // the hardware sine and cosine take revolutions; reduce to [0, 1) first
        const float rev = __builtin_amdgcn_fractf(d * rth * 0.15915494309189535f);
        scs[tid] = __builtin_amdgcn_cosf(rev);
        ssn[tid] = __builtin_amdgcn_sinf(rev);
    }
    __syncthreads();
    const int wave = tid / 64, lane = tid % 64;

    const float dsk = a.D ? a.D[hi] : 0.f;
    // with the output norm, what is staged: each rank row of y (or of Y, before the
    // gate), or the gated and contracted O' (after the gate)
    const bool stage_ranks = ONORM && !(a.fused && a.norm_after_gate);
    const bool stage_o = ONORM && a.fused && a.norm_after_gate;

    // ---- this thread's columns: coefficients in registers
    float bl[R][V], bhc[R][V], cl[R][V], ch[R][V], pl[R][V], ph[R][V];
    float cs[V], sn[V];
    unpack<V>(*reinterpret_cast<const vec *>(scs + n0), cs);
    unpack<V>(*reinterpret_cast<const vec *>(ssn + n0), sn);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        unpack<V>(*reinterpret_cast<const vec *>(sB + r * N + n0), bl[r]);
        unpack<V>(*reinterpret_cast<const vec *>(sB + r * N + HALF + n0), bhc[r]);
        unpack<V>(*reinterpret_cast<const vec *>(sC + r * N + n0), cl[r]);
        unpack<V>(*reinterpret_cast<const vec *>(sC + r * N + HALF + n0), ch[r]);
        unpack<V>(*reinterpret_cast<const vec *>(sBp + r * N + n0), pl[r]);
        unpack<V>(*reinterpret_cast<const vec *>(sBp + r * N + HALF + n0), ph[r]);
    }
    // R_t is linear, so R_t (alpha H + beta B_prev x_prev^T) = (alpha R_t) H +
    // (R_t beta B_prev) x_prev^T: the rotation is folded into alpha (acs, asn) and
    // into the beta B_prev columns once here, not applied per state element
    float acs[V], asn[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
        acs[c] = alpha * cs[c];
        asn[c] = alpha * sn[c];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float u = pl[r][c], v = ph[r][c];
            pl[r][c] = cs[c] * u - sn[c] * v;
            ph[r][c] = sn[c] * u + cs[c] * v;
        }
    }
    // the skip term D x enters the partial sums of each row's first lane only
    const float dq = (q == 0) ? dsk : 0.f;

    // ---- stream the state rows
    const int64_t ybase = rowX;  // y has the x layout
    void *gy = a.fused ? nullptr : io_at<BF16>(a.y, ybase);
    void *go = a.fused ? io_at<BF16>(a.o, rowP) : nullptr;
    for (int kb = 0; kb < passes; kb += KB) {
        if (kb > 0) {
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int p = prow + (kb + k) * ROWS;
                if (kb + k < passes && p < P) {
                    lo[k] = __builtin_nontemporal_load(reinterpret_cast<const svec *>(hbase + (int64_t)p * N + n0));
                    hiv[k] = __builtin_nontemporal_load(reinterpret_cast<const svec *>(hbase + (int64_t)p * N + HALF + n0));
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
                xv[r] = sx[p * R + r];
                xpv[r] = sxp[p * R + r];
            }
            float l[V], h[V];
            unpack_state<BS, V>(lo[k], l);
            unpack_state<BS, V>(hiv[k], h);
            // the skip term D x enters the sum of the row's first lane, so every
            // reduction below carries it
            float yacc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) yacc[r] = dq * xv[r];
#pragma unroll
            for (int c = 0; c < V; ++c) {
                // (l, h) <- alpha R_t (l, h) + (R_t beta B_prev) x_prev + gamma B x
                float nu = acs[c] * l[c] - asn[c] * h[c];
                float nv = asn[c] * l[c] + acs[c] * h[c];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    nu += pl[r][c] * xpv[r];
                    nv += ph[r][c] * xpv[r];
                    nu += bl[r][c] * xv[r];
                    nv += bhc[r][c] * xv[r];
                }
                l[c] = nu;
                h[c] = nv;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    yacc[r] += cl[r][c] * nu;
                    yacc[r] += ch[r][c] * nv;
                }
            }
            __builtin_nontemporal_store(pack_state<BS, V>(l), reinterpret_cast<svec *>(hbase + (int64_t)p * N + n0));
            __builtin_nontemporal_store(pack_state<BS, V>(h), reinterpret_cast<svec *>(hbase + (int64_t)p * N + HALF + n0));
            if (stage_ranks) {
                // every rank row of the output, skip included, into LDS for the norm
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float v = group_sum<NQ>(yacc[r]);
                    if (q == 0) sy[r * P + p] = v;
                }
            } else if (a.fused) {
                // the gate is linear in y: contract the ranks first, then reduce once
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) v += sgt[p * R + r] * yacc[r];
                v = group_sum<NQ>(v);
                if (q == 0) {
                    if (stage_o)
                        sy[p] = v;
                    else
                        st_io_u<BF16>(go, p, v);
                }
            } else if constexpr (R == 2 || R == 4) {
                // reduce-scatter over the NQ lanes of the row: at the top log2(R)
                // bits of the lane group a lane keeps half of its partial sums and
                // adds the partner's matching half; the low bits then sum one value.
                // A lane with group index q ends with the sum of rank
                // q / (NQ / R).
                constexpr int LNQ = (NQ >= 64) ? 6 : (NQ >= 32) ? 5 : (NQ >= 16) ? 4 : (NQ >= 8) ? 3 : (NQ >= 4) ? 2 : 1;
                constexpr int LR = (R == 2) ? 1 : 2;
                static_assert(LNQ >= LR, "the row needs at least R lanes");
                float vals[R];
#pragma unroll
                for (int r = 0; r < R; ++r) vals[r] = yacc[r];
                scatter_step<LNQ - 1, R / 2>(vals, q);
                if constexpr (LR == 2) scatter_step<LNQ - 2, 1>(vals, q);
                const float v = tree_sum_low<LNQ - LR>(vals[0]);
                const int rk = q / (NQ / R);
                if (q % (NQ / R) == 0) st_io_u<BF16>(gy, rk * P + p, v);
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) yacc[r] = group_sum<NQ>(yacc[r]);
                if (q == 0) {
#pragma unroll
                    for (int r = 0; r < R; ++r) st_io_u<BF16>(gy, r * P + p, yacc[r]);
                }
            }
        }
    }

    if constexpr (ONORM) {
        // grouped output RMSNorm over the P channels of each staged vector
        __syncthreads();
        const int nvec = stage_o ? 1 : R;
        for (int k = wave; k < nvec; k += kThreads / 64) {
            float ss = 0.f;
            for (int p = lane; p < P; p += 64) ss += sy[k * P + p] * sy[k * P + p];
            ss = wave_sum(ss);
            if (lane == 0) srn[k] = 1.0f / sqrtf(ss / (float)P + a.eps);
        }
        __syncthreads();
        const float *wn = a.out_normw ? a.out_normw + hi * P : nullptr;
        const int64_t rowP = (bi * a.H + hi) * P;
        if (!a.fused) {
            for (int e = tid; e < R * P; e += kThreads) {
                const int p = e % P;
                st_io<BF16>(a.y, ybase + e, sy[e] * srn[e / P] * (wn ? wn[p] : 1.f));
            }
        } else if (stage_o) {
            for (int p = tid; p < P; p += kThreads) st_io<BF16>(a.o, rowP + p, sy[p] * srn[0] * (wn ? wn[p] : 1.f));
        } else {
            // normalised Y, then the gate and the rank contraction
            for (int p = tid; p < P; p += kThreads) {
                float v = 0.f;
                for (int r = 0; r < R; ++r) v += sgt[p * R + r] * sy[r * P + p] * srn[r];
                st_io<BF16>(a.o, rowP + p, v * (wn ? wn[p] : 1.f));
            }
        }
    }
}

template <bool BF16, bool BS, int N, bool ONORM>
hipError_t launch_nn(const DecodeArgs &a, hipStream_t s) {
    const size_t smem = sizeof(float) * (3 * a.R * N + N + (a.fused ? 3 : 2) * a.R * a.P +
                                         (a.onorm ? a.R * a.P + a.R : 0));
    dim3 grid((unsigned)(a.b * a.H)), block(kThreads);
    switch (a.R) {
        case 1: hipLaunchKernelGGL((decode_kernel<BF16, BS, N, 1, 4, 2, ONORM>), grid, block, smem, s, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<BF16, BS, N, 2, 2, 4, ONORM>), grid, block, smem, s, a); break;
        case 3: hipLaunchKernelGGL((decode_kernel<BF16, BS, N, 3, 2, 4, ONORM>), grid, block, smem, s, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<BF16, BS, N, 4, 2, 4, ONORM>), grid, block, smem, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16, bool BS, int N>
hipError_t launch_n(const DecodeArgs &a, hipStream_t s) {
    return a.onorm ? launch_nn<BF16, BS, N, true>(a, s) : launch_nn<BF16, BS, N, false>(a, s);
}

template <bool BF16, bool BS>
hipError_t launch_io(const DecodeArgs &a, hipStream_t s) {
    switch (a.N) {
        case 16: return launch_n<BF16, BS, 16>(a, s);
        case 32: return launch_n<BF16, BS, 32>(a, s);
        case 64: return launch_n<BF16, BS, 64>(a, s);
        case 128: return launch_n<BF16, BS, 128>(a, s);
        case 256: return launch_n<BF16, BS, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    if (a.b * a.H == 0) return hipSuccess;
    if (a.bf16_state) return a.bf16 ? launch_io<true, true>(a, s) : launch_io<false, true>(a, s);
    return a.bf16 ? launch_io<true, false>(a, s) : launch_io<false, false>(a, s);
}

}  // namespace m3i
