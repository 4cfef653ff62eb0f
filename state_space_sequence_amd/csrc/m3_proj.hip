// The MIMO projections of the Mamba-3 paper's App. C as two stand-alone
// elementwise kernels: the rank expansion of the input before the core, and the
// gate with the rank contraction after it. The fused prefill and decode do the
// same inside the core kernels; these exist for callers that run the core on
// its own, and they are the unfused baseline the fused path is measured against.
//
//   expand:   x[., h, r, p] = W_X[h, p, r] * x'[., h, p]
//   gate:     o[., h, p]    = sum_r W_O[h, p, r] * y[., h, r, p] * SiLU(W_Z[h, p, r] * z'[., h, p])
//
// Both are bound by HBM: a thread moves 8 consecutive channels p of one head
// (16 bytes of bf16 or 32 of fp32 per access) for a run of tokens, with the
// head's weights for those channels loaded once. (One thread per (token, head)
// row re-read 8 R weights per row: about 4 GB of cache traffic per gate call on
// a b8 L4096 H64 rank-4 layer, which bound it at 1.4 TB/s of HBM.)
#include "m3_internal.h"

namespace m3i {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;  // channels per thread

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t i, float *v) {
    if constexpr (BF16) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    } else {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 a = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + i);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + i + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = a[k];
            v[k + 4] = b[k];
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void store8(void *base, int64_t i, const float *v) {
    if constexpr (BF16) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)f32_to_bf16_bits(v[2 * k]) | ((uint32_t)f32_to_bf16_bits(v[2 * k + 1]) << 16);
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + i) = w;
    } else {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + i) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

// the thread's weights W[h][p0..p0+7][0..R-1]: 8 R consecutive floats, 16-byte
// aligned (p0 is a multiple of 8), read as 2 R vector loads
template <int R>
__device__ __forceinline__ void load_w(const float *W, int64_t h, int P, int p0, float *w) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 *src = reinterpret_cast<const f32x4 *>(W + (h * P + p0) * R);
#pragma unroll
    for (int k = 0; k < 2 * R; ++k) {
        const f32x4 v = src[k];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[4 * k + j] = v[j];
    }
}

// Grid: x = blocks of kTokSlots tokens times kTokIter trips, y = head. A thread
// owns channels p0..p0+7 of one head (its weights are loaded once) and walks
// tokens tok0, tok0 + kTokSlots, ...: rows (token, head) are H apart, and the
// P / 8 threads of one token cover its P channels contiguously.
constexpr int kTokIter = 16;

template <bool BF16, int R>
__global__ __launch_bounds__(kThreads) void expand_kernel(const void *xin, const float *W, void *xout, int64_t ntok,
                                                          int64_t H, int P) {
    const int pb = P / kVec, slots = kThreads / pb;
    if ((int)threadIdx.x >= slots * pb) return;  // P / 8 need not divide the block
    const int h = blockIdx.y;
    const int p0 = (int)(threadIdx.x % pb) * kVec;
    const int64_t t0 = (int64_t)blockIdx.x * slots * kTokIter + threadIdx.x / pb;
    float w[kVec * R];  // w[p * R + r]
    load_w<R>(W, h, P, p0, w);
    for (int it = 0; it < kTokIter; ++it) {
        const int64_t tok = t0 + (int64_t)it * slots;
        if (tok >= ntok) break;
        const int64_t row = tok * H + h;
        float x[kVec];
        load8<BF16>(xin, row * P + p0, x);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float o[kVec];
#pragma unroll
            for (int k = 0; k < kVec; ++k) o[k] = w[k * R + r] * x[k];
            store8<BF16>(xout, (row * R + r) * P + p0, o);
        }
    }
}

template <bool BF16, int R>
__global__ __launch_bounds__(kThreads) void gate_kernel(const void *y, const void *z, const float *WZ, const float *WO,
                                                        void *o, int64_t ntok, int64_t H, int P) {
    const int pb = P / kVec, slots = kThreads / pb;
    if ((int)threadIdx.x >= slots * pb) return;  // P / 8 need not divide the block
    const int h = blockIdx.y;
    const int p0 = (int)(threadIdx.x % pb) * kVec;
    const int64_t t0 = (int64_t)blockIdx.x * slots * kTokIter + threadIdx.x / pb;
    float wz[kVec * R], wo[kVec * R];
    load_w<R>(WZ, h, P, p0, wz);
    load_w<R>(WO, h, P, p0, wo);
    for (int it = 0; it < kTokIter; ++it) {
        const int64_t tok = t0 + (int64_t)it * slots;
        if (tok >= ntok) break;
        const int64_t row = tok * H + h;
        float zz[kVec], acc[kVec];
        load8<BF16>(z, row * P + p0, zz);
#pragma unroll
        for (int k = 0; k < kVec; ++k) acc[k] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float yv[kVec];
            load8<BF16>(y, (row * R + r) * P + p0, yv);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                const float g = wz[k * R + r] * zz[k];
                const float silu = g / (1.f + __expf(-g));
                acc[k] = __builtin_fmaf(wo[k * R + r] * yv[k], silu, acc[k]);
            }
        }
        store8<BF16>(o, row * P + p0, acc);
    }
}

inline dim3 proj_grid(int64_t ntok, int64_t H, int P) {
    const int slots = kThreads / (P / kVec);
    const int64_t per = (int64_t)slots * kTokIter;
    return dim3((unsigned)((ntok + per - 1) / per), (unsigned)H);
}

template <bool BF16>
hipError_t launch_expand_io(const void *xin, const float *W, void *xout, int64_t ntok, int64_t H, int P, int R,
                            hipStream_t s) {
    const dim3 grid = proj_grid(ntok, H, P), block(kThreads);
    switch (R) {
        case 1: hipLaunchKernelGGL((expand_kernel<BF16, 1>), grid, block, 0, s, xin, W, xout, ntok, H, P); break;
        case 2: hipLaunchKernelGGL((expand_kernel<BF16, 2>), grid, block, 0, s, xin, W, xout, ntok, H, P); break;
        case 3: hipLaunchKernelGGL((expand_kernel<BF16, 3>), grid, block, 0, s, xin, W, xout, ntok, H, P); break;
        case 4: hipLaunchKernelGGL((expand_kernel<BF16, 4>), grid, block, 0, s, xin, W, xout, ntok, H, P); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_gate_io(const void *y, const void *z, const float *WZ, const float *WO, void *o, int64_t ntok,
                          int64_t H, int P, int R, hipStream_t s) {
    const dim3 grid = proj_grid(ntok, H, P), block(kThreads);
    switch (R) {
        case 1: hipLaunchKernelGGL((gate_kernel<BF16, 1>), grid, block, 0, s, y, z, WZ, WO, o, ntok, H, P); break;
        case 2: hipLaunchKernelGGL((gate_kernel<BF16, 2>), grid, block, 0, s, y, z, WZ, WO, o, ntok, H, P); break;
        case 3: hipLaunchKernelGGL((gate_kernel<BF16, 3>), grid, block, 0, s, y, z, WZ, WO, o, ntok, H, P); break;
        case 4: hipLaunchKernelGGL((gate_kernel<BF16, 4>), grid, block, 0, s, y, z, WZ, WO, o, ntok, H, P); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Shape checks shared by both entry points; rows = batch * seqlen tokens
m3_status proj_check(const m3_shape *s, int64_t *rows) {
    if (!s) return M3_ERR_INVALID_ARG;
    if (s->batch < 0 || s->seqlen < 0 || s->nheads < 1 || s->headdim < 1 || s->rank < 1) return M3_ERR_INVALID_ARG;
    if (s->io_dtype != M3_F32 && s->io_dtype != M3_BF16) return M3_ERR_INVALID_ARG;
    if (s->headdim % kVec != 0 || s->headdim > kVec * kThreads || s->rank > 4) return M3_ERR_UNSUPPORTED;
    if (s->batch > (1LL << 31) || s->seqlen > (1LL << 40) || s->nheads > 65535) return M3_ERR_UNSUPPORTED;
    if (s->seqlen > 0 && s->batch > (1LL << 40) / s->seqlen) return M3_ERR_UNSUPPORTED;
    *rows = s->batch * s->seqlen;  // tokens; the heads are the grid's y
    return M3_OK;
}

bool al16(const void *p) { return (((uintptr_t)p) & 15u) == 0; }

}  // namespace
}  // namespace m3i

using namespace m3i;

extern "C" {

m3_status m3_expand_ranks(const m3_shape *shape, const void *x_in, const float *W_X, void *x_out, void *stream) {
    int64_t rows = 0;
    m3_status st = proj_check(shape, &rows);
    if (st != M3_OK) return st;
    if (rows == 0) return M3_OK;
    if (!x_in || !W_X || !x_out) return M3_ERR_INVALID_ARG;
    if (!al16(x_in) || !al16(W_X) || !al16(x_out)) return M3_ERR_MISALIGNED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int P = (int)shape->headdim, R = (int)shape->rank;
    const hipError_t e = shape->io_dtype == M3_BF16
                             ? launch_expand_io<true>(x_in, W_X, x_out, rows, shape->nheads, P, R, s)
                             : launch_expand_io<false>(x_in, W_X, x_out, rows, shape->nheads, P, R, s);
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status m3_gate_contract(const m3_shape *shape, const void *y, const void *z_in, const float *W_Z,
                           const float *W_O, void *o, void *stream) {
    int64_t rows = 0;
    m3_status st = proj_check(shape, &rows);
    if (st != M3_OK) return st;
    if (rows == 0) return M3_OK;
    if (!y || !z_in || !W_Z || !W_O || !o) return M3_ERR_INVALID_ARG;
    if (!al16(y) || !al16(z_in) || !al16(W_Z) || !al16(W_O) || !al16(o)) return M3_ERR_MISALIGNED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int P = (int)shape->headdim, R = (int)shape->rank;
    const hipError_t e = shape->io_dtype == M3_BF16
                             ? launch_gate_io<true>(y, z_in, W_Z, W_O, o, rows, shape->nheads, P, R, s)
                             : launch_gate_io<false>(y, z_in, W_Z, W_O, o, rows, shape->nheads, P, R, s);
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // extern "C"
