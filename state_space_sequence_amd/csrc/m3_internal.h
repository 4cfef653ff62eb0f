// Internal declarations shared by the HIP sources of libm3 (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "m3.h"

namespace m3i {

// Flattened, validated arguments handed from the C ABI to the launchers.
struct ScanArgs {
    int64_t b, L, H, G, P, N, R, C;  // C = chunk (tokens)
    float eps;
    bool bf16;      // io dtype
    bool has_prev;  // x_prev / Braw_prev given
    const void *x, *Braw, *Craw;
    const float *dt, *A, *lam, *theta;
    const float *B_bias, *C_bias, *B_normw, *C_normw;
    const float *h0;
    const void *x_prev, *Braw_prev;
    void *y;
    float *h_final;
};

struct DecodeArgs {
    int64_t b, H, G, P, N, R;
    float eps;
    bool bf16;
    bool has_prev;
    const void *x, *Braw, *Craw;
    const float *dt, *A, *lam, *theta;
    const float *B_bias, *C_bias, *B_normw, *C_normw;
    const void *x_prev, *Braw_prev;
    float *h;
    void *y;
};

// Segment-split bookkeeping for the matrix-core prefill (state passing).
struct SplitPlan {
    int nseg;          // segments per sequence
    int64_t seg_chunks;  // chunks per segment (last one may be shorter)
    float *seg_state;  // [b,H,nseg,P,N]: pass-1 end states, then incoming states
    float *seg_decay;  // [b,H,nseg]     total log-decay of each segment
    float *seg_angle;  // [b,H,nseg,N/2] total rotation angle of each segment, in revolutions mod 1
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_scan_generic(const ScanArgs &a, hipStream_t s);
hipError_t launch_scan_mfma(const ScanArgs &a, const SplitPlan &sp, hipStream_t s);

// matrix-core prefill planning (m3_scan_mfma.hip)
bool mfma_kernel_available();
int mfma_auto_segments(int64_t chains, int64_t nchunks);
size_t mfma_workspace_bytes(int64_t chains, int nseg, int64_t P, int64_t N);
void mfma_workspace_carve(void *ws, int64_t chains, int nseg, int64_t P, int64_t N, SplitPlan *sp);

// limits of the individual kernels (checked by the C ABI before launching)
constexpr int kGenericMaxN = 128;
constexpr int kGenericMaxP = 128;
constexpr int kGenericMaxRows = 64;      // chunk * rank
constexpr int kGenericMaxNP = 8192;      // N * P
constexpr int kDecodeMaxP = 256;
constexpr int kDecodeMaxR = 4;

// ----------------------------------------------------------------- device ---
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

// round to nearest even (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float ld_io(const void *p, int64_t i) {
    if constexpr (BF16)
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else
        return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st_io(void *p, int64_t i, float v) {
    if constexpr (BF16)
        static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(v);
    else
        static_cast<float *>(p)[i] = v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace m3i
