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
    // fused projections (fused == W_X given): x / x_prev are X' without the rank axis
    bool fused;
    const void *z;
    const float *W_X, *W_Z, *W_O;
    void *o;
    // output epilogue: skip D[h] x, grouped output RMSNorm (gain [H,P] or NULL)
    const float *D, *out_normw;
    bool onorm, norm_after_gate;
    // matrix-core path: B and C after BCNorm and its gain (scaled by a power of two,
    // see the prefill), one row of N/2 f16 pairs (n, n + N/2) per (token, group, rank)
    unsigned *Bq, *Cq;
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
    void *h;          // [b,H,P,N] fp32, or bf16 when bf16_state
    bool bf16_state;  // state stored as bf16 (rounded to nearest even), arithmetic in fp32
    void *y;
    // fused projections (fused == W_X given): x / x_prev are X' [b,H,P]
    bool fused;
    const void *z;
    const float *W_X, *W_Z, *W_O;
    void *o;
    const float *D, *out_normw;
    bool onorm, norm_after_gate;
    int64_t hpg;  // heads per group, H / G
};

// Segment-split bookkeeping for the matrix-core prefill (state passing).
struct SplitPlan {
    int nseg;          // segments per sequence
    int64_t seg_chunks;  // chunks per segment (last one may be shorter)
    float *seg_state;  // [b,H,nseg,P,N]: pass-1 end states, then incoming states
    float *seg_decay;  // [b,H,nseg]     total log-decay of each segment
    float *seg_angle;  // [b,H,nseg,N/2] total rotation angle of each segment, in revolutions mod 1
};

// gradient pointers of the prefill backward (m3_scan_grads)
struct BwdIO {
    const void *dy;
    const float *dh_final;
    float *dx, *dBraw, *dCraw, *ddt, *dA, *dlam, *dtheta, *dB_bias, *dC_bias, *dB_normw, *dC_normw, *dh0,
        *dx_prev, *dBraw_prev;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
// lowmem: the windowed low-memory schedule (shapes with scan_bwd_lowmem_ok only), with
// `windows` windows (0: the count that minimises the workspace)
hipError_t launch_scan_bwd(const ScanArgs &a, const BwdIO &io, void *ws, bool lowmem, int windows, hipStream_t s);
size_t scan_bwd_workspace_bytes(const ScanArgs &a, bool lowmem, int windows);
bool scan_bwd_lowmem_ok(const ScanArgs &a);
int scan_bwd_windows(const ScanArgs &a, bool lowmem, int windows);
size_t scan_bwd_smem_bytes(const ScanArgs &a);
hipError_t launch_scan_generic(const ScanArgs &a, hipStream_t s);
hipError_t launch_scan_mfma(const ScanArgs &a, const SplitPlan &sp, hipStream_t s);

// matrix-core prefill planning (m3_scan_mfma.hip)
bool mfma_kernel_available();
int mfma_auto_segments(int64_t chains, int64_t nchunks);
// rows: raw B (or C) rows, b * L * G * R; chains: b * H
size_t mfma_workspace_bytes(int64_t rows, int64_t chains, int nseg, int64_t P, int64_t N);
void mfma_workspace_carve(void *ws, int64_t rows, int64_t chains, int nseg, int64_t P, int64_t N, ScanArgs *a,
                          SplitPlan *sp);

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

// ---- cross-lane exchanges without LDS round trips: DPP lane moves inside a
// 16-lane row and the gfx950 row swaps across rows

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// The two halves a row swap brings together: for B = 4 lanes l and l ^ 16, for
// B = 5 lanes l and l ^ 32. Returns (first, second) with first + second equal, in
// the lower lane, to a + partner's a and, in the upper lane, to b + partner's b.
template <int B>
__device__ __forceinline__ void row_swap(float a, float b, float &first, float &second) {
    static_assert(B == 4 || B == 5, "row swaps pair bit 4 or bit 5");
    if constexpr (B == 4) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        first = __uint_as_float(p[0]);
        second = __uint_as_float(p[1]);
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        first = __uint_as_float(p[0]);
        second = __uint_as_float(p[1]);
    }
}

// x of a partner lane whose index differs from this lane's in bit B (B <= 3). For
// B = 2 and B = 3 the pairing (mirror of 8 / 16 lanes) also flips the lower bits;
// callers rely only on it being an involution that flips bit B.
template <int B>
__device__ __forceinline__ float lane_partner(float x) {
    static_assert(B >= 0 && B <= 3, "DPP pairings cover bits 0..3");
    if constexpr (B == 0) return dpp_mov<0xB1>(x);        // quad_perm [1,0,3,2]
    else if constexpr (B == 1) return dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    else if constexpr (B == 2) return dpp_mov<0x141>(x);  // row_half_mirror
    else return dpp_mov<0x140>(x);                        // row_mirror
}

// x summed over the aligned group of G lanes (G a power of two, at most 64); the
// low bits go first, so every mirror pairing meets lanes that already hold equal sums
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    // No contraction: a caller's product fused into the first step had become a
    // zeroed register, a DPP move and an FMA instead of one DPP add.
#pragma clang fp contract(off)
    if constexpr (G >= 2) x += lane_partner<0>(x);
    if constexpr (G >= 4) x += lane_partner<1>(x);
    if constexpr (G >= 8) x += lane_partner<2>(x);
    if constexpr (G >= 16) x += lane_partner<3>(x);
    if constexpr (G >= 32) {
        float f, s;
        row_swap<4>(x, x, f, s);
        x = f + s;
    }
    if constexpr (G >= 64) {
        float f, s;
        row_swap<5>(x, x, f, s);
        x = f + s;
    }
    return x;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

}  // namespace m3i
