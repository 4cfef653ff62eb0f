/* libm3 calibration probes: the ceilings the mixer's kernels are measured
 * against, taken on the device itself.
 *
 * The prefill and decode kernels are judged against two hardware limits: HBM
 * bandwidth for the decode step (the decode's arithmetic intensity is far below
 * the matrix-core ridge: Mamba-3 paper, §3.3, the arithmetic-intensity argument
 * for decode) and dense bf16 matrix-core throughput for the prefill's
 * intra-chunk contraction (§3.3, chunked algorithm). The spec sheet gives the
 * peaks; these probes give what one kernel can reach on the device at hand, and
 * the shader clock it ran at.
 *
 * Conventions as in m3.h: plain device pointers and sizes, the stream is a
 * hipStream_t passed as void*, every argument is checked on the host before any
 * HIP call, work is enqueued on the stream and nothing is allocated, freed or
 * synchronised. Status codes are m3_status.
 */
#ifndef M3_PROBE_H
#define M3_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "m3.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stream copy: dst[i] = src[i] for `bytes` bytes, in 16 KiB tiles of 256 lanes x
 * four 16-byte non-temporal accesses; `blocks` workgroups walk the tiles with a
 * stride of the grid (0: one workgroup per tile, a single pass).
 * src and dst are device pointers, 16-byte aligned, not overlapping; bytes is a
 * multiple of 16. HBM traffic is `bytes` read plus `bytes` written; a size well
 * above the 256 MB last-level cache measures HBM.
 * Errors: M3_ERR_INVALID_ARG (null pointer with bytes > 0, bytes not a multiple
 * of 16, overlapping buffers, blocks < 0), M3_ERR_MISALIGNED, M3_ERR_HIP. */
m3_status m3_probe_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream);

/* Dense bf16 matrix-core loop: `blocks` workgroups of 4 waves; each wave runs
 * `iters` rounds of 2 independent v_mfma_f32_16x16x32_bf16 (16x16x32, fp32
 * accumulate), i.e. blocks * 4 * iters * 2 * 16384 flops in total; 8 workgroups
 * per compute unit fill the SIMDs with 8 waves each. Operands are
 * derived from `seed` so nothing folds away.
 *   out   device, float[blocks]: one checksum per workgroup (the sum of its
 *         accumulators), finite for any seed;
 *   clock device, int64[2 * blocks] or NULL: per workgroup, the shader-clock
 *         cycles (s_memtime) and the constant-clock ticks (s_memrealtime, at
 *         wall_clock_khz of m3_probe_device_facts) wave 0 spent in the loop, so
 *         cycles / ticks * wall_clock_khz is the shader clock in kHz.
 * Errors: M3_ERR_INVALID_ARG (out NULL, blocks < 1, iters < 1), M3_ERR_HIP. */
m3_status m3_probe_mfma_bf16(float *out, int64_t *clock, int blocks, int iters, float seed, void *stream);

/* Device facts from the HIP runtime for device `dev`: compute units, peak shader
 * clock (kHz), memory clock (kHz), memory bus width (bits), the rate of the
 * constant clock m3_probe_mfma_bf16 reads (kHz), L2 bytes, LDS bytes per
 * workgroup, wave size and the architecture name. Host only; no work is enqueued.
 * Errors: M3_ERR_INVALID_ARG (facts NULL), M3_ERR_HIP (no such device). */
typedef struct {
    int32_t compute_units;
    int32_t clock_khz;
    int32_t memory_clock_khz;
    int32_t memory_bus_bits;
    int32_t wall_clock_khz;
    int64_t l2_bytes;
    int64_t lds_bytes_per_block;
    int32_t wave_size;
    char arch[64];
} m3_device_facts;

m3_status m3_probe_device_facts(int dev, m3_device_facts *facts);

#ifdef __cplusplus
}
#endif

#endif /* M3_PROBE_H */
