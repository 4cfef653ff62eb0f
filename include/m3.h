/*
 * m3.h -- C ABI of the MI355X (gfx950) Mamba-3 SSM mixer core.
 *
 * The library computes the selective state-space recurrence of Mamba-3:
 *
 *   B_t[r] = RMSNorm_N(Braw_t[r]) * B_normw + B_bias[h, r]     (same for C)
 *            -- Mamba-3 paper, §3.4: BC normalisation, then a head-specific,
 *               channel-wise bias
 *   alpha_t = exp(dt_t A_t), beta_t = (1 - lam_t) dt_t exp(dt_t A_t),
 *   gamma_t = lam_t dt_t                      -- §3.1.1, Proposition 1
 *   H_t = R_t (alpha_t H_{t-1} + beta_t sum_r B_{t-1}[r] X_{t-1}[r]^T)
 *         + gamma_t sum_r B_t[r] X_t[r]^T     -- App. B.3 eq. 25 (real form of the
 *                                               complex exponential-trapezoidal SSM),
 *                                               rank-R input of App. C
 *   y_t[r] = H_t^T C_t[r]                     -- App. C, Y_t = H_t^T C_t
 *
 * where R_t rotates every state coordinate pair (i, i + N/2), i < N/2, by the
 * angle dt_t * theta_t[i] (counter-clockwise: [[cos, -sin], [sin, cos]]; §3.2.1,
 * Proposition 2, with the state stacked as [real half; imaginary half]). The
 * prefill evaluates this with the chunked algorithm of §3.3 and the rotary
 * "RoPE trick" of §3.2.2 (Proposition 4); decode applies one step directly.
 *
 * Tensor layouts are dense, row-major, contiguous; b = batch, L = seqlen,
 * H = nheads, G = ngroups (head h uses group h / (H/G)), P = headdim,
 * N = dstate, R = rank (1 = SISO):
 *   x, x-like outputs    [b, L, H, R, P]   io dtype (fp32 or bf16)
 *   Braw, Craw           [b, L, G, R, N]   io dtype (raw projections, before BCNorm)
 *   dt, A, lam           [b, L, H]         fp32 (dt > 0 after softplus, A < 0,
 *                                                lam in [0, 1] after sigmoid)
 *   theta                [b, L, G, N/2]    fp32 (rotation frequencies; angle = dt*theta)
 *   B_bias, C_bias       [H, R, N]         fp32
 *   B_normw, C_normw     [N]               fp32, optional (NULL = ones)
 *   state h              [b, H, P, N]      fp32 (physical frame)
 *   x_prev               [b, H, R, P]      io dtype, Braw_prev [b, G, R, N] io dtype
 *
 * Ownership: the caller owns every buffer, including the workspace. The library
 * keeps no state between calls, never allocates, frees or synchronises, and
 * enqueues its kernels on the caller's stream (a hipStream_t passed as void*;
 * NULL = the default stream). It is re-entrant.
 *
 * Errors: every argument is checked on the host before any HIP call; a failed
 * check returns a negative status and enqueues nothing. M3_ERR_HIP means a
 * kernel launch was rejected by the runtime. Faults inside a kernel surface at
 * the caller's next synchronisation, as HIP errors. No C++ exception crosses
 * this interface. All device pointers must be 16-byte aligned.
 */
#ifndef M3_H
#define M3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    M3_OK = 0,
    M3_ERR_INVALID_ARG = -1,         /* NULL where a tensor is required, bad sizes */
    M3_ERR_UNSUPPORTED = -2,         /* valid shape that no kernel here handles */
    M3_ERR_MISALIGNED = -3,          /* a device pointer is not 16-byte aligned */
    M3_ERR_WORKSPACE_TOO_SMALL = -4, /* ws_bytes < m3_scan_workspace_bytes(shape) */
    M3_ERR_HIP = -5                  /* the HIP runtime rejected a launch */
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

/* flags */
#define M3_FLAG_FORCE_GENERIC 1u /* use the fp32 vector-ALU chunked kernel even where
                                    the bf16 matrix-core kernel applies */
#define M3_FLAG_BF16_STATE 2u    /* decode only: the state h is stored as bf16 [b,H,P,N],
                                    read, updated in fp32 and written back rounded to
                                    nearest even (the Mamba-3 paper times decode with
                                    fp32 and with bf16 state, §4.4 Table 6). m3_scan_fwd
                                    rejects it with M3_ERR_INVALID_ARG. */
#define M3_FLAG_OUT_NORM 4u      /* grouped output RMSNorm: every output row of P
                                    channels (one head, one token, one rank row of y)
                                    becomes v / sqrt(mean(v^2) + eps) * out_normw[h][:],
                                    eps the BCNorm eps. The optional Mamba-2 norm that
                                    BCNorm makes optional (Mamba-3 paper §3.4), studied
                                    grouped and before/after the gate in §4.1.2 Table 4
                                    and App. E Table 9. With the fused gate the norm is
                                    applied to each rank row of Y before the gate. */
#define M3_FLAG_NORM_AFTER_GATE 8u /* with M3_FLAG_OUT_NORM and the fused gate (W_X set):
                                    norm O' (after the gate and the rank contraction)
                                    instead of Y. M3_ERR_INVALID_ARG without both. */
#define M3_FLAG_BWD_LOW_MEMORY 16u /* m3_scan_bwd only, N = 128, P = 64, R in {1, 2, 4}: the
                                      windowed schedule. The forward sweep keeps a state
                                      checkpoint every k chunks; then, last window first,
                                      each window of k chunks has its states recomputed
                                      from its checkpoint, its reverse sweep run and its
                                      per-head dB, dC, d theta sums reduced before the next
                                      window reuses the buffers. k minimises the workspace
                                      (about sqrt of the chunk count); shape->nsegments > 0
                                      asks for that many windows instead (fewer: less
                                      launch overhead, more memory). Same results, bit
                                      for bit, for about one more forward sweep of time;
                                      m3_scan_bwd_workspace_bytes gives the smaller size
                                      for a shape with this flag. Without the flag the
                                      backward ignores nsegments. */

typedef struct {
    int64_t batch;     /* b >= 0 */
    int64_t seqlen;    /* L >= 0 (decode: ignored) */
    int64_t nheads;    /* H >= 1 */
    int64_t ngroups;   /* G >= 1, H % G == 0 */
    int64_t headdim;   /* P */
    int64_t dstate;    /* N, even */
    int64_t rank;      /* R >= 1 */
    int64_t chunk;     /* tokens per chunk (prefill). The matrix-core kernel needs
                          chunk * rank == 64 (the pages' rule: 64 / mimo_rank) */
    int32_t io_dtype;  /* m3_dtype of x, Braw, Craw, x_prev, Braw_prev, y */
    uint32_t flags;    /* M3_FLAG_* */
    float eps;         /* BCNorm epsilon (added to the mean square) */
    int32_t nsegments; /* prefill sequence split: 0 = automatic, 1 = none,
                          k > 1 = split every sequence into k segments whose end
                          states are combined in a second pass (state passing) */
} m3_shape;

/* Prefill (chunked scan) arguments. */
typedef struct {
    const void *x;         /* [b,L,H,R,P] io */
    const void *Braw;      /* [b,L,G,R,N] io */
    const void *Craw;      /* [b,L,G,R,N] io */
    const float *dt;       /* [b,L,H] */
    const float *A;        /* [b,L,H] */
    const float *lam;      /* [b,L,H] */
    const float *theta;    /* [b,L,G,N/2] */
    const float *B_bias;   /* [H,R,N] */
    const float *C_bias;   /* [H,R,N] */
    const float *B_normw;  /* [N] or NULL */
    const float *C_normw;  /* [N] or NULL */
    const float *h0;       /* [b,H,P,N] initial state or NULL (zero) */
    const void *x_prev;    /* [b,H,R,P] io: token before position 0, or NULL */
    const void *Braw_prev; /* [b,G,R,N] io: its raw B, or NULL. Both or neither:
                              with them, position 0 gets the beta term of the
                              trapezoid; without, it has none (§3.1.3 unrolling
                              starts from h_0 = gamma_0 B_0 x_0) */
    void *y;               /* out [b,L,H,R,P] io (not written, may be NULL, with W_X set) */
    float *h_final;        /* out [b,H,P,N] state after position L-1, or NULL */
    /* Fused MIMO projections and output gate (Mamba-3 paper App. C), all NULL to
     * leave them out. With W_X set, x and x_prev hold X' [b,L,H,P] and [b,H,P]
     * (no rank axis); the kernel forms X[r][p] = W_X[h][p][r] X'[p], runs the
     * recurrence, and writes o[p] = sum_r W_O[h][p][r] Y[r][p] SiLU(W_Z[h][p][r] Z'[p])
     * instead of y. Needs the bf16 matrix-core shape (M3_ERR_UNSUPPORTED otherwise). */
    const void *z;         /* [b,L,H,P] io: Z' */
    const float *W_X;      /* [H,P,R] rank expansion of X' */
    const float *W_Z;      /* [H,P,R] rank expansion of Z' */
    const float *W_O;      /* [H,P,R] contraction of the gated output over the ranks */
    void *o;               /* out [b,L,H,P] io */
    /* Output epilogue. D: skip term y += D[h] x on every rank row (with W_X set,
     * x is the expanded X), the D term of the SSM output equation y = C h + D x
     * (szyisi.cn article on Mamba-3, state space model section). NULL = none. */
    const float *D;        /* [H] */
    const float *out_normw; /* [H,P] gain of the output norm (M3_FLAG_OUT_NORM); NULL = ones */
} m3_scan_io;

/* Decode (single token) arguments: the per-token tensors have no L axis. */
typedef struct {
    const void *x;         /* [b,H,R,P] io */
    const void *Braw;      /* [b,G,R,N] io */
    const void *Craw;      /* [b,G,R,N] io */
    const float *dt;       /* [b,H] */
    const float *A;        /* [b,H] */
    const float *lam;      /* [b,H] */
    const float *theta;    /* [b,G,N/2] */
    const float *B_bias;   /* [H,R,N] */
    const float *C_bias;   /* [H,R,N] */
    const float *B_normw;  /* [N] or NULL */
    const float *C_normw;  /* [N] or NULL */
    const void *x_prev;    /* [b,H,R,P] io, previous token, or NULL (first token) */
    const void *Braw_prev; /* [b,G,R,N] io, or NULL; both or neither */
    void *h;               /* in/out [b,H,P,N] state, updated in place: fp32, or bf16
                              with M3_FLAG_BF16_STATE */
    void *y;               /* out [b,H,R,P] io (not written, may be NULL, with W_X set) */
    /* Fused MIMO projections and gate, as in m3_scan_io: x and x_prev are X' [b,H,P] */
    const void *z;         /* [b,H,P] io: Z' */
    const float *W_X;      /* [H,P,R] */
    const float *W_Z;      /* [H,P,R] */
    const float *W_O;      /* [H,P,R] */
    void *o;               /* out [b,H,P] io */
    const float *D;        /* [H] skip term, as in m3_scan_io, or NULL */
    const float *out_normw; /* [H,P] output-norm gain, as in m3_scan_io, or NULL */
} m3_decode_io;

/* Gradients of the prefill (m3_scan_bwd): upstream gradients in, the gradient of
 * <dy, y> + <dh_final, h_final> with respect to every forward input out. All
 * outputs are fp32 and fully overwritten. */
typedef struct {
    const void *dy;          /* [b,L,H,R,P] io: gradient of y */
    const float *dh_final;   /* [b,H,P,N] gradient of h_final, or NULL (zero) */
    float *dx;               /* [b,L,H,R,P] */
    float *dBraw;            /* [b,L,G,R,N] */
    float *dCraw;            /* [b,L,G,R,N] */
    float *ddt;              /* [b,L,H] */
    float *dA;               /* [b,L,H] */
    float *dlam;             /* [b,L,H] */
    float *dtheta;           /* [b,L,G,N/2] */
    float *dB_bias;          /* [H,R,N] */
    float *dC_bias;          /* [H,R,N] */
    float *dB_normw;         /* [N]: required when the forward had B_normw, else NULL */
    float *dC_normw;         /* [N]: required when the forward had C_normw, else NULL */
    float *dh0;              /* [b,H,P,N] gradient of the initial state, or NULL (not wanted) */
    float *dx_prev;          /* [b,H,R,P]: required when the forward had x_prev, else NULL */
    float *dBraw_prev;       /* [b,G,R,N]: likewise */
} m3_scan_grads;

/* What m3_scan_fwd will launch for a shape (for logs and tests). */
typedef struct {
    int32_t kernel;         /* 0 = fp32 vector-ALU chunked kernel, 1 = bf16 matrix-core kernel */
    int32_t nsegments;      /* segments per sequence (1 = single pass) */
    int64_t workgroups;     /* workgroups of the main (output) pass */
    size_t workspace_bytes; /* bytes of caller workspace required */
} m3_plan;

/* Chunked-scan prefill: y for every position and the final state.
 * Chunked algorithm of §3.3 (quadratic masked form inside a chunk, §3.1.3 eq. 7
 * mask; linear state passing between chunks) on B and C rotated by the
 * cumulative angle (§3.2.2, Proposition 4). Returns M3_OK or a negative status.
 * workspace may be NULL when m3_scan_workspace_bytes returns 0. The bf16
 * matrix-core path always takes one: B and C after BCNorm and its gain, computed
 * once per (token, group, rank) row rather than once per head (2 * b*L*G*R * N/2
 * f16 pairs, 4 * b*L*G*R*N bytes), then, when the sequence is split, the segment
 * records. Its contents need not be initialised and are not kept. */
m3_status m3_scan_fwd(const m3_shape *shape, const m3_scan_io *io, void *workspace,
                      size_t ws_bytes, void *stream);

/* m3_scan_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, kernels and results as m3_scan_fwd, but the workspace is a device
 * array inside the library, fixed at m3_scan_noalloc_max_workspace_bytes()
 * (256 MiB) per GPU, held by each GPU the library runs on until the process
 * ends. Every automatic plan with at most 2^18 raw B rows (b*L*G*R) fits: the
 * normalised rows take 128 MiB there and the segment records at most ~36 MB.
 * The call allocates and frees nothing. On its first use on a device it looks up
 * that device's copy of the array (a host-side query, no allocation). A plan
 * whose workspace exceeds the maximum returns M3_ERR_WORKSPACE_TOO_SMALL before
 * any HIP call; the caller then splits the batch.
 * Calls on one GPU share its array, which keeps the last call's contents; no
 * part of it needs to start at zero. Calls that overlap on one GPU (on different
 * streams, or replayed graphs running concurrently) race on the array: the
 * caller serialises them. */
m3_status m3_scan_fwd_noalloc(const m3_shape *shape, const m3_scan_io *io, void *stream);

/* The fixed workspace size of m3_scan_fwd_noalloc, in bytes. */
size_t m3_scan_noalloc_max_workspace_bytes(void);

/* Bytes of device workspace m3_scan_fwd needs for this shape (0 if none). */
size_t m3_scan_workspace_bytes(const m3_shape *shape);

/* Fill *plan with what m3_scan_fwd would launch; validates like m3_scan_fwd
 * (without the pointer checks). */
m3_status m3_scan_plan(const m3_shape *shape, m3_plan *plan);

/* One decode step in place: h <- R_t(alpha h + beta B_prev x_prev^T) + gamma B x^T,
 * y = h^T C (App. B.3 eq. 25 with App. C's rank-R form). Decode requires
 * N in {16, 32, 64, 128, 256}, P <= 256, R <= 4. */
m3_status m3_decode_step(const m3_shape *shape, const m3_decode_io *io, void *stream);

/* Prefill backward: the gradients of the chunked scan for training (the forward
 * being m3_scan_fwd with the same shape and io). The pages give no backward; this
 * is the adjoint of the chunked algorithm of §3.3 in the rotated frame of §3.2.2
 * (Proposition 4), taken term by term: masked scores, carried state, decay,
 * trapezoid weights (§3.1.3 eq. 7), rotation angles and BCNorm + bias (§3.4).
 * Computed in fp32 for io fp32 or bf16, any L; shapes as for the fp32 prefill
 * kernel (N, P <= 128, N * P <= 8192, R <= 4) with N and P multiples of 4. shape->chunk is not used: the
 * backward picks its own chunk (32 / R tokens), the result does not depend on it.
 * The fused projections and the output epilogue are not differentiated here
 * (M3_ERR_UNSUPPORTED when io->W_X or io->D is set or M3_FLAG_OUT_NORM is on);
 * io->y and io->h_final are not read. The workspace (m3_scan_bwd_workspace_bytes)
 * holds chunk-start states and per-head partial gradients. */
m3_status m3_scan_bwd(const m3_shape *shape, const m3_scan_io *io, const m3_scan_grads *grads,
                      void *workspace, size_t ws_bytes, void *stream);

/* Bytes of device workspace m3_scan_bwd needs for this shape. */
size_t m3_scan_bwd_workspace_bytes(const m3_shape *shape);

/* The MIMO projections of App. C as stand-alone steps, for callers that run the
 * core without the fused form (and the unfused baseline of the fused path). Both
 * use shape->batch, seqlen (1 for a decode token), nheads, headdim P (a multiple
 * of 8), rank R (<= 4) and io_dtype; rows are the batch * seqlen * nheads (token,
 * head) pairs. Weights are [H,P,R] fp32. Pointers 16-byte aligned; nothing is
 * allocated; M3_ERR_UNSUPPORTED for P % 8 != 0, P > 2048 or R > 4, or more than
 * 65535 heads.
 *
 * m3_expand_ranks: the rank expansion X = W_X (.) X' of App. C,
 *   x_out[b,L,H,R,P][r][p] = W_X[h][p][r] * x_in[b,L,H,P][p]            (io dtype) */
m3_status m3_expand_ranks(const m3_shape *shape, const void *x_in, const float *W_X, void *x_out, void *stream);

/* m3_gate_contract: App. C's gate and rank contraction after the core,
 *   o[b,L,H,P][p] = sum_r W_O[h][p][r] * y[b,L,H,R,P][r][p] * SiLU(W_Z[h][p][r] * z_in[b,L,H,P][p])
 * with SiLU(v) = v / (1 + e^-v); y, z_in, o in the io dtype, accumulated in fp32. */
m3_status m3_gate_contract(const m3_shape *shape, const void *y, const void *z_in, const float *W_Z,
                           const float *W_O, void *o, void *stream);

/* Human-readable name of a status code (static string). */
const char *m3_status_str(m3_status status);

/* Library ABI version (major * 100 + minor). */
int m3_version(void);

#ifdef __cplusplus
}
#endif
#endif /* M3_H */
