// Matrix-core chunked-scan prefill of the Mamba-3 SSM core for gfx950.
//
// Shape: bf16 io, N = 128 state, P = 64 head dim, 64 rows per chunk where a row
// is a (token, rank) pair: chunk = 64 / R tokens (the pages' rule "64 / mimo_rank"
// for bf16; Mamba-3 paper §3.3 "chunked algorithm for MIMO", with the chunk
// chosen so that the intra-chunk tile stays 64 x 64).
//
// Method (see the fp32 kernel for the same algebra written plainly):
//   rotated frame (§3.2.2 Proposition 4 / App. B.3): B_bar = R(-Phi) B,
//   C_bar = R(-Phi) C, Phi = cumulative dt*theta from the workgroup's first token;
//   folded trapezoid weights w_s = lam_s dt_s + (1-lam_{s+1}) dt_{s+1};
//   per chunk (SSD chunked algorithm, §3.3, mask of §3.1.3 eq. 7):
//     S^T = B_bar C_bar^T                        (MFMA, K = N)
//     P^T = S^T o L^T,  L[t,s] = exp(cs_t - cs_s) w_s (s<t), gamma_t (s=t)
//     Y   = diag(exp(cs_t)) C_bar H~ + P X        (MFMA, K = N and K = rows)
//     H~ <- exp(cs_end) H~ + B_bar^T diag(exp(cs_end - cs_s) w_s) X   (MFMA, K = rows)
//   final state H = R(Phi_end) H~.
//
// One workgroup (4 waves) owns one (batch, head) chain, or one segment of it
// when the sequence is split (state passing, App. G.2: pass 1 computes each
// segment's end state from zero, a combine kernel chains them, pass 2 produces
// the outputs from the right incoming states). Wave w:
//   * rotates the 16 rows 16w..16w+15 of the chunk (each lane: one row, 32 of
//     the 128 state columns, i.e. 16 rotation pairs (i, i+64)), which leaves the
//     lane holding exactly its MFMA fragments of B_bar and C_bar;
//   * owns output rows 16w..16w+15 (S^T blocks s <= t, mask, Y);
//   * owns state columns n in [16w, 16w+16) and [64+16w, 64+16w+16) (so each
//     rotation pair of the state is held by one lane) for all 64 p.
// MFMA: v_mfma_f32_16x16x32_bf16. Operand fragments: lane l holds row l%16 and
// K-slots 8*(l/16)..+7; the accumulator holds rows 4*(l/16)..+3 of column l%16.
// P^T comes out of the first MFMA already in the A-operand layout of P (K-slots
// taken in accumulator order), so it never goes through LDS.
//
// LDS (bf16 tiles with rows padded by 16 bytes, ~69 KiB, two workgroups
// per CU): B_bar [row][n], B_bar*scale transposed [n][row], X transposed
// [p][row], the bf16 copy of the state transposed [p][n] for the Y_off product,
// and small per-row scalar tables.
#include <type_traits>

#include "m3_internal.h"

namespace m3i {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kN = 128, kP = 64, kRows = 64, kHalf = 64;
// LDS row strides (elements): 16 bytes of padding per row puts the 8 rows that
// one 16-byte fragment read touches on 8 different bank groups
constexpr int kLdN = kN + 8;     // tiles with 128 columns (B_bar, state)
constexpr int kLdR = kRows + 8;  // tiles with 64 columns (B_bar^T, X^T)

// Column order of the B_bar^T and X^T tiles: rows 32m + 16h + 4g + j (h, j < 2, 4) sit at slot
// 32m + 8g + 4h + j. A lane's K-slots of a 16x16x32 product against the score accumulators (rows
// 32m + 4g + j and 32m + 16 + 4g + j) are then one 16-byte read; the state update reads the same
// slots from both of its operands, so its K order only changes with the slot order.
__device__ __forceinline__ constexpr int row_slot(int w, int lg) { return 32 * (w >> 1) + 8 * lg + 4 * (w & 1); }
constexpr int kThreads = 256;
constexpr int kCUs = 256;  // MI355X compute units: 2 resident workgroups each
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInv2Pi = 0.15915494309189535f;

// kFull: one pass over the whole sequence. Segment split (state passing):
//   kPass1 + combine + kPass2: end states only, then every segment again from its
//     incoming state (used with the output norm, which is not linear in y);
//   kLocal + combine + kCorrect: every segment's outputs and end state from a
//     zero state, then the outputs corrected for the incoming state. The
//     recurrence is linear in its initial state: a token's output gains
//     e^{cs_t} C_bar_t^T H_in, with cs_t the decay from the segment start, and
//     nothing else. The correction pass rotates only C, has no input term and
//     stops once the decay since the segment start falls below e^kCorrectStop,
//     where the term is far below the output's rounding.
enum Mode { kFull = 0, kPass1 = 1, kPass2 = 2, kLocal = 3, kCorrect = 4 };
constexpr float kCorrectStop = -80.f;

// A value the compiler cannot see through: lane-derived indices computed from it
// inside the chunk loop are recomputed each iteration instead of being hoisted
// out of the loop and kept live (or spilled) across it.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float dpp_row_shr(float v, int k) {
    // lanes whose source falls outside their 16-lane row read 0
    int r;
    switch (k) {
        case 1: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false); break;
        case 4: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false); break;
        default: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false); break;
    }
    return __int_as_float(r);
}

// Angles are kept in revolutions (turns): the hardware sine/cosine take them
// directly, and the running total can be reduced mod 1 without changing any
// rotation, which keeps its fp32 resolution over long sequences.
__device__ __forceinline__ void sincos_rev(float x, float &s, float &c) {
    const float rev = __builtin_amdgcn_fractf(x);
    s = __builtin_amdgcn_sinf(rev);
    c = __builtin_amdgcn_cosf(rev);
}

// x summed over lanes l, l^16, l^32, l^48 (the four 16-lane rows of the wave),
// through the gfx950 row swaps instead of an LDS round trip
__device__ __forceinline__ float sum_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A quad permute whose result is an operand rather than an addend: every lane has a
// source, so no "old" value is materialised (an update with old = 0 costs a zeroing
// move where the permute is not folded into an add).
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
    static_assert(CTRL <= 0xFF, "quad permutes only");
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Rotation of f16 pairs v = (lo, hi) by their angles, in fp32 (v_dot2_f32_f16):
// lo' = cos lo + sin hi = dot(v, (cos, sin)), hi' = cos hi - sin lo =
// dot(v, (-sin, cos)); cs = (cos, sin) and sc = (sin, cos) of each pair's angle,
// the second product negating the low half of sc through the encoding's neg_lo.
// Written out because the compiler's form of the builtin accumulates into its
// destination and needs a zeroing move per product, and does not fold the
// negation. A vector instruction that reads a dot product's result needs 3 wait
// states after it, which the compiler inserts only for dot instructions it
// emitted itself: each block ends with s_nop 2, and its outputs are early-clobber
// (written while inputs are still read).
__device__ __forceinline__ void rot_pairs2(h2 v0, h2 v1, h2 cs0, h2 sc0, h2 cs1, h2 sc1, float &l0, float &h0,
                                           float &l1, float &h1) {
    asm("v_dot2_f32_f16 %0, %4, %6, 0\n\t"
        "v_dot2_f32_f16 %1, %4, %7, 0 neg_lo:[0,1,0]\n\t"
        "v_dot2_f32_f16 %2, %5, %8, 0\n\t"
        "v_dot2_f32_f16 %3, %5, %9, 0 neg_lo:[0,1,0]\n\t"
        "s_nop 2"
        : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1)
        : "v"(v0), "v"(v1), "v"(cs0), "v"(sc0), "v"(cs1), "v"(sc1));
}
// two rows (B and C) sharing the angles of two slots
__device__ __forceinline__ void rot_pairs4(h2 b0, h2 b1, h2 c0, h2 c1, h2 cs0, h2 sc0, h2 cs1, h2 sc1, float *ob,
                                           float *oc) {
    asm("v_dot2_f32_f16 %0, %8, %12, 0\n\t"
        "v_dot2_f32_f16 %1, %8, %13, 0 neg_lo:[0,1,0]\n\t"
        "v_dot2_f32_f16 %2, %9, %14, 0\n\t"
        "v_dot2_f32_f16 %3, %9, %15, 0 neg_lo:[0,1,0]\n\t"
        "v_dot2_f32_f16 %4, %10, %12, 0\n\t"
        "v_dot2_f32_f16 %5, %10, %13, 0 neg_lo:[0,1,0]\n\t"
        "v_dot2_f32_f16 %6, %11, %14, 0\n\t"
        "v_dot2_f32_f16 %7, %11, %15, 0 neg_lo:[0,1,0]\n\t"
        "s_nop 2"
        : "=&v"(ob[0]), "=&v"(ob[1]), "=&v"(ob[2]), "=&v"(ob[3]), "=&v"(oc[0]), "=&v"(oc[1]), "=&v"(oc[2]),
          "=&v"(oc[3])
        : "v"(b0), "v"(b1), "v"(c0), "v"(c1), "v"(cs0), "v"(sc0), "v"(cs1), "v"(sc1));
}

// Smallest e with m <= 2^e for finite m > 0 (-126 for m == 0), clamped to
// [-126, 100]; exact, from the bits.
__device__ __forceinline__ int exp_ceil(float m) {
    if (!(m > 0.f)) return -126;
    const unsigned u = __float_as_uint(m);
    int e = (int)((u >> 23) & 0xff) - 127;
    if (u & 0x7fffff) ++e;
    return e < -126 ? -126 : (e > 100 ? 100 : e);
}

struct alignas(16) Smem {
    alignas(16) __bf16 Bb[kRows * kLdN];  // B_bar [row][n]
    alignas(16) __bf16 Bt[kN * kLdR];     // B_bar * cst, [n][row slot] (row slots: row_slot())
    alignas(16) __bf16 Xt[kP * kLdR];     // X, [p][row slot]
    alignas(16) __bf16 St[kP * kLdN];     // bf16 state, [p][n]
    alignas(16) float l2cs[kRows];        // per row: log2(e) * chunk-local cumulative log decay
    alignas(16) float wgt[kRows];         // per row: folded weight w of the row's token
    alignas(16) float gam[kRows];         // per row: gamma
    alignas(16) float eoff[kRows];        // per row: exp(cs) (carried-state output scale)
    alignas(16) float cstt[kRows];        // per row: exp(cs_end - cs) w (state-input weight)
    alignas(16) float ftab[kRows];        // per row t >= 16: exp(cs_t - cs_ref), ref = last row of the block before t's
    alignas(16) float tw[3][kRows];       // [w-1][s]: exp(cs_ref(w) - cs_s) w_s for s < 16w, else 0
    alignas(16) float tok[3][kRows];      // dt, A, lambda of each row's token (next chunk's, staged)
    alignas(16) float tokn[4];            // dt, lambda of the token after that chunk
    alignas(16) float angtot[4][kHalf];   // per wave: angle total of its rows (revolutions)
    alignas(16) float carry[kHalf];       // cumulative angle before the current chunk, mod 1 revolution
    alignas(16) float woff[4][kHalf];     // per wave: angle offset of its rows (carry + earlier waves' totals)
    alignas(16) unsigned bq[2][4][kHalf];  // B / C bias of this head per rank, f16 pairs (n, n + 64), scaled
    alignas(16) float mx[4][4];           // prologue: per-wave maxima of |gain| and |bias|
    alignas(16) float onw[kP];            // output-norm gain of this head (ones when absent)
};

// with the fused rank projections: W_X, W_Z, W_O of this head, [rank][p]
struct SmemFused : Smem {
    alignas(16) float fw[3][4][kP];
};

struct ChainPos {
    int64_t chain, seg, c_begin, c_end;
};

__device__ __forceinline__ ChainPos chain_of_block(const ScanArgs &a, const SplitPlan &sp, int mode) {
    // Blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous range
    // of (segment, chain) so heads that share B, C, theta share an L2.
    const int64_t nchains = a.b * a.H;
    const int64_t nseg = (mode == kFull) ? 1 : sp.nseg;
    const int64_t total = nchains * nseg;
    const int64_t id = blockIdx.x;
    int64_t lin = id;
    if (total % 8 == 0) lin = (id % 8) * (total / 8) + id / 8;
    ChainPos cp;
    cp.seg = lin / nchains;
    cp.chain = lin % nchains;
    const int64_t nchunks = (a.L + a.C - 1) / a.C;
    if (mode == kFull) {
        cp.c_begin = 0;
        cp.c_end = nchunks;
    } else {
        cp.c_begin = cp.seg * sp.seg_chunks;
        cp.c_end = cp.c_begin + sp.seg_chunks < nchunks ? cp.c_begin + sp.seg_chunks : nchunks;
    }
    return cp;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: Hillis-Steele
// inside each 16-lane row, then the row totals carried by row broadcasts.
__device__ __forceinline__ float wave_incl_scan(float v) {
#pragma clang fp contract(off)  // a caller's product fused into the first step takes its DPP add apart
    v += dpp_row_shr(v, 1);
    v += dpp_row_shr(v, 2);
    v += dpp_row_shr(v, 4);
    v += dpp_row_shr(v, 8);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return v;
}

// Per-lane constants of the chunk loop (fixed for the workgroup's lifetime).
struct Lane {
    int l, lr, lg, row, r_row, t_row;
    int offX;  // element offset of this lane's row in a chunk's x (and y) block
};

template <int R>
__device__ __forceinline__ Lane make_lane(int l, int w, int64_t H) {
    Lane ln;
    ln.l = l;
    ln.lr = l & 15;
    ln.lg = l >> 4;
    ln.row = 16 * w + ln.lr;
    ln.r_row = ln.row % R;
    ln.t_row = ln.row / R;
    ln.offX = (ln.t_row * (int)H * R + ln.r_row) * kP;
    return ln;
}

// Uniform (per workgroup and chunk) bases of a chunk's blocks. With the fused
// projections x is X' and z is Z' (one row of P per token, no rank axis) and the
// output goes to o, also one row per token.
struct ChunkBase {
    const unsigned *qB, *qC;  // normalised B, C rows (f16 pairs)
    const __bf16 *x, *z;
    const float *th;
    const float *dt, *A, *lam;
    __bf16 *y;
};

template <int R, bool FUSED>
__device__ __forceinline__ ChunkBase chunk_base(const ScanArgs &a, int64_t bi, int64_t hi, int64_t g, int64_t c0) {
    ChunkBase cb;
    const int64_t t0 = bi * a.L + c0;  // first token of the chunk
    cb.qB = a.Bq + (t0 * a.G + g) * R * kHalf;
    cb.qC = a.Cq + (t0 * a.G + g) * R * kHalf;
    cb.th = a.theta + (t0 * a.G + g) * kHalf;
    constexpr int XR = FUSED ? 1 : R;  // x rows per token
    cb.x = static_cast<const __bf16 *>(a.x) + (t0 * a.H + hi) * XR * kP;
    cb.y = static_cast<__bf16 *>(FUSED ? a.o : a.y) + (t0 * a.H + hi) * XR * kP;
    cb.z = FUSED ? static_cast<const __bf16 *>(a.z) + (t0 * a.H + hi) * kP : nullptr;
    cb.dt = a.dt + t0 * a.H + hi;
    cb.A = a.A + t0 * a.H + hi;
    cb.lam = a.lam + t0 * a.H + hi;
    return cb;
}

// Global inputs of one chunk for one lane: its row's normalised B and C pairs
// (pairs 8lg..8lg+7 and 32+8lg..32+8lg+7), theta and X (MFMA fragment layout).
// Loaded one chunk ahead so the loads are in flight while the previous chunk is
// computed.
struct ChunkRegs {
    u32x4 qb[4], qc[4];
    bf16x8 xf[2];
    bf16x4 zf[4];  // fused projections: Z' of the row's token at the lane's output columns
    f32x4 th[4];  // theta of the lane's angle slots: all 4 blocks for R = 1, its own 4 / R blocks otherwise
};

// nv: tokens of the chunk; avail: tokens from the chunk's first one to the end
// of the sequence (capped at C + 1).
template <int MODE, int R, bool FUSED>
__device__ __forceinline__ void load_chunk(const ChunkBase &cb, const Lane &ln, int nv, int avail, int64_t G,
                                           int64_t H, ChunkRegs &cr) {
    // Every load is unconditional, from a clamped index; the consumer zeroes what
    // lies past the chunk. Offsets are all formed before the first load is issued:
    // address arithmetic interleaved with the loads had let a 32-bit multiply-add
    // take a just-loaded register as its unused high half, and the wave then
    // waited for that load.
    // fragment rows past the end read the last token's data: finite values whose
    // weights, gamma, state weight and angle increment are all zero, and whose
    // outputs are not stored
    const int tr = ln.t_row < nv ? ln.t_row : nv - 1;
    int offBC = (tr * (int)G * R + ln.r_row) * kHalf + 8 * ln.lg;
    int oth = tr * (int)G * kHalf;
    int offx = FUSED ? tr * (int)H * kP : (tr * (int)H * R + ln.r_row) * kP;
    asm volatile("" : "+v"(offBC), "+v"(oth), "+v"(offx));
    // angle slot block b (4 channels) of lane group lg starts at channel
    // 32 (b >> 1) + 8 lg + 4 (b & 1), i.e. float4 8 (b >> 1) + 2 lg + (b & 1). The R
    // rank lanes of a token share its angles: rank r owns blocks (4 / R) r ..
    auto load_theta = [&]() {
        const f32x4 *pt = reinterpret_cast<const f32x4 *>(cb.th + oth);
#pragma unroll
        for (int q = 0; q < 4 / R; ++q) {
            const int b = (4 / R) * ln.r_row + q;
            cr.th[q] = pt[8 * (b >> 1) + 2 * ln.lg + (b & 1)];
        }
    };
    auto load_pairs = [&]() {
        const u32x4 *pb = reinterpret_cast<const u32x4 *>(cb.qB + offBC);
        const u32x4 *pc = reinterpret_cast<const u32x4 *>(cb.qC + offBC);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int o = (k >> 1) * 8 + (k & 1);  // pairs 8lg + 4k (k < 2), 32 + 8lg + 4(k - 2)
            if constexpr (MODE != kCorrect) cr.qb[k] = pb[o];
            if constexpr (MODE != kPass1) cr.qc[k] = pc[o];
        }
    };
    auto load_z = [&]() {
        if constexpr (FUSED && MODE != kPass1) {
            // columns p = 16pb + 4lg..+3 of the output rows this lane holds
            const bf16x4 *pz = reinterpret_cast<const bf16x4 *>(cb.z + offx + 4 * ln.lg);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) cr.zf[pb] = pz[4 * pb];
        }
    };
    auto load_x = [&]() {
        if constexpr (MODE != kCorrect) {
            const bf16x8 *px = reinterpret_cast<const bf16x8 *>(cb.x + offx);
            cr.xf[0] = px[ln.lg];
            cr.xf[1] = px[4 + ln.lg];
        }
    };
    // A wait for a load also waits for every load issued before it. For R > 1 the
    // loads go in the order of first use: theta (the chunk top's angle prefix), Z'
    // (the fused gate factor, also at the top), X, then the B / C pairs (after B1):
    // MIMO-4 1.138 -> 1.121 ms, long 0.973 -> 0.956 ms, fused 1.277 -> 1.262 ms. For
    // R = 1 that order was 4% slower; its pairs go first.
    if constexpr (R == 1) {
        load_pairs();
        load_theta();
        load_x();
        load_z();
    } else {
        load_theta();
        load_z();
        load_x();
        load_pairs();
    }
}

// Token scalars of chunk cc for this wave's 16 rows, one load per lane: lane
// groups 0, 1, 2 take dt, A, lambda of row 16w + lr (token (16w + lr) / R); lane
// group 3 takes the dt (even lr) or lambda (odd lr) of the token after the chunk.
// Tokens are H floats apart, so a per-lane load of all 64 rows by every wave
// touched 4x the cache lines. Indices are clamped into the sequence; the reader
// zeroes what lies past it.
typedef __attribute__((address_space(1))) const float gfloat;  // global memory

// sbase: this lane's array (scalar_base) offset to head hi.
template <int R>
__device__ __forceinline__ float load_scalars(const ScanArgs &a, gfloat *sbase, int64_t bi, int64_t cc,
                                              const Lane &ln) {
    constexpr int C = kRows / R;
    const int64_t c0 = cc * C;
    const int nv = (int)((a.L - c0) < C ? (a.L - c0) : C);
    const int avail = (int)((a.L - c0) < C + 1 ? (a.L - c0) : C + 1);
    const int t = ln.lg < 3 ? (ln.row / R < nv ? ln.row / R : nv - 1) : (C < avail ? C : avail - 1);
    int ot = t * (int)a.H;
    asm volatile("" : "+v"(ot));
    return sbase[(bi * a.L + c0) * a.H + ot];
}

// The array a lane of load_scalars reads (dt, A or lambda), offset to head hi.
// The three pointers pass through an empty asm so that the per-lane choice is a
// register select: a short-circuit condition had been compiled to divergent
// branches that left the odd lanes of group 3 on the dt pointer, and a plain
// select to a per-lane load of the pointer from the argument block.
__device__ __forceinline__ gfloat *scalar_base(const ScanArgs &a, int64_t hi, int lg, int lr) {
    gfloat *pd = (gfloat *)a.dt, *pa = (gfloat *)a.A, *pl = (gfloat *)a.lam;
    asm("" : "+s"(pd), "+s"(pa), "+s"(pl));
    const int k = lg < 3 ? lg : 2 * (lr & 1);  // 0: dt, 1: A, 2: lambda
    return (k == 0 ? pd : (k == 1 ? pa : pl)) + hi;
}

// bf16x8 fragment with a single 1.0 at slot j (none when j is outside 0..7)
__device__ __forceinline__ bf16x8 unit_fragment(int j) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 u;
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = (j == 2 * k ? 0x3F80u : 0u) | (j == 2 * k + 1 ? 0x3F800000u : 0u);
    return __builtin_bit_cast(bf16x8, u);
}

// X' (fused projections) or x of the previous token, element (r, p)
template <int R, bool FUSED>
__device__ __forceinline__ float prev_x(const ScanArgs &a, int64_t bi, int64_t hi, int r, int p) {
    if constexpr (FUSED) {
        const __bf16 *xp = static_cast<const __bf16 *>(a.x_prev) + (bi * a.H + hi) * kP;
        return a.W_X[(hi * kP + p) * R + r] * (float)xp[p];
    } else {
        const __bf16 *xp = static_cast<const __bf16 *>(a.x_prev) + ((bi * a.H + hi) * R) * kP;
        return (float)xp[r * kP + p];
    }
}

template <int MODE, int R, bool FUSED, bool ONORM>
__global__ __launch_bounds__(kThreads, 2) void scan_mfma_kernel(ScanArgs a, SplitPlan sp) {
    constexpr int C = kRows / R;  // tokens per chunk
    __shared__ typename std::conditional<FUSED, SmemFused, Smem>::type sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const ChainPos pos = chain_of_block(a, sp, MODE);
    const int64_t chain = pos.chain;
    const int64_t bi = chain / a.H, hi = chain % a.H, g = hi / (a.H / a.G);
    const int64_t L = a.L, H = a.H, G = a.G;

    const int l = tid & 63, lr = l & 15, lg = l >> 4;

    // ---------------------------------------------------------------- prologue
    // Scales of the f16 rotation inputs. The normalised rows hold u g 2^-eg, with
    // |u| <= sqrt(N) after BCNorm and max |g| <= 2^eg, so they stay below sqrt(N).
    // This head adds its bias scaled by 2^-k, with k >= eg the least exponent that
    // keeps |bias| 2^-k <= 2^14: the f16 sums stay finite for any gains and biases.
    // The rotated B_bar and C_bar are then 2^-kB and 2^-kC times the true ones; the
    // per-row tables of the chunk loop carry the inverse powers of two (exact).
    h2 rrB, rrC;  // 2^(eg - k) per matrix: the factor of the normalised rows
    float sB, sC, sBC;
    {
        float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
        if (tid < kN) {
            m0 = a.B_normw ? fabsf(a.B_normw[tid]) : 1.f;
            m1 = a.C_normw ? fabsf(a.C_normw[tid]) : 1.f;
        }
        for (int e = tid; e < R * kN; e += kThreads) {
            m2 = fmaxf(m2, fabsf(a.B_bias[hi * R * kN + e]));
            m3 = fmaxf(m3, fabsf(a.C_bias[hi * R * kN + e]));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            m0 = fmaxf(m0, __shfl_xor(m0, o));
            m1 = fmaxf(m1, __shfl_xor(m1, o));
            m2 = fmaxf(m2, __shfl_xor(m2, o));
            m3 = fmaxf(m3, __shfl_xor(m3, o));
        }
        if (l == 0) {
            sm.mx[w][0] = m0;
            sm.mx[w][1] = m1;
            sm.mx[w][2] = m2;
            sm.mx[w][3] = m3;
        }
        __syncthreads();
        f32x4 m = *reinterpret_cast<const f32x4 *>(&sm.mx[0][0]);
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(&sm.mx[k][0]);
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = fmaxf(m[j], v[j]);
        }
        const int egB = max(0, exp_ceil(m[0])), egC = max(0, exp_ceil(m[1]));
        const int kB = __builtin_amdgcn_readfirstlane(max(egB, exp_ceil(m[2]) - 14));
        const int kC = __builtin_amdgcn_readfirstlane(max(egC, exp_ceil(m[3]) - 14));
        const _Float16 fB = (_Float16)ldexpf(1.f, egB - kB), fC = (_Float16)ldexpf(1.f, egC - kC);
        rrB = h2{fB, fB};
        rrC = h2{fC, fC};
        sB = ldexpf(1.f, kB);
        sC = ldexpf(1.f, kC);
        sBC = ldexpf(1.f, kB + kC);
        for (int e = tid; e < 2 * R * kHalf; e += kThreads) {
            const int which = e / (R * kHalf), r = (e / kHalf) % R, i = e % kHalf;
            const float *bsrc = (which == 0 ? a.B_bias : a.C_bias) + (hi * R + r) * kN;
            const int k = which == 0 ? kB : kC;
            const h2 v = {(_Float16)ldexpf(bsrc[i], -k), (_Float16)ldexpf(bsrc[i + kHalf], -k)};
            sm.bq[which][r][i] = __builtin_bit_cast(unsigned, v);
        }
    }
    if (tid < kHalf) sm.carry[tid] = 0.f;
    if constexpr (ONORM) {
        if (tid < kP) sm.onw[tid] = a.out_normw ? a.out_normw[hi * kP + tid] : 1.f;
    }
    // skip term D x: added to the diagonal of the masked scores (P[t][t] += D), so
    // the X^T P^T product carries it
    const float dsk = (MODE != kPass1 && MODE != kCorrect && a.D) ? a.D[hi] : 0.f;
    if constexpr (FUSED) {
        // global W is [H][P][R]: e runs over (p, r) of this head, rank fastest
        for (int e = tid; e < 3 * R * kP; e += kThreads) {
            const int which = e / (R * kP), rem = e % (R * kP);
            const float *W = (which == 0) ? a.W_X : ((which == 1) ? a.W_Z : a.W_O);
            sm.fw[which][rem % R][rem / R] = W[hi * (R * kP) + rem];
        }
    }

    // state fragments: acc[q][pb] holds state[n = 16(w+4q) + 4lg + j][p = 16pb + lr]
    f32x4 acc[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[q][pb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (MODE == kCorrect) {
        // segment 0 has nothing to correct without an initial state or previous token
        if (pos.seg == 0 && !a.h0 && !a.has_prev) return;
    }
    if constexpr (MODE == kFull || MODE == kPass2 || MODE == kCorrect) {
        const float *src = nullptr;
        if (MODE == kFull)
            src = a.h0 ? a.h0 + chain * (kP * kN) : nullptr;
        else
            src = sp.seg_state + (chain * sp.nseg + pos.seg) * (kP * kN);
        if (src) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const int n0 = 16 * (w + 4 * q) + 4 * lg, p = 16 * pb + lr;
                    acc[q][pb] = *reinterpret_cast<const f32x4 *>(src + p * kN + n0);
                }
        }
    }
    if constexpr (MODE == kFull) {
        if (a.has_prev && L > 0) {
            // fold (1 - lam_0) dt_0 B_{-1} x_{-1}^T into the starting state
            const __bf16 *bp = static_cast<const __bf16 *>(a.Braw_prev) + ((bi * G + g) * R) * kN;
            float rsr[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float v0 = (float)bp[r * kN + 2 * l], v1 = (float)bp[r * kN + 2 * l + 1];
                rsr[r] = __builtin_amdgcn_rsqf(wave_sum(v0 * v0 + v1 * v1) * (1.f / kN) + a.eps);
            }
            const int64_t o0 = (bi * L) * H + hi;
            const float f = (1.f - a.lam[o0]) * a.dt[o0];
            const float *bb = a.B_bias + (hi * R) * kN;
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int pb = 0; pb < 4; ++pb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = 16 * (w + 4 * q) + 4 * lg + j, p = 16 * pb + lr;
                        const float wn = a.B_normw ? a.B_normw[n] : 1.f;
                        float s = 0.f;
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            s += ((float)bp[r * kN + n] * rsr[r] * wn + bb[r * kN + n]) *
                                 prev_x<R, FUSED>(a, bi, hi, r, p);
                        acc[q][pb][j] += f * s;
                    }
        }
    }
    if constexpr (MODE != kPass1) {
        // bf16 copy of the state for the first chunk's carried-state output
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int n0 = 16 * (w + 4 * q) + 4 * lg, p = 16 * pb + lr;
                bf16x4 v = {(__bf16)acc[q][pb][0], (__bf16)acc[q][pb][1], (__bf16)acc[q][pb][2],
                            (__bf16)acc[q][pb][3]};
                *reinterpret_cast<bf16x4 *>(&sm.St[p * kLdN + n0]) = v;
            }
    }
    // selection fragments for the transposes: E_h[k][c] = 1 when k == 16h + c,
    // with k = 8lg + slot and c = lr
    const bf16x8 e0 = unit_fragment(lr - 8 * lg), e1 = unit_fragment(16 + lr - 8 * lg);
    // token scalars: the first chunk's staged now, the next one's in flight (each
    // later chunk's are loaded two chunks ahead and staged before B2 of the chunk
    // before it)
    gfloat *const sbase = scalar_base(a, hi, lg, lr);
    float scal = 0.f;
    if (pos.c_begin < pos.c_end) {
        const Lane ln0 = make_lane<R>(l, w, H);
        const float s0 = load_scalars<R>(a, sbase, bi, pos.c_begin, ln0);
        if (lg < 3) sm.tok[lg][ln0.row] = s0;
        else if (w == 0 && lr < 2) sm.tokn[lr] = s0;
        scal = load_scalars<R>(a, sbase, bi, pos.c_begin + 1 < pos.c_end ? pos.c_begin + 1 : pos.c_begin, ln0);
    }
    __syncthreads();

    float logdecay_total = 0.f;
    float newcarry = 0.f;

    ChunkRegs cr;
    if (pos.c_begin < pos.c_end) {
        const int64_t c0 = pos.c_begin * C;
        const int nv = (int)((L - c0) < C ? (L - c0) : C);
        const int avail = (int)((L - c0) < C + 1 ? (L - c0) : C + 1);
        load_chunk<MODE, R, FUSED>(chunk_base<R, FUSED>(a, bi, hi, g, c0), make_lane<R>(tid & 63, w, H), nv, avail,
                                   G, H, cr);
    }

    // lane constants of the diagonal mask block (lane: row t = 16w + lr, columns s = 16w + 4lg + j):
    // 1 where s's token precedes t's, 1 where it is t's token, and the skip D on t's own entry.
    // Kept across the loop: recomputed per chunk they cost a compare and a select each.
    f32x4 mbef, msame, mskip;
    {
        const int lr0 = tid & 15, lg0 = (tid & 63) >> 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sj = (4 * lg0 + j) / R, tj = lr0 / R;  // tokens relative to 16w / R
            mbef[j] = sj < tj ? 1.f : 0.f;
            msame[j] = sj == tj ? 1.f : 0.f;
            mskip[j] = (4 * lg0 + j == lr0) ? dsk : 0.f;
        }
    }

    for (int64_t c = pos.c_begin; c < pos.c_end; ++c) {
        // Wave priorities by phase: the two workgroups of a CU share each SIMD and
        // are rarely in the same phase. Favouring the rotation (2) and the score,
        // mask and output stage (3) over the rest (0) lets the wave that the next
        // barrier waits on issue first: 0.428 -> 0.368 ms for SISO b8 L4096.
        __builtin_amdgcn_s_setprio(0);
        const int64_t c0 = c * C;
        const int nv = (int)((L - c0) < C ? (L - c0) : C);
        const ChunkBase cb = chunk_base<R, FUSED>(a, bi, hi, g, c0);
        // lane-derived indices, recomputed per chunk (see opaque())
        const Lane ln = make_lane<R>(opaque(tid & 63), w, H);
        const int l = ln.l, lr = ln.lr, lg = ln.lg, row = ln.row, r_row = ln.r_row, t_row = ln.t_row;

        // ---- this chunk's inputs, loaded during the previous chunk
        const bool valid = t_row < nv;
        // token scalars (staged before B2 of the previous chunk): row l's token, the
        // next token's (row l + R, or the token after the chunk), the fragment row's;
        // zero for tokens past the chunk and a look-ahead past the sequence
        const int avail = (int)((L - c0) < C + 1 ? (L - c0) : C + 1);
        const bool tin = l / R < nv, tnx = l / R + 1 < avail;
        const bool lastt = l + R >= kRows;
        const int lnx = lastt ? kRows - 1 : l + R;
        const float d0 = sm.tok[0][l], a0_ = sm.tok[1][l], l0 = sm.tok[2][l];
        const float dsh = sm.tok[0][lnx], lsh = sm.tok[2][lnx], dnl = sm.tokn[0], lmnl = sm.tokn[1];
        const float drw = sm.tok[0][row];
        const float d = tin ? d0 : 0.f, av = tin ? a0_ : 0.f, lm = tin ? l0 : 0.f;
        const float dn = tnx ? (lastt ? dnl : dsh) : 0.f, lmn = tnx ? (lastt ? lmnl : lsh) : 0.f;
        const float drow = valid ? drw : 0.f;
        u32x4 qb[4], qc[4];
        bf16x8 xf[2];
        f32x4 th[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            qb[k] = cr.qb[k];
            qc[k] = cr.qc[k];
        }
#pragma unroll
        for (int k = 0; k < 4 / R; ++k) th[k] = cr.th[k];
        if constexpr (MODE != kCorrect) {
            xf[0] = cr.xf[0];
            xf[1] = cr.xf[1];
        }
        // fused gate factor W_O SiLU(W_Z Z') of the row's token and rank at the lane's
        // output columns (App. C), formed here, off the output stage's critical path
        f32x4 gz[4];
        if constexpr (FUSED && MODE != kPass1) {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const f32x4 wz = *reinterpret_cast<const f32x4 *>(&sm.fw[1][r_row][16 * pb + 4 * lg]);
                const f32x4 wo = *reinterpret_cast<const f32x4 *>(&sm.fw[2][r_row][16 * pb + 4 * lg]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float zz = wz[j] * (float)cr.zf[pb][j];
                    float gv = wo[j] * (zz * __builtin_amdgcn_rcpf(1.f + __expf(-zz)));
                    asm volatile("" : "+v"(gv));  // formed here, not sunk to its use
                    gz[pb][j] = gv;
                }
            }
        }
        if constexpr (FUSED && MODE != kCorrect) {
            // rank expansion X = W_X (.) X' for this lane's rank (App. C), rounded
            // to bf16 like any other matrix-core operand
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&sm.fw[0][r_row][32 * hh + 8 * lg]);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&sm.fw[0][r_row][32 * hh + 8 * lg + 4]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xf[hh][j] = (__bf16)((float)xf[hh][j] * w0[j]);
                    xf[hh][j + 4] = (__bf16)((float)xf[hh][j + 4] * w1[j]);
                }
            }
        }
        // ---- token scalars in row layout (lane l = row l, token l / R): decay
        // prefix over the tokens (one term per token), folded weights
        const float cs = wave_incl_scan((l % R == 0) ? d * av : 0.f);
        const float gm = lm * d;
        const float wt = gm + (1.f - lmn) * dn;
        const float cs_end = lane_value(cs, 63);
        // per-row tables; the previous chunk's reads of them ended before its last barrier.
        // The mask weights carry 2^(kB + kC), the state-input weights 2^kB and the
        // carried-state output scale 2^kC: the inverse scales of B_bar and C_bar.
        {
            const float l2c = cs * kLog2e;
            const float wtm = wt * sBC;
            if (w == 0) {
                sm.l2cs[l] = l2c;
                sm.wgt[l] = wtm;
                sm.gam[l] = gm * sBC;
                sm.eoff[l] = __expf(cs) * sC;
            } else if (w == 1) {
                sm.cstt[l] = __expf(cs_end - cs) * wt * sB;
                // factor of row t against the last row of the block before its own
                const float ref = (l < 32) ? lane_value(l2c, 15) : ((l < 48) ? lane_value(l2c, 31) : lane_value(l2c, 47));
                sm.ftab[l] = __builtin_amdgcn_exp2f(fminf(l2c - ref, 0.f));
            } else {
                // decay from row s to the last row of block wb-1, times w_s (rows s < 16wb)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int wb = (w == 2) ? 1 + k : 3;
                    if (w == 2 || k == 0) {
                        const float ref = lane_value(l2c, 16 * wb - 1);
                        sm.tw[wb - 1][l] = (l < 16 * wb) ? __builtin_amdgcn_exp2f(fminf(ref - l2c, 0.f)) * wtm : 0.f;
                    }
                }
            }
        }

        // ---- angles: prefix over the tokens of this wave's rows (16-lane DPP rows)
        // slot k (0..15) is channel i = 8lg + k (k < 8) or 32 + 8lg + (k - 8)
        // (in revolutions: dt theta / 2 pi). A lane computes the 4 / R slot blocks
        // its rank owns (load_chunk); the token's other rank lanes hold the rest.
        constexpr int NB = 4 / R;  // owned blocks of 4 slots
        const float drev = drow * kInv2Pi;
        float ph[4 * NB];
        {
            // (no contraction: fused into the first step's product, each add with a
            // neighbour's value took a zeroed register and a separate DPP move
            // instead of one DPP add)
#pragma clang fp contract(off)
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) ph[4 * q + j] = drev * th[q][j];
#pragma unroll
            for (int sh = R; sh < 16; sh <<= 1)
#pragma unroll
                for (int k = 0; k < 4 * NB; ++k) ph[k] += dpp_row_shr(ph[k], sh);
            // formed here by every lane: the last step had been placed in the join of the
            // branch below, as a zeroed register, a DPP move and a separate add
#pragma unroll
            for (int k = 0; k < 4 * NB; ++k) asm volatile("" : "+v"(ph[k]));
        }
        if (lr >= 16 - R) {  // the wave's last token: its rank lanes hold every block
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int b = NB * r_row + q;
                *reinterpret_cast<f32x4 *>(&sm.angtot[w][32 * (b >> 1) + 8 * lg + 4 * (b & 1)]) =
                    f32x4{ph[4 * q + 0], ph[4 * q + 1], ph[4 * q + 2], ph[4 * q + 3]};
            }
        }
        __syncthreads();  // B1
        __builtin_amdgcn_s_setprio(2);

        // ---- X^T through the matrix core: T = X-fragment x selection, exact for
        // bf16 operands; the output lane holds rows 16w + 4lg..+3 of column lr.
        // Written after B1, which every wave passes only once its state update of
        // the previous chunk (a reader of every column of X^T) is done.
        if constexpr (MODE != kCorrect) {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const f32x4 t = mfma(xf[pb >> 1], (pb & 1) ? e1 : e0, f32x4{0.f, 0.f, 0.f, 0.f});
                const bf16x4 v = {(__bf16)t[0], (__bf16)t[1], (__bf16)t[2], (__bf16)t[3]};
                *reinterpret_cast<bf16x4 *>(&sm.Xt[(16 * pb + lr) * kLdR + row_slot(w, lg)]) = v;
            }
        }

        // ---- rotate into the frame of the workgroup's first token: add the carry
        // and the totals of the earlier waves' rows. Lane l forms that offset for
        // channel l once (branch-free, uniform 0/1 weights) into the wave's LDS
        // row; each lane then adds it to its 16 slots.
        {
            const float f0 = (w > 0) ? 1.f : 0.f, f1 = (w > 1) ? 1.f : 0.f, f2 = (w > 2) ? 1.f : 0.f;
            float o = sm.carry[l];
            o = __builtin_fmaf(f0, sm.angtot[0][l], o);
            o = __builtin_fmaf(f1, sm.angtot[1][l], o);
            sm.woff[w][l] = __builtin_fmaf(f2, sm.angtot[2][l], o);
            // the wave reads other lanes' entries: its LDS accesses complete in order
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int b = NB * r_row + q;
                const f32x4 of = *reinterpret_cast<const f32x4 *>(&sm.woff[w][32 * (b >> 1) + 8 * lg + 4 * (b & 1)]);
#pragma unroll
                for (int k = 0; k < 4; ++k) ph[4 * q + k] += of[k];
            }
        }
        if (w == 0)
            newcarry = __builtin_amdgcn_fractf(sm.carry[l] + sm.angtot[0][l] + sm.angtot[1][l] + sm.angtot[2][l] +
                                               sm.angtot[3][l]);
        // sine and cosine of the owned slots, packed as f16 (cos, sin) and (sin, cos);
        // slot block b comes from the token's rank lane b / NB (a DPP quad permute
        // within the token's R lanes)
        unsigned csp[4 * NB], scp[4 * NB];
#pragma unroll
        for (int k = 0; k < 4 * NB; ++k) {
            float sn, cn;
            sincos_rev(ph[k], sn, cn);
            csp[k] = __builtin_bit_cast(unsigned, h2{(_Float16)cn, (_Float16)sn});
            scp[k] = __builtin_bit_cast(unsigned, h2{(_Float16)sn, (_Float16)cn});
        }
        auto slot_pair = [&](const unsigned *src, int sl) -> h2 {  // sl: compile-time slot 0..15
            if constexpr (R == 1) {
                return __builtin_bit_cast(h2, src[sl]);
            } else {
                const int b = sl >> 2, ro = b / NB, k = 4 * (b % NB) + (sl & 3);
                const float v = __uint_as_float(src[k]);
                float t;
                // every lane of a group of R takes lane (group base + ro)
                if constexpr (R == 4) {
                    if (ro == 0) t = quad_perm<0x00>(v);
                    else if (ro == 1) t = quad_perm<0x55>(v);
                    else if (ro == 2) t = quad_perm<0xAA>(v);
                    else t = quad_perm<0xFF>(v);
                } else {  // R == 2: quad_perm [ro, ro, 2 + ro, 2 + ro]
                    t = ro == 0 ? quad_perm<0xA0>(v) : quad_perm<0xF5>(v);
                }
                return __builtin_bit_cast(h2, __float_as_uint(t));
            }
        };
        // B~ = normalised row times 2^(eg - k) plus the scaled bias (one packed f16
        // multiply-add per channel pair), then rotated in fp32 and rounded to bf16.
        // Rows past the end of the sequence need no zeroing: their weights w, gamma
        // and cst are 0 and their outputs are not stored.
        bf16x8 bfr[4], cfr[4];
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            const int i0 = 32 * ks2 + 8 * lg;  // first of this lane's 8 pairs
            u32x4 bb[2], bc[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if constexpr (MODE != kCorrect) bb[hh] = *reinterpret_cast<const u32x4 *>(&sm.bq[0][r_row][i0 + 4 * hh]);
                if constexpr (MODE != kPass1) bc[hh] = *reinterpret_cast<const u32x4 *>(&sm.bq[1][r_row][i0 + 4 * hh]);
            }
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const h2 cs0 = slot_pair(csp, 8 * ks2 + j), sc0 = slot_pair(scp, 8 * ks2 + j);
                const h2 cs1 = slot_pair(csp, 8 * ks2 + j + 1), sc1 = slot_pair(scp, 8 * ks2 + j + 1);
                // (vector elements go through scalars: a bit cast of an element
                // lvalue was compiled as a cast of the vector's first element)
                h2 vb[2], vc[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int jj = j + e;
                    if constexpr (MODE != kCorrect) {
                        const unsigned qv = qb[2 * ks2 + (jj >> 2)][jj & 3], bv = bb[jj >> 2][jj & 3];
                        vb[e] = __builtin_bit_cast(h2, qv) * rrB + __builtin_bit_cast(h2, bv);
                    }
                    if constexpr (MODE != kPass1) {
                        const unsigned qv = qc[2 * ks2 + (jj >> 2)][jj & 3], bv = bc[jj >> 2][jj & 3];
                        vc[e] = __builtin_bit_cast(h2, qv) * rrC + __builtin_bit_cast(h2, bv);
                    }
                }
                float ob[4], oc[4];
                if constexpr (MODE != kCorrect && MODE != kPass1)
                    rot_pairs4(vb[0], vb[1], vc[0], vc[1], cs0, sc0, cs1, sc1, ob, oc);
                else if constexpr (MODE == kPass1)
                    rot_pairs2(vb[0], vb[1], cs0, sc0, cs1, sc1, ob[0], ob[1], ob[2], ob[3]);
                else
                    rot_pairs2(vc[0], vc[1], cs0, sc0, cs1, sc1, oc[0], oc[1], oc[2], oc[3]);
                if constexpr (MODE != kCorrect) {
                    bfr[ks2][j] = (__bf16)ob[0];
                    bfr[ks2 + 2][j] = (__bf16)ob[1];
                    bfr[ks2][j + 1] = (__bf16)ob[2];
                    bfr[ks2 + 2][j + 1] = (__bf16)ob[3];
                }
                if constexpr (MODE != kPass1) {
                    cfr[ks2][j] = (__bf16)oc[0];
                    cfr[ks2 + 2][j] = (__bf16)oc[1];
                    cfr[ks2][j + 1] = (__bf16)oc[2];
                    cfr[ks2 + 2][j + 1] = (__bf16)oc[3];
                }
            }
        }
        if constexpr (MODE != kPass1 && MODE != kCorrect) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                *reinterpret_cast<bf16x8 *>(&sm.Bb[row * kLdN + 32 * ks + 8 * lg]) = bfr[ks];
        }
        // ---- B_bar^T scaled by cst through the matrix core; the scale belongs to
        // the output rows 16w + 4lg + j
        if constexpr (MODE != kCorrect) {
            const f32x4 cs4 = *reinterpret_cast<const f32x4 *>(&sm.cstt[16 * w + 4 * lg]);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const f32x4 t = mfma(bfr[nb >> 1], (nb & 1) ? e1 : e0, f32x4{0.f, 0.f, 0.f, 0.f}) * cs4;
                const bf16x4 v = {(__bf16)t[0], (__bf16)t[1], (__bf16)t[2], (__bf16)t[3]};
                *reinterpret_cast<bf16x4 *>(&sm.Bt[(16 * nb + lr) * kLdR + row_slot(w, lg)]) = v;
            }
        }
        // the next chunk's token scalars (every wave read this chunk's before B1)
        if (lg < 3) sm.tok[lg][row] = scal;
        else if (w == 0 && lr < 2) sm.tokn[lr] = scal;
        __syncthreads();  // B2

        // ---- the next chunk's inputs. A burst of every wave's loads right after B2
        // filled the CU's queue of outstanding misses and blocked the issuing waves
        // for a memory latency. Measured best (with the phase priorities): one burst
        // before the state update, for every R.
        const int64_t c1 = c0 + C;
        const bool more = c + 1 < pos.c_end;
        const int nv1 = (int)((L - c1) < C ? (L - c1) : C);
        const int avail1 = (int)((L - c1) < C + 1 ? (L - c1) : C + 1);

        __builtin_amdgcn_s_setprio(3);
        if constexpr (MODE != kPass1) {
            // the stage with the wave index as a constant: the causal block structure
            // is then straight-line code for each wave
            auto stage_m = [&](auto wc) __attribute__((always_inline)) {
                constexpr int w = decltype(wc)::value;
            // the correction pass has no input term: only the carried-state output
            bf16x8 pfr[2];
            if constexpr (MODE != kCorrect) {
            // ---- S^T blocks (s-block sb <= w) for this wave's t-block
            f32x4 sT[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                sT[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (sb <= w) {
                    const int srow = 16 * sb + lr;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 av_ = *reinterpret_cast<const bf16x8 *>(&sm.Bb[srow * kLdN + 32 * ks + 8 * lg]);
                        sT[sb] = mfma(av_, cfr[ks], sT[sb]);
                    }
                }
            }
            // ---- mask: lane holds S^T[s = 16sb + 4lg + j][t = 16w + lr]
            // (all table reads first, no LDS wait inside the uniform branches below)
            const float l2t = sm.l2cs[row], gmt = sm.gam[row], ft = sm.ftab[row];
            const f32x4 l2s = *reinterpret_cast<const f32x4 *>(&sm.l2cs[16 * w + 4 * lg]);
            const f32x4 ws = *reinterpret_cast<const f32x4 *>(&sm.wgt[16 * w + 4 * lg]);
            f32x4 tws[3];
#pragma unroll
            for (int sb = 0; sb < 3; ++sb)
                tws[sb] = *reinterpret_cast<const f32x4 *>(&sm.tw[w > 0 ? w - 1 : 0][16 * sb + 4 * lg]);
            // diagonal block w: exp(cs_t - cs_s) w_s below the diagonal, gamma on it
            f32x4 mdiag;
            const f32x4 dadd = mskip;  // the row's own entry
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = __builtin_amdgcn_exp2f(fminf(l2t - l2s[j], 0.f)) * ws[j];
                mdiag[j] = mbef[j] * e + msame[j] * gmt;
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb < w) {
                    // every s token precedes every t token: the decay splits at the
                    // last row of block w-1, exp(cs_t - cs_ref) exp(cs_ref - cs_s),
                    // both factors at most 1
#pragma unroll
                    for (int j = 0; j < 4; ++j) sT[sb][j] *= tws[sb < 3 ? sb : 2][j] * ft;
                } else if (sb == w) {
                    sT[sb] = sT[sb] * mdiag + dadd;
                }
            }
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pfr[m2][j] = (__bf16)sT[2 * m2][j];
                    pfr[m2][j + 4] = (__bf16)sT[2 * m2 + 1][j];
                }
            }
            // ---- Y^T = (St C_bar^T) diag(exp(cs)) + X^T P^T ; lane: column t = row, rows p
            const float eo = sm.eoff[row];
            auto y_block = [&](int pb) -> f32x4 {
                const int p = 16 * pb + lr;
                f32x4 yv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 sv = *reinterpret_cast<const bf16x8 *>(&sm.St[p * kLdN + 32 * ks + 8 * lg]);
                    yv = mfma(sv, cfr[ks], yv);
                }
                yv *= eo;
                if constexpr (MODE == kCorrect) return yv;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    if (2 * m2 <= w) {
                        // rows 32m2 + 4lg + j and 32m2 + 16 + 4lg + j: one read (row_slot)
                        const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(&sm.Xt[p * kLdR + 32 * m2 + 8 * lg]);
                        yv = mfma(xv, pfr[m2], yv);
                    }
                }
                return yv;
            };
            // gate and rank contraction (App. C): sum over the R lanes of the token of
            // W_O Y SiLU(W_Z Z'); every lane of the token ends with the sum
            auto gate_block = [&](int pb, const f32x4 &yv) -> f32x4 {
                if constexpr (FUSED) {
                    // (no contraction: fused into the product, each rank-sum step took a
                    // zeroed register, a DPP move and an FMA instead of one DPP add)
#pragma clang fp contract(off)
                    f32x4 ov;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // formed here by every lane: sunk into the writer's branch, the last
                        // step had become a zeroed register, a DPP move and a separate add
                        float t = group_sum<R>(yv[j] * gz[pb][j]);
                        if constexpr (R > 1) asm volatile("" : "+v"(t));
                        ov[j] = t;
                    }
                    return ov;
                } else {
                    return yv;
                }
            };
            __bf16 *const orow = FUSED ? cb.y + t_row * (int)H * kP : cb.y + ln.offX;
            auto store_block = [&](int pb, const f32x4 &v) {
                bf16x4 *dst = reinterpret_cast<bf16x4 *>(orow + 16 * pb + 4 * lg);
                f32x4 t = v;
                if constexpr (MODE == kCorrect) {  // add to the local pass's output
                    const bf16x4 old = *dst;
                    t = f32x4{(float)old[0], (float)old[1], (float)old[2], (float)old[3]} + v;
                }
                const bf16x4 o = {(__bf16)t[0], (__bf16)t[1], (__bf16)t[2], (__bf16)t[3]};
                *dst = o;
            };
            // the token's rank-0 lane stores the gated output
            const bool writer = valid && (!FUSED || r_row == 0);
            if constexpr (!ONORM) {
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const f32x4 yv = y_block(pb);
                    if constexpr (FUSED) {
                        const f32x4 ov = gate_block(pb, yv);
                        if (writer) store_block(pb, ov);
                    } else if (writer) {
                        store_block(pb, yv);
                    }
                }
            } else {
                // grouped output RMSNorm: a row's 64 channels sit in lanes lr + 16 lg
                // (16 each), so the mean square is a 16-term sum and a sum over rows
                f32x4 v4[4], wn[4];
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    v4[pb] = y_block(pb);
                    wn[pb] = *reinterpret_cast<const f32x4 *>(&sm.onw[16 * pb + 4 * lg]);
                }
                auto norm4 = [&]() {
                    float ss = 0.f;
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
                        for (int j = 0; j < 4; ++j) ss = __builtin_fmaf(v4[pb][j], v4[pb][j], ss);
                    const float rs = __builtin_amdgcn_rsqf(sum_over_rows(ss) * (1.f / kP) + a.eps);
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) v4[pb] = v4[pb] * wn[pb] * rs;
                };
                const bool after = FUSED && a.norm_after_gate;
                if (!after) norm4();  // each rank row of y (of Y, before the gate)
                if constexpr (FUSED) {
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) v4[pb] = gate_block(pb, v4[pb]);
                    if (after) norm4();  // O', after the gate and the rank contraction
                }
                if (writer) {
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) store_block(pb, v4[pb]);
                }
            }
            };
            switch (w) {
                case 0: stage_m(std::integral_constant<int, 0>{}); break;
                case 1: stage_m(std::integral_constant<int, 1>{}); break;
                case 2: stage_m(std::integral_constant<int, 2>{}); break;
                default: stage_m(std::integral_constant<int, 3>{}); break;
            }
            __syncthreads();  // B3: St and Bb reads done
            __builtin_amdgcn_s_setprio(0);
        }

        if (more) load_chunk<MODE, R, FUSED>(chunk_base<R, FUSED>(a, bi, hi, g, c1), ln, nv1, avail1, G, H, cr);
        scal = load_scalars<R>(a, sbase, bi, c + 2 < pos.c_end ? c + 2 : pos.c_end - 1, ln);

        // ---- state update: acc[q][pb] = exp(cs_end) acc + Bt-rows x Xt
        const float dec = __expf(cs_end);
        logdecay_total += cs_end;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) acc[q][pb] *= dec;
#pragma unroll
        for (int m2 = 0; m2 < (MODE == kCorrect ? 0 : 2); ++m2) {
            bf16x8 xb[4];
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
                xb[pb] = *reinterpret_cast<const bf16x8 *>(&sm.Xt[(16 * pb + lr) * kLdR + 32 * m2 + 8 * lg]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int n = 16 * (w + 4 * q) + lr;
                const bf16x8 bt = *reinterpret_cast<const bf16x8 *>(&sm.Bt[n * kLdR + 32 * m2 + 8 * lg]);
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) acc[q][pb] = mfma(bt, xb[pb], acc[q][pb]);
            }
        }
        if constexpr (MODE != kPass1) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const int n0 = 16 * (w + 4 * q) + 4 * lg, p = 16 * pb + lr;
                    bf16x4 v = {(__bf16)acc[q][pb][0], (__bf16)acc[q][pb][1], (__bf16)acc[q][pb][2],
                                (__bf16)acc[q][pb][3]};
                    *reinterpret_cast<bf16x4 *>(&sm.St[p * kLdN + n0]) = v;
                }
        }
        // carry was last read before B2 of this chunk; the next read is after B1 of the next
        if (w == 0) sm.carry[l] = newcarry;
        if constexpr (MODE == kCorrect) {
            // every later output's share of the incoming state is below e^kCorrectStop
            // (logdecay_total is the same in every wave)
            if (logdecay_total < kCorrectStop) break;
        }
    }
    __syncthreads();

    // ------------------------------------------------------------- epilogue
    if constexpr (MODE == kCorrect) return;  // the combine wrote the final state
    const bool last_seg = (MODE == kFull) || (pos.c_end * C >= L);
    float *dst = nullptr;
    if (MODE == kPass1 || MODE == kLocal)
        dst = sp.seg_state + (chain * sp.nseg + pos.seg) * (kP * kN);
    else if (last_seg)
        dst = a.h_final ? a.h_final + chain * (kP * kN) : nullptr;
    if (dst) {
        // back to the physical frame: H = R(Phi) H~ on pairs (n, n + 64)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = 16 * w + 4 * lg + j;
            float sn, cn;
            sincos_rev(sm.carry[i], sn, cn);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const float u = acc[0][pb][j], v = acc[1][pb][j];
                acc[0][pb][j] = cn * u - sn * v;
                acc[1][pb][j] = sn * u + cn * v;
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int n0 = 16 * (w + 4 * q) + 4 * lg, p = 16 * pb + lr;
                *reinterpret_cast<f32x4 *>(dst + p * kN + n0) = acc[q][pb];
            }
    }
    if constexpr (MODE == kPass1 || MODE == kLocal) {
        if (tid < kHalf) sp.seg_angle[(chain * sp.nseg + pos.seg) * kHalf + tid] = sm.carry[tid];
        if (tid == 0) sp.seg_decay[chain * sp.nseg + pos.seg] = logdecay_total;
    }
}

// Chain the segment end states: H_in[0] = h0 (+ fold of the previous token);
// H_in[k+1] = exp(D_k) R(Phi_k) H_in[k] + E_k. Overwrites E_k with H_in[k]; with
// write_final, H_in[nseg] (the state after the last token) goes to h_final.
// kCombineSplit workgroups per chain, each kCombineRows rows p of the N x P state (a
// thread two channel pairs); the end states of kCombineBurst segments are loaded at
// once, since only the stores depend on the carried state. (One workgroup per chain
// walking the segments one load round trip at a time had taken 34 us for 48 chains
// of 21 segments.)
constexpr int kCombineSplit = 8;
constexpr int kCombineRows = kP / kCombineSplit;
constexpr int kCombineBurst = 8;
template <int R, bool FUSED>
__global__ __launch_bounds__(kThreads) void combine_kernel(ScanArgs a, SplitPlan sp, bool write_final) {
    constexpr int KE = kCombineRows * kHalf / kThreads;  // channel pairs per thread
    static_assert(KE * kThreads == kCombineRows * kHalf, "the rows of a part fill the workgroup");
    __shared__ float rsp[4];
    const int tid = threadIdx.x;
    const int64_t chain = blockIdx.x / kCombineSplit;
    const int p0 = (int)(blockIdx.x % kCombineSplit) * kCombineRows;
    const int64_t bi = chain / a.H, hi = chain % a.H, g = hi / (a.H / a.G);
    const int i = tid % kHalf;  // this thread's rotation channel
    float lo[KE], hiv[KE];
#pragma unroll
    for (int k = 0; k < KE; ++k) {
        const int p = p0 + (tid + kThreads * k) / kHalf;
        lo[k] = a.h0 ? a.h0[(chain * kP + p) * kN + i] : 0.f;
        hiv[k] = a.h0 ? a.h0[(chain * kP + p) * kN + i + kHalf] : 0.f;
    }
    if (a.has_prev && a.L > 0) {
        const __bf16 *bp = static_cast<const __bf16 *>(a.Braw_prev) + ((bi * a.G + g) * R) * kN;
        const int wv = tid >> 6, l = tid & 63;
        if (wv < R) {
            const float v0 = (float)bp[wv * kN + 2 * l], v1 = (float)bp[wv * kN + 2 * l + 1];
            const float ss = wave_sum(v0 * v0 + v1 * v1);
            if (l == 0) rsp[wv] = __builtin_amdgcn_rsqf(ss * (1.f / kN) + a.eps);
        }
        __syncthreads();
        const int64_t o0 = (bi * a.L) * a.H + hi;
        const float f = (1.f - a.lam[o0]) * a.dt[o0];
        const float *bb = a.B_bias + (hi * R) * kN;
        const float wl = a.B_normw ? a.B_normw[i] : 1.f, wh = a.B_normw ? a.B_normw[i + kHalf] : 1.f;
#pragma unroll
        for (int k = 0; k < KE; ++k) {
            const int p = p0 + (tid + kThreads * k) / kHalf;
            float sl = 0.f, sh = 0.f;
            for (int r = 0; r < R; ++r) {
                const float xv = prev_x<R, FUSED>(a, bi, hi, r, p);
                sl += ((float)bp[r * kN + i] * rsp[r] * wl + bb[r * kN + i]) * xv;
                sh += ((float)bp[r * kN + i + kHalf] * rsp[r] * wh + bb[r * kN + i + kHalf]) * xv;
            }
            lo[k] += f * sl;
            hiv[k] += f * sh;
        }
    }
    float *const E0 = sp.seg_state + chain * sp.nseg * (int64_t)(kP * kN);
    for (int s0 = 0; s0 < sp.nseg; s0 += kCombineBurst) {
        // the burst's end states, decays and angles (indices clamped into the segments)
        float el[kCombineBurst][KE], eh[kCombineBurst][KE], dec[kCombineBurst], ang[kCombineBurst];
#pragma unroll
        for (int j = 0; j < kCombineBurst; ++j) {
            const int sc = s0 + j < sp.nseg ? s0 + j : sp.nseg - 1;
            const float *E = E0 + sc * (int64_t)(kP * kN);
#pragma unroll
            for (int k = 0; k < KE; ++k) {
                const int p = p0 + (tid + kThreads * k) / kHalf;
                el[j][k] = E[p * kN + i];
                eh[j][k] = E[p * kN + i + kHalf];
            }
            dec[j] = sp.seg_decay[chain * sp.nseg + sc];
            ang[j] = sp.seg_angle[(chain * sp.nseg + sc) * kHalf + i];
        }
#pragma unroll
        for (int j = 0; j < kCombineBurst; ++j) {
            if (s0 + j < sp.nseg) {
                float *E = E0 + (s0 + j) * (int64_t)(kP * kN);
                const float dc = __expf(dec[j]);
                float sn, cn;
                sincos_rev(ang[j], sn, cn);
#pragma unroll
                for (int k = 0; k < KE; ++k) {
                    const int p = p0 + (tid + kThreads * k) / kHalf;
                    E[p * kN + i] = lo[k];
                    E[p * kN + i + kHalf] = hiv[k];
                    const float u = lo[k], v = hiv[k];
                    lo[k] = dc * (cn * u - sn * v) + el[j][k];
                    hiv[k] = dc * (sn * u + cn * v) + eh[j][k];
                }
            }
        }
    }
    if (write_final && a.h_final) {
#pragma unroll
        for (int k = 0; k < KE; ++k) {
            const int p = p0 + (tid + kThreads * k) / kHalf;
            a.h_final[(chain * kP + p) * kN + i] = lo[k];
            a.h_final[(chain * kP + p) * kN + i + kHalf] = hiv[k];
        }
    }
}

// BCNorm of every raw B and C row (Mamba-3 paper §3.4, "BCNorm"), once per
// (token, group, rank) row instead of once per head that reads it:
// u = x / sqrt(mean(x^2) + eps) times the gain, scaled by 2^-eg with
// max |g| <= 2^eg, stored as f16 pairs (n, n + N/2) -- the rotation's operand
// layout. 16 lanes per row, lane k taking pairs 4k..4k+3, 4 rows per pass; blockIdx.y is 0 for B
// and 1 for C. Every row of both outputs is written.
__global__ __launch_bounds__(256) void bcnorm_pairs_kernel(const __bf16 *Bm, const __bf16 *Cm, const float *gB,
                                                           const float *gC, float eps, int64_t rows, unsigned *qB,
                                                           unsigned *qC) {
    const bool isC = blockIdx.y != 0;
    const __bf16 *src = isC ? Cm : Bm;
    const float *gn = isC ? gC : gB;
    unsigned *dst = isC ? qC : qB;
    const int k = threadIdx.x & 15;
    f32x4 gl = {1.f, 1.f, 1.f, 1.f}, gh = {1.f, 1.f, 1.f, 1.f};
    if (gn) {
        gl = *reinterpret_cast<const f32x4 *>(gn + 4 * k);
        gh = *reinterpret_cast<const f32x4 *>(gn + kHalf + 4 * k);
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(gl[j]), fabsf(gh[j])));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    const float sc = ldexpf(1.f, -max(0, exp_ceil(m)));
    gl *= sc;
    gh *= sc;
    // 4 rows per 16-lane group and pass: their loads go out together (indices clamped
    // into the rows; a row past the end is computed and not stored)
    constexpr int RP = 4;
    for (int64_t r0 = (int64_t)blockIdx.x * 16 * RP + (threadIdx.x >> 4); r0 < rows; r0 += (int64_t)gridDim.x * 16 * RP) {
        bf16x4 lo[RP], hi[RP];
#pragma unroll
        for (int q = 0; q < RP; ++q) {
            const int64_t r = r0 + 16 * q < rows ? r0 + 16 * q : rows - 1;
            lo[q] = *reinterpret_cast<const bf16x4 *>(src + r * kN + 4 * k);
            hi[q] = *reinterpret_cast<const bf16x4 *>(src + r * kN + kHalf + 4 * k);
        }
#pragma unroll
        for (int q = 0; q < RP; ++q) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = (float)lo[q][j], b = (float)hi[q][j];
                ss = __builtin_fmaf(a, a, __builtin_fmaf(b, b, ss));
            }
            ss = group_sum<16>(ss);  // the row's 16 lanes (DPP)
            const float rs = __builtin_amdgcn_rsqf(ss * (1.f / kN) + eps);
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                out[j] = __builtin_bit_cast(
                    unsigned, h2{(_Float16)((float)lo[q][j] * rs * gl[j]), (_Float16)((float)hi[q][j] * rs * gh[j])});
            if (r0 + 16 * q < rows) *reinterpret_cast<u32x4 *>(dst + (r0 + 16 * q) * kHalf + 4 * k) = out;
        }
    }
}

template <int R, bool FUSED, bool ONORM>
hipError_t launch_rw(const ScanArgs &a, const SplitPlan &sp, hipStream_t s) {
    const int64_t chains = a.b * a.H;
    if (sp.nseg <= 1) {
        hipLaunchKernelGGL((scan_mfma_kernel<kFull, R, FUSED, ONORM>), dim3((unsigned)chains), dim3(kThreads), 0,
                           s, a, sp);
        return hipGetLastError();
    }
    const unsigned nblk = (unsigned)(chains * sp.nseg);
    if constexpr (!ONORM) {
        // local outputs and end states, the combine (which also writes the final
        // state), then the correction of each segment's outputs for its incoming state
        hipLaunchKernelGGL((scan_mfma_kernel<kLocal, R, FUSED, false>), dim3(nblk), dim3(kThreads), 0, s, a,
                           sp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((combine_kernel<R, FUSED>), dim3((unsigned)(chains * kCombineSplit)), dim3(kThreads), 0, s, a,
                           sp, true);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((scan_mfma_kernel<kCorrect, R, FUSED, false>), dim3(nblk), dim3(kThreads), 0, s, a,
                           sp);
        return hipGetLastError();
    }
    // the output norm is not linear in y: end states first, then every segment
    // again from its incoming state. Pass 1 produces no output, so it takes no norm
    hipLaunchKernelGGL((scan_mfma_kernel<kPass1, R, FUSED, false>), dim3(nblk), dim3(kThreads), 0, s, a, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((combine_kernel<R, FUSED>), dim3((unsigned)(chains * kCombineSplit)), dim3(kThreads), 0, s, a, sp,
                       false);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_mfma_kernel<kPass2, R, FUSED, ONORM>), dim3(nblk), dim3(kThreads), 0, s, a, sp);
    return hipGetLastError();
}

template <int R, bool FUSED>
hipError_t launch_rf(const ScanArgs &a, const SplitPlan &sp, hipStream_t s) {
    return a.onorm ? launch_rw<R, FUSED, true>(a, sp, s) : launch_rw<R, FUSED, false>(a, sp, s);
}

template <int R>
hipError_t launch_r(const ScanArgs &a, const SplitPlan &sp, hipStream_t s) {
    return a.fused ? launch_rf<R, true>(a, sp, s) : launch_rf<R, false>(a, sp, s);
}

}  // namespace

bool mfma_kernel_available() { return true; }

int mfma_auto_segments(int64_t chains, int64_t nchunks) {
    // One resident wave of workgroups is 2 per CU. Split only when the chains
    // alone leave most of them idle, and keep segments at least 8 chunks long.
    // Start from the most segments that fit one wave; take more (up to two
    // waves) only when they fill the waves at least 3 points better, since each
    // segment adds a first pass over its chunks. Measured: 192 chains, 2 -> 5
    // segments, 10-17% faster; 48 chains, 10 -> 21, 2% faster; 64, 96 and 128
    // chains (already >= 94% full with one wave) 4-5% slower with twice the
    // segments.
    const int64_t slots = 2 * kCUs;
    if (chains * 4 >= slots * 3) return 1;
    const int64_t c = chains > 0 ? chains : 1;
    const int64_t cap = nchunks / 8 > 1 ? nchunks / 8 : 1;
    int64_t best = slots / c;
    if (best > cap) best = cap;
    if (best < 1) best = 1;
    auto fill = [&](int64_t n) {
        const int64_t wg = c * n, waves = (wg + slots - 1) / slots;
        return (double)wg / (double)(waves * slots);
    };
    double fb = fill(best);
    const int64_t n1 = best;
    for (int64_t n = n1 + 1; n <= 2 * n1 + 1 && n <= cap; ++n) {
        const double f = fill(n);
        if (f > fb + 0.03) {
            best = n;
            fb = f;
        }
    }
    return (int)best;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: the normalised B and C rows, then (with a split) the segment records.
size_t mfma_workspace_bytes(int64_t rows, int64_t chains, int nseg, int64_t P, int64_t N) {
    size_t b = 2 * align256(sizeof(unsigned) * rows * (N / 2));
    if (nseg > 1)
        b += align256(sizeof(float) * chains * nseg * P * N) + align256(sizeof(float) * chains * nseg) +
             align256(sizeof(float) * chains * nseg * (N / 2));
    return b;
}

void mfma_workspace_carve(void *ws, int64_t rows, int64_t chains, int nseg, int64_t P, int64_t N, ScanArgs *a,
                          SplitPlan *sp) {
    char *p = static_cast<char *>(ws);
    a->Bq = reinterpret_cast<unsigned *>(p);
    p += align256(sizeof(unsigned) * rows * (N / 2));
    a->Cq = reinterpret_cast<unsigned *>(p);
    p += align256(sizeof(unsigned) * rows * (N / 2));
    if (nseg > 1) {
        sp->seg_state = reinterpret_cast<float *>(p);
        p += align256(sizeof(float) * chains * nseg * P * N);
        sp->seg_decay = reinterpret_cast<float *>(p);
        p += align256(sizeof(float) * chains * nseg);
        sp->seg_angle = reinterpret_cast<float *>(p);
    }
}

hipError_t launch_scan_mfma(const ScanArgs &a, const SplitPlan &sp, hipStream_t s) {
    if (a.b * a.H == 0) return hipSuccess;
    const int64_t rows = a.b * a.L * a.G * a.R;
    if (rows > 0) {
        const int64_t nb = (rows + 63) / 64;  // 64 rows per block of 256 (16 lanes a row, 4 rows each)
        hipLaunchKernelGGL(bcnorm_pairs_kernel, dim3((unsigned)(nb < 16384 ? nb : 16384), 2), dim3(256), 0, s,
                           static_cast<const __bf16 *>(a.Braw), static_cast<const __bf16 *>(a.Craw), a.B_normw,
                           a.C_normw, a.eps, rows, a.Bq, a.Cq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    switch (a.R) {
        case 1: return launch_r<1>(a, sp, s);
        case 2: return launch_r<2>(a, sp, s);
        case 4: return launch_r<4>(a, sp, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace m3i
