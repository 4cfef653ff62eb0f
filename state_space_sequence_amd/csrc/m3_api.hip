// C ABI of libm3: argument validation, plan selection, launches.
// Every check runs on the host before any HIP call (see include/m3.h).
#include <math.h>
#include <string.h>

#include <mutex>

#include "m3_internal.h"

namespace m3i {
namespace {

// grid-stride element loops over n floats, with a grid of at most kFillBlocks
constexpr int64_t kFillBlocks = 65536;

unsigned fill_grid(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < kFillBlocks ? g : kFillBlocks);
}

__global__ void state_copy_kernel(const float *h0, float *hf, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        hf[i] = h0 ? h0[i] : 0.f;
}

bool aligned16(const void *p) { return p == nullptr || (((uintptr_t)p) & 15u) == 0; }

constexpr int64_t kMaxGrid = 0x7fffffff;  // workgroups of one launch

__global__ void fill_zero_kernel(float *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

hipError_t zero(float *p, int64_t n, hipStream_t s) {
    if (!p || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(fill_grid(n)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

struct Plan {
    int kernel;       // 0 generic, 1 matrix-core
    int nseg;         // segments per sequence
    int64_t seg_chunks;
    int64_t workgroups;
    size_t ws_bytes;
};

bool mfma_applicable(const m3_shape &s) {
    // (a chunk's per-lane element offsets are 32-bit: at most 2^18 heads)
    return s.io_dtype == M3_BF16 && s.dstate == 128 && s.headdim == 64 && s.chunk * s.rank == 64 &&
           s.nheads <= (1 << 18) &&
           (s.rank == 1 || s.rank == 2 || s.rank == 4) &&
           !(s.flags & M3_FLAG_FORCE_GENERIC) && mfma_kernel_available();
}

bool generic_applicable(const m3_shape &s) {
    return s.dstate <= kGenericMaxN && s.headdim <= kGenericMaxP && s.dstate * s.headdim <= kGenericMaxNP &&
           s.chunk * s.rank <= kGenericMaxRows;
}

m3_status check_shape(const m3_shape *s) {
    if (!s) return M3_ERR_INVALID_ARG;
    if (s->batch < 0 || s->seqlen < 0 || s->nheads < 1 || s->ngroups < 1 || s->headdim < 1 || s->dstate < 2 ||
        s->rank < 1 || s->chunk < 1)
        return M3_ERR_INVALID_ARG;
    if (s->nheads % s->ngroups != 0 || s->dstate % 2 != 0) return M3_ERR_INVALID_ARG;
    if (s->io_dtype != M3_F32 && s->io_dtype != M3_BF16) return M3_ERR_INVALID_ARG;
    if (!(s->eps >= 0.f) || !isfinite(s->eps)) return M3_ERR_INVALID_ARG;
    if (s->nsegments < 0) return M3_ERR_INVALID_ARG;
    // (the bf16-state flag is decode only)
    if (s->flags & ~(M3_FLAG_FORCE_GENERIC | M3_FLAG_OUT_NORM | M3_FLAG_NORM_AFTER_GATE | M3_FLAG_BWD_LOW_MEMORY))
        return M3_ERR_INVALID_ARG;
    if (s->batch > (1LL << 31) || s->nheads > (1LL << 20) || s->seqlen > (1LL << 40)) return M3_ERR_UNSUPPORTED;
    // every launch takes at most one workgroup per (batch, head) chain and segment,
    // and the grid is a 32-bit count; tokens and elements stay far below 64-bit overflow
    if (s->batch * s->nheads > kMaxGrid || (s->seqlen > 0 && s->batch > (1LL << 40) / s->seqlen) ||
        s->headdim > (1 << 16) || s->dstate > (1 << 16) || s->rank > (1 << 10))
        return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

m3_status make_plan(const m3_shape &s, Plan *pl) {
    if (s.flags & M3_FLAG_BWD_LOW_MEMORY) return M3_ERR_INVALID_ARG;  // a backward flag
    Plan p{};
    const int64_t nchunks = (s.seqlen + s.chunk - 1) / s.chunk;
    if (mfma_applicable(s)) {
        p.kernel = 1;
        int nseg = s.nsegments;
        if (nseg == 0) nseg = mfma_auto_segments(s.batch * s.nheads, nchunks);
        if (nseg < 1) nseg = 1;
        if (nseg > nchunks && nchunks > 0) nseg = (int)nchunks;
        if (nchunks == 0) nseg = 1;
        p.nseg = nseg;
        p.seg_chunks = nseg > 1 ? (nchunks + nseg - 1) / nseg : nchunks;
        if (nseg > 1) p.nseg = (int)((nchunks + p.seg_chunks - 1) / p.seg_chunks);
        p.workgroups = s.batch * s.nheads * p.nseg;
        if (p.workgroups > kMaxGrid) return M3_ERR_UNSUPPORTED;
        const int64_t rows = s.batch * s.seqlen * s.ngroups * s.rank;  // raw B (C) rows
        if (rows > (1LL << 44)) return M3_ERR_UNSUPPORTED;
        p.ws_bytes = mfma_workspace_bytes(rows, s.batch * s.nheads, p.nseg, s.headdim, s.dstate);
    } else if (generic_applicable(s)) {
        if (s.nsegments > 1) return M3_ERR_UNSUPPORTED;  // the fp32 kernel runs each chain in one pass
        p.kernel = 0;
        p.nseg = 1;
        p.seg_chunks = nchunks;
        p.workgroups = s.batch * s.nheads;
        p.ws_bytes = 0;
    } else {
        return M3_ERR_UNSUPPORTED;
    }
    *pl = p;
    return M3_OK;
}

// Device-resident scratch of the allocation-free prefill entry point: the
// matrix-core path's workspace (normalised B and C rows, and the segment split's
// end states, decays and angles). Each GPU the library runs on holds its own copy
// until the process ends. Host code never passes the array's name to a kernel:
// its device address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kScratchBytes = size_t(256) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device a call's work runs on: the stream's, or the current one for the
// null stream.
hipError_t call_device(hipStream_t s, int *dev) {
    if (s) return hipStreamGetDevice(s, dev);
    return hipGetDevice(dev);
}

// Device address of this device's scratch array, looked up on first use.
hipError_t scratch_address(hipStream_t s, void **out) {
    int dev = 0;
    hipError_t e = call_device(s, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace m3i

using namespace m3i;

extern "C" {

const char *m3_status_str(m3_status st) {
    switch (st) {
        case M3_OK: return "ok";
        case M3_ERR_INVALID_ARG: return "invalid argument";
        case M3_ERR_UNSUPPORTED: return "unsupported shape";
        case M3_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case M3_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case M3_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

int m3_version(void) { return 104; }

// Output epilogue flags against the pointers: the gain needs the norm flag, and
// the after-gate position needs the norm and the fused gate.
static bool epilogue_ok(uint32_t flags, bool fused, const float *out_normw) {
    const bool onorm = (flags & M3_FLAG_OUT_NORM) != 0;
    if (out_normw && !onorm) return false;
    if ((flags & M3_FLAG_NORM_AFTER_GATE) && !(onorm && fused)) return false;
    return true;
}

m3_status m3_scan_plan(const m3_shape *shape, m3_plan *plan) {
    m3_status st = check_shape(shape);
    if (st != M3_OK) return st;
    if (!plan) return M3_ERR_INVALID_ARG;
    Plan p;
    st = make_plan(*shape, &p);
    if (st != M3_OK) return st;
    plan->kernel = p.kernel;
    plan->nsegments = p.nseg;
    plan->workgroups = p.workgroups;
    plan->workspace_bytes = p.ws_bytes;
    return M3_OK;
}

size_t m3_scan_workspace_bytes(const m3_shape *shape) {
    if (check_shape(shape) != M3_OK) return 0;
    Plan p;
    if (make_plan(*shape, &p) != M3_OK) return 0;
    return p.ws_bytes;
}

// m3_scan_fwd with the workspace either the caller's or, for noalloc, this
// device's scratch array (checked against its size before any HIP call).
static m3_status scan_fwd(const m3_shape *shape, const m3_scan_io *io, void *workspace, size_t ws_bytes,
                          void *stream, bool noalloc) {
    m3_status st = check_shape(shape);
    if (st != M3_OK) return st;
    if (!io) return M3_ERR_INVALID_ARG;
    const m3_shape &s = *shape;
    if ((io->x_prev == nullptr) != (io->Braw_prev == nullptr)) return M3_ERR_INVALID_ARG;
    const bool work = s.batch * s.seqlen > 0;
    const bool fused = io->W_X != nullptr;
    if (fused && (!io->W_Z || !io->W_O)) return M3_ERR_INVALID_ARG;
    if (!fused && (io->W_Z || io->W_O || io->z || io->o)) return M3_ERR_INVALID_ARG;
    if (!epilogue_ok(s.flags, fused, io->out_normw)) return M3_ERR_INVALID_ARG;
    if (work && (!io->x || !io->Braw || !io->Craw || !io->dt || !io->A || !io->lam || !io->theta ||
                 !io->B_bias || !io->C_bias || (fused ? (!io->z || !io->o) : !io->y)))
        return M3_ERR_INVALID_ARG;
    const void *ptrs[] = {io->x, io->Braw, io->Craw, io->dt, io->A, io->lam, io->theta, io->B_bias,
                          io->C_bias, io->B_normw, io->C_normw, io->h0, io->x_prev, io->Braw_prev,
                          io->y, io->h_final, workspace, io->z, io->W_X, io->W_Z, io->W_O, io->o,
                          io->D, io->out_normw};
    for (const void *p : ptrs)
        if (!aligned16(p)) return M3_ERR_MISALIGNED;
    Plan p;
    st = make_plan(s, &p);
    if (st != M3_OK) return st;
    if (fused && p.kernel != 1) return M3_ERR_UNSUPPORTED;  // the fp32 kernel does not take the fused form
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (noalloc) {
        // nothing in the scratch array needs clearing: the BCNorm pass writes every
        // normalised row before the scan reads it, pass 1 writes every segment
        // record before the combine reads it, and the combine writes every
        // incoming state before pass 2 reads it
        if (p.ws_bytes > kScratchBytes) return M3_ERR_WORKSPACE_TOO_SMALL;
        workspace = nullptr;
        ws_bytes = 0;
        if (p.ws_bytes > 0) {
            if (scratch_address(hs, &workspace) != hipSuccess) return M3_ERR_HIP;
            ws_bytes = kScratchBytes;
        }
    }
    if (p.ws_bytes > 0 && (workspace == nullptr || ws_bytes < p.ws_bytes)) return M3_ERR_WORKSPACE_TOO_SMALL;

    ScanArgs a{};
    a.b = s.batch; a.L = s.seqlen; a.H = s.nheads; a.G = s.ngroups; a.P = s.headdim; a.N = s.dstate;
    a.R = s.rank; a.C = s.chunk; a.eps = s.eps; a.bf16 = (s.io_dtype == M3_BF16);
    a.has_prev = io->x_prev != nullptr;
    a.x = io->x; a.Braw = io->Braw; a.Craw = io->Craw; a.dt = io->dt; a.A = io->A; a.lam = io->lam;
    a.theta = io->theta; a.B_bias = io->B_bias; a.C_bias = io->C_bias; a.B_normw = io->B_normw;
    a.C_normw = io->C_normw; a.h0 = io->h0; a.x_prev = io->x_prev; a.Braw_prev = io->Braw_prev;
    a.y = io->y; a.h_final = io->h_final;
    a.fused = fused; a.z = io->z; a.W_X = io->W_X; a.W_Z = io->W_Z; a.W_O = io->W_O; a.o = io->o;
    a.D = io->D; a.out_normw = io->out_normw;
    a.onorm = (s.flags & M3_FLAG_OUT_NORM) != 0;
    a.norm_after_gate = (s.flags & M3_FLAG_NORM_AFTER_GATE) != 0;

    hipError_t e = hipSuccess;
    if (s.batch * s.nheads == 0) return M3_OK;
    if (s.seqlen == 0) {
        if (io->h_final) {
            const int64_t n = s.batch * s.nheads * s.headdim * s.dstate;
            hipLaunchKernelGGL(state_copy_kernel, dim3(fill_grid(n)), dim3(256), 0, hs, io->h0,
                               io->h_final, n);
            e = hipGetLastError();
        }
        return e == hipSuccess ? M3_OK : M3_ERR_HIP;
    }
    if (p.kernel == 0) {
        e = launch_scan_generic(a, hs);
    } else {
        SplitPlan sp{};
        sp.nseg = p.nseg;
        sp.seg_chunks = p.seg_chunks;
        mfma_workspace_carve(workspace, s.batch * s.seqlen * s.ngroups * s.rank, s.batch * s.nheads, p.nseg,
                             s.headdim, s.dstate, &a, &sp);
        e = launch_scan_mfma(a, sp, hs);
    }
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status m3_scan_fwd(const m3_shape *shape, const m3_scan_io *io, void *workspace, size_t ws_bytes,
                      void *stream) {
    return scan_fwd(shape, io, workspace, ws_bytes, stream, false);
}

m3_status m3_scan_fwd_noalloc(const m3_shape *shape, const m3_scan_io *io, void *stream) {
    return scan_fwd(shape, io, nullptr, 0, stream, true);
}

size_t m3_scan_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

// Backward limits: those of the fp32 prefill kernel (the backward keeps every
// tile of a 32-row chunk in LDS), and N, P multiples of 4 (16-byte row reads).
static bool bwd_shape_ok(const m3_shape &s) {
    // the group reduction runs one wave per raw B/C row, four to a workgroup
    return s.dstate <= kGenericMaxN && s.headdim <= kGenericMaxP && s.dstate * s.headdim <= kGenericMaxNP &&
           s.rank <= 4 && s.dstate % 4 == 0 && s.headdim % 4 == 0 &&
           s.batch * s.seqlen * s.ngroups * s.rank / 4 < kMaxGrid;
}

static ScanArgs bwd_args(const m3_shape &s, const m3_scan_io *io) {
    ScanArgs a{};
    a.b = s.batch; a.L = s.seqlen; a.H = s.nheads; a.G = s.ngroups; a.P = s.headdim; a.N = s.dstate;
    a.R = s.rank; a.C = s.chunk; a.eps = s.eps; a.bf16 = (s.io_dtype == M3_BF16);
    if (io) {
        a.has_prev = io->x_prev != nullptr;
        a.x = io->x; a.Braw = io->Braw; a.Craw = io->Craw; a.dt = io->dt; a.A = io->A; a.lam = io->lam;
        a.theta = io->theta; a.B_bias = io->B_bias; a.C_bias = io->C_bias; a.B_normw = io->B_normw;
        a.C_normw = io->C_normw; a.h0 = io->h0; a.x_prev = io->x_prev; a.Braw_prev = io->Braw_prev;
    }
    return a;
}

size_t m3_scan_bwd_workspace_bytes(const m3_shape *shape) {
    if (check_shape(shape) != M3_OK || !bwd_shape_ok(*shape)) return 0;
    const ScanArgs a = bwd_args(*shape, nullptr);
    const bool lowmem = (shape->flags & M3_FLAG_BWD_LOW_MEMORY) != 0;
    if (shape->flags & ~(M3_FLAG_FORCE_GENERIC | M3_FLAG_BWD_LOW_MEMORY)) return 0;
    if (lowmem && !scan_bwd_lowmem_ok(a)) return 0;
    return scan_bwd_workspace_bytes(a, lowmem, lowmem ? (int)shape->nsegments : 0);
}

m3_status m3_scan_bwd(const m3_shape *shape, const m3_scan_io *io, const m3_scan_grads *gr, void *workspace,
                      size_t ws_bytes, void *stream) {
    m3_status st = check_shape(shape);
    if (st != M3_OK) return st;
    if (!io || !gr) return M3_ERR_INVALID_ARG;
    const m3_shape &s = *shape;
    if (s.flags & ~(M3_FLAG_FORCE_GENERIC | M3_FLAG_BWD_LOW_MEMORY))
        return (s.flags & M3_FLAG_OUT_NORM) ? M3_ERR_UNSUPPORTED : M3_ERR_INVALID_ARG;
    const bool lowmem = (s.flags & M3_FLAG_BWD_LOW_MEMORY) != 0;
    if (io->W_X || io->W_Z || io->W_O || io->z || io->o || io->D || io->out_normw) return M3_ERR_UNSUPPORTED;
    if ((io->x_prev == nullptr) != (io->Braw_prev == nullptr)) return M3_ERR_INVALID_ARG;
    if (!bwd_shape_ok(s)) return M3_ERR_UNSUPPORTED;
    const bool work = s.batch * s.seqlen > 0;
    const bool prev = io->x_prev != nullptr;
    // every gradient of an input that is present is required, and none of an absent one
    if ((gr->dB_normw == nullptr) != (io->B_normw == nullptr) || (gr->dC_normw == nullptr) != (io->C_normw == nullptr) ||
        (gr->dx_prev == nullptr) != !prev || (gr->dBraw_prev == nullptr) != !prev)
        return M3_ERR_INVALID_ARG;
    if (!gr->dB_bias || !gr->dC_bias) return M3_ERR_INVALID_ARG;
    if (work && (!io->x || !io->Braw || !io->Craw || !io->dt || !io->A || !io->lam || !io->theta || !io->B_bias ||
                 !io->C_bias || !gr->dy || !gr->dx || !gr->dBraw || !gr->dCraw || !gr->ddt || !gr->dA ||
                 !gr->dlam || !gr->dtheta))
        return M3_ERR_INVALID_ARG;
    const void *ptrs[] = {io->x, io->Braw, io->Craw, io->dt, io->A, io->lam, io->theta, io->B_bias, io->C_bias,
                          io->B_normw, io->C_normw, io->h0, io->x_prev, io->Braw_prev, gr->dy, gr->dh_final,
                          gr->dx, gr->dBraw, gr->dCraw, gr->ddt, gr->dA, gr->dlam, gr->dtheta, gr->dB_bias,
                          gr->dC_bias, gr->dB_normw, gr->dC_normw, gr->dh0, gr->dx_prev, gr->dBraw_prev, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return M3_ERR_MISALIGNED;
    const ScanArgs a = bwd_args(s, io);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const int64_t HRN = s.nheads * s.rank * s.dstate;
    if (!work) {
        // no token: the bias and gain gradients are zero, dh0 = dh_final (h_final = h0),
        // and the previous token is never used
        const int64_t nst = s.batch * s.nheads * s.headdim * s.dstate;
        if ((e = zero(gr->dB_bias, HRN, hs)) != hipSuccess || (e = zero(gr->dC_bias, HRN, hs)) != hipSuccess ||
            (e = zero(gr->dB_normw, s.dstate, hs)) != hipSuccess || (e = zero(gr->dC_normw, s.dstate, hs)) != hipSuccess ||
            (e = zero(gr->dx_prev, s.batch * s.nheads * s.rank * s.headdim, hs)) != hipSuccess ||
            (e = zero(gr->dBraw_prev, s.batch * s.ngroups * s.rank * s.dstate, hs)) != hipSuccess)
            return M3_ERR_HIP;
        if (gr->dh0 && nst > 0) {
            hipLaunchKernelGGL(state_copy_kernel, dim3(fill_grid(nst)), dim3(256), 0, hs, gr->dh_final,
                               gr->dh0, nst);
            if (hipGetLastError() != hipSuccess) return M3_ERR_HIP;
        }
        return M3_OK;
    }
    if (lowmem && !scan_bwd_lowmem_ok(a)) return M3_ERR_UNSUPPORTED;
    const int windows = lowmem ? (int)s.nsegments : 0;
    const size_t need = scan_bwd_workspace_bytes(a, lowmem, windows);
    if (workspace == nullptr || ws_bytes < need) return M3_ERR_WORKSPACE_TOO_SMALL;
    BwdIO bio{};
    bio.dy = gr->dy; bio.dh_final = gr->dh_final; bio.dx = gr->dx; bio.dBraw = gr->dBraw; bio.dCraw = gr->dCraw;
    bio.ddt = gr->ddt; bio.dA = gr->dA; bio.dlam = gr->dlam; bio.dtheta = gr->dtheta; bio.dB_bias = gr->dB_bias;
    bio.dC_bias = gr->dC_bias; bio.dB_normw = gr->dB_normw; bio.dC_normw = gr->dC_normw; bio.dh0 = gr->dh0;
    bio.dx_prev = gr->dx_prev; bio.dBraw_prev = gr->dBraw_prev;
    e = launch_scan_bwd(a, bio, workspace, lowmem, windows, hs);
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status m3_decode_step(const m3_shape *shape, const m3_decode_io *io, void *stream) {
    if (!shape || !io) return M3_ERR_INVALID_ARG;
    const m3_shape &s = *shape;
    if (s.batch < 0 || s.nheads < 1 || s.ngroups < 1 || s.headdim < 1 || s.dstate < 2 || s.rank < 1)
        return M3_ERR_INVALID_ARG;
    if (s.nheads % s.ngroups != 0 || s.dstate % 2 != 0) return M3_ERR_INVALID_ARG;
    if (s.flags & ~(M3_FLAG_BF16_STATE | M3_FLAG_OUT_NORM | M3_FLAG_NORM_AFTER_GATE)) return M3_ERR_INVALID_ARG;
    if (s.io_dtype != M3_F32 && s.io_dtype != M3_BF16) return M3_ERR_INVALID_ARG;
    if (!(s.eps >= 0.f) || !isfinite(s.eps)) return M3_ERR_INVALID_ARG;
    if ((io->x_prev == nullptr) != (io->Braw_prev == nullptr)) return M3_ERR_INVALID_ARG;
    const int64_t N = s.dstate;
    if (!(N == 16 || N == 32 || N == 64 || N == 128 || N == 256) || s.headdim > kDecodeMaxP ||
        s.rank > kDecodeMaxR || s.batch > (1LL << 31) || s.nheads > (1LL << 20) || s.batch * s.nheads > kMaxGrid)
        return M3_ERR_UNSUPPORTED;
    const bool fused = io->W_X != nullptr;
    if (fused && (!io->W_Z || !io->W_O)) return M3_ERR_INVALID_ARG;
    if (!fused && (io->W_Z || io->W_O || io->z || io->o)) return M3_ERR_INVALID_ARG;
    if (!epilogue_ok(s.flags, fused, io->out_normw)) return M3_ERR_INVALID_ARG;
    if (s.batch > 0 && (!io->x || !io->Braw || !io->Craw || !io->dt || !io->A || !io->lam || !io->theta ||
                        !io->B_bias || !io->C_bias || !io->h || (fused ? (!io->z || !io->o) : !io->y)))
        return M3_ERR_INVALID_ARG;
    const void *ptrs[] = {io->x, io->Braw, io->Craw, io->dt, io->A, io->lam, io->theta, io->B_bias,
                          io->C_bias, io->B_normw, io->C_normw, io->x_prev, io->Braw_prev, io->h, io->y,
                          io->z, io->W_X, io->W_Z, io->W_O, io->o, io->D, io->out_normw};
    for (const void *p : ptrs)
        if (!aligned16(p)) return M3_ERR_MISALIGNED;
    if (s.batch == 0) return M3_OK;
    DecodeArgs a{};
    a.b = s.batch; a.H = s.nheads; a.G = s.ngroups; a.P = s.headdim; a.N = s.dstate; a.R = s.rank;
    a.hpg = s.nheads / s.ngroups;
    a.eps = s.eps; a.bf16 = (s.io_dtype == M3_BF16); a.has_prev = io->x_prev != nullptr;
    a.x = io->x; a.Braw = io->Braw; a.Craw = io->Craw; a.dt = io->dt; a.A = io->A; a.lam = io->lam;
    a.theta = io->theta; a.B_bias = io->B_bias; a.C_bias = io->C_bias; a.B_normw = io->B_normw;
    a.C_normw = io->C_normw; a.x_prev = io->x_prev; a.Braw_prev = io->Braw_prev; a.h = io->h; a.y = io->y;
    a.bf16_state = (s.flags & M3_FLAG_BF16_STATE) != 0;
    a.fused = fused; a.z = io->z; a.W_X = io->W_X; a.W_Z = io->W_Z; a.W_O = io->W_O; a.o = io->o;
    a.D = io->D; a.out_normw = io->out_normw;
    a.onorm = (s.flags & M3_FLAG_OUT_NORM) != 0;
    a.norm_after_gate = (s.flags & M3_FLAG_NORM_AFTER_GATE) != 0;
    hipError_t e = launch_decode(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // extern "C"
