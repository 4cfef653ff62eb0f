"""Thin Python binding of libm3 (include/m3.h): argument marshalling only.

Every step of the mixer runs in the library's HIP kernels; this module checks
every tensor against the shape and dtype the call implies (the C ABI sees raw
pointers only, so a short or mistyped buffer would be read or written past its
end on the GPU), then that tensors are contiguous GPU tensors on one device,
fills the C structs and passes raw pointers plus the current stream. All checks
raise before the library is called. If the library is not built, importing this
module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libm3.so")

M3_OK = 0
M3_F32, M3_BF16 = 0, 1
M3_FLAG_FORCE_GENERIC = 1
M3_FLAG_BF16_STATE = 2
M3_FLAG_OUT_NORM = 4
M3_FLAG_NORM_AFTER_GATE = 8
M3_FLAG_BWD_LOW_MEMORY = 16


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("ngroups", ctypes.c_int64), ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("rank", ctypes.c_int64), ("chunk", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("eps", ctypes.c_float), ("nsegments", ctypes.c_int32),
    ]


class ScanIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "Braw", "Craw", "dt", "A", "lam", "theta", "B_bias", "C_bias", "B_normw", "C_normw",
        "h0", "x_prev", "Braw_prev", "y", "h_final", "z", "W_X", "W_Z", "W_O", "o", "D", "out_normw")]


class DecodeIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "Braw", "Craw", "dt", "A", "lam", "theta", "B_bias", "C_bias", "B_normw", "C_normw",
        "x_prev", "Braw_prev", "h", "y", "z", "W_X", "W_Z", "W_O", "o", "D", "out_normw")]


class ScanGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dy", "dh_final", "dx", "dBraw", "dCraw", "ddt", "dA", "dlam", "dtheta", "dB_bias", "dC_bias",
        "dB_normw", "dC_normw", "dh0", "dx_prev", "dBraw_prev")]


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("nsegments", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


class DeviceFacts(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int32), ("clock_khz", ctypes.c_int32),
                ("memory_clock_khz", ctypes.c_int32), ("memory_bus_bits", ctypes.c_int32),
                ("wall_clock_khz", ctypes.c_int32), ("l2_bytes", ctypes.c_int64),
                ("lds_bytes_per_block", ctypes.c_int64), ("wave_size", ctypes.c_int32),
                ("arch", ctypes.c_char * 64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libm3.so is not built (%s); run __graft_entry__.build() or "
                          "python state_space_sequence_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.m3_scan_fwd.restype = ctypes.c_int
    lib.m3_scan_fwd.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ScanIO), ctypes.c_void_p,
                                ctypes.c_size_t, ctypes.c_void_p]
    lib.m3_scan_bwd.restype = ctypes.c_int
    lib.m3_scan_bwd.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ScanIO), ctypes.POINTER(ScanGrads),
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.m3_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.m3_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Shape)]
    lib.m3_decode_step.restype = ctypes.c_int
    lib.m3_decode_step.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(DecodeIO), ctypes.c_void_p]
    lib.m3_scan_fwd_noalloc.restype = ctypes.c_int
    lib.m3_scan_fwd_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ScanIO), ctypes.c_void_p]
    lib.m3_scan_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
    lib.m3_scan_noalloc_max_workspace_bytes.argtypes = []
    lib.m3_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.m3_scan_workspace_bytes.argtypes = [ctypes.POINTER(Shape)]
    lib.m3_scan_plan.restype = ctypes.c_int
    lib.m3_scan_plan.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Plan)]
    lib.m3_status_str.restype = ctypes.c_char_p
    lib.m3_status_str.argtypes = [ctypes.c_int]
    lib.m3_version.restype = ctypes.c_int
    lib.m3_expand_ranks.restype = ctypes.c_int
    lib.m3_expand_ranks.argtypes = [ctypes.POINTER(Shape)] + [ctypes.c_void_p] * 4
    lib.m3_gate_contract.restype = ctypes.c_int
    lib.m3_gate_contract.argtypes = [ctypes.POINTER(Shape)] + [ctypes.c_void_p] * 6
    lib.m3_probe_copy.restype = ctypes.c_int
    lib.m3_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.m3_probe_mfma_bf16.restype = ctypes.c_int
    lib.m3_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_void_p]
    lib.m3_probe_device_facts.restype = ctypes.c_int
    lib.m3_probe_device_facts.argtypes = [ctypes.c_int, ctypes.POINTER(DeviceFacts)]
    return lib


lib = _load()


class M3Error(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__("libm3: %s (%d)" % (lib.m3_status_str(code).decode(), code))


def _check(rc: int):
    if rc != M3_OK:
        raise M3Error(rc)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(name, t, shape, dtype, device=None):
    """Raise unless t is None or a tensor of exactly this shape and dtype (dtype may
    be a tuple of allowed dtypes) and, when given, on the device of that index."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.dtype is not dtype and not (isinstance(dtype, tuple) and t.dtype in dtype):
        raise TypeError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.shape != shape:
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if device is not None and t.get_device() != device:
        raise ValueError("%s: on device %d, expected %d (the device of the inputs)" % (name, t.get_device(), device))


def _expect_all(specs, device):
    """specs: (name, tensor, shape tuple, dtype); device: get_device() of the inputs."""
    for name, t, shape, dtype in specs:
        if t is not None:
            _expect(name, t, shape, dtype, device)


def _need(name, t):
    if t is None:
        raise ValueError("%s is required" % name)


def _scan_specs(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, h0, x_prev, Braw_prev,
                *, b, L, H, G, R, P, N, io, xr=True):
    """(name, tensor, shape, dtype) of the prefill inputs; xr: x and x_prev carry the
    rank axis (False for the fused projections' X')."""
    f32 = torch.float32
    xs = (b, L, H, R, P) if xr else (b, L, H, P)
    xps = (b, H, R, P) if xr else (b, H, P)
    return [("x", x, xs, io), ("Braw", Braw, (b, L, G, R, N), io), ("Craw", Craw, (b, L, G, R, N), io),
            ("dt", dt, (b, L, H), f32), ("A", A, (b, L, H), f32), ("lam", lam, (b, L, H), f32),
            ("theta", theta, (b, L, G, N // 2), f32), ("B_bias", B_bias, (H, R, N), f32),
            ("C_bias", C_bias, (H, R, N), f32), ("B_normw", B_normw, (N,), f32),
            ("C_normw", C_normw, (N,), f32), ("h0", h0, (b, H, P, N), f32),
            ("x_prev", x_prev, xps, io), ("Braw_prev", Braw_prev, (b, G, R, N), io)]


def _epilogue_specs(D, out_normw, H, P):
    return [("D", D, (H,), torch.float32), ("out_normw", out_normw, (H, P), torch.float32)]


def _weight_specs(W_X, W_Z, W_O, H, P, R):
    f32 = torch.float32
    return [("W_X", W_X, (H, P, R), f32), ("W_Z", W_Z, (H, P, R), f32), ("W_O", W_O, (H, P, R), f32)]


def _decode_specs(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, x_prev, Braw_prev, h,
                  *, b, H, G, R, P, N, io, xr=True):
    f32 = torch.float32
    xs = (b, H, R, P) if xr else (b, H, P)
    return [("x", x, xs, io), ("Braw", Braw, (b, G, R, N), io), ("Craw", Craw, (b, G, R, N), io),
            ("dt", dt, (b, H), f32), ("A", A, (b, H), f32), ("lam", lam, (b, H), f32),
            ("theta", theta, (b, G, N // 2), f32), ("B_bias", B_bias, (H, R, N), f32),
            ("C_bias", C_bias, (H, R, N), f32), ("B_normw", B_normw, (N,), f32),
            ("C_normw", C_normw, (N,), f32), ("x_prev", x_prev, xs, io),
            ("Braw_prev", Braw_prev, (b, G, R, N), io), ("h", h, (b, H, P, N), (f32, torch.bfloat16))]


def _dims5(name, t, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor" % name)
    if t.dim() != ndim:
        raise ValueError("%s: expected %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    return tuple(t.shape)


def _io_dtype(t):
    if t.dtype == torch.bfloat16:
        return M3_BF16
    if t.dtype == torch.float32:
        return M3_F32
    raise TypeError("io tensors must be float32 or bfloat16, got %s" % t.dtype)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(batch, seqlen, nheads, ngroups, headdim, dstate, rank, chunk, io_dtype, eps=1e-5,
               flags=0, nsegments=0) -> Shape:
    return Shape(batch, seqlen, nheads, ngroups, headdim, dstate, rank, chunk, io_dtype, flags, eps, nsegments)


def _norm_flags(out_norm) -> int:
    """out_norm: False/None (no output norm), True or "pre" (norm y, or Y before the
    gate), "post" (norm O' after the gate; fused form only)."""
    if not out_norm:
        return 0
    if out_norm is True or out_norm == "pre":
        return M3_FLAG_OUT_NORM
    if out_norm == "post":
        return M3_FLAG_OUT_NORM | M3_FLAG_NORM_AFTER_GATE
    raise ValueError("out_norm must be False, True, 'pre' or 'post'")


def scan_shape(x, Braw, chunk, eps=1e-5, *, force_generic=False, nsegments=0, out_norm=False) -> Shape:
    b, L, H, R, P = x.shape
    G, N = Braw.shape[2], Braw.shape[4]
    return make_shape(b, L, H, G, P, N, R, chunk, _io_dtype(x), eps,
                      (M3_FLAG_FORCE_GENERIC if force_generic else 0) | _norm_flags(out_norm), nsegments)


def plan(shape: Shape) -> Plan:
    p = Plan()
    _check(lib.m3_scan_plan(ctypes.byref(shape), ctypes.byref(p)))
    return p


def workspace_bytes(shape: Shape) -> int:
    return int(lib.m3_scan_workspace_bytes(ctypes.byref(shape)))


def scan_fwd(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, *, chunk=64, eps=1e-5,
             B_normw=None, C_normw=None, h0=None, x_prev=None, Braw_prev=None,
             y=None, h_final=None, want_state=True, workspace=None, nsegments=0,
             force_generic=False, D=None, out_norm=False, out_normw=None, stream=None):
    """Chunked-scan prefill (m3_scan_fwd). Shapes: x [b,L,H,R,P], Braw/Craw [b,L,G,R,N],
    dt/A/lam [b,L,H], theta [b,L,G,N/2], biases [H,R,N]; optional skip D [H] and output
    norm (out_norm=True, gain out_normw [H,P]). Returns (y, h_final)."""
    b, L, H, R, P = _dims5("x", x, 5)
    _, _, G, _, N = _dims5("Braw", Braw, 5)
    io = x.dtype
    _io_dtype(x)
    _expect_all(_scan_specs(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, h0, x_prev,
                            Braw_prev, b=b, L=L, H=H, G=G, R=R, P=P, N=N, io=io)
                + _epilogue_specs(D, out_normw, H, P)
                + [("y", y, (b, L, H, R, P), io), ("h_final", h_final, (b, H, P, N), torch.float32),
                   ("workspace", workspace, (None if workspace is None else workspace.numel(),), torch.uint8)],
                x.get_device())
    shape = scan_shape(x, Braw, chunk, eps, force_generic=force_generic, nsegments=nsegments,
                       out_norm=out_norm)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None and want_state:
        h_final = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    ws = workspace_bytes(shape)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=x.device)
    io = ScanIO(_ptr(x), _ptr(Braw), _ptr(Craw), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                _ptr(B_bias), _ptr(C_bias), _ptr(B_normw), _ptr(C_normw), _ptr(h0),
                _ptr(x_prev), _ptr(Braw_prev), _ptr(y), _ptr(h_final))
    io.D, io.out_normw = _ptr(D), _ptr(out_normw)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.m3_scan_fwd(ctypes.byref(shape), ctypes.byref(io), _ptr(workspace), wsb, _stream(stream)))
    return y, h_final


def scan_fwd_noalloc(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, y, h_final, *, chunk=64, eps=1e-5,
                     B_normw=None, C_normw=None, h0=None, x_prev=None, Braw_prev=None, nsegments=0,
                     force_generic=False, D=None, out_norm=False, out_normw=None, stream=None):
    """m3_scan_fwd_noalloc: scan_fwd for callers that cannot allocate. The caller
    passes the outputs y [b,L,H,R,P] (io dtype) and h_final [b,H,P,N] fp32 (or None);
    the workspace (normalised B and C rows, segment records) is the library's per-GPU array. Nothing is
    allocated here either. Returns (y, h_final)."""
    b, L, H, R, P = _dims5("x", x, 5)
    _, _, G, _, N = _dims5("Braw", Braw, 5)
    _io_dtype(x)
    _need("y", y)
    _expect_all(_scan_specs(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, h0, x_prev,
                            Braw_prev, b=b, L=L, H=H, G=G, R=R, P=P, N=N, io=x.dtype)
                + _epilogue_specs(D, out_normw, H, P)
                + [("y", y, (b, L, H, R, P), x.dtype), ("h_final", h_final, (b, H, P, N), torch.float32)],
                x.get_device())
    shape = scan_shape(x, Braw, chunk, eps, force_generic=force_generic, nsegments=nsegments,
                       out_norm=out_norm)
    io = ScanIO(_ptr(x), _ptr(Braw), _ptr(Craw), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                _ptr(B_bias), _ptr(C_bias), _ptr(B_normw), _ptr(C_normw), _ptr(h0),
                _ptr(x_prev), _ptr(Braw_prev), _ptr(y), _ptr(h_final))
    io.D, io.out_normw = _ptr(D), _ptr(out_normw)
    _check(lib.m3_scan_fwd_noalloc(ctypes.byref(shape), ctypes.byref(io), _stream(stream)))
    return y, h_final


def noalloc_max_workspace_bytes() -> int:
    return int(lib.m3_scan_noalloc_max_workspace_bytes())


def scan_fused_fwd(x_in, z_in, W_X, W_Z, W_O, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, *,
                   chunk=64, eps=1e-5, B_normw=None, C_normw=None, h0=None, x_prev_in=None,
                   Braw_prev=None, o=None, h_final=None, want_state=True, workspace=None,
                   nsegments=0, D=None, out_norm=None, out_normw=None, stream=None):
    """Prefill with the fused MIMO projections and gate (m3_scan_fwd with W_X set).
    x_in, z_in [b,L,H,P] (X', Z'), W_X/W_Z/W_O [H,P,R], x_prev_in [b,H,P] or None;
    skip D [H], output norm out_norm None / "pre" / "post" with gain out_normw [H,P].
    Returns (o [b,L,H,P], h_final)."""
    b, L, H, P = _dims5("x_in", x_in, 4)
    R = _dims5("W_X", W_X, 3)[2]
    _, _, G, _, N = _dims5("Braw", Braw, 5)
    io = x_in.dtype
    iot = _io_dtype(x_in)
    _expect_all(_scan_specs(x_in, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, h0,
                            x_prev_in, Braw_prev, b=b, L=L, H=H, G=G, R=R, P=P, N=N, io=io, xr=False)
                + _weight_specs(W_X, W_Z, W_O, H, P, R) + _epilogue_specs(D, out_normw, H, P)
                + [("z_in", z_in, (b, L, H, P), io), ("o", o, (b, L, H, P), io),
                   ("h_final", h_final, (b, H, P, N), torch.float32),
                   ("workspace", workspace, (None if workspace is None else workspace.numel(),), torch.uint8)],
                x_in.get_device())
    shape = make_shape(b, L, H, G, P, N, R, chunk, iot, eps, _norm_flags(out_norm), nsegments)
    if o is None:
        o = torch.empty_like(x_in)
    if h_final is None and want_state:
        h_final = torch.empty((b, H, P, N), dtype=torch.float32, device=x_in.device)
    ws = workspace_bytes(shape)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=x_in.device)
    io = ScanIO(_ptr(x_in), _ptr(Braw), _ptr(Craw), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                _ptr(B_bias), _ptr(C_bias), _ptr(B_normw), _ptr(C_normw), _ptr(h0),
                _ptr(x_prev_in), _ptr(Braw_prev), None, _ptr(h_final),
                _ptr(z_in), _ptr(W_X), _ptr(W_Z), _ptr(W_O), _ptr(o), _ptr(D), _ptr(out_normw))
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.m3_scan_fwd(ctypes.byref(shape), ctypes.byref(io), _ptr(workspace), wsb, _stream(stream)))
    return o, h_final


def scan_bwd_workspace_bytes(shape: Shape) -> int:
    return int(lib.m3_scan_bwd_workspace_bytes(ctypes.byref(shape)))


def scan_bwd(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, dy, *, eps=1e-5, B_normw=None,
             C_normw=None, h0=None, x_prev=None, Braw_prev=None, dh_final=None, want_dh0=True,
             workspace=None, grads=None, low_memory=False, windows=0, stream=None):
    """Prefill backward (m3_scan_bwd): gradients of <dy, y> + <dh_final, h_final> with
    respect to the forward inputs (same tensors as scan_fwd). Returns a dict of fp32
    tensors named like the inputs (x, Braw, ..., h0, x_prev, Braw_prev when present).
    low_memory: the windowed schedule (M3_FLAG_BWD_LOW_MEMORY), same results in a
    smaller workspace for about one more forward sweep of time; windows > 0 sets the
    number of windows (0: the count that minimises the workspace)."""
    b, L, H, R, P = _dims5("x", x, 5)
    _, _, G, _, N = _dims5("Braw", Braw, 5)
    iot = _io_dtype(x)
    _expect_all(_scan_specs(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, h0, x_prev,
                            Braw_prev, b=b, L=L, H=H, G=G, R=R, P=P, N=N, io=x.dtype)
                + [("dy", dy, (b, L, H, R, P), x.dtype), ("dh_final", dh_final, (b, H, P, N), torch.float32),
                   ("workspace", workspace, (None if workspace is None else workspace.numel(),), torch.uint8)],
                x.get_device())
    _need("dy", dy)
    shape = make_shape(b, L, H, G, P, N, R, max(1, 64 // R), iot, eps,
                       M3_FLAG_BWD_LOW_MEMORY if low_memory else 0, windows if low_memory else 0)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    if grads is None:
        grads = {"x": torch.empty(x.shape, **f32), "Braw": torch.empty(Braw.shape, **f32),
                 "Craw": torch.empty(Craw.shape, **f32), "dt": torch.empty(dt.shape, **f32),
                 "A": torch.empty(A.shape, **f32), "lam": torch.empty(lam.shape, **f32),
                 "theta": torch.empty(theta.shape, **f32), "B_bias": torch.empty(B_bias.shape, **f32),
                 "C_bias": torch.empty(C_bias.shape, **f32)}
        if B_normw is not None:
            grads["B_normw"] = torch.empty(B_normw.shape, **f32)
        if C_normw is not None:
            grads["C_normw"] = torch.empty(C_normw.shape, **f32)
        if want_dh0:
            grads["h0"] = torch.empty((b, H, P, N), **f32)
        if x_prev is not None:
            grads["x_prev"] = torch.empty(x_prev.shape, **f32)
            grads["Braw_prev"] = torch.empty(Braw_prev.shape, **f32)
    # every gradient buffer is fp32 and shaped like the input it belongs to
    gshape = {"x": x.shape, "Braw": Braw.shape, "Craw": Craw.shape, "dt": dt.shape, "A": A.shape,
              "lam": lam.shape, "theta": theta.shape, "B_bias": B_bias.shape, "C_bias": C_bias.shape,
              "B_normw": (N,), "C_normw": (N,), "h0": (b, H, P, N), "x_prev": (b, H, R, P),
              "Braw_prev": (b, G, R, N)}
    for k, t in grads.items():
        if k not in gshape:
            raise ValueError("grads: unknown entry %r" % k)
        _expect("grads[%r]" % k, t, tuple(gshape[k]), torch.float32, x.get_device())
    ws = scan_bwd_workspace_bytes(shape)
    if workspace is None and ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    io = ScanIO(_ptr(x), _ptr(Braw), _ptr(Craw), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                _ptr(B_bias), _ptr(C_bias), _ptr(B_normw), _ptr(C_normw), _ptr(h0),
                _ptr(x_prev), _ptr(Braw_prev), None, None)
    gd = grads.get
    gs = ScanGrads(_ptr(dy), _ptr(dh_final), _ptr(gd("x")), _ptr(gd("Braw")), _ptr(gd("Craw")), _ptr(gd("dt")),
                   _ptr(gd("A")), _ptr(gd("lam")), _ptr(gd("theta")), _ptr(gd("B_bias")), _ptr(gd("C_bias")),
                   _ptr(gd("B_normw")), _ptr(gd("C_normw")), _ptr(gd("h0")), _ptr(gd("x_prev")),
                   _ptr(gd("Braw_prev")))
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.m3_scan_bwd(ctypes.byref(shape), ctypes.byref(io), ctypes.byref(gs), _ptr(workspace), wsb,
                           _stream(stream)))
    return grads


def decode_step(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, h, *, eps=1e-5,
                B_normw=None, C_normw=None, x_prev=None, Braw_prev=None, y=None, D=None,
                out_norm=False, out_normw=None, stream=None):
    """One decode step (m3_decode_step). x [b,H,R,P], Braw/Craw [b,G,R,N], dt/A/lam [b,H],
    theta [b,G,N/2], h [b,H,P,N] updated in place: fp32, or bf16 (then the step runs with
    M3_FLAG_BF16_STATE); skip D and output norm as in scan_fwd. Returns y [b,H,R,P]."""
    b, H, R, P = _dims5("x", x, 4)
    _, G, _, N = _dims5("Braw", Braw, 4)
    iot = _io_dtype(x)
    _need("h", h)
    _expect_all(_decode_specs(x, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw, x_prev,
                              Braw_prev, h, b=b, H=H, G=G, R=R, P=P, N=N, io=x.dtype)
                + _epilogue_specs(D, out_normw, H, P) + [("y", y, (b, H, R, P), x.dtype)], x.get_device())
    flags = (M3_FLAG_BF16_STATE if h.dtype == torch.bfloat16 else 0) | _norm_flags(out_norm)
    shape = make_shape(b, 1, H, G, P, N, R, 1, iot, eps, flags)
    if y is None:
        y = torch.empty_like(x)
    io = DecodeIO(_ptr(x), _ptr(Braw), _ptr(Craw), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                  _ptr(B_bias), _ptr(C_bias), _ptr(B_normw), _ptr(C_normw), _ptr(x_prev),
                  _ptr(Braw_prev), _ptr(h), _ptr(y))
    io.D, io.out_normw = _ptr(D), _ptr(out_normw)
    _check(lib.m3_decode_step(ctypes.byref(shape), ctypes.byref(io), _stream(stream)))
    return y


def decode_fused_step(x_in, z_in, W_X, W_Z, W_O, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, h, *,
                      eps=1e-5, B_normw=None, C_normw=None, x_prev_in=None, Braw_prev=None, o=None,
                      D=None, out_norm=None, out_normw=None, stream=None):
    """One decode step with the fused projections. x_in, z_in [b,H,P], W_* [H,P,R],
    h [b,H,P,N] (fp32 or bf16) updated in place. Returns o [b,H,P]."""
    b, H, P = _dims5("x_in", x_in, 3)
    R = _dims5("W_X", W_X, 3)[2]
    _, G, _, N = _dims5("Braw", Braw, 4)
    iot = _io_dtype(x_in)
    _need("h", h)
    _expect_all(_decode_specs(x_in, Braw, Craw, dt, A, lam, theta, B_bias, C_bias, B_normw, C_normw,
                              x_prev_in, Braw_prev, h, b=b, H=H, G=G, R=R, P=P, N=N, io=x_in.dtype, xr=False)
                + _weight_specs(W_X, W_Z, W_O, H, P, R) + _epilogue_specs(D, out_normw, H, P)
                + [("z_in", z_in, (b, H, P), x_in.dtype), ("o", o, (b, H, P), x_in.dtype)], x_in.get_device())
    flags = (M3_FLAG_BF16_STATE if h.dtype == torch.bfloat16 else 0) | _norm_flags(out_norm)
    shape = make_shape(b, 1, H, G, P, N, R, 1, iot, eps, flags)
    if o is None:
        o = torch.empty_like(x_in)
    io = DecodeIO(_ptr(x_in), _ptr(Braw), _ptr(Craw), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                  _ptr(B_bias), _ptr(C_bias), _ptr(B_normw), _ptr(C_normw), _ptr(x_prev_in),
                  _ptr(Braw_prev), _ptr(h), None, _ptr(z_in), _ptr(W_X), _ptr(W_Z), _ptr(W_O), _ptr(o),
                  _ptr(D), _ptr(out_normw))
    _check(lib.m3_decode_step(ctypes.byref(shape), ctypes.byref(io), _stream(stream)))
    return o


# ---------------------------------------------------------------- helpers ---
def to_device(inp: dict, io: str, device="cuda"):
    """Move a numpy input dict (from state_space_sequence_amd.inputs) to the GPU:
    io tensors in bf16 or fp32 (bf16 values are exact), the rest fp32."""
    io_keys = ("x", "Braw", "Craw", "x_prev", "Braw_prev", "x_in", "z_in", "x_prev_in")
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(v).to(device)
        if k in io_keys and io == "bf16":
            t = t.to(torch.bfloat16)
        out[k] = t.contiguous()
    return out


# -------------------------------------------- unfused projections (App. C) ---
def expand_ranks(x_in, W_X, x_out=None, stream=None):
    """m3_expand_ranks: x_in [..., H, P] (io dtype), W_X [H, P, R] fp32 ->
    x_out [..., H, R, P] with x_out[..., h, r, p] = W_X[h, p, r] * x_in[..., h, p]."""
    H, P = x_in.shape[-2], x_in.shape[-1]
    R = _dims5("W_X", W_X, 3)[2]
    iot = _io_dtype(x_in)
    lead = tuple(x_in.shape[:-2])
    _expect_all([("W_X", W_X, (H, P, R), torch.float32),
                 ("x_out", x_out, lead + (H, R, P), x_in.dtype)], x_in.get_device())
    if x_out is None:
        x_out = torch.empty(lead + (H, R, P), dtype=x_in.dtype, device=x_in.device)
    rows = 1
    for v in lead:
        rows *= int(v)
    shape = make_shape(rows, 1, H, 1, P, 2, R, 1, iot)
    _check(lib.m3_expand_ranks(ctypes.byref(shape), _ptr(x_in), _ptr(W_X), _ptr(x_out), _stream(stream)))
    return x_out


def gate_contract(y, z_in, W_Z, W_O, o=None, stream=None):
    """m3_gate_contract: y [..., H, R, P], z_in [..., H, P] (io dtype), W_Z, W_O [H, P, R]
    fp32 -> o [..., H, P] = sum_r W_O * y * SiLU(W_Z * z_in)."""
    H, R, P = y.shape[-3], y.shape[-2], y.shape[-1]
    iot = _io_dtype(y)
    lead = tuple(y.shape[:-3])
    _expect_all([("z_in", z_in, lead + (H, P), y.dtype), ("W_Z", W_Z, (H, P, R), torch.float32),
                 ("W_O", W_O, (H, P, R), torch.float32), ("o", o, lead + (H, P), y.dtype)], y.get_device())
    _need("z_in", z_in)
    if o is None:
        o = torch.empty(lead + (H, P), dtype=y.dtype, device=y.device)
    rows = 1
    for v in lead:
        rows *= int(v)
    shape = make_shape(rows, 1, H, 1, P, 2, R, 1, iot)
    _check(lib.m3_gate_contract(ctypes.byref(shape), _ptr(y), _ptr(z_in), _ptr(W_Z), _ptr(W_O), _ptr(o),
                                _stream(stream)))
    return o


# ------------------------------------------------------ calibration probes ---
def probe_copy(src, dst, blocks=0, stream=None):
    """m3_probe_copy: dst <- src (same number of bytes, uint8 or any dtype, contiguous)."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("probe_copy: src and dst sizes differ")
    _check(lib.m3_probe_copy(_ptr(src), _ptr(dst), nb, int(blocks), _stream(stream)))


def probe_mfma_bf16(blocks, iters, seed=1.0, out=None, clock=None, stream=None):
    """m3_probe_mfma_bf16: returns (out float[blocks], clock int64[2*blocks]) on the GPU;
    flops = blocks * 4 * iters * 2 * 16384."""
    dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty(blocks, dtype=torch.float32, device=dev)
    if clock is None:
        clock = torch.empty(2 * blocks, dtype=torch.int64, device=dev)
    _expect("out", out, (blocks,), torch.float32)
    _expect("clock", clock, (2 * blocks,), torch.int64)
    _check(lib.m3_probe_mfma_bf16(_ptr(out), _ptr(clock), int(blocks), int(iters), float(seed), _stream(stream)))
    return out, clock


def probe_mfma_flops(blocks, iters) -> int:
    return blocks * 4 * iters * 2 * 16 * 16 * 32 * 2


def device_facts(dev=0) -> dict:
    f = DeviceFacts()
    _check(lib.m3_probe_device_facts(int(dev), ctypes.byref(f)))
    return {"compute_units": f.compute_units, "clock_mhz": f.clock_khz / 1e3,
            "memory_clock_mhz": f.memory_clock_khz / 1e3, "memory_bus_bits": f.memory_bus_bits,
            "wall_clock_mhz": f.wall_clock_khz / 1e3, "l2_bytes": f.l2_bytes,
            "lds_bytes_per_block": f.lds_bytes_per_block, "wave_size": f.wave_size,
            "arch": f.arch.decode(errors="replace")}
