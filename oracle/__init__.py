"""CPU fp64 oracle for the Mamba-3 SSM mixer core (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never touches it, and it never touches the product path.

``scan`` runs the plain sequential recurrence of ``m3_oracle.c`` (see the header
there for the definition and its sources on the pages). Inputs are the float32
arrays made by ``state_space_sequence_amd.inputs``; outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB = os.path.join(_HERE, "_m3_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    """The compiled oracle. M3_ORACLE_LIB names another build of the same source to
    load instead (the sanitizer test runs the pins against an ASan/UBSan build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("M3_ORACLE_LIB")
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        f = lib.m3o_scan
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_long] * 7 + [ctypes.c_double] + [ctypes.c_void_p] * 16 + [ctypes.c_int]
        lib.m3o_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().m3o_max_threads())


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"], "oracle inputs are contiguous float32"
    return a.ctypes.data


def scan(inp: dict, shape, *, nthreads: int = 0, want_state: bool = True):
    """Run the oracle recurrence. Returns (y [b,L,H,R,P], h_final [b,H,P,N]) in float64."""
    lib = _load()
    b, L, H, G = shape.batch, shape.seqlen, shape.nheads, shape.ngroups
    P, N, R = shape.headdim, shape.dstate, shape.rank
    arr = {k: (None if v is None else np.ascontiguousarray(v, dtype=np.float32)) for k, v in inp.items()}
    y = np.empty((b, L, H, R, P), dtype=np.float64)
    hf = np.empty((b, H, P, N), dtype=np.float64) if want_state else None
    rc = lib.m3o_scan(b, L, H, G, P, N, R, float(shape.eps),
                      _ptr(arr["x"]), _ptr(arr["Braw"]), _ptr(arr["Craw"]),
                      _ptr(arr["dt"]), _ptr(arr["A"]), _ptr(arr["lam"]), _ptr(arr["theta"]),
                      _ptr(arr["B_bias"]), _ptr(arr["C_bias"]),
                      _ptr(arr.get("B_normw")), _ptr(arr.get("C_normw")),
                      _ptr(arr.get("h0")), _ptr(arr.get("x_prev")), _ptr(arr.get("Braw_prev")),
                      y.ctypes.data, None if hf is None else hf.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle scan failed with code %d" % rc)
    return y, hf


def decode(inp: dict, shape, *, nthreads: int = 0):
    """One decode step = the recurrence at L=1 from state ``h`` with the previous
    token (if given). Per-token tensors carry no L axis. Returns (y [b,H,R,P], h_new)."""
    s = shape.replace(seqlen=1)
    d = {}
    for k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta"):
        d[k] = np.ascontiguousarray(inp[k][:, None])
    for k in ("B_bias", "C_bias", "B_normw", "C_normw", "x_prev", "Braw_prev"):
        d[k] = inp.get(k)
    d["h0"] = inp["h"]
    y, h = scan(d, s, nthreads=nthreads)
    return y[:, 0], h


# ---------------------------------------------------------------------------
# Fused MIMO projections and output gate (Mamba-3 paper, App. C "MIMO for
# Mamba-3"): inside a head, the rank-R input is the per-rank scaling of one
# P-vector, the gate Z is formed the same way, the SSM output Y (P x R) is
# gated by SiLU(Z) and contracted back to P with per-(p, r) weights.
# Weights are per head: W_X, W_Z, W_O of shape [H, P, R].

def expand_ranks(v, W):
    """App. C, X_t = contract(PR, P -> PR)(W_X, X'_t): out[..., h, r, p] = W[h, p, r] * v[..., h, p].
    v has shape [..., H, P]; returns float64 [..., H, R, P]."""
    v = np.asarray(v, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return v[..., None, :] * np.swapaxes(W, -1, -2)


def silu(z):
    """App. C's residual function uses SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def gate_contract(y, z_in, W_Z, W_O):
    """App. C: Z = W_Z (.) Z' (as for X), Y' = Y (.) SiLU(Z), O' = contract(PR, PR -> P)(W_O', Y'):
    O'[..., h, p] = sum_r W_O[h, p, r] * Y[..., h, r, p] * SiLU(Z[..., h, r, p])."""
    z = expand_ranks(z_in, W_Z)
    gated = np.asarray(y, dtype=np.float64) * silu(z)
    return np.einsum("...hrp,hpr->...hp", gated, np.asarray(W_O, dtype=np.float64))


def scan_fused(inp: dict, shape, *, nthreads: int = 0, want_state: bool = True):
    """Prefill with the fused projections: inputs carry x_in [b,L,H,P] (X'), z_in [b,L,H,P] (Z'),
    W_X / W_Z / W_O [H,P,R] and, optionally, x_prev_in [b,H,P]. Returns (O' [b,L,H,P], h_final)."""
    d = dict(inp)
    d["x"] = expand_ranks(inp["x_in"], inp["W_X"]).astype(np.float32)
    xp = inp.get("x_prev_in")
    d["x_prev"] = None if xp is None else expand_ranks(xp, inp["W_X"]).astype(np.float32)
    y, h = scan(d, shape, nthreads=nthreads, want_state=want_state)
    return gate_contract(y, inp["z_in"], inp["W_Z"], inp["W_O"]), h


def decode_fused(inp: dict, shape, *, nthreads: int = 0):
    """One decode step with the fused projections (per-token tensors without the L axis:
    x_in, z_in [b,H,P], x_prev_in [b,H,P] or absent). Returns (O' [b,H,P], h_new)."""
    d = dict(inp)
    d["x"] = expand_ranks(inp["x_in"], inp["W_X"]).astype(np.float32)
    xp = inp.get("x_prev_in")
    d["x_prev"] = None if xp is None else expand_ranks(xp, inp["W_X"]).astype(np.float32)
    y, h = decode(d, shape, nthreads=nthreads)
    return gate_contract(y, inp["z_in"], inp["W_Z"], inp["W_O"]), h


# ---------------------------------------------------------------------------
# Skip term and output norm. The skip is the D term of the SSM output equation
# (szyisi.cn article on Mamba-3, section introducing state space models:
# y = C h + D x), one weight per head, added to every rank row of y. The
# optional output RMSNorm is the Mamba-2 norm that BCNorm makes optional
# (Mamba-3 paper §3.4 "BC / QK normalization"), studied in §4.1.2 / Table 4 and
# App. E Table 9 as grouped or default, before or after the gate. Built here:
# the grouped form with one group per head (RMS over that head's P channels of
# one token and rank row), with a per-channel gain [H, P], ε the BCNorm ε.

def d_skip(y, x, D):
    """y + D[h] x for y, x of shape [..., H, R, P] and D of shape [H]."""
    y = np.asarray(y, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return y + np.asarray(D, dtype=np.float64)[:, None, None] * x


def out_rmsnorm(v, w, eps, *, rank_axis: bool):
    """Grouped output RMSNorm: v / sqrt(mean over the last axis (P) of v^2 + eps), times
    the gain w [H, P] (ones when None). v is [..., H, R, P] (rank_axis) or [..., H, P]."""
    v = np.asarray(v, dtype=np.float64)
    out = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + float(eps))
    if w is not None:
        w = np.asarray(w, dtype=np.float64)
        out = out * (w[:, None, :] if rank_axis else w)
    return out


def scan_out(inp: dict, shape, *, out_norm: bool = False, nthreads: int = 0):
    """Prefill with the skip term (inp["D"], [H], optional) and, if out_norm, the grouped
    output RMSNorm (gain inp["out_normw"], optional) on y. Returns (y, h_final)."""
    y, h = scan(inp, shape, nthreads=nthreads)
    if inp.get("D") is not None:
        y = d_skip(y, inp["x"], inp["D"])
    if out_norm:
        y = out_rmsnorm(y, inp.get("out_normw"), shape.eps, rank_axis=True)
    return y, h


def decode_out(inp: dict, shape, *, out_norm: bool = False, nthreads: int = 0):
    """decode with the skip term and the optional output norm (see scan_out)."""
    y, h = decode(inp, shape, nthreads=nthreads)
    if inp.get("D") is not None:
        y = d_skip(y, inp["x"], inp["D"])
    if out_norm:
        y = out_rmsnorm(y, inp.get("out_normw"), shape.eps, rank_axis=True)
    return y, h


def _gated_out(y, x, inp, eps, out_norm):
    """Y (+ D X), normed before the gate ("pre") or O' normed after the gate and the
    rank contraction ("post"), or neither (None)."""
    if inp.get("D") is not None:
        y = d_skip(y, x, inp["D"])
    if out_norm == "pre":
        y = out_rmsnorm(y, inp.get("out_normw"), eps, rank_axis=True)
    o = gate_contract(y, inp["z_in"], inp["W_Z"], inp["W_O"])
    if out_norm == "post":
        o = out_rmsnorm(o, inp.get("out_normw"), eps, rank_axis=False)
    return o


def scan_fused_out(inp: dict, shape, *, out_norm=None, nthreads: int = 0):
    """scan_fused with the skip term on Y (D times the expanded X) and the output norm
    before ("pre") or after ("post") the gate. Returns (O', h_final)."""
    d = dict(inp)
    d["x"] = expand_ranks(inp["x_in"], inp["W_X"]).astype(np.float32)
    xp = inp.get("x_prev_in")
    d["x_prev"] = None if xp is None else expand_ranks(xp, inp["W_X"]).astype(np.float32)
    y, h = scan(d, shape, nthreads=nthreads)
    return _gated_out(y, d["x"], inp, shape.eps, out_norm), h


def decode_fused_out(inp: dict, shape, *, out_norm=None, nthreads: int = 0):
    """decode_fused with the skip term and the output norm (see scan_fused_out)."""
    d = dict(inp)
    d["x"] = expand_ranks(inp["x_in"], inp["W_X"]).astype(np.float32)
    xp = inp.get("x_prev_in")
    d["x_prev"] = None if xp is None else expand_ranks(xp, inp["W_X"]).astype(np.float32)
    y, h = decode(d, shape, nthreads=nthreads)
    return _gated_out(y, d["x"], inp, shape.eps, out_norm), h


# ---------------------------------------------------------------------------
# Gradients of the prefill (training backward). The pages give no backward
# derivation, so the oracle takes the plainest one: the derivative of the
# forward's definition. ``scan_torch`` restates the sequential physical-frame
# recurrence of m3_oracle.c (same definition, written independently with torch
# float64 tensors on the CPU, one token at a time), and ``scan_grads`` applies
# reverse-mode differentiation (torch.autograd, a library primitive) to it.
# Pinned by: its forward agreeing with the C oracle, and its gradients agreeing
# with central finite differences of the C oracle.

GRAD_INPUTS = ("x", "Braw", "Craw", "dt", "A", "lam", "theta", "B_bias", "C_bias",
               "B_normw", "C_normw", "h0", "x_prev", "Braw_prev")


def scan_torch(t: dict, shape):
    """The recurrence on torch float64 tensors t[...] (same layouts as scan). Returns
    (y [b,L,H,R,P], h_final [b,H,P,N])."""
    import torch
    b, L, H, G = shape.batch, shape.seqlen, shape.nheads, shape.ngroups
    P, N, R = shape.headdim, shape.dstate, shape.rank
    half = N // 2
    gi = torch.arange(H) // (H // G)  # group of each head

    def bc(raw, w, bias):  # raw [b,H,R,N] -> BCNorm (RMS over N) * gain + bias
        inv = 1.0 / torch.sqrt((raw * raw).mean(dim=-1, keepdim=True) + shape.eps)
        out = raw * inv
        if w is not None:
            out = out * w
        return out + bias

    def rot(Hs, ang):  # rotate pairs (i, i + N/2) of Hs [b,H,N,P] by ang [b,H,N/2]
        c, s = torch.cos(ang)[..., None], torch.sin(ang)[..., None]
        lo, hi = Hs[:, :, :half], Hs[:, :, half:]
        return torch.cat([c * lo - s * hi, s * lo + c * hi], dim=2)

    Hs = t["h0"].transpose(-1, -2) if t.get("h0") is not None else torch.zeros(b, H, N, P, dtype=torch.float64)
    prev = None
    if t.get("x_prev") is not None:
        prev = (bc(t["Braw_prev"][:, gi], t.get("B_normw"), t["B_bias"]), t["x_prev"])
    ys = []
    for k in range(L):
        d, a, lm = t["dt"][:, k], t["A"][:, k], t["lam"][:, k]  # [b,H]
        Bk = bc(t["Braw"][:, k][:, gi], t.get("B_normw"), t["B_bias"])  # [b,H,R,N]
        Ck = bc(t["Craw"][:, k][:, gi], t.get("C_normw"), t["C_bias"])
        xk = t["x"][:, k]  # [b,H,R,P]
        alpha = torch.exp(d * a)
        u = alpha[..., None, None] * Hs
        if prev is not None:
            beta = (1.0 - lm) * d * alpha
            u = u + beta[..., None, None] * torch.einsum("bhrn,bhrp->bhnp", prev[0], prev[1])
        ang = d[..., None] * t["theta"][:, k][:, gi]  # [b,H,N/2]
        Hs = rot(u, ang) + (lm * d)[..., None, None] * torch.einsum("bhrn,bhrp->bhnp", Bk, xk)
        ys.append(torch.einsum("bhrn,bhnp->bhrp", Ck, Hs))
        prev = (Bk, xk)
    y = torch.stack(ys, dim=1) if L > 0 else torch.zeros(b, 0, H, R, P, dtype=torch.float64)
    return y, Hs.transpose(-1, -2)


def scan_grads(inp: dict, shape, dy, dh_final=None):
    """Gradients of <dy, y> + <dh_final, h_final> with respect to every input that is
    present (GRAD_INPUTS order; absent inputs are skipped). Returns a dict of float64
    arrays with the inputs' shapes."""
    import torch
    t, names = {}, []
    for k in GRAD_INPUTS:
        v = inp.get(k)
        if v is None:
            continue
        t[k] = torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
        names.append(k)
    y, hf = scan_torch(t, shape)
    outs, gouts = [y], [torch.tensor(np.asarray(dy, dtype=np.float64))]
    if dh_final is not None:
        outs.append(hf)
        gouts.append(torch.tensor(np.asarray(dh_final, dtype=np.float64)))
    g = torch.autograd.grad(outs, [t[k] for k in names], gouts, allow_unused=True)
    return {k: (np.zeros(inp[k].shape) if gk is None else gk.detach().numpy()) for k, gk in zip(names, g)}
