"""Seeded synthetic inputs for the Mamba-3 SSM mixer core.

This module only draws numbers. It holds none of the mixer's arithmetic, so the
GPU path and the CPU oracle can both take their inputs from here without sharing
any part of the computation.

Value recipe (Mamba-3 paper, §3.1-§3.4 and App. A.3/F for what each tensor is;
the distributions themselves are this project's synthetic stand-in, no dataset):

  x          ~ N(0, 1)                     [b, L, H, R, P]
  Braw, Craw ~ N(0, 1)                     [b, L, G, R, N]   (BCNorm happens in the mixer)
  dt         = softplus(N(0, 1))           [b, L, H]         (step size, already positive)
  A          = -exp(U(ln 1, ln 16))        [b, L, H]         (negative decay rate)
               slow-decay variant: -exp(U(ln 1e-3, ln 1e-1))
  lam        = sigmoid(N(0, 1))            [b, L, H]         (trapezoid mix in [0, 1])
  theta      ~ U(-pi, pi)                  [b, L, G, N/2]    (rotation frequency; angle = dt*theta)
  B_bias, C_bias ~ N(0, 0.1^2)             [H, R, N]
  h0         ~ N(0, 1)                     [b, H, P, N]      (optional initial state)
  x_prev, Braw_prev ~ N(0, 1)              [b, H, R, P], [b, G, R, N] (optional previous token)
  B_normw, C_normw = 1 + 0.1 N(0, 1)       [N]               (optional BCNorm gains)

Draw order is fixed (the order above). Large normal arrays are drawn in float32
with numpy's PCG64 generator. Where the io dtype is bf16, x / Braw / Craw /
x_prev / Braw_prev are rounded to bf16 (round to nearest even) and returned as
float32 arrays holding exactly those bf16 values, so every consumer reads the
same numbers.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Shape",
    "WORKLOADS",
    "round_bf16",
    "make_scan_inputs",
    "make_decode_inputs",
    "make_fused_scan_inputs",
    "make_fused_decode_inputs",
    "epilogue_extras",
    "slice_chain",
]


@dataclasses.dataclass(frozen=True)
class Shape:
    batch: int
    seqlen: int
    nheads: int
    ngroups: int
    headdim: int  # P
    dstate: int  # N
    rank: int = 1  # R (1 = SISO)
    chunk: int = 64  # chunk length in tokens
    io: str = "bf16"  # "f32" or "bf16": dtype of x, Braw, Craw and y
    eps: float = 1e-5

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# Named workloads, each described by what it is.
WORKLOADS = {
    # tiny SISO layer, all fp32 (b1 L256 H2 P16 N16)
    "tiny_siso_f32": Shape(1, 256, 2, 1, 16, 16, 1, 64, "f32"),
    # 1.5B-scale SISO prefill (b8 L4096 H64 P64 N128, chunk 64)
    "siso_prefill_1p5b": Shape(8, 4096, 64, 1, 64, 128, 1, 64, "bf16"),
    # 1.5B-scale MIMO rank-4 prefill (chunk 16 = 64/R)
    "mimo4_prefill_1p5b": Shape(8, 4096, 64, 1, 64, 128, 4, 16, "bf16"),
    # long-context MIMO rank-4 prefill (b2 L32768, 24 heads x P64, N128)
    "mimo4_prefill_long": Shape(2, 32768, 24, 1, 64, 128, 4, 16, "bf16"),
    # decode steps: batch 128, 64 heads x P64, fp32 state
    "decode_siso_n128": Shape(128, 1, 64, 1, 64, 128, 1, 1, "bf16"),
    "decode_mimo4_n128": Shape(128, 1, 64, 1, 64, 128, 4, 1, "bf16"),
    "decode_siso_n64": Shape(128, 1, 64, 1, 64, 64, 1, 1, "bf16"),
    "decode_mimo4_n64": Shape(128, 1, 64, 1, 64, 64, 4, 1, "bf16"),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return np.where(z > 20.0, z, np.log1p(np.exp(np.minimum(z, 20.0))))


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z.astype(np.float64)))


def make_scan_inputs(
    shape: Shape,
    seed: int,
    *,
    slow_decay: bool = False,
    with_h0: bool = False,
    with_prev: bool = False,
    with_normw: bool = False,
    bias_std: float = 0.1,
) -> dict:
    """Draw one set of prefill inputs. Returns a dict of float32 numpy arrays.

    Optional tensors that are not requested are returned as None.
    """
    b, L, H, G = shape.batch, shape.seqlen, shape.nheads, shape.ngroups
    P, N, R = shape.headdim, shape.dstate, shape.rank
    if N % 2:
        raise ValueError("dstate must be even")
    if H % G:
        raise ValueError("nheads must be a multiple of ngroups")
    rng = np.random.Generator(np.random.PCG64(seed))
    bf = shape.io == "bf16"

    def io_cast(a):
        return round_bf16(a) if bf else np.ascontiguousarray(a, dtype=np.float32)

    x = io_cast(_normal(rng, (b, L, H, R, P)))
    Braw = io_cast(_normal(rng, (b, L, G, R, N)))
    Craw = io_cast(_normal(rng, (b, L, G, R, N)))
    dt = _softplus(_normal(rng, (b, L, H))).astype(np.float32)
    lo, hi = (math.log(1e-3), math.log(1e-1)) if slow_decay else (math.log(1.0), math.log(16.0))
    A = (-np.exp(rng.uniform(lo, hi, size=(b, L, H)))).astype(np.float32)
    lam = _sigmoid(_normal(rng, (b, L, H))).astype(np.float32)
    theta = rng.uniform(-math.pi, math.pi, size=(b, L, G, N // 2)).astype(np.float32)
    B_bias = (bias_std * rng.standard_normal(size=(H, R, N))).astype(np.float32)
    C_bias = (bias_std * rng.standard_normal(size=(H, R, N))).astype(np.float32)
    h0 = _normal(rng, (b, H, P, N)) if with_h0 else None
    if with_prev:
        x_prev = io_cast(_normal(rng, (b, H, R, P)))
        Braw_prev = io_cast(_normal(rng, (b, G, R, N)))
    else:
        x_prev = Braw_prev = None
    if with_normw:
        B_normw = (1.0 + 0.1 * rng.standard_normal(size=(N,))).astype(np.float32)
        C_normw = (1.0 + 0.1 * rng.standard_normal(size=(N,))).astype(np.float32)
    else:
        B_normw = C_normw = None
    return dict(
        x=x, Braw=Braw, Craw=Craw, dt=dt, A=A, lam=lam, theta=theta,
        B_bias=B_bias, C_bias=C_bias, B_normw=B_normw, C_normw=C_normw,
        h0=h0, x_prev=x_prev, Braw_prev=Braw_prev,
    )


def make_decode_inputs(shape: Shape, seed: int, *, first_token: bool = False,
                       with_normw: bool = False) -> dict:
    """Inputs for one decode step: the prefill recipe at L=1 with a state h ~ N(0,1)
    and (unless ``first_token``) the previous token's x and Braw. Per-token tensors
    lose their L axis: x [b,H,R,P], Braw/Craw [b,G,R,N], dt/A/lam [b,H], theta [b,G,N/2].
    """
    s = shape.replace(seqlen=1)
    d = make_scan_inputs(s, seed, with_h0=True, with_prev=not first_token, with_normw=with_normw)
    out = dict(d)
    for k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta"):
        out[k] = np.ascontiguousarray(d[k][:, 0])
    out["h"] = out.pop("h0")
    return out


def _fused_extras(shape: Shape, seed: int, lead: tuple, with_prev: bool) -> dict:
    """Draws for the fused MIMO projections and gate: X', Z' ~ N(0,1) of shape
    lead + (H, P) in the io dtype; per-head weights W_X, W_Z ~ 1 + 0.5 N(0,1) and
    W_O ~ N(0,1)/sqrt(R), shape [H, P, R], fp32; X' of the previous token when asked."""
    H, P, R = shape.nheads, shape.headdim, shape.rank
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    bf = shape.io == "bf16"

    def io_cast(a):
        return round_bf16(a) if bf else np.ascontiguousarray(a, dtype=np.float32)

    out = dict(
        x_in=io_cast(_normal(rng, lead + (H, P))),
        z_in=io_cast(_normal(rng, lead + (H, P))),
        W_X=(1.0 + 0.5 * rng.standard_normal(size=(H, P, R))).astype(np.float32),
        W_Z=(1.0 + 0.5 * rng.standard_normal(size=(H, P, R))).astype(np.float32),
        W_O=(rng.standard_normal(size=(H, P, R)) / math.sqrt(R)).astype(np.float32),
    )
    out["x_prev_in"] = io_cast(_normal(rng, (lead[0], H, P))) if with_prev else None
    return out


def make_fused_scan_inputs(shape: Shape, seed: int, **kw) -> dict:
    """Prefill inputs for the fused projections: the make_scan_inputs draws (B, C, dt,
    A, lambda, theta, biases, optional h0 / gains / previous raw B) with x replaced by
    X' [b,L,H,P] and the gate and weights added (x and x_prev are None)."""
    d = make_scan_inputs(shape, seed, **kw)
    d.update(_fused_extras(shape, seed, (shape.batch, shape.seqlen), d["x_prev"] is not None))
    d["x"] = None
    d["x_prev"] = None
    return d


def make_fused_decode_inputs(shape: Shape, seed: int, *, first_token: bool = False,
                             with_normw: bool = False) -> dict:
    """Decode inputs for the fused projections: make_decode_inputs with x replaced
    by X' [b,H,P], plus Z' [b,H,P], the weights and (unless first_token) X' of the
    previous token."""
    d = make_decode_inputs(shape, seed, first_token=first_token, with_normw=with_normw)
    d.update(_fused_extras(shape, seed, (shape.batch,), not first_token))
    d["x"] = None
    d["x_prev"] = None
    return d


def epilogue_extras(shape: Shape, seed: int, *, with_D: bool = True, with_normw: bool = True) -> dict:
    """Draws for the skip term and the output norm: D ~ 1 + 0.5 N(0,1) per head [H] and
    the output-norm gain out_normw ~ 1 + 0.1 N(0,1) per (head, channel) [H, P], fp32, from
    a generator of their own (seed + 104729) so every other draw is unchanged."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    H, P = shape.nheads, shape.headdim
    D = (1.0 + 0.5 * rng.standard_normal(size=(H,))).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(size=(H, P))).astype(np.float32)
    return {"D": D if with_D else None, "out_normw": w if with_normw else None}


def slice_chain(inp: dict, shape: Shape, b: int, h: int) -> tuple[dict, Shape]:
    """Cut the prefill inputs of one (batch, head) chain out of a full input set,
    as a batch-1, one-head, one-group problem. Chains are independent, so this is
    how a sampled subset of a large workload is checked."""
    hpg = shape.nheads // shape.ngroups
    g = h // hpg
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif k in ("x", "dt", "A", "lam", "x_in", "z_in"):
            out[k] = np.ascontiguousarray(v[b:b + 1, :, h:h + 1])
        elif k in ("Braw", "Craw", "theta"):
            out[k] = np.ascontiguousarray(v[b:b + 1, :, g:g + 1])
        elif k in ("B_bias", "C_bias", "W_X", "W_Z", "W_O", "D", "out_normw"):
            out[k] = np.ascontiguousarray(v[h:h + 1])
        elif k in ("h0", "x_prev", "x_prev_in"):
            out[k] = np.ascontiguousarray(v[b:b + 1, h:h + 1])
        elif k == "Braw_prev":
            out[k] = np.ascontiguousarray(v[b:b + 1, g:g + 1])
        else:  # norm gains: shared
            out[k] = v
    return out, shape.replace(batch=1, nheads=1, ngroups=1)
