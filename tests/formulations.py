"""Independent formulations of the Mamba-3 SSM core used to pin the oracle.

Each one follows a *different* statement of the method on the pages than the
oracle's physical-frame real recurrence, so agreement between them is evidence
that neither has a dropped term, wrong sign or swapped index:

* ``complex_form``   -- the complex-valued SSM discretised with the exponential-
                        trapezoidal rule (Mamba-3 paper, App. B.3, the step before
                        eq. 25): an N/2-dim complex state, transition
                        exp(dt (A + i theta)), beta term rotated by exp(i dt theta),
                        input B + i B_hat, output Re((C + i C_hat)^T h).
* ``rotated_frame``  -- the "RoPE trick" (§3.2.2, Proposition 4 / App. B.3): a plain
                        scalar-decay recurrence on B and C rotated by the cumulative
                        angle, state carried in the rotated frame.
* ``brute_force``    -- the masked parallel form Y = (L o C B^T) X of §3.1.3 with the
                        mask built entry by entry from the explicit products printed
                        there, plus the cumulative rotation between positions s and t.
* ``mamba2``         -- the exponential-Euler (Mamba-2) update of §2.2 / §3.1.1 eq. 4.
* ``classic_trapezoid`` -- the ordinary trapezoid rule (average of the endpoints).

All work on one chain: Bn, Cn [L, R, N] already normalised (+bias), x [L, R, P],
dt, A, lam [L], theta [L, N/2]. States are [N, P].
"""
from __future__ import annotations

import numpy as np


def norm_bias(raw, gain, bias, eps):
    """RMS norm over the last axis, optional gain, plus bias (float64)."""
    raw = np.asarray(raw, dtype=np.float64)
    inv = 1.0 / np.sqrt(np.mean(raw * raw, axis=-1, keepdims=True) + eps)
    g = 1.0 if gain is None else np.asarray(gain, dtype=np.float64)
    return raw * inv * g + np.asarray(bias, dtype=np.float64)


def chain_inputs(inp, shape, b=0, h=0):
    """Normalised per-chain tensors from an input dict (float64)."""
    hpg = shape.nheads // shape.ngroups
    g = h // hpg
    eps = shape.eps
    Bn = norm_bias(inp["Braw"][b, :, g], inp.get("B_normw"), inp["B_bias"][h], eps)
    Cn = norm_bias(inp["Craw"][b, :, g], inp.get("C_normw"), inp["C_bias"][h], eps)
    d = dict(
        Bn=Bn, Cn=Cn,
        x=inp["x"][b, :, h].astype(np.float64),
        dt=inp["dt"][b, :, h].astype(np.float64),
        A=inp["A"][b, :, h].astype(np.float64),
        lam=inp["lam"][b, :, h].astype(np.float64),
        theta=inp["theta"][b, :, g].astype(np.float64),
        h0=None, Bp=None, xp=None,
    )
    if inp.get("h0") is not None:
        d["h0"] = inp["h0"][b, h].astype(np.float64).T.copy()  # [N, P]
    if inp.get("x_prev") is not None and inp.get("Braw_prev") is not None:
        d["Bp"] = norm_bias(inp["Braw_prev"][b, g], inp.get("B_normw"), inp["B_bias"][h], eps)
        d["xp"] = inp["x_prev"][b, h].astype(np.float64)
    return d


def _coeffs(dt, A, lam):
    alpha = np.exp(dt * A)
    beta = (1.0 - lam) * dt * alpha
    gamma = lam * dt
    return alpha, beta, gamma


def complex_form(Bn, Cn, x, dt, A, lam, theta, h0=None, Bp=None, xp=None):
    L, R, N = Bn.shape
    P = x.shape[-1]
    M = N // 2
    alpha, beta, gamma = _coeffs(dt, A, lam)
    Bc = Bn[..., :M] + 1j * Bn[..., M:]          # B + i B_hat     (B := [B; B_hat])
    Cc = Cn[..., :M] - 1j * Cn[..., M:]          # C + i C_hat     (C := [C; -C_hat])
    hc = np.zeros((M, P), complex) if h0 is None else h0[:M] + 1j * h0[M:]
    prev = None
    if Bp is not None:
        prev = (Bp[:, :M] + 1j * Bp[:, M:], xp)
    y = np.zeros((L, R, P))
    for t in range(L):
        rot = np.exp(1j * dt[t] * theta[t])[:, None]           # e^{i dt theta}
        hc = np.exp(dt[t] * A[t]) * rot * hc
        if prev is not None:
            hc = hc + beta[t] * rot * np.einsum("rm,rp->mp", prev[0], prev[1])
        hc = hc + gamma[t] * np.einsum("rm,rp->mp", Bc[t], x[t])
        y[t] = np.real(np.einsum("rm,mp->rp", Cc[t], hc))
        prev = (Bc[t], x[t])
    h = np.concatenate([hc.real, hc.imag], axis=0)
    return y, h


def _rot(v, ang):
    """Rotate the pairs (i, i+N/2) of v[..., N] by angles ang[N/2] (counter-clockwise)."""
    M = v.shape[-1] // 2
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = v[..., :M], v[..., M:]
    return np.concatenate([c * lo - s * hi, s * lo + c * hi], axis=-1)


def rotated_frame(Bn, Cn, x, dt, A, lam, theta, h0=None, Bp=None, xp=None):
    L, R, N = Bn.shape
    P = x.shape[-1]
    alpha, beta, gamma = _coeffs(dt, A, lam)
    Phi = np.cumsum(dt[:, None] * theta, axis=0)                # Phi_t = sum_{s<=t} dt_s theta_s
    Bbar = _rot(Bn, -Phi[:, None, :])                            # prod R_s^T applied to B_t
    Cbar = _rot(Cn, -Phi[:, None, :])
    ht = np.zeros((N, P)) if h0 is None else h0.copy()
    prev = None if Bp is None else (Bp, xp)                      # frame at t=-1 is the identity
    y = np.zeros((L, R, P))
    for t in range(L):
        ht = alpha[t] * ht
        if prev is not None:
            ht = ht + beta[t] * np.einsum("rn,rp->np", prev[0], prev[1])
        ht = ht + gamma[t] * np.einsum("rn,rp->np", Bbar[t], x[t])
        y[t] = np.einsum("rn,np->rp", Cbar[t], ht)
        prev = (Bbar[t], x[t])
    h = _rot(ht.T, Phi[-1]).T if L else ht
    return y, h


def brute_force(Bn, Cn, x, dt, A, lam, theta):
    """y = M x with M[(t,r),(s,j)] = L[t,s] * C_t[r]^T R(Phi_t - Phi_s) B_s[j];
    zero initial state and no previous token."""
    L, R, N = Bn.shape
    P = x.shape[-1]
    alpha, beta, gamma = _coeffs(dt, A, lam)
    Lm = np.zeros((L, L))
    for t in range(L):
        Lm[t, t] = gamma[t]
        for s in range(t):
            prod = 1.0
            for k in range(s + 2, t + 1):       # alpha_{t...s+2}
                prod *= alpha[k]
            Lm[t, s] = prod * (gamma[s] * alpha[s + 1] + beta[s + 1])
    Phi = np.cumsum(dt[:, None] * theta, axis=0)
    Mm = np.zeros((L, R, L, R))
    for t in range(L):
        for s in range(t + 1):
            Bs = _rot(Bn[s], Phi[t] - Phi[s])   # R(Phi_t - Phi_s) B_s[j]
            Mm[t, :, s, :] = Lm[t, s] * (Cn[t] @ Bs.T)
    y = Mm.reshape(L * R, L * R) @ x.reshape(L * R, P)
    return y.reshape(L, R, P), Lm


def mamba2(Bn, Cn, x, dt, A):
    """Exponential-Euler update h = exp(dt A) h + dt B x (no rotation)."""
    L, R, N = Bn.shape
    h = np.zeros((N, x.shape[-1]))
    y = np.zeros((L, R, x.shape[-1]))
    for t in range(L):
        h = np.exp(dt[t] * A[t]) * h + dt[t] * np.einsum("rn,rp->np", Bn[t], x[t])
        y[t] = Cn[t] @ h
    return y, h


def classic_trapezoid(Bn, Cn, x, dt, A):
    """Trapezoid rule on the exponentially adjusted system: the state input is the
    average of the decayed left endpoint and the right endpoint (lambda = 1/2)."""
    L, R, N = Bn.shape
    h = np.zeros((N, x.shape[-1]))
    y = np.zeros((L, R, x.shape[-1]))
    for t in range(L):
        a = np.exp(dt[t] * A[t])
        v = np.einsum("rn,rp->np", Bn[t], x[t])
        if t == 0:
            h = a * h + 0.5 * dt[t] * v
        else:
            vp = np.einsum("rn,rp->np", Bn[t - 1], x[t - 1])
            h = a * h + 0.5 * dt[t] * (a * vp + v)
        y[t] = Cn[t] @ h
    return y, h
