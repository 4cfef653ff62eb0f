"""Pins for the CPU oracle: it is checked against values and properties the pages
and the mathematics fix, never against itself or the GPU path.

Each test names what it pins. A plausible mistake in the oracle (dropped beta
term, beta without the exp(dt A) factor, (1-lam) on the wrong endpoint, wrong
rotation sign or pairing, a transposed state, a wrong rank sum) fails at least
one of them; ``test_planted_mistakes_are_caught`` checks that claim by planting
such mistakes into a copy of the oracle's C source and rebuilding it.
"""
from __future__ import annotations

import json
import math
import os
import re
import subprocess
import tempfile
import ctypes

import numpy as np
import pytest

import oracle
from state_space_sequence_amd.inputs import Shape, make_scan_inputs, slice_chain
from tests import formulations as F

HERE = os.path.dirname(os.path.abspath(__file__))


def small(R=1, L=37, N=8, P=3, H=2, G=1, io="f32", **kw):
    return Shape(batch=2, seqlen=L, nheads=H, ngroups=G, headdim=P, dstate=N, rank=R,
                 chunk=16, io=io, eps=1e-5, **kw)


def relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- golden ----
def test_golden_hand_derived():
    """Worked example derived by hand (tests/golden/trapezoid_rotation_n2.json)."""
    with open(os.path.join(HERE, "golden", "trapezoid_rotation_n2.json")) as f:
        g = json.load(f)
    s = g["shape"]
    shape = Shape(s["batch"], s["seqlen"], s["nheads"], s["ngroups"], s["headdim"], s["dstate"],
                  s["rank"], 64, "f32", s["eps"])
    I = g["inputs"]
    f32 = lambda v, sh: np.asarray(v, dtype=np.float32).reshape(sh)
    L = shape.seqlen
    inp = dict(
        x=f32(I["x"], (1, L, 1, 1, 1)),
        Braw=f32(I["Braw"], (1, L, 1, 1, 2)), Craw=f32(I["Craw"], (1, L, 1, 1, 2)),
        dt=f32(I["dt"], (1, L, 1)), A=f32(I["A"], (1, L, 1)), lam=f32(I["lam"], (1, L, 1)),
        theta=f32(I["theta"], (1, L, 1, 1)),
        B_bias=np.zeros((1, 1, 2), np.float32), C_bias=np.zeros((1, 1, 2), np.float32),
        B_normw=None, C_normw=None, h0=None, x_prev=None, Braw_prev=None)
    y, h = oracle.scan(inp, shape)
    np.testing.assert_allclose(y.reshape(-1), g["expected"]["y"], rtol=0, atol=2e-6)
    np.testing.assert_allclose(h.reshape(-1), g["expected"]["h_final"], rtol=0, atol=2e-6)


# ------------------------------------------------- special cases (I1-I3) ----
def _chain_case(shape, seed, **kw):
    inp = make_scan_inputs(shape, seed, **kw)
    return inp


def test_lambda_one_is_mamba2():
    """lam = 1 removes the beta term: exponential-Euler (Mamba-2) update (§3.1.1 Rem. 2)."""
    shape = small(R=2)
    inp = _chain_case(shape, 1)
    inp["lam"][:] = 1.0
    inp["theta"][:] = 0.0
    y, h = oracle.scan(inp, shape)
    for b in range(shape.batch):
        for hh in range(shape.nheads):
            c = F.chain_inputs(inp, shape, b, hh)
            y2, h2 = F.mamba2(c["Bn"], c["Cn"], c["x"], c["dt"], c["A"])
            assert relerr(y[b, :, hh], y2) < 1e-12
            assert relerr(h[b, hh].T, h2) < 1e-12


def test_lambda_one_matches_mamba2_ssd_mask():
    """With lam = 1 and no rotation the parallel mask is decay * Diag(gamma) (§2.3)."""
    shape = small(R=1, L=20)
    inp = _chain_case(shape, 2)
    inp["lam"][:] = 1.0
    inp["theta"][:] = 0.0
    y, _ = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 0, 0)
    L = shape.seqlen
    a = np.exp(c["dt"] * c["A"])
    Lm = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            Lm[t, s] = np.prod(a[s + 1:t + 1]) * c["dt"][s]
    Y = (Lm * (c["Cn"][:, 0] @ c["Bn"][:, 0].T)) @ c["x"][:, 0]
    assert relerr(y[0, :, 0, 0], Y) < 1e-12


def test_lambda_half_is_classic_trapezoid():
    """lam = 1/2 is the ordinary trapezoid rule (§3.1.1 Rem. 2)."""
    shape = small(R=2)
    inp = _chain_case(shape, 3)
    inp["lam"][:] = 0.5
    inp["theta"][:] = 0.0
    y, h = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 1, 1)
    y2, h2 = F.classic_trapezoid(c["Bn"], c["Cn"], c["x"], c["dt"], c["A"])
    assert relerr(y[1, :, 1], y2) < 1e-12
    assert relerr(h[1, 1].T, h2) < 1e-12


def test_no_decay_no_rotation_is_prefix_sum():
    """alpha = 1 (A = 0), no rotation: the state is a weighted prefix sum of B x^T with
    weights lam_s dt_s + (1 - lam_{s+1}) dt_{s+1} for s < t and lam_t dt_t for s = t
    (the 2-band convolution of §3.1.2 / §3.1.3 with alpha = 1); with lam = 1 it is
    exactly numpy.cumsum of dt B x^T."""
    shape = small(R=1, L=30, N=4, P=2)
    inp = _chain_case(shape, 4)
    inp["A"][:] = 0.0
    inp["theta"][:] = 0.0
    y, h = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 0, 1)
    v = np.einsum("tn,tp->tnp", c["Bn"][:, 0], c["x"][:, 0])
    lam, dt = c["lam"], c["dt"]
    w = lam * dt
    w[:-1] += (1.0 - lam[1:]) * dt[1:]
    hs = np.cumsum(w[:-1, None, None] * v[:-1], axis=0)
    h_last = hs[-1] + lam[-1] * dt[-1] * v[-1]
    assert relerr(h[0, 1].T, h_last) < 1e-12
    # lam = 1: plain cumulative sum
    inp["lam"][:] = 1.0
    y, h = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 0, 1)
    H = np.cumsum(c["dt"][:, None, None] * np.einsum("tn,tp->tnp", c["Bn"][:, 0], c["x"][:, 0]), axis=0)
    Y = np.einsum("tn,tnp->tp", c["Cn"][:, 0], H)
    assert relerr(y[0, :, 1, 0], Y) < 1e-12


# -------------------------------------------------------- rotation (I4-I5) --
def test_rotation_preserves_pair_norms():
    """R_t is orthogonal (App. B.2): with alpha = 1 and no input after t0 + 1 the norm
    of every state pair (i, i + N/2) stays constant."""
    shape = small(R=1, L=25, N=8, P=3, H=1)
    inp = _chain_case(shape, 5)
    inp["A"][:] = 0.0
    inp["x"][:, 6:] = 0.0
    ys = []
    norms = []
    for L in range(8, 25, 4):
        s = shape.replace(seqlen=L)
        sub = {k: (v[:, :L] if (v is not None and k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta")) else v)
               for k, v in inp.items()}
        _, h = oracle.scan(sub, s)
        st = h[0, 0].T  # [N, P]
        M = shape.dstate // 2
        norms.append(np.hypot(st[:M], st[M:]))
    for nrm in norms[1:]:
        np.testing.assert_allclose(nrm, norms[0], rtol=1e-12, atol=0)


def test_parity_toy_and_rotation_direction():
    """State tracking of parity with a 2-D rotation (§3.2): N = 2, A = 0, lam = 1,
    dt = 1, one impulse at t0; theta_t = pi * bit_t gives y = 2 cos(pi * #bits) with
    C = (1, 0) direction, and y = 2 sin(Psi) with C = (0, 1) pins the rotation sense
    R(theta) = [[cos, -sin], [sin, cos]] (Proposition 2)."""
    L, t0 = 24, 3
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2, size=L)
    shape = Shape(1, L, 1, 1, 1, 2, 1, 64, "f32", 0.0)
    base = dict(
        x=np.zeros((1, L, 1, 1, 1), np.float32),
        Braw=np.tile(np.array([1.0, 0.0], np.float32), (1, L, 1, 1, 1)),
        dt=np.ones((1, L, 1), np.float32), A=np.zeros((1, L, 1), np.float32),
        lam=np.ones((1, L, 1), np.float32),
        theta=(math.pi * bits).astype(np.float32).reshape(1, L, 1, 1),
        B_bias=np.zeros((1, 1, 2), np.float32), C_bias=np.zeros((1, 1, 2), np.float32),
        B_normw=None, C_normw=None, h0=None, x_prev=None, Braw_prev=None)
    base["x"][0, t0] = 1.0
    # raw B = (1, 0) normalises to (sqrt 2, 0); raw C likewise
    base["Craw"] = np.tile(np.array([1.0, 0.0], np.float32), (1, L, 1, 1, 1))
    y, _ = oracle.scan(base, shape)
    psi = np.pi * np.concatenate([[0] * (t0 + 1), np.cumsum(bits[t0 + 1:])])
    exp_y = np.where(np.arange(L) >= t0, 2.0 * np.cos(psi), 0.0)
    np.testing.assert_allclose(y.reshape(-1), exp_y, atol=1e-6)
    assert set(np.round(y.reshape(-1)[t0:]).astype(int)) <= {-2, 2}
    # direction: a pi/3 rotation per step, read out on the second coordinate
    base["theta"][:] = np.float32(math.pi / 3)
    base["Craw"] = np.tile(np.array([0.0, 1.0], np.float32), (1, L, 1, 1, 1))
    y, _ = oracle.scan(base, shape)
    ang = (np.arange(L) - t0) * np.float64(np.float32(math.pi / 3))
    exp_y = np.where(np.arange(L) >= t0, 2.0 * np.sin(ang), 0.0)
    np.testing.assert_allclose(y.reshape(-1), exp_y, atol=1e-6)


# ------------------------------------------------ other formulations (I6-I9) -
@pytest.mark.parametrize("R", [1, 2])
@pytest.mark.parametrize("state", [False, True])
def test_complex_form_twin(R, state):
    """The N/2-dim complex SSM with exp-trapezoidal discretisation (App. B.3) equals
    the real recurrence with B = [B; B_hat], C = [C; -C_hat], pairs (i, i + N/2)."""
    shape = small(R=R, N=10)
    inp = _chain_case(shape, 10 + R, with_h0=state, with_prev=state, with_normw=state)
    y, h = oracle.scan(inp, shape)
    for b in range(shape.batch):
        for hh in range(shape.nheads):
            c = F.chain_inputs(inp, shape, b, hh)
            y2, h2 = F.complex_form(**c)
            assert relerr(y[b, :, hh], y2) < 1e-11
            assert relerr(h[b, hh].T, h2) < 1e-11


@pytest.mark.parametrize("R", [1, 3])
def test_rotated_frame_twin(R):
    """RoPE trick (Proposition 4): scalar-decay recurrence on cumulatively rotated
    B and C, final state rotated back, equals the physical recurrence."""
    shape = small(R=R, N=6, L=50)
    inp = _chain_case(shape, 20 + R, with_h0=True, with_prev=True)
    y, h = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 1, 0)
    y2, h2 = F.rotated_frame(**c)
    assert relerr(y[1, :, 0], y2) < 1e-11
    assert relerr(h[1, 0].T, h2) < 1e-11


@pytest.mark.parametrize("R", [1, 2])
def test_brute_force_masked_matrix(R):
    """Parallel form Y = (L o C B^T) X with the mask of §3.1.3 built from the
    printed products, and the cumulative rotation between s and t."""
    shape = small(R=R, N=8, P=4, L=24)
    inp = _chain_case(shape, 30 + R)
    y, _ = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 0, 1)
    y2, Lm = F.brute_force(c["Bn"], c["Cn"], c["x"], c["dt"], c["A"], c["lam"], c["theta"])
    assert relerr(y[0, :, 1], y2) < 1e-11
    # the mask factors as (1-semiseparable decay) x (2-band beta/gamma), eq. 7
    a, bt, gm = np.exp(c["dt"] * c["A"]), (1 - c["lam"]) * c["dt"] * np.exp(c["dt"] * c["A"]), c["lam"] * c["dt"]
    L = shape.seqlen
    L1 = np.array([[np.prod(a[s + 1:t + 1]) if s <= t else 0.0 for s in range(L)] for t in range(L)])
    L2 = np.diag(gm) + np.diag(bt[1:], -1)
    assert relerr(L1 @ L2, Lm) < 1e-12


# ------------------------------------------------------- order of accuracy --
def _one_step_error(lam, step, a=-0.7, omega=3.0, tau0=0.4):
    """Local error of one oracle step on h' = a h + cos(omega tau) against the exact
    solution; B is the constant vector (1, 1) (raw (1, 1), eps = 0, no bias)."""
    f32 = np.float32
    a32, d32 = f32(a), f32(step)
    ad, dd = float(a32), float(d32)

    def hp(tau):
        return (-ad * math.cos(omega * tau) + omega * math.sin(omega * tau)) / (ad * ad + omega * omega)

    h_start = f32(0.3)
    tau1 = tau0 + dd
    exact = (float(h_start) - hp(tau0)) * math.exp(ad * dd) + hp(tau1)
    shape = Shape(1, 1, 1, 1, 1, 2, 1, 64, "f32", 0.0)
    inp = dict(
        x=np.array([math.cos(omega * tau1)], f32).reshape(1, 1, 1, 1, 1),
        Braw=np.ones((1, 1, 1, 1, 2), f32), Craw=np.ones((1, 1, 1, 1, 2), f32),
        dt=np.full((1, 1, 1), d32, f32), A=np.full((1, 1, 1), a32, f32),
        lam=np.full((1, 1, 1), lam, f32), theta=np.zeros((1, 1, 1, 1), f32),
        B_bias=np.zeros((1, 1, 2), f32), C_bias=np.zeros((1, 1, 2), f32),
        B_normw=None, C_normw=None,
        h0=np.full((1, 1, 1, 2), h_start, f32),
        x_prev=np.array([math.cos(omega * tau0)], f32).reshape(1, 1, 1, 1),
        Braw_prev=np.ones((1, 1, 1, 2), f32))
    _, h = oracle.scan(inp, shape)
    return abs(h[0, 0, 0, 0] - exact)


@pytest.mark.parametrize("lam,order", [(0.5, 3.0), (1.0, 2.0), (0.0, 2.0)])
def test_local_error_order(lam, order):
    """App. A.2: the local error is O(dt^3) when lam = 1/2 and O(dt^2) otherwise.
    This pins that beta carries exp(dt A) and that (1 - lam) weights the left endpoint."""
    steps = [0.08, 0.04, 0.02, 0.01]
    errs = [_one_step_error(lam, s) for s in steps]
    slopes = [math.log2(errs[i] / errs[i + 1]) for i in range(len(errs) - 1)]
    assert all(abs(sl - order) < 0.25 for sl in slopes), (errs, slopes)


# ---------------------------------------------------------- structure -------
def test_mimo_is_sum_of_siso():
    """Eqs. 12-14: y^(i) = sum_j SSM(B^(j), C^(i), x^(j)); the state is the sum."""
    R = 3
    shape = small(R=R, N=6, P=2, L=21, H=1)
    inp = _chain_case(shape, 40)
    y, h = oracle.scan(inp, shape)
    s1 = shape.replace(rank=1)
    ysum = np.zeros_like(y)
    hsum = np.zeros_like(h)
    for j in range(R):
        for i in range(R):
            sub = dict(inp)
            sub["x"] = np.ascontiguousarray(inp["x"][:, :, :, j:j + 1])
            sub["Braw"] = np.ascontiguousarray(inp["Braw"][:, :, :, j:j + 1])
            sub["Craw"] = np.ascontiguousarray(inp["Craw"][:, :, :, i:i + 1])
            sub["B_bias"] = np.ascontiguousarray(inp["B_bias"][:, j:j + 1])
            sub["C_bias"] = np.ascontiguousarray(inp["C_bias"][:, i:i + 1])
            yj, hj = oracle.scan(sub, s1)
            ysum[:, :, :, i] += yj[:, :, :, 0]
            if i == 0:
                hsum += hj
    assert relerr(y, ysum) < 1e-12
    assert relerr(h, hsum) < 1e-12


def test_rank_one_mimo_equals_siso_layout():
    shape = small(R=1)
    inp = _chain_case(shape, 41)
    y, h = oracle.scan(inp, shape)
    c = F.chain_inputs(inp, shape, 0, 0)
    y2, h2 = F.complex_form(**c)
    assert relerr(y[0, :, 0], y2) < 1e-11


def _cut(inp, a, b):
    keys = ("x", "Braw", "Craw", "dt", "A", "lam", "theta")
    return {k: (np.ascontiguousarray(v[:, a:b]) if (v is not None and k in keys) else v) for k, v in inp.items()}


@pytest.mark.parametrize("R", [1, 2])
def test_segment_state_passing(R):
    """Processing a sequence in two halves and passing (state, last x, last Braw)
    equals one pass (App. G.2 state passing); one more decode step equals the
    prefill of L+1 tokens."""
    shape = small(R=R, L=40, N=8, P=3)
    inp = _chain_case(shape, 50 + R, with_h0=True, with_prev=True)
    y, h = oracle.scan(inp, shape)
    m = 17
    y1, h1 = oracle.scan(_cut(inp, 0, m), shape.replace(seqlen=m))
    second = _cut(inp, m, shape.seqlen)
    second["h0"] = h1.astype(np.float32)
    second["x_prev"] = np.ascontiguousarray(inp["x"][:, m - 1])
    second["Braw_prev"] = np.ascontiguousarray(inp["Braw"][:, m - 1])
    y2, h2 = oracle.scan(second, shape.replace(seqlen=shape.seqlen - m))
    # h1 passes through float32: compare at float32 resolution
    assert relerr(np.concatenate([y1, y2], axis=1), y) < 1e-6
    assert relerr(h2, h) < 1e-6
    # prefill(L-1) + decode(L-1) == prefill(L)[L-1]
    Lm1 = shape.seqlen - 1
    ya, ha = oracle.scan(_cut(inp, 0, Lm1), shape.replace(seqlen=Lm1))
    dec = {k: (np.ascontiguousarray(inp[k][:, Lm1]) if k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta") else inp[k])
           for k in inp}
    dec["h"] = ha.astype(np.float32)
    dec["x_prev"] = np.ascontiguousarray(inp["x"][:, Lm1 - 1])
    dec["Braw_prev"] = np.ascontiguousarray(inp["Braw"][:, Lm1 - 1])
    yd, hd = oracle.decode(dec, shape)
    assert relerr(yd, y[:, Lm1]) < 1e-6
    assert relerr(hd, h) < 1e-6


def test_groups_equal_replicated_heads_and_linearity():
    """Heads of one group share B, C and theta (§3.3 MIMO instantiation): G = 1 equals
    G = H with those tensors replicated. y is linear in x at zero initial state."""
    shape = small(R=2, H=4, G=1)
    inp = _chain_case(shape, 60)
    y, h = oracle.scan(inp, shape)
    rep = dict(inp)
    for k in ("Braw", "Craw", "theta"):
        rep[k] = np.ascontiguousarray(np.repeat(inp[k], 4, axis=2))
    y2, h2 = oracle.scan(rep, shape.replace(ngroups=4))
    assert relerr(y2, y) < 1e-14 and relerr(h2, h) < 1e-14
    # linearity in x
    other = _chain_case(shape, 61)
    both = dict(inp)
    both["x"] = inp["x"] + other["x"]
    o2 = dict(inp)
    o2["x"] = other["x"]
    ya, _ = oracle.scan(o2, shape)
    yb, _ = oracle.scan(both, shape)
    assert relerr(yb, y + ya) < 1e-5  # x + x' is rounded to float32


def test_bcnorm_is_rms_and_scale_invariant():
    """BCNorm is an RMS norm over N (§3.4): scaling a raw row does not change y
    (eps = 0), and a gain multiplies the normalised row channel-wise."""
    shape = small(R=2).replace(eps=0.0)
    inp = _chain_case(shape, 70)
    y, h = oracle.scan(inp, shape)
    sc = dict(inp)
    sc["Braw"] = inp["Braw"] * np.float32(4.0)
    sc["Craw"] = inp["Craw"] * np.float32(0.25)
    y2, h2 = oracle.scan(sc, shape)
    assert relerr(y2, y) < 1e-12 and relerr(h2, h) < 1e-12
    # a uniform gain of 2 on B with zero bias doubles y
    z = dict(inp)
    z["B_bias"] = np.zeros_like(inp["B_bias"])
    y3, _ = oracle.scan(z, shape)
    z["B_normw"] = np.full(shape.dstate, 2.0, np.float32)
    y4, _ = oracle.scan(z, shape)
    assert relerr(y4, 2 * y3) < 1e-12


def test_chain_slicing_matches_full_run():
    """A chain cut out with slice_chain gives the same result as in the full run
    (how large workloads are checked on sampled chains)."""
    shape = small(R=2, H=4, G=2)
    inp = _chain_case(shape, 80, with_h0=True, with_prev=True)
    y, h = oracle.scan(inp, shape)
    sub, s1 = slice_chain(inp, shape, 1, 3)
    ys, hs = oracle.scan(sub, s1)
    assert relerr(ys[0, :, 0], y[1, :, 3]) == 0.0
    assert relerr(hs[0, 0], h[1, 3]) == 0.0


# ---------------------------------------------------- planted mistakes ------
MUTANTS = {
    "beta_without_decay": ("const double beta = (1.0 - l) * d * alpha;", "const double beta = (1.0 - l) * d;"),
    "lambda_on_left": ("const double beta = (1.0 - l) * d * alpha;", "const double beta = l * d * alpha;"),
    "no_beta_term": ("v += beta * s;", "v += 0.0 * s;"),
    "rotation_sign": ("Hs[i * P + p] = c * u - s * v;", "Hs[i * P + p] = c * u + s * v;"),
    "beta_not_rotated": ("U[n * P + p] = v;", "U[n * P + p] = alpha * Hs[n * P + p];"),
    "adjacent_pairs": ("""double u = U[i * P + p], v = U[(i + half) * P + p];
                    Hs[i * P + p] = c * u - s * v;
                    Hs[(i + half) * P + p] = s * u + c * v;""",
                       """double u = U[(2 * i) * P + p], v = U[(2 * i + 1) * P + p];
                    Hs[(2 * i) * P + p] = c * u - s * v;
                    Hs[(2 * i + 1) * P + p] = s * u + c * v;"""),
    "norm_without_mean": ("ms /= (double)N;", "ms /= 1.0;"),
    "current_B_in_beta": ("s += Bp[r * N + n] * xp[r * P + p];", "s += Bn[r * N + n] * xp[r * P + p];"),
}


def _build_mutant(src, name, old, new, tmpdir):
    assert src.count(old) >= 1, name
    code = src.replace(old, new, 1)
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(code)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"])
    return so


def test_planted_mistakes_are_caught(monkeypatch):
    """Each planted mistake in a copy of the oracle makes some pin above fail."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "m3_oracle.c")).read()
    checks = [test_golden_hand_derived, test_lambda_half_is_classic_trapezoid,
              lambda: test_complex_form_twin(2, True), lambda: test_brute_force_masked_matrix(2),
              lambda: test_local_error_order(0.5, 3.0), test_bcnorm_is_rms_and_scale_invariant,
              test_parity_toy_and_rotation_direction]
    with tempfile.TemporaryDirectory() as td:
        for name, (old, new) in MUTANTS.items():
            so = _build_mutant(src, name, old, new, td)
            lib = ctypes.CDLL(so)
            lib.m3o_scan.restype = ctypes.c_int
            lib.m3o_scan.argtypes = [ctypes.c_long] * 7 + [ctypes.c_double] + [ctypes.c_void_p] * 16 + [ctypes.c_int]
            lib.m3o_max_threads.restype = ctypes.c_int
            monkeypatch.setattr(oracle, "_lib", lib)
            caught = 0
            for chk in checks:
                try:
                    chk()
                except AssertionError:
                    caught += 1
            assert caught > 0, "planted mistake %s was not caught" % name
        monkeypatch.setattr(oracle, "_lib", None)
