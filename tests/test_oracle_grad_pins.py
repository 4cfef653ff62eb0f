"""Pins for the oracle's prefill gradients (scan_grads): its forward restatement
agrees with the C oracle, and every gradient agrees with central finite
differences of the C oracle (independent code) along random directions. Inputs
are rounded to bf16 so that the float32 perturbations the C oracle takes are
exact."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from state_space_sequence_amd.inputs import Shape, make_scan_inputs, round_bf16


def case(R, G=1, H=2, prev=True, normw=True, h0=True, L=11, N=8, P=5, seed=0):
    s = Shape(batch=2, seqlen=L, nheads=H, ngroups=G, headdim=P, dstate=N, rank=R, chunk=4, io="f32",
              eps=1e-5)
    inp = make_scan_inputs(s, seed=seed, with_h0=h0, with_prev=prev, with_normw=normw)
    inp = {k: (None if v is None else round_bf16(v)) for k, v in inp.items()}
    return s, inp


def test_torch_forward_matches_c_oracle():
    import torch
    for R, G, H in ((1, 1, 2), (3, 2, 4)):
        s, inp = case(R, G, H)
        t = {k: torch.tensor(v, dtype=torch.float64) for k, v in inp.items() if v is not None}
        y, h = oracle.scan_torch(t, s)
        yc, hc = oracle.scan(inp, s)
        assert np.max(np.abs(y.numpy() - yc)) < 1e-12 * max(1.0, np.max(np.abs(yc)))
        assert np.max(np.abs(h.numpy() - hc)) < 1e-12 * max(1.0, np.max(np.abs(hc)))


@pytest.mark.parametrize("R,G,H,prev", [(1, 1, 2, True), (2, 2, 4, True), (3, 1, 3, False)])
def test_gradients_match_finite_differences(R, G, H, prev):
    s, inp = case(R, G, H, prev=prev, seed=R)
    rng = np.random.default_rng(100 + R)
    dy = rng.standard_normal((s.batch, s.seqlen, H, R, s.headdim))
    dhf = rng.standard_normal((s.batch, H, s.headdim, s.dstate))
    g = oracle.scan_grads(inp, s, dy, dhf)

    def objective(d):
        y, h = oracle.scan(d, s)
        return float(np.sum(dy * y) + np.sum(dhf * h))

    eps = 2.0 ** -12
    for name, gk in g.items():
        v = rng.choice([-1.0, 1.0], size=inp[name].shape).astype(np.float32)
        if name == "dt":  # stay positive: step sizes are softplus outputs
            v = np.abs(v)
        dp, dm = dict(inp), dict(inp)
        dp[name] = (inp[name] + eps * v).astype(np.float32)
        dm[name] = (inp[name] - eps * v).astype(np.float32)
        assert np.array_equal(dp[name].astype(np.float64) - inp[name], eps * v)  # exact steps
        fd = (objective(dp) - objective(dm)) / (2 * eps)
        an = float(np.sum(gk * v))
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, fd, an)


def test_unused_inputs_have_zero_gradient_paths():
    """Without h0 and the previous token their gradients are simply not produced."""
    s, inp = case(1, prev=False, h0=False, normw=False)
    g = oracle.scan_grads(inp, s, np.ones((s.batch, s.seqlen, s.nheads, 1, s.headdim)))
    assert set(g) == {"x", "Braw", "Craw", "dt", "A", "lam", "theta", "B_bias", "C_bias"}
