"""GPU parity of the bf16 matrix-core chunked prefill against the oracle.

Small shapes are compared element by element over the whole output (several
chunks plus a ragged tail). The full-size workloads run in the launch
configuration the benchmark times; the oracle then recomputes sampled
(batch, head) chains in full (chains are independent)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_amd.inputs import WORKLOADS, Shape, make_scan_inputs, slice_chain
from tests.gpu_helpers import TOL_BF16, gpu_decode, gpu_scan, relerr

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def plan_of(shape, **kw):
    from state_space_sequence_amd import m3
    s = m3.make_shape(shape.batch, shape.seqlen, shape.nheads, shape.ngroups, shape.headdim, shape.dstate,
                      shape.rank, shape.chunk, m3.M3_BF16, shape.eps, kw.get("flags", 0), kw.get("nsegments", 0))
    return m3.plan(s)


SMALL = [
    # (b, L, H, G, R, chunk, state, prev, normw, slow)
    (2, 200, 4, 1, 1, 64, False, False, False, False),
    (1, 331, 2, 2, 1, 64, True, True, True, True),
    (2, 100, 3, 1, 4, 16, False, False, False, True),
    (1, 250, 2, 1, 4, 16, True, True, False, False),
    (2, 129, 2, 1, 2, 32, True, False, True, True),
    (1, 1, 2, 1, 1, 64, True, True, False, False),
    (1, 64, 2, 1, 4, 16, False, False, False, False),
]


@pytest.mark.parametrize("case", SMALL)
def test_mfma_prefill_matches_oracle(case):
    b, L, H, G, R, C, state, prev, normw, slow = case
    shape = Shape(b, L, H, G, 64, 128, R, C, "bf16")
    assert plan_of(shape).kernel == 1
    say("mfma prefill", case)
    inp = make_scan_inputs(shape, seed=21, slow_decay=slow, with_h0=state, with_prev=prev, with_normw=normw)
    y, h = gpu_scan(inp, shape)
    yr, hr = oracle.scan(inp, shape)
    ey, eh = relerr(y, yr), relerr(h, hr)
    say("  err y %.2e  h %.2e" % (ey, eh))
    assert ey < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("R,C", [(1, 64), (4, 16)])
def test_mfma_agrees_with_fp32_kernel(R, C):
    """Same bf16 inputs through the matrix-core kernel and the fp32 kernel."""
    shape = Shape(2, 300, 2, 1, 64, 128, R, C, "bf16")
    inp = make_scan_inputs(shape, seed=22, slow_decay=True, with_h0=True, with_prev=True)
    y1, h1 = gpu_scan(inp, shape)
    y0, h0 = gpu_scan(inp, shape, force_generic=True)
    yr, hr = oracle.scan(inp, shape)
    say("R=%d mfma %.2e fp32 %.2e (y vs oracle)" % (R, relerr(y1, yr), relerr(y0, yr)))
    assert relerr(y1, y0) < TOL_BF16 and relerr(h1, h0) < TOL_BF16


@pytest.mark.parametrize("R,C,nseg,slow,state", [(1, 64, 3, True, True), (4, 16, 5, True, True),
                                                 (2, 32, 2, True, True), (1, 64, 4, False, False),
                                                 (4, 16, 6, False, True), (4, 16, 3, True, False)])
def test_segment_split_matches_single_pass(R, C, nseg, slow, state):
    """State passing between segments (local pass + combine + correction of each
    segment's outputs for its incoming state) gives the single-pass result. With
    fast decay the correction stops after the first chunk or two of a segment;
    with slow decay it runs through every segment."""
    shape = Shape(2, 700, 2, 1, 64, 128, R, C, "bf16")
    assert plan_of(shape, nsegments=nseg).nsegments == nseg
    inp = make_scan_inputs(shape, seed=23, slow_decay=slow, with_h0=state, with_prev=state)
    y1, h1 = gpu_scan(inp, shape, nsegments=1)
    ys, hs = gpu_scan(inp, shape, nsegments=nseg)
    yr, hr = oracle.scan(inp, shape)
    say("nseg=%d err y %.2e h %.2e; vs single %.2e" % (nseg, relerr(ys, yr), relerr(hs, hr), relerr(ys, y1)))
    assert relerr(ys, yr) < TOL_BF16 and relerr(hs, hr) < TOL_BF16
    assert relerr(ys, y1) < 1e-2 and relerr(hs, h1) < 1e-2


@pytest.mark.parametrize("R,C", [(1, 64), (4, 16)])
def test_mfma_large_gains_and_biases(R, C):
    """BCNorm gains and biases far from 1. The matrix-core path holds the
    normalised B and C in f16 for the rotation, scaled per head by powers of two
    (the gain exponent, raised further where a bias needs it) that the per-row
    tables undo exactly. Head 0 has B biases ~1e7 (scale beyond the gain's), head
    1 C biases ~1e5; B gains ~400, C gains ~1e-3. Each head is checked against
    the oracle on its own scale."""
    shape = Shape(2, 150, 3, 1, 64, 128, R, C, "bf16")
    inp = make_scan_inputs(shape, seed=26, with_normw=True, slow_decay=True)
    inp["B_normw"] = (inp["B_normw"] * 400.0).astype(np.float32)
    inp["C_normw"] = (inp["C_normw"] * 1e-3).astype(np.float32)
    inp["B_bias"][0] *= 1e8
    inp["C_bias"][1] *= 1e6
    y, h = gpu_scan(inp, shape)
    yr, hr = oracle.scan(inp, shape)
    assert np.isfinite(y).all() and np.isfinite(h).all()
    for hh in range(shape.nheads):
        ey = relerr(y[:, :, hh], yr[:, :, hh])
        eh = relerr(h[:, hh], hr[:, hh])
        say("R=%d head %d: |y| %.2e err y %.2e h %.2e" % (R, hh, np.abs(yr[:, :, hh]).max(), ey, eh))
        assert ey < TOL_BF16 and eh < TOL_BF16


def test_mfma_deterministic():
    shape = Shape(2, 256, 4, 1, 64, 128, 1, 64, "bf16")
    inp = make_scan_inputs(shape, seed=24)
    y1, h1 = gpu_scan(inp, shape)
    y2, h2 = gpu_scan(inp, shape)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_mfma_prefill_then_decode():
    """prefill(L-1) on the matrix-core path, one decode step == prefill(L) at L-1."""
    shape = Shape(2, 193, 2, 1, 64, 128, 4, 16, "bf16")
    inp = make_scan_inputs(shape, seed=25, slow_decay=True)
    Lm1 = shape.seqlen - 1
    keys = ("x", "Braw", "Craw", "dt", "A", "lam", "theta")
    part = {k: (np.ascontiguousarray(v[:, :Lm1]) if k in keys else v) for k, v in inp.items()}
    _, h_part = gpu_scan(part, shape.replace(seqlen=Lm1))
    dec = {k: (np.ascontiguousarray(inp[k][:, Lm1]) if k in keys else inp[k]) for k in inp}
    dec["h"] = h_part.astype(np.float32)
    dec["x_prev"] = np.ascontiguousarray(inp["x"][:, Lm1 - 1])
    dec["Braw_prev"] = np.ascontiguousarray(inp["Braw"][:, Lm1 - 1])
    yd, hd = gpu_decode(dec, shape)
    yr, hr = oracle.scan(inp, shape)
    assert relerr(yd, yr[:, Lm1]) < TOL_BF16
    assert relerr(hd, hr) < TOL_BF16


# ----------------------------------------------------- full-size workloads --
def _sampled(name, chains, seed, slow=False):
    shape = WORKLOADS[name]
    say("workload", name, shape)
    inp = make_scan_inputs(shape, seed=seed, slow_decay=slow)
    p = plan_of(shape)
    say("  plan: kernel %d, %d segments, %d workgroups" % (p.kernel, p.nsegments, p.workgroups))
    assert p.kernel == 1
    y, h = gpu_scan(inp, shape)
    assert np.isfinite(y).all() and np.isfinite(h).all()
    for (b, hh) in chains:
        sub, s1 = slice_chain(inp, shape, b, hh)
        yr, hr = oracle.scan(sub, s1)
        ey = relerr(y[b:b + 1, :, hh:hh + 1], yr)
        eh = relerr(h[b:b + 1, hh:hh + 1], hr)
        say("  chain (%d,%d): err y %.2e h %.2e" % (b, hh, ey, eh))
        assert ey < TOL_BF16 and eh < TOL_BF16
    return p


def test_siso_prefill_1p5b_sampled():
    _sampled("siso_prefill_1p5b", [(0, 0), (3, 37), (7, 63)], seed=1)


def test_mimo4_prefill_1p5b_sampled():
    _sampled("mimo4_prefill_1p5b", [(0, 5), (6, 60)], seed=2)


def test_mimo4_prefill_long_sampled():
    p = _sampled("mimo4_prefill_long", [(0, 0), (1, 23)], seed=4)
    assert p.nsegments > 1  # 48 chains: split into segments with state passing
