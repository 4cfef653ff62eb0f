"""GPU parity of the fused MIMO projections and output gate (Mamba-3 paper,
App. C) against the oracle: prefill on the matrix-core kernel (single pass and
segment split), decode with fp32 and bf16 state, and prefill followed by decode.
err = max|o_gpu - o_ref| / max|o_ref| with the same bars as the unfused paths."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from state_space_sequence_amd.inputs import (WORKLOADS, Shape, make_fused_decode_inputs, make_fused_scan_inputs,
                                             round_bf16, slice_chain)
from tests.gpu_helpers import TOL_BF16, TOL_F32, gpu_decode_fused, gpu_scan_fused, relerr

pytestmark = pytest.mark.gpu

TOL_BF16_STATE = 4e-3  # bf16 state: unit roundoff 2^-8 of an 8-significant-bit format


def say(*a):
    print(*a, flush=True)


def plan_of(shape, nsegments=0):
    from state_space_sequence_amd import m3
    s = m3.make_shape(shape.batch, shape.seqlen, shape.nheads, shape.ngroups, shape.headdim, shape.dstate,
                      shape.rank, shape.chunk, m3.M3_BF16, shape.eps, 0, nsegments)
    return m3.plan(s)


PREFILL = [
    # (b, L, H, G, R, chunk, state, prev, normw, slow)
    (2, 100, 3, 1, 4, 16, False, False, False, True),
    (1, 250, 2, 1, 4, 16, True, True, True, False),
    (2, 129, 2, 1, 2, 32, True, True, False, True),
    (2, 200, 2, 2, 1, 64, True, True, True, False),
    (1, 1, 2, 1, 4, 16, True, True, False, False),
    (1, 17, 2, 1, 4, 16, False, True, False, False),
]


@pytest.mark.parametrize("case", PREFILL)
def test_fused_prefill_matches_oracle(case):
    b, L, H, G, R, C, state, prev, normw, slow = case
    shape = Shape(b, L, H, G, 64, 128, R, C, "bf16")
    assert plan_of(shape).kernel == 1
    say("fused prefill", case)
    inp = make_fused_scan_inputs(shape, seed=31, slow_decay=slow, with_h0=state, with_prev=prev,
                                 with_normw=normw)
    o, h = gpu_scan_fused(inp, shape)
    orf, hr = oracle.scan_fused(inp, shape)
    eo, eh = relerr(o, orf), relerr(h, hr)
    say("  err o %.2e  h %.2e" % (eo, eh))
    assert o.shape == (b, L, H, 64)
    assert eo < TOL_BF16 and eh < TOL_BF16


@pytest.mark.parametrize("R,C,nseg", [(4, 16, 5), (2, 32, 3)])
def test_fused_segment_split(R, C, nseg):
    """Two passes + combine (the previous token's X' folded in the combine) give the
    single-pass result and the oracle's."""
    shape = Shape(2, 700, 2, 1, 64, 128, R, C, "bf16")
    assert plan_of(shape, nseg).nsegments == nseg
    inp = make_fused_scan_inputs(shape, seed=32, slow_decay=True, with_h0=True, with_prev=True)
    o1, h1 = gpu_scan_fused(inp, shape, nsegments=1)
    os_, hs = gpu_scan_fused(inp, shape, nsegments=nseg)
    orf, hr = oracle.scan_fused(inp, shape)
    say("nseg=%d err o %.2e h %.2e; vs single %.2e" % (nseg, relerr(os_, orf), relerr(hs, hr), relerr(os_, o1)))
    assert relerr(os_, orf) < TOL_BF16 and relerr(hs, hr) < TOL_BF16
    assert relerr(os_, o1) < 1e-2 and relerr(hs, h1) < 1e-2


def test_fused_state_equals_unfused_state():
    """The fused prefill's final state is the unfused prefill's on x = W_X (.) X'
    (the gate only touches the output); both on the GPU, x rounded to bf16 as the
    kernel rounds its operand."""
    from tests.gpu_helpers import gpu_scan
    shape = Shape(1, 160, 2, 1, 64, 128, 4, 16, "bf16")
    inp = make_fused_scan_inputs(shape, seed=33, with_h0=True, with_prev=True)
    _, hf = gpu_scan_fused(inp, shape)
    un = dict(inp)
    un["x"] = round_bf16(oracle.expand_ranks(inp["x_in"], inp["W_X"]))
    un["x_prev"] = round_bf16(oracle.expand_ranks(inp["x_prev_in"], inp["W_X"]))
    _, hu = gpu_scan(un, shape)
    say("fused vs unfused state %.2e" % relerr(hf, hu))
    assert relerr(hf, hu) < 1e-3


def test_fused_prefill_then_decode():
    """fused prefill(L-1) then one fused decode step == fused prefill(L) at token L-1."""
    shape = Shape(2, 97, 2, 1, 64, 128, 4, 16, "bf16")
    inp = make_fused_scan_inputs(shape, seed=34, slow_decay=True, with_prev=True)
    Lm1 = shape.seqlen - 1
    keys = ("x_in", "z_in", "Braw", "Craw", "dt", "A", "lam", "theta")
    part = {k: (np.ascontiguousarray(v[:, :Lm1]) if k in keys else v) for k, v in inp.items()}
    _, h_part = gpu_scan_fused(part, shape.replace(seqlen=Lm1))
    dec = {k: (np.ascontiguousarray(inp[k][:, Lm1]) if k in keys else inp[k]) for k in inp}
    dec["h"] = h_part.astype(np.float32)
    dec.pop("h0", None)
    dec["x_prev_in"] = np.ascontiguousarray(inp["x_in"][:, Lm1 - 1])
    dec["Braw_prev"] = np.ascontiguousarray(inp["Braw"][:, Lm1 - 1])
    od, hd = gpu_decode_fused(dec, shape.replace(seqlen=1, chunk=1))
    orf, hr = oracle.scan_fused(inp, shape)
    say("prefill+decode: err o %.2e h %.2e" % (relerr(od, orf[:, Lm1]), relerr(hd, hr)))
    assert relerr(od, orf[:, Lm1]) < TOL_BF16
    assert relerr(hd, hr) < TOL_BF16


DECODE = [
    # (b, H, G, P, N, R, io, first_token, normw)
    (3, 4, 1, 64, 128, 4, "bf16", False, False),
    (3, 4, 2, 64, 64, 4, "bf16", True, True),
    (2, 3, 1, 64, 128, 1, "bf16", False, True),
    (2, 2, 1, 32, 256, 2, "f32", False, False),
    (2, 2, 1, 48, 16, 4, "f32", False, True),
    (1, 2, 1, 128, 128, 3, "f32", True, False),
    (1, 2, 1, 200, 64, 4, "f32", False, True),  # R P > 512
]


@pytest.mark.parametrize("case", DECODE)
def test_fused_decode_matches_oracle(case):
    b, H, G, P, N, R, io, first, normw = case
    shape = Shape(b, 1, H, G, P, N, R, 1, io)
    say("fused decode", case)
    inp = make_fused_decode_inputs(shape, seed=35, first_token=first, with_normw=normw)
    o, h = gpu_decode_fused(inp, shape)
    orf, hr = oracle.decode_fused(inp, shape)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    eo, eh = relerr(o, orf), relerr(h, hr)
    say("  err o %.2e  h %.2e" % (eo, eh))
    assert eo < tol and eh < tol


@pytest.mark.parametrize("N,R", [(128, 4), (64, 1)])
def test_fused_decode_bf16_state(N, R):
    shape = Shape(2, 1, 4, 1, 64, N, R, 1, "bf16")
    inp = make_fused_decode_inputs(shape, seed=36)
    inp["h"] = round_bf16(inp["h"])
    o, h = gpu_decode_fused(inp, shape, bf16_state=True)
    orf, hr = oracle.decode_fused(inp, shape)
    eo, eh = relerr(o, orf), relerr(h, hr)
    say("bf16 state N%d R%d: err o %.2e h %.2e" % (N, R, eo, eh))
    assert eo < TOL_BF16 and eh < TOL_BF16_STATE


# ----------------------------------------------------- full-size workloads --
def _sampled_fused(name, chains, seed):
    shape = WORKLOADS[name]
    say("fused workload", name, shape)
    inp = make_fused_scan_inputs(shape, seed=seed)
    p = plan_of(shape)
    say("  plan: kernel %d, %d segments, %d workgroups" % (p.kernel, p.nsegments, p.workgroups))
    o, h = gpu_scan_fused(inp, shape)
    assert np.isfinite(o).all() and np.isfinite(h).all()
    for (b, hh) in chains:
        sub, s1 = slice_chain(inp, shape, b, hh)
        orf, hr = oracle.scan_fused(sub, s1)
        eo = relerr(o[b:b + 1, :, hh:hh + 1], orf)
        eh = relerr(h[b:b + 1, hh:hh + 1], hr)
        say("  chain (%d,%d): err o %.2e h %.2e" % (b, hh, eo, eh))
        assert eo < TOL_BF16 and eh < TOL_BF16
    return p


def test_fused_mimo4_prefill_1p5b_sampled():
    _sampled_fused("mimo4_prefill_1p5b", [(1, 7), (7, 62)], seed=5)


def test_fused_mimo4_prefill_long_sampled():
    p = _sampled_fused("mimo4_prefill_long", [(1, 11)], seed=6)
    assert p.nsegments > 1


@pytest.mark.parametrize("bf16_state", [False, True])
def test_fused_decode_mimo4_n128_sampled(bf16_state):
    """Full decode workload, state in fp32 or bf16; the oracle recomputes a few
    (batch, head) pairs."""
    shape = WORKLOADS["decode_mimo4_n128"]
    inp = make_fused_decode_inputs(shape, seed=7)
    if bf16_state:
        inp["h"] = round_bf16(inp["h"])
    o, h = gpu_decode_fused(inp, shape, bf16_state=bf16_state)
    for (b, hh) in [(0, 0), (77, 31), (127, 63)]:
        sub = {}
        for k, v in inp.items():
            if v is None:
                sub[k] = None
            elif k in ("x_in", "z_in", "dt", "A", "lam", "x_prev_in", "h"):
                sub[k] = np.ascontiguousarray(v[b:b + 1, hh:hh + 1])
            elif k in ("Braw", "Craw", "theta", "Braw_prev"):
                sub[k] = np.ascontiguousarray(v[b:b + 1])
            elif k in ("B_bias", "C_bias", "W_X", "W_Z", "W_O"):
                sub[k] = np.ascontiguousarray(v[hh:hh + 1])
            else:
                sub[k] = v
        orf, hr = oracle.decode_fused(sub, shape.replace(batch=1, nheads=1))
        eo, eh = relerr(o[b:b + 1, hh:hh + 1], orf), relerr(h[b:b + 1, hh:hh + 1], hr)
        say("  (%d,%d): err o %.2e h %.2e" % (b, hh, eo, eh))
        assert eo < TOL_BF16 and eh < (TOL_BF16_STATE if bf16_state else TOL_BF16)
