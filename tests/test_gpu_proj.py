"""GPU parity of the stand-alone MIMO projection steps (Mamba-3 paper, App. C):
the rank expansion before the core and the gate with the rank contraction after
it, against the oracle's expand_ranks and gate_contract; and the unfused pipeline
(expand, core, gate) against the oracle's fused prefill."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_amd.inputs import Shape, make_fused_scan_inputs, round_bf16
from tests.gpu_helpers import TOL_BF16, gpu_scan_fused, relerr

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _draw(shape, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    lead = (shape[0], shape[1])
    H, P, R = shape[2], shape[3], shape[4]
    f32 = np.float32
    return (rng.standard_normal(lead + (H, P)).astype(f32), rng.standard_normal(lead + (H, R, P)).astype(f32),
            (1 + 0.5 * rng.standard_normal((H, P, R))).astype(f32), (1 + 0.5 * rng.standard_normal((H, P, R))).astype(f32),
            (rng.standard_normal((H, P, R)) / np.sqrt(R)).astype(f32))


# bf16 io: one rounding of the output (2^-9 of the largest value, with margin);
# fp32 io: fp32 arithmetic and the hardware exponential in SiLU
TOL = {"bf16": 5e-3, "f32": 1e-5}


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dims", [(2, 37, 3, 64, 4), (1, 5, 2, 128, 2), (3, 1, 4, 8, 1), (1, 9, 2, 24, 3)])
def test_expand_and_gate_match_oracle(io, dims):
    from state_space_sequence_amd import m3
    b, L, H, P, R = dims
    xin, y, WX, WZ, WO = _draw(dims, seed=61)
    z = _draw(dims, seed=62)[0]
    if io == "bf16":
        xin, y, z = round_bf16(xin), round_bf16(y), round_bf16(z)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dev = lambda a, d=dt: torch.from_numpy(a).cuda().to(d).contiguous()
    xo = m3.expand_ranks(dev(xin), dev(WX, torch.float32))
    o = m3.gate_contract(dev(y), dev(z), dev(WZ, torch.float32), dev(WO, torch.float32))
    torch.cuda.synchronize()
    ex = relerr(xo.float().cpu().numpy(), oracle.expand_ranks(xin, WX))
    eo = relerr(o.float().cpu().numpy(), oracle.gate_contract(y, z, WZ, WO))
    say("proj", io, dims, "expand %.2e gate %.2e" % (ex, eo))
    assert ex < TOL[io] and eo < TOL[io]


@pytest.mark.parametrize("R,C", [(4, 16), (2, 32)])
def test_unfused_pipeline_matches_fused_oracle(R, C):
    """expand_ranks -> scan_fwd -> gate_contract gives the fused prefill's output."""
    from state_space_sequence_amd import m3
    shape = Shape(2, 150, 3, 1, 64, 128, R, C, "bf16")
    inp = make_fused_scan_inputs(shape, seed=63, slow_decay=True, with_h0=True)
    d = m3.to_device(inp, shape.io)
    x = m3.expand_ranks(d["x_in"], d["W_X"])
    y, h = m3.scan_fwd(x, d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"],
                       chunk=C, eps=shape.eps, h0=d["h0"])
    o = m3.gate_contract(y, d["z_in"], d["W_Z"], d["W_O"])
    torch.cuda.synchronize()
    orf, hr = oracle.scan_fused(inp, shape)
    o_f, h_f = gpu_scan_fused(inp, shape)
    eo, eh = relerr(o.float().cpu().numpy(), orf), relerr(h.cpu().numpy(), hr)
    say("pipeline R=%d: o %.2e h %.2e; fused kernel o %.2e" % (R, eo, eh, relerr(o_f, orf)))
    assert eo < TOL_BF16 and eh < TOL_BF16
