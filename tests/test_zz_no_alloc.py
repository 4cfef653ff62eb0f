"""GPU check of the allocation-free prefill entry point (m3_scan_fwd_noalloc): it
gives exactly what m3_scan_fwd gives with a caller-allocated workspace, on two
calls in a row, the second on a smaller input, so what the first call left in
the library's scratch array cannot leak into the second."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_amd.inputs import Shape, make_scan_inputs, slice_chain
from tests.gpu_helpers import TOL_BF16, relerr

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _both(shape, seed, **kw):
    from state_space_sequence_amd import m3
    inp = make_scan_inputs(shape, seed=seed, slow_decay=True, with_h0=True, with_prev=True)
    d = m3.to_device(inp, shape.io)
    args = (d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"])
    opt = dict(chunk=shape.chunk, eps=shape.eps, h0=d["h0"], x_prev=d["x_prev"], Braw_prev=d["Braw_prev"], **kw)
    y1, h1 = m3.scan_fwd(*args, **opt)
    y2 = torch.full_like(y1, float("nan"))
    h2 = torch.full_like(h1, float("nan"))
    m3.scan_fwd_noalloc(*args, y2, h2, **opt)
    torch.cuda.synchronize()
    sh = m3.scan_shape(d["x"], d["Braw"], shape.chunk, shape.eps, nsegments=kw.get("nsegments", 0))
    return inp, m3.plan(sh), (y1, h1), (y2, h2)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_scan_fwd_on_two_calls(order):
    cases = [(Shape(2, 8192, 4, 1, 64, 128, 4, 16, "bf16"), 51), (Shape(1, 2048, 2, 1, 64, 128, 1, 64, "bf16"), 52)]
    for shape, seed in cases:
        inp, p, (y1, h1), (y2, h2) = _both(shape, seed)
        say("noalloc", shape, "plan: %d segments, workspace %d bytes" % (p.nsegments, p.workspace_bytes))
        assert p.nsegments > 1 and p.workspace_bytes > 0  # the scratch array is used
        assert torch.equal(y1, y2) and torch.equal(h1, h2)
        sub, s1 = slice_chain(inp, shape, 0, shape.nheads - 1)
        yr, hr = oracle.scan(sub, s1)
        ey = relerr(y2[:1, :, -1:].float().cpu().numpy(), yr)
        eh = relerr(h2[:1, -1:].cpu().numpy(), hr)
        say("  vs oracle: y %.2e h %.2e" % (ey, eh))
        assert ey < TOL_BF16 and eh < TOL_BF16


def test_noalloc_without_split_and_forced_split():
    # no split: the scratch array holds only the normalised B and C rows
    inp, p, (y1, h1), (y2, h2) = _both(Shape(4, 640, 64, 1, 64, 128, 1, 64, "bf16"), 53)
    assert p.nsegments == 1 and p.workspace_bytes == 2 * 4 * 640 * 64 * 4
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    # a forced split that still fits the array
    inp, p, (y1, h1), (y2, h2) = _both(Shape(2, 1024, 8, 1, 64, 128, 2, 32, "bf16"), 54, nsegments=6)
    assert p.nsegments == 6
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
