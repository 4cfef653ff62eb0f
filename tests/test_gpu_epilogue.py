"""GPU parity of the output epilogue (skip term D x and grouped output RMSNorm)
against the oracle's scan_out / scan_fused_out / decode_out / decode_fused_out:
the matrix-core prefill (plain and fused, single pass and segment split), the
fp32 prefill kernel, and the decode step (plain and fused, fp32 and bf16 state)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from state_space_sequence_amd.inputs import (Shape, epilogue_extras, make_decode_inputs, make_fused_decode_inputs,
                                             make_fused_scan_inputs, make_scan_inputs, round_bf16)
from tests.gpu_helpers import (TOL_BF16, TOL_F32, gpu_decode, gpu_decode_fused, gpu_scan, gpu_scan_fused,
                               relerr)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def check(name, got, ref, tol):
    e = relerr(got, ref)
    say("  %s err %.2e" % (name, e))
    assert e < tol, name


MFMA = [
    # (b, L, H, R, chunk, D, norm, gain, prev, nseg)
    (2, 200, 3, 1, 64, True, False, False, False, 1),
    (2, 150, 2, 4, 16, True, True, True, True, 1),
    (1, 129, 2, 2, 32, False, True, False, False, 1),
    (2, 300, 2, 4, 16, True, True, True, True, 3),
    (1, 77, 2, 1, 64, True, True, True, True, 1),
]


@pytest.mark.parametrize("case", MFMA)
def test_mfma_epilogue(case):
    b, L, H, R, C, withD, norm, gain, prev, nseg = case
    shape = Shape(b, L, H, 1, 64, 128, R, C, "bf16")
    say("mfma epilogue", case)
    inp = make_scan_inputs(shape, seed=41, slow_decay=True, with_h0=True, with_prev=prev)
    inp.update(epilogue_extras(shape, 41, with_D=withD, with_normw=gain))
    y, h = gpu_scan(inp, shape, out_norm=norm, nsegments=nseg)
    yr, hr = oracle.scan_out(inp, shape, out_norm=norm)
    check("y", y, yr, TOL_BF16)
    check("h", h, hr, TOL_BF16)


GENERIC = [
    # (b, L, H, P, N, R, chunk, io, D, norm, gain)
    (2, 100, 2, 16, 16, 1, 64, "f32", True, True, True),
    (1, 70, 3, 32, 64, 2, 16, "f32", True, False, False),
    (2, 45, 2, 24, 32, 3, 8, "f32", False, True, False),
    (1, 90, 2, 64, 128, 4, 16, "bf16", True, True, True),
]


@pytest.mark.parametrize("case", GENERIC)
def test_fp32_kernel_epilogue(case):
    b, L, H, P, N, R, C, io, withD, norm, gain = case
    shape = Shape(b, L, H, 1, P, N, R, C, io)
    say("fp32 kernel epilogue", case)
    inp = make_scan_inputs(shape, seed=42, with_h0=True, with_prev=True)
    inp.update(epilogue_extras(shape, 42, with_D=withD, with_normw=gain))
    y, h = gpu_scan(inp, shape, out_norm=norm, force_generic=True)
    yr, hr = oracle.scan_out(inp, shape, out_norm=norm)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    check("y", y, yr, tol)
    check("h", h, hr, tol)


FUSED = [
    # (b, L, H, R, chunk, D, out_norm, gain, nseg)
    (2, 120, 2, 4, 16, True, None, False, 1),
    (2, 120, 2, 4, 16, True, "pre", True, 1),
    (1, 99, 3, 2, 32, True, "post", True, 1),
    (2, 400, 2, 4, 16, False, "post", False, 4),
    (1, 64, 2, 1, 64, True, "pre", True, 1),
]


@pytest.mark.parametrize("case", FUSED)
def test_fused_epilogue(case):
    b, L, H, R, C, withD, out_norm, gain, nseg = case
    shape = Shape(b, L, H, 1, 64, 128, R, C, "bf16")
    say("fused epilogue", case)
    inp = make_fused_scan_inputs(shape, seed=43, slow_decay=True, with_h0=True, with_prev=True)
    inp.update(epilogue_extras(shape, 43, with_D=withD, with_normw=gain))
    o, h = gpu_scan_fused(inp, shape, out_norm=out_norm, nsegments=nseg)
    orf, hr = oracle.scan_fused_out(inp, shape, out_norm=out_norm)
    check("o", o, orf, TOL_BF16)
    check("h", h, hr, TOL_BF16)


DECODE = [
    # (b, H, P, N, R, io, D, norm, gain, bf16_state)
    (3, 4, 64, 128, 1, "bf16", True, False, False, False),
    (3, 4, 64, 128, 4, "bf16", True, False, False, False),
    (2, 3, 64, 64, 2, "bf16", True, True, True, False),
    (2, 2, 32, 256, 3, "f32", True, True, False, False),
    (2, 2, 48, 16, 4, "f32", False, True, True, False),
    (2, 4, 64, 128, 4, "bf16", True, True, True, True),
]


@pytest.mark.parametrize("case", DECODE)
def test_decode_epilogue(case):
    b, H, P, N, R, io, withD, norm, gain, bs = case
    shape = Shape(b, 1, H, 1, P, N, R, 1, io)
    say("decode epilogue", case)
    inp = make_decode_inputs(shape, seed=44)
    inp.update(epilogue_extras(shape, 44, with_D=withD, with_normw=gain))
    if bs:
        inp["h"] = round_bf16(inp["h"])
    y, h = gpu_decode(inp, shape, bf16_state=bs, out_norm=norm)
    yr, hr = oracle.decode_out(inp, shape, out_norm=norm)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    check("y", y, yr, tol)
    check("h", h, hr, 4e-3 if bs else tol)


FUSED_DECODE = [
    # (b, H, P, N, R, io, D, out_norm, gain)
    (3, 4, 64, 128, 4, "bf16", True, None, False),
    (3, 4, 64, 128, 4, "bf16", True, "pre", True),
    (2, 2, 64, 64, 2, "bf16", True, "post", True),
    (2, 2, 32, 128, 3, "f32", True, "pre", False),
    (2, 2, 40, 32, 1, "f32", False, "post", True),
]


@pytest.mark.parametrize("case", FUSED_DECODE)
def test_fused_decode_epilogue(case):
    b, H, P, N, R, io, withD, out_norm, gain = case
    shape = Shape(b, 1, H, 1, P, N, R, 1, io)
    say("fused decode epilogue", case)
    inp = make_fused_decode_inputs(shape, seed=45)
    inp.update(epilogue_extras(shape, 45, with_D=withD, with_normw=gain))
    o, h = gpu_decode_fused(inp, shape, out_norm=out_norm)
    orf, hr = oracle.decode_fused_out(inp, shape, out_norm=out_norm)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    check("o", o, orf, tol)
    check("h", h, hr, tol)


def test_skip_only_changes_the_output():
    """The state after a prefill with D equals the one without it (the skip is output only)."""
    shape = Shape(1, 130, 2, 1, 64, 128, 4, 16, "bf16")
    inp = make_scan_inputs(shape, seed=46)
    _, h0 = gpu_scan(inp, shape)
    inp.update(epilogue_extras(shape, 46))
    _, h1 = gpu_scan(inp, shape, out_norm=True)
    assert np.array_equal(h0, h1)
