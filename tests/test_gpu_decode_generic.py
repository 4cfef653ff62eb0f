"""GPU parity: fused decode kernel and fp32 chunked prefill kernel vs the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from state_space_sequence_amd.inputs import WORKLOADS, Shape, make_decode_inputs, make_scan_inputs, round_bf16
from tests.gpu_helpers import TOL_BF16, TOL_F32, gpu_decode, gpu_scan, relerr

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ decode --
DECODE_CASES = [
    # (b, H, G, P, N, R, io, first_token, normw)
    (3, 4, 1, 16, 16, 1, "f32", False, False),
    (2, 4, 2, 64, 64, 2, "f32", False, True),
    (2, 6, 3, 32, 128, 4, "f32", True, False),
    (2, 4, 4, 64, 256, 3, "f32", False, False),
    (4, 8, 1, 64, 128, 1, "bf16", False, False),
    (4, 8, 1, 64, 64, 4, "bf16", False, True),
    (1, 2, 1, 200, 32, 2, "bf16", True, False),
    # every lane-group width of the output reductions: 64-lane rows (both row
    # swaps), 4-lane rows with R = 4 (no tree), 32-lane SISO rows
    (1, 3, 1, 48, 256, 4, "bf16", False, False),
    (2, 2, 1, 16, 256, 2, "f32", False, True),
    (2, 3, 1, 16, 16, 4, "f32", True, False),
    (1, 2, 1, 32, 256, 1, "f32", False, False),
    # R P > 512: x elements past the first two per thread of the set-up
    (1, 2, 1, 256, 64, 4, "f32", True, True),
    (2, 2, 1, 160, 128, 4, "bf16", False, False),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_decode_matches_oracle(case):
    b, H, G, P, N, R, io, first, normw = case
    shape = Shape(b, 1, H, G, P, N, R, 1, io)
    say("decode", case)
    inp = make_decode_inputs(shape, seed=11, first_token=first, with_normw=normw)
    y, h = gpu_decode(inp, shape)
    yr, hr = oracle.decode(inp, shape)
    # the state is fp32 throughout: fp32 bar for h on both io dtypes
    assert relerr(h, hr) < TOL_F32
    assert relerr(y, yr) < (TOL_F32 if io == "f32" else TOL_BF16)


@pytest.mark.parametrize("name", ["decode_siso_n128", "decode_mimo4_n128", "decode_siso_n64", "decode_mimo4_n64"])
def test_decode_full_workloads(name):
    shape = WORKLOADS[name]
    say("decode workload", name)
    inp = make_decode_inputs(shape, seed=3)
    y, h = gpu_decode(inp, shape)
    yr, hr = oracle.decode(inp, shape)
    assert relerr(h, hr) < TOL_F32
    assert relerr(y, yr) < TOL_BF16


# ----------------------------------------------------- fp32 chunked prefill --
def test_tiny_siso_f32_workload():
    shape = WORKLOADS["tiny_siso_f32"]
    say("prefill tiny_siso_f32")
    inp = make_scan_inputs(shape, seed=0)
    y, h = gpu_scan(inp, shape)
    yr, hr = oracle.scan(inp, shape)
    assert relerr(y, yr) < TOL_F32
    assert relerr(h, hr) < TOL_F32


GENERIC_CASES = [
    # (b, L, H, G, P, N, R, chunk, io, state, prev, normw, slow)
    (2, 100, 2, 1, 16, 16, 1, 64, "f32", False, False, False, True),     # ragged tail
    (1, 256, 3, 3, 8, 32, 2, 16, "f32", True, True, True, True),         # MIMO, G = H
    (2, 77, 4, 2, 32, 64, 4, 16, "f32", True, False, False, False),      # MIMO R=4, ragged
    (1, 5, 2, 1, 16, 16, 1, 64, "f32", False, True, False, False),       # shorter than a chunk
    (1, 192, 2, 1, 64, 128, 1, 64, "f32", True, True, False, True),      # 1.5B-like head shape
    (2, 130, 2, 1, 64, 128, 1, 64, "bf16", False, False, False, True),   # bf16 io, fp32 math
    # at the fp32 kernel's limits (N, P <= 128, N P <= 8192, chunk R <= 64)
    (1, 90, 2, 1, 128, 64, 1, 64, "f32", True, True, False, True),       # P = 128
    (1, 70, 2, 1, 64, 128, 2, 32, "f32", False, True, True, False),      # N = 128, R = 2
    (1, 40, 1, 1, 128, 16, 4, 16, "bf16", True, False, False, True),     # P = 128, R = 4
]


@pytest.mark.parametrize("case", GENERIC_CASES)
def test_generic_prefill_matches_oracle(case):
    b, L, H, G, P, N, R, C, io, state, prev, normw, slow = case
    shape = Shape(b, L, H, G, P, N, R, C, io)
    say("generic prefill", case)
    inp = make_scan_inputs(shape, seed=5, slow_decay=slow, with_h0=state, with_prev=prev, with_normw=normw)
    y, h = gpu_scan(inp, shape, force_generic=True)
    yr, hr = oracle.scan(inp, shape)
    assert relerr(h, hr) < TOL_F32
    assert relerr(y, yr) < (TOL_F32 if io == "f32" else TOL_BF16)


def test_generic_chunk_size_invariance():
    """The chunked result does not depend on the chunk length (exact re-association)."""
    shape = Shape(1, 150, 2, 1, 16, 32, 1, 64, "f32")
    inp = make_scan_inputs(shape, seed=8, slow_decay=True, with_h0=True, with_prev=True)
    y64, h64 = gpu_scan(inp, shape, force_generic=True)
    for c in (1, 7, 16, 50):
        y, h = gpu_scan(inp, shape.replace(chunk=c), force_generic=True)
        assert relerr(y, y64) < 1e-5 and relerr(h, h64) < 1e-5, c


def test_prefill_then_decode_continues_the_sequence():
    """prefill(L-1) then one decode step equals prefill(L) at position L-1 (state passing)."""
    shape = Shape(2, 65, 2, 1, 16, 32, 2, 16, "f32")
    inp = make_scan_inputs(shape, seed=9, slow_decay=True)
    y_full, h_full = gpu_scan(inp, shape, force_generic=True)
    Lm1 = shape.seqlen - 1
    part = {k: (np.ascontiguousarray(v[:, :Lm1]) if k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta") else v)
            for k, v in inp.items()}
    _, h_part = gpu_scan(part, shape.replace(seqlen=Lm1), force_generic=True)
    dec = {k: (np.ascontiguousarray(inp[k][:, Lm1]) if k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta") else inp[k])
           for k in inp}
    dec["h"] = h_part.astype(np.float32)
    dec["x_prev"] = np.ascontiguousarray(inp["x"][:, Lm1 - 1])
    dec["Braw_prev"] = np.ascontiguousarray(inp["Braw"][:, Lm1 - 1])
    yd, hd = gpu_decode(dec, shape)
    assert relerr(yd, y_full[:, Lm1]) < 1e-5
    assert relerr(hd, h_full) < 1e-5


def test_empty_sequence_copies_state():
    shape = Shape(2, 0, 2, 1, 16, 16, 1, 64, "f32")
    inp = make_scan_inputs(shape.replace(seqlen=1), seed=1, with_h0=True)
    inp = {k: (np.ascontiguousarray(v[:, :0]) if k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta") else v)
           for k, v in inp.items()}
    y, h = gpu_scan(inp, shape)
    assert y.size == 0
    np.testing.assert_array_equal(h, inp["h0"])


def test_generic_is_deterministic():
    shape = Shape(2, 90, 3, 1, 16, 32, 2, 16, "f32")
    inp = make_scan_inputs(shape, seed=12)
    y1, h1 = gpu_scan(inp, shape, force_generic=True)
    y2, h2 = gpu_scan(inp, shape, force_generic=True)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


# ---- decode with the state stored in bf16 (read and written as bf16, updated in fp32)
BF16_STATE_CASES = [
    # (b, H, G, P, N, R, io, first_token)
    (3, 4, 1, 64, 128, 1, "bf16", False),
    (2, 4, 1, 64, 128, 4, "bf16", False),
    (2, 6, 2, 32, 64, 2, "f32", True),
    (1, 3, 1, 48, 256, 4, "bf16", False),
    (2, 2, 1, 16, 16, 3, "f32", False),
]
# A state rounded to nearest even in bf16 (8 significant bits) is within half an
# ulp of the fp32 result: at most 2^-8 of the largest power of two not above the
# element, so at most 2^-8 = 3.9e-3 against the largest element; the fp32
# arithmetic adds ~1e-6.
TOL_BF16_STATE = 4e-3


@pytest.mark.gpu
@pytest.mark.parametrize("case", BF16_STATE_CASES)
def test_decode_bf16_state_matches_oracle(case):
    b, H, G, P, N, R, io, first = case
    shape = Shape(b, 1, H, G, P, N, R, 1, io)
    say("decode bf16 state", case)
    inp = make_decode_inputs(shape, seed=12, first_token=first)
    inp["h"] = round_bf16(inp["h"])  # the stored state is bf16: both sides start from its values
    y, h = gpu_decode(inp, shape, bf16_state=True)
    yr, hr = oracle.decode(inp, shape)
    say("err y %.2e h %.2e" % (relerr(y, yr), relerr(h, hr)))
    assert relerr(h, hr) < TOL_BF16_STATE
    # y comes from the fp32 update before the state is rounded
    assert relerr(y, yr) < (TOL_F32 if io == "f32" else TOL_BF16)
    # the stored state is exactly representable in bf16
    assert np.array_equal(round_bf16(h.astype(np.float32)), h.astype(np.float32))


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["decode_siso_n128", "decode_mimo4_n128", "decode_siso_n64", "decode_mimo4_n64"])
def test_decode_bf16_state_full_workloads(name):
    """The four decode workloads at full size (b128 H64 P64), state stored in bf16,
    in the launch configuration the benchmark times."""
    shape = WORKLOADS[name]
    say("decode bf16 state workload", name)
    inp = make_decode_inputs(shape, seed=3)
    inp["h"] = round_bf16(inp["h"])
    y, h = gpu_decode(inp, shape, bf16_state=True)
    yr, hr = oracle.decode(inp, shape)
    say("err y %.2e h %.2e" % (relerr(y, yr), relerr(h, hr)))
    assert relerr(h, hr) < TOL_BF16_STATE
    assert relerr(y, yr) < TOL_BF16
    assert np.array_equal(round_bf16(h.astype(np.float32)), h.astype(np.float32))


@pytest.mark.gpu
def test_decode_bf16_state_several_steps():
    """Eight chained steps with a bf16 state against the oracle stepped the same
    way (its state rounded to bf16 between steps, by the test)."""
    shape = Shape(2, 1, 4, 1, 64, 128, 4, 1, "bf16")
    steps = [make_decode_inputs(shape, seed=40 + k, first_token=(k == 0)) for k in range(8)]
    h_ref = round_bf16(steps[0]["h"]).astype(np.float64)
    import torch
    from state_space_sequence_amd import m3
    h_gpu = torch.from_numpy(h_ref.astype(np.float32)).cuda().to(torch.bfloat16)
    for k, inp in enumerate(steps):
        if k > 0:  # the previous token's x and raw B carry the trapezoid's second term
            inp["x_prev"], inp["Braw_prev"] = steps[k - 1]["x"], steps[k - 1]["Braw"]
        inp["h"] = h_ref.astype(np.float32)
        yr, hr = oracle.decode(inp, shape)
        d = m3.to_device(inp, shape.io)
        y = m3.decode_step(d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"],
                           d["B_bias"], d["C_bias"], h_gpu, eps=shape.eps,
                           x_prev=d.get("x_prev"), Braw_prev=d.get("Braw_prev"))
        torch.cuda.synchronize()
        yg = y.float().cpu().numpy()
        hg = h_gpu.float().cpu().numpy()
        say("step %d err y %.2e h %.2e" % (k, relerr(yg, yr), relerr(hg, hr)))
        # one rounding per step on each side, not always to the same neighbour
        assert relerr(yg, yr) < TOL_BF16 and relerr(hg, hr) < 4 * TOL_BF16_STATE
        # the GPU keeps its own chained state; the oracle's is rounded the same way
        h_ref = round_bf16(hr.astype(np.float32)).astype(np.float64)


@pytest.mark.gpu
def test_decode_steps_replayed_from_a_graph():
    """Four decode steps captured once in a HIP graph and replayed three times,
    with eager steps on a copy of the state between the replays: every replay
    gives the eager result bit for bit (the same kernel on the same inputs)."""
    import torch
    from state_space_sequence_amd import m3
    shape = Shape(2, 1, 24, 1, 64, 128, 4, 1, "bf16")
    inp = make_decode_inputs(shape, seed=21)
    d = m3.to_device(inp, shape.io)
    base = (d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"])
    kw = dict(eps=shape.eps, x_prev=d["x_prev"], Braw_prev=d["Braw_prev"])
    h_graph, h_eager = d["h"].clone(), d["h"].clone()
    y_graph, y_eager = torch.empty_like(d["x"]), torch.empty_like(d["x"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, on a scratch state
        h_tmp = d["h"].clone()
        m3.decode_step(*base, h_tmp, y=y_graph, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(4):
            m3.decode_step(*base, h_graph, y=y_graph, **kw)
    torch.cuda.synchronize()
    h_graph.copy_(d["h"])  # capture launches nothing: start both from the same state
    for rep in range(3):
        say("graph replay", rep)
        graph.replay()
        for _ in range(4):
            m3.decode_step(*base, h_eager, y=y_eager, **kw)
        torch.cuda.synchronize()
        assert torch.equal(h_graph, h_eager)
        assert torch.equal(y_graph, y_eager)
        # eager work between replays
        h_eager.mul_(1.0)
    # the chained result also matches the oracle stepped four times per replay
    hr = inp["h"].astype(np.float64)
    for _ in range(12):
        step = dict(inp)
        step["h"] = hr.astype(np.float32)
        _, hr = oracle.decode(step, shape)
    assert relerr(h_graph.cpu().numpy(), hr) < TOL_F32
