"""GPU parity of the prefill backward (m3_scan_bwd) against the oracle's
gradients (autograd of the restated recurrence, itself pinned to finite
differences of the C oracle). Every gradient the call returns is compared
element by element, err = max|g_gpu - g_ref| / max|g_ref|."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from state_space_sequence_amd.inputs import Shape, make_scan_inputs, round_bf16
from tests.gpu_helpers import gpu_scan_bwd, relerr

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-4  # fp32 arithmetic on bf16-exact or fp32 inputs


def say(*a):
    print(*a, flush=True)


def upstream(shape, seed, with_dh, io):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((shape.batch, shape.seqlen, shape.nheads, shape.rank, shape.headdim)).astype(np.float32)
    if io == "bf16":
        dy = round_bf16(dy)
    dh = rng.standard_normal((shape.batch, shape.nheads, shape.headdim, shape.dstate)).astype(np.float32) \
        if with_dh else None
    return dy, dh


CASES = [
    # (b, L, H, G, P, N, R, io, prev, h0, normw, dh_final, slow)
    (2, 70, 2, 1, 16, 16, 1, "f32", True, True, True, True, True),
    (1, 45, 4, 2, 32, 64, 2, "f32", True, False, False, True, False),
    (2, 33, 3, 1, 24, 32, 3, "f32", False, True, True, False, True),
    (1, 100, 2, 1, 64, 128, 4, "bf16", True, True, False, True, True),
    (2, 64, 2, 1, 64, 128, 1, "bf16", False, False, False, False, False),
    (1, 1, 2, 1, 16, 32, 2, "f32", True, True, True, True, False),
    # the head shape N = 128, P = 64 runs on the matrix cores (R in {1, 2, 4})
    (2, 77, 2, 1, 64, 128, 2, "f32", True, True, True, True, True),
    (1, 40, 3, 3, 64, 128, 1, "f32", False, True, False, True, False),
    (1, 5, 2, 1, 64, 128, 4, "bf16", True, False, True, False, False),
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_oracle(case):
    b, L, H, G, P, N, R, io, prev, h0, normw, dhf, slow = case
    shape = Shape(b, L, H, G, P, N, R, max(1, 64 // R), io)
    say("backward", case)
    inp = make_scan_inputs(shape, seed=51, slow_decay=slow, with_h0=h0, with_prev=prev, with_normw=normw)
    dy, dh = upstream(shape, 52, dhf, io)
    got = gpu_scan_bwd(inp, shape, dy, dh)
    ref = oracle.scan_grads(inp, shape, dy, dh)
    if "h0" not in ref:  # the gradient with respect to a zero initial state
        z = dict(inp)
        z["h0"] = np.zeros((b, H, P, N), dtype=np.float32)
        ref["h0"] = oracle.scan_grads(z, shape, dy, dh)["h0"]
    worst = 0.0
    for k in ref:
        e = relerr(got[k], ref[k])
        worst = max(worst, e)
        say("  d%-9s err %.2e" % (k, e))
    assert set(got) == set(ref)
    assert worst < TOL_BWD


@pytest.mark.parametrize("N,P", [(64, 32), (128, 64)])
def test_backward_is_deterministic(N, P):
    shape = Shape(2, 90, 3, 1, P, N, 2, 32, "f32")
    inp = make_scan_inputs(shape, seed=53, with_h0=True, with_prev=True, with_normw=True)
    dy, dh = upstream(shape, 54, True, "f32")
    g1 = gpu_scan_bwd(inp, shape, dy, dh)
    g2 = gpu_scan_bwd(inp, shape, dy, dh)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("name,b,h", [("siso_prefill_1p5b", 5, 41), ("mimo4_prefill_1p5b", 2, 17)])
def test_backward_prefill_1p5b_sampled(name, b, h):
    """The full b8 L4096 H64 workload (SISO, and MIMO rank 4) through the backward; the
    oracle recomputes the per-chain gradients (dx, dt, A, lam, h0) of one sampled
    (batch, head) chain."""
    from state_space_sequence_amd.inputs import WORKLOADS, slice_chain
    shape = WORKLOADS[name]
    say("backward workload", shape)
    inp = make_scan_inputs(shape, seed=55)
    dy, _ = upstream(shape, 56, False, "bf16")
    got = gpu_scan_bwd(inp, shape, dy, None)
    for k, v in got.items():
        assert np.isfinite(v).all(), k
    sub, s1 = slice_chain(inp, shape, b, h)
    sub["h0"] = np.zeros((1, 1, shape.headdim, shape.dstate), dtype=np.float32)
    ref = oracle.scan_grads(sub, s1, np.ascontiguousarray(dy[b:b + 1, :, h:h + 1]))
    pairs = {"x": got["x"][b:b + 1, :, h:h + 1], "dt": got["dt"][b:b + 1, :, h:h + 1],
             "A": got["A"][b:b + 1, :, h:h + 1], "lam": got["lam"][b:b + 1, :, h:h + 1],
             "h0": got["h0"][b:b + 1, h:h + 1]}
    for k, v in pairs.items():
        e = relerr(v, ref[k])
        say("  chain (%d,%d) d%-4s err %.2e" % (b, h, k, e))
        assert e < TOL_BWD, k


LOWMEM = [
    # (b, L, H, G, R, io, prev, h0, normw, dh_final, slow)
    (2, 700, 3, 1, 1, "bf16", True, True, True, True, True),    # 22 chunks: several windows, ragged tail
    (1, 301, 2, 1, 4, "f32", True, False, False, True, True),   # R = 4: 38 chunks of 8 tokens
    (2, 77, 2, 1, 2, "f32", False, True, True, False, False),
    (1, 5, 2, 1, 4, "bf16", True, True, False, True, False),     # one chunk, one window
]


@pytest.mark.parametrize("case", LOWMEM)
def test_backward_low_memory_is_bit_identical(case):
    """The windowed low-memory schedule (M3_FLAG_BWD_LOW_MEMORY) recomputes each
    window's states from a checkpoint of the exact fp32 state and keeps every sum in
    the same order: every gradient equals the one-pass result bit for bit."""
    from state_space_sequence_amd import m3
    b, L, H, G, R, io, prev, h0, normw, dhf, slow = case
    shape = Shape(b, L, H, G, 64, 128, R, max(1, 64 // R), io)
    say("low-memory backward", case)
    inp = make_scan_inputs(shape, seed=57, slow_decay=slow, with_h0=h0, with_prev=prev, with_normw=normw)
    dy, dh = upstream(shape, 58, dhf, io)
    g1 = gpu_scan_bwd(inp, shape, dy, dh)
    g2 = gpu_scan_bwd(inp, shape, dy, dh, low_memory=True)
    s0 = m3.make_shape(b, L, H, G, 64, 128, R, max(1, 64 // R), m3.M3_BF16 if io == "bf16" else m3.M3_F32)
    s1 = m3.make_shape(b, L, H, G, 64, 128, R, max(1, 64 // R), m3.M3_BF16 if io == "bf16" else m3.M3_F32,
                       flags=m3.M3_FLAG_BWD_LOW_MEMORY)
    say("  workspace %d -> %d bytes" % (m3.scan_bwd_workspace_bytes(s0), m3.scan_bwd_workspace_bytes(s1)))
    assert set(g1) == set(g2)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("windows", [1, 3, 22])
def test_backward_low_memory_window_count(windows):
    """A caller-chosen window count (shape nsegments with the flag): 22 chunks in 1,
    3 (8 + 8 + 6 chunks) or 22 windows, all bit-identical to the one-pass result."""
    shape = Shape(2, 700, 2, 1, 64, 128, 1, 64, "bf16")
    inp = make_scan_inputs(shape, seed=61, slow_decay=True, with_h0=True, with_prev=True, with_normw=True)
    dy, dh = upstream(shape, 62, True, "bf16")
    g1 = gpu_scan_bwd(inp, shape, dy, dh)
    g2 = gpu_scan_bwd(inp, shape, dy, dh, low_memory=True, windows=windows)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


def test_backward_low_memory_mimo4_1p5b_bit_identical():
    """The full MIMO rank-4 b8 L4096 H64 backward, one pass and windowed (32 windows
    of 16 chunks), compared bit for bit on the GPU; the windowed workspace is
    about 1.3 GB against 18 GB."""
    import torch
    from state_space_sequence_amd import m3
    from state_space_sequence_amd.inputs import WORKLOADS
    shape = WORKLOADS["mimo4_prefill_1p5b"]
    inp = make_scan_inputs(shape, seed=59)
    d = m3.to_device(inp, shape.io)
    del inp
    dy, _ = upstream(shape, 60, False, "bf16")
    dyt = torch.from_numpy(dy).cuda().to(torch.bfloat16)
    del dy
    args = (d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"], dyt)
    g1 = m3.scan_bwd(*args, eps=shape.eps)
    g2 = m3.scan_bwd(*args, eps=shape.eps, low_memory=True)
    torch.cuda.synchronize()
    s1 = m3.make_shape(shape.batch, shape.seqlen, shape.nheads, shape.ngroups, shape.headdim, shape.dstate,
                       shape.rank, shape.chunk, m3.M3_BF16, flags=m3.M3_FLAG_BWD_LOW_MEMORY)
    ws = m3.scan_bwd_workspace_bytes(s1)
    say("windowed workspace %.2f GB" % (ws / 1e9))
    assert ws < 1.5e9
    for k in g1:
        assert torch.isfinite(g1[k]).all(), k
        assert torch.equal(g1[k], g2[k]), k
