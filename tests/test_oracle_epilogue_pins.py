"""Pins for the oracle's skip term (D x) and grouped output RMSNorm.

The skip is checked where the state is provably zero (B = 0 after BCNorm and
bias), so y reduces to D x exactly. The norm is checked against hand-worked
rows, its grouping (one group per head and rank row), and its position relative
to the gate through a constant gate."""
from __future__ import annotations

import math

import numpy as np

import oracle
from state_space_sequence_amd.inputs import (Shape, epilogue_extras, make_decode_inputs, make_fused_scan_inputs,
                                             make_scan_inputs)


def small(R=2, L=21, N=8, P=6, H=3):
    return Shape(batch=2, seqlen=L, nheads=H, ngroups=1, headdim=P, dstate=N, rank=R, chunk=16, io="f32",
                 eps=1e-5)


def zero_state_inputs(s, seed):
    """Raw B and both biases zero: BCNorm gives 0 / sqrt(eps) = 0, so B = 0 and the state never leaves 0."""
    inp = make_scan_inputs(s, seed=seed)
    inp["Braw"] = np.zeros_like(inp["Braw"])
    inp["B_bias"] = np.zeros_like(inp["B_bias"])
    inp.update(epilogue_extras(s, seed))
    return inp


def test_skip_alone_when_the_state_is_zero():
    s = small(R=3)
    inp = zero_state_inputs(s, 1)
    y, h = oracle.scan_out(inp, s)
    assert np.all(h == 0.0)
    x = inp["x"].astype(np.float64)
    for hh in range(s.nheads):
        assert np.array_equal(y[:, :, hh], float(inp["D"][hh]) * x[:, :, hh])


def test_skip_without_D_is_the_core():
    s = small()
    inp = make_scan_inputs(s, seed=2)
    y0, _ = oracle.scan(inp, s)
    y1, _ = oracle.scan_out(inp, s)
    assert np.array_equal(y0, y1)


def test_norm_of_hand_worked_rows():
    """With y = x (zero state, D = 1): a row alternating 3, 4 has mean square 12.5, so the
    normalised row alternates 3 / sqrt(12.5 + eps) and 4 / sqrt(12.5 + eps); a constant row c
    becomes c / sqrt(c^2 + eps)."""
    s = small(R=1, P=4, L=3, H=2)
    inp = zero_state_inputs(s, 3)
    inp["D"] = np.ones_like(inp["D"])
    inp["out_normw"] = None
    x = np.zeros_like(inp["x"])
    x[:, :, 0] = np.array([3.0, 4.0, 3.0, 4.0], dtype=np.float32)
    x[:, :, 1] = -0.25
    inp["x"] = x
    y, _ = oracle.scan_out(inp, s, out_norm=True)
    r = math.sqrt(12.5 + 1e-5)
    assert np.allclose(y[:, :, 0, 0], np.array([3, 4, 3, 4]) / r, rtol=1e-14, atol=0)
    assert np.allclose(y[:, :, 1, 0], -0.25 / math.sqrt(0.0625 + 1e-5), rtol=1e-14, atol=0)


def _scaled_row_check(s, inp, hh, r):
    y1, _ = oracle.scan_out(inp, s, out_norm=True)
    inp2 = dict(inp)
    x2 = inp["x"].copy()
    x2[:, :, hh, r] *= 1000.0
    inp2["x"] = x2
    y2, _ = oracle.scan_out(inp2, s, out_norm=True)
    k = hh * s.rank + r
    rows1 = y1.reshape(-1, s.nheads * s.rank, s.headdim)
    rows2 = y2.reshape(-1, s.nheads * s.rank, s.headdim)
    assert np.array_equal(np.delete(rows1, k, axis=1), np.delete(rows2, k, axis=1))
    # the scaled row changes only through eps / mean-square (small rows early in the sequence)
    assert np.max(np.abs(rows2[:, k] - rows1[:, k])) < 1e-2


def test_norm_group_is_one_head():
    """SISO from a zero state: y of a head is linear in that head's x alone, so scaling it by
    1000 scales that head's y; the normalised output of that head is unchanged (to the eps
    effect) and every other head's is unchanged bit for bit."""
    s = small(R=1)
    inp = make_scan_inputs(s, seed=4)
    inp.update(epilogue_extras(s, 4))
    _scaled_row_check(s, inp, 1, 0)


def test_norm_group_is_one_rank_row():
    """MIMO mixes ranks through the state, so take the zero-state case (y = D x): scaling one
    rank row of x scales only that row of y, and the norm is per rank row."""
    s = small(R=2)
    inp = zero_state_inputs(s, 9)
    _scaled_row_check(s, inp, 2, 1)


def test_norm_gain_multiplies_channels():
    s = small(R=1)
    inp = make_scan_inputs(s, seed=5)
    inp.update(epilogue_extras(s, 5, with_D=False))
    y1, _ = oracle.scan_out(inp, s, out_norm=True)
    w = inp.pop("out_normw")
    y0, _ = oracle.scan_out(inp, s, out_norm=True)
    assert np.allclose(y1, y0 * w[None, None, :, None, :].astype(np.float64), rtol=1e-14, atol=0)


def test_norm_position_against_a_constant_gate():
    """R = 1, W_O = 1, W_Z Z' = ln 3 everywhere: the gate is the constant (3/4) ln 3.
    Before the gate the norm leaves the factor on the output; after it the norm removes it."""
    s = small(R=1).replace(eps=1e-12)  # so the eps term does not blur the comparison
    inp = make_fused_scan_inputs(s, seed=6)
    inp.update(epilogue_extras(s, 6))
    inp["W_O"] = np.ones_like(inp["W_O"])
    inp["W_Z"] = np.ones_like(inp["W_Z"])
    inp["z_in"] = np.full_like(inp["z_in"], math.log(3.0))
    pre, _ = oracle.scan_fused_out(inp, s, out_norm="pre")
    post, _ = oracle.scan_fused_out(inp, s, out_norm="post")
    z = float(np.float32(math.log(3.0)))  # Z' is stored in float32
    g = z / (1.0 + math.exp(-z))           # = (3/4) ln 3 up to that rounding
    assert abs(g - 0.75 * math.log(3.0)) < 1e-7
    assert np.max(np.abs(pre - g * post)) / np.max(np.abs(pre)) < 1e-9


def test_fused_skip_uses_the_expanded_x():
    """Zero state: Y = D (W_X (.) X'), so O'[p] = D sum_r W_O[p,r] W_X[p,r] X'[p] SiLU(W_Z[p,r] Z'[p]),
    written here with explicit loops."""
    s = small(R=2, L=5, P=3, H=2)
    inp = make_fused_scan_inputs(s, seed=7)
    inp["Braw"] = np.zeros_like(inp["Braw"])
    inp["B_bias"] = np.zeros_like(inp["B_bias"])
    inp.update(epilogue_extras(s, 7, with_normw=False))
    o, _ = oracle.scan_fused_out(inp, s)
    ref = np.zeros(o.shape)
    for b in range(s.batch):
        for t in range(s.seqlen):
            for h in range(s.nheads):
                for p in range(s.headdim):
                    acc = 0.0
                    for r in range(s.rank):
                        xr = float(np.float32(float(inp["W_X"][h, p, r]) * float(inp["x_in"][b, t, h, p])))
                        zz = float(inp["W_Z"][h, p, r]) * float(inp["z_in"][b, t, h, p])
                        acc += float(inp["W_O"][h, p, r]) * float(inp["D"][h]) * xr * zz / (1.0 + math.exp(-zz))
                    ref[b, t, h, p] = acc
    assert np.max(np.abs(o - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_decode_epilogue_equals_prefill_at_one_token():
    s = small(R=2, L=1)
    inp = make_scan_inputs(s, seed=8, with_h0=True, with_prev=True)
    inp.update(epilogue_extras(s, 8))
    y, h = oracle.scan_out(inp, s, out_norm=True)
    dec = dict(inp)
    for k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta"):
        dec[k] = np.ascontiguousarray(inp[k][:, 0])
    dec["h"] = dec.pop("h0")
    yd, hd = oracle.decode_out(dec, s, out_norm=True)
    assert np.array_equal(yd, y[:, 0]) and np.array_equal(hd, h)
