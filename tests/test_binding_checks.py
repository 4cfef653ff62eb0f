"""Host-side checks of the Python binding (no GPU needed): every tensor is checked
against the shape and dtype the call implies, and the binding raises before the
library is called. The tensors here live on the CPU; the shape and dtype checks
come before the device check, so a mistake is named even without a GPU, and a
well-formed call on CPU tensors fails only at the device check."""
from __future__ import annotations

import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "state_space_sequence_amd", "libm3.so")


@pytest.fixture(scope="module")
def m3():
    if not os.path.exists(LIB):
        from state_space_sequence_amd import build
        build.build()
    from state_space_sequence_amd import m3 as mod
    return mod


@pytest.fixture
def no_library_call(m3, monkeypatch):
    """Any call into the library's compute entry points fails the test."""
    def boom(*a, **k):
        raise AssertionError("the library was called")
    for name in ("m3_scan_fwd", "m3_decode_step", "m3_scan_bwd"):
        monkeypatch.setattr(m3.lib, name, boom)
    return m3


b, L, H, G, R, P, N = 2, 64, 4, 1, 1, 64, 128


def scan_inputs(io=torch.bfloat16):
    f32 = torch.float32
    return dict(x=torch.zeros(b, L, H, R, P, dtype=io), Braw=torch.zeros(b, L, G, R, N, dtype=io),
                Craw=torch.zeros(b, L, G, R, N, dtype=io), dt=torch.zeros(b, L, H, dtype=f32),
                A=torch.zeros(b, L, H, dtype=f32), lam=torch.zeros(b, L, H, dtype=f32),
                theta=torch.zeros(b, L, G, N // 2, dtype=f32), B_bias=torch.zeros(H, R, N, dtype=f32),
                C_bias=torch.zeros(H, R, N, dtype=f32))


def call_scan(m3, d, **kw):
    return m3.scan_fwd(d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"],
                       d["C_bias"], **kw)


def test_well_formed_cpu_call_stops_at_the_device_check(no_library_call):
    with pytest.raises(ValueError, match="GPU"):
        call_scan(no_library_call, scan_inputs())


@pytest.mark.parametrize("key,bad", [
    ("Braw", lambda d: d["Braw"].float()),                       # io dtype differs from x
    ("Craw", lambda d: d["Craw"][:, :-1].contiguous()),          # short in L
    ("dt", lambda d: d["dt"].to(torch.bfloat16)),                # scalars are fp32
    ("A", lambda d: d["A"][:, :, :2].contiguous()),
    ("lam", lambda d: d["lam"].double()),
    ("theta", lambda d: torch.zeros(b, L, G, N, dtype=torch.float32)),  # N, not N/2
    ("B_bias", lambda d: torch.zeros(H, R, N // 2, dtype=torch.float32)),
    ("C_bias", lambda d: d["C_bias"].to(torch.bfloat16)),
])
def test_scan_input_mismatch_raises(no_library_call, key, bad):
    d = scan_inputs()
    d[key] = bad(d)
    with pytest.raises((TypeError, ValueError), match=key):
        call_scan(no_library_call, d)


@pytest.mark.parametrize("kw,name", [
    (lambda: dict(h0=torch.zeros(b, H, P, N - 2)), "h0"),
    (lambda: dict(h0=torch.zeros(b, H, P, N, dtype=torch.bfloat16)), "h0"),
    (lambda: dict(x_prev=torch.zeros(b, H, R, P), Braw_prev=torch.zeros(b, G, R, N, dtype=torch.bfloat16)),
     "x_prev"),
    (lambda: dict(x_prev=torch.zeros(b, H, R, P, dtype=torch.bfloat16), Braw_prev=torch.zeros(b, G, R, N - 2,
                                                                                               dtype=torch.bfloat16)),
     "Braw_prev"),
    (lambda: dict(y=torch.zeros(b, L - 1, H, R, P, dtype=torch.bfloat16)), "y"),
    (lambda: dict(y=torch.zeros(b, L, H, R, P)), "y"),
    (lambda: dict(h_final=torch.zeros(b, H, P, N // 2)), "h_final"),
    (lambda: dict(B_normw=torch.zeros(N + 1)), "B_normw"),
    (lambda: dict(D=torch.zeros(H + 1)), "D"),
    (lambda: dict(out_norm=True, out_normw=torch.zeros(H, P, dtype=torch.float64)), "out_normw"),
    (lambda: dict(workspace=torch.zeros(64, dtype=torch.float32)), "workspace"),
])
def test_scan_optional_mismatch_raises(no_library_call, kw, name):
    with pytest.raises((TypeError, ValueError), match=name):
        call_scan(no_library_call, scan_inputs(), **kw())


def test_scan_x_rank_and_dtype(no_library_call):
    d = scan_inputs()
    d["x"] = d["x"][:, :, :, 0]
    with pytest.raises(ValueError, match="x"):
        call_scan(no_library_call, d)
    d = scan_inputs()
    d["x"] = d["x"].double()
    with pytest.raises(TypeError):
        call_scan(no_library_call, d)


def decode_inputs(io=torch.bfloat16, Rk=4):
    f32 = torch.float32
    return dict(x=torch.zeros(b, H, Rk, P, dtype=io), Braw=torch.zeros(b, G, Rk, N, dtype=io),
                Craw=torch.zeros(b, G, Rk, N, dtype=io), dt=torch.zeros(b, H, dtype=f32),
                A=torch.zeros(b, H, dtype=f32), lam=torch.zeros(b, H, dtype=f32),
                theta=torch.zeros(b, G, N // 2, dtype=f32), B_bias=torch.zeros(H, Rk, N, dtype=f32),
                C_bias=torch.zeros(H, Rk, N, dtype=f32), h=torch.zeros(b, H, P, N, dtype=f32))


def call_decode(m3, d, **kw):
    return m3.decode_step(d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"],
                          d["C_bias"], d["h"], **kw)


def test_decode_well_formed_stops_at_device(no_library_call):
    with pytest.raises(ValueError, match="GPU"):
        call_decode(no_library_call, decode_inputs())


@pytest.mark.parametrize("key,bad", [
    ("h", lambda d: torch.zeros(b, H, P, N // 2)),
    ("h", lambda d: d["h"].half()),
    ("Braw", lambda d: torch.zeros(b, G, 1, N, dtype=torch.bfloat16)),   # rank differs from x
    ("theta", lambda d: torch.zeros(b, G, N // 2 + 1)),
    ("dt", lambda d: torch.zeros(b, H + 1)),
    ("B_bias", lambda d: torch.zeros(H, 1, N)),
])
def test_decode_mismatch_raises(no_library_call, key, bad):
    d = decode_inputs()
    d[key] = bad(d)
    with pytest.raises((TypeError, ValueError), match=key):
        call_decode(no_library_call, d)


def test_decode_output_and_prev(no_library_call):
    with pytest.raises(ValueError, match="y"):
        call_decode(no_library_call, decode_inputs(), y=torch.zeros(b, H, 1, P, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="x_prev"):
        call_decode(no_library_call, decode_inputs(), x_prev=torch.zeros(b, H, 4, P - 1, dtype=torch.bfloat16),
                    Braw_prev=torch.zeros(b, G, 4, N, dtype=torch.bfloat16))


def fused_scan_inputs(Rk=4):
    d = scan_inputs()
    f32 = torch.float32
    d["x"] = torch.zeros(b, L, H, P, dtype=torch.bfloat16)
    d["z"] = torch.zeros(b, L, H, P, dtype=torch.bfloat16)
    for k in ("Braw", "Craw"):
        d[k] = torch.zeros(b, L, G, Rk, N, dtype=torch.bfloat16)
    for k in ("B_bias", "C_bias"):
        d[k] = torch.zeros(H, Rk, N, dtype=f32)
    for k in ("W_X", "W_Z", "W_O"):
        d[k] = torch.zeros(H, P, Rk, dtype=f32)
    return d


def call_fused(m3, d, **kw):
    return m3.scan_fused_fwd(d["x"], d["z"], d["W_X"], d["W_Z"], d["W_O"], d["Braw"], d["Craw"], d["dt"], d["A"],
                             d["lam"], d["theta"], d["B_bias"], d["C_bias"], chunk=16, **kw)


def test_fused_scan_checks(no_library_call):
    with pytest.raises(ValueError, match="GPU"):
        call_fused(no_library_call, fused_scan_inputs())
    for key, bad in (("z", torch.zeros(b, L, H, P)), ("W_Z", torch.zeros(H, P, 2)),
                     ("W_O", torch.zeros(H, P - 1, 4))):
        d = fused_scan_inputs()
        d[key] = bad
        with pytest.raises((TypeError, ValueError), match=key):
            call_fused(no_library_call, d)
    with pytest.raises(ValueError, match="o"):
        call_fused(no_library_call, fused_scan_inputs(), o=torch.zeros(b, L, H, 4, P, dtype=torch.bfloat16))


def test_fused_decode_checks(no_library_call):
    m3 = no_library_call
    d = decode_inputs()
    xin = torch.zeros(b, H, P, dtype=torch.bfloat16)
    W = torch.zeros(H, P, 4)
    args = lambda z: (xin, z, W, W, W, d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"],
                      d["C_bias"], d["h"])
    with pytest.raises(ValueError, match="GPU"):
        m3.decode_fused_step(*args(torch.zeros(b, H, P, dtype=torch.bfloat16)))
    with pytest.raises(TypeError, match="z_in"):
        m3.decode_fused_step(*args(torch.zeros(b, H, P)))


def test_backward_checks(no_library_call):
    m3 = no_library_call
    d = scan_inputs(torch.float32)
    args = (d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"])
    with pytest.raises(ValueError, match="GPU"):
        m3.scan_bwd(*args, torch.zeros(b, L, H, R, P))
    with pytest.raises(TypeError, match="dy"):
        m3.scan_bwd(*args, torch.zeros(b, L, H, R, P, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dh_final"):
        m3.scan_bwd(*args, torch.zeros(b, L, H, R, P), dh_final=torch.zeros(b, H, P, N + 2))
    with pytest.raises(ValueError, match="grads"):
        m3.scan_bwd(*args, torch.zeros(b, L, H, R, P), grads={"x": torch.zeros(b, L, H, R, P - 1)})
