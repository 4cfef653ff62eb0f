"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/m3.h declares, validates its arguments before any HIP call and
plans the expected kernel for each workload."""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
LIB = os.path.join(ROOT, "state_space_sequence_amd", "libm3.so")


@pytest.fixture(scope="module")
def m3():
    if not os.path.exists(LIB):
        from state_space_sequence_amd import build
        build.build()
    from state_space_sequence_amd import m3 as mod
    return mod


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        names |= set(re.findall(r"\b(m3_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function(m3):
    names = declared_functions()
    assert "m3_scan_fwd" in names and "m3_decode_step" in names and "m3_probe_copy" in names
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), "libm3.so does not export %s" % n


def test_status_strings_and_version(m3):
    assert m3.lib.m3_version() >= 100
    for code in (0, -1, -2, -3, -4, -5):
        assert m3.lib.m3_status_str(code)
    assert m3.lib.m3_status_str(0) == b"ok"


def _shape(m3, **kw):
    d = dict(batch=2, seqlen=100, nheads=4, ngroups=1, headdim=64, dstate=128, rank=1, chunk=64,
             io_dtype=m3.M3_BF16, eps=1e-5)
    d.update(kw)
    return m3.make_shape(d["batch"], d["seqlen"], d["nheads"], d["ngroups"], d["headdim"], d["dstate"],
                         d["rank"], d["chunk"], d["io_dtype"], d["eps"], d.get("flags", 0), d.get("nsegments", 0))


def _scan(m3, shape, io=None, ws=None, wsb=0):
    if io is None:
        io = m3.ScanIO()
    return m3.lib.m3_scan_fwd(ctypes.byref(shape), ctypes.byref(io), ws, wsb, None)


FUSED_FIELDS = ("z", "W_X", "W_Z", "W_O", "o")


def _fake_io(m3, base=0x100000, misalign=None, drop=None, fused=False):
    io = m3.ScanIO()
    for i, (name, _) in enumerate(m3.ScanIO._fields_):
        if name in ("B_normw", "C_normw", "h0", "x_prev", "Braw_prev", "h_final", "D", "out_normw"):
            continue
        if (name in FUSED_FIELDS) != fused and name in FUSED_FIELDS + ("y",):
            continue
        setattr(io, name, base + 0x1000 * (i + 1))
    if misalign:
        setattr(io, misalign, getattr(io, misalign) + 4)
    if drop:
        setattr(io, drop, None)
    return io


@pytest.mark.parametrize("field,value", [
    ("batch", -1), ("seqlen", -3), ("nheads", 0), ("ngroups", 3), ("dstate", 7), ("rank", 0),
    ("chunk", 0), ("io_dtype", 5), ("eps", float("nan")), ("headdim", 0)])
def test_invalid_shapes_rejected_on_host(m3, field, value):
    s = _shape(m3, **{field: value})
    assert _scan(m3, s, _fake_io(m3)) == -1


def test_null_io_and_missing_tensor(m3):
    s = _shape(m3)
    assert m3.lib.m3_scan_fwd(ctypes.byref(s), None, None, 0, None) == -1
    assert m3.lib.m3_scan_fwd(None, None, None, 0, None) == -1
    for name in ("x", "Braw", "Craw", "dt", "A", "lam", "theta", "B_bias", "C_bias", "y"):
        assert _scan(m3, s, _fake_io(m3, drop=name)) == -1, name


def test_fused_fields_validated(m3):
    s = _shape(m3, rank=4)
    # each fused pointer but y is required once W_X is set
    for name in FUSED_FIELDS:
        assert _scan(m3, s, _fake_io(m3, fused=True, drop=name)) == -1, name
    # a fused pointer without W_X is an error, not silently ignored
    for name in ("z", "W_Z", "W_O", "o"):
        io = _fake_io(m3)
        setattr(io, name, 0x900000)
        assert _scan(m3, s, io) == -1, name
    for name in ("z", "W_X", "o"):
        assert _scan(m3, s, _fake_io(m3, fused=True, misalign=name)) == -3, name
    # the fp32 kernel does not take the fused form
    assert _scan(m3, _shape(m3, rank=4, io_dtype=m3.M3_F32, dstate=64, headdim=32),
                 _fake_io(m3, fused=True)) == -2


def test_decode_fused_fields_validated(m3):
    s = _shape(m3, rank=4, seqlen=1, chunk=1)
    def dio(fused, drop=None):
        io = m3.DecodeIO()
        for i, (name, _) in enumerate(m3.DecodeIO._fields_):
            if name in ("B_normw", "C_normw", "x_prev", "Braw_prev", "D", "out_normw"):
                continue
            if (name in FUSED_FIELDS) != fused and name in FUSED_FIELDS + ("y",):
                continue
            setattr(io, name, 0x100000 + 0x1000 * (i + 1))
        if drop:
            setattr(io, drop, None)
        return io
    for name in FUSED_FIELDS + ("h",):
        assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(dio(True, name)), None) == -1, name
    io = dio(False)
    io.z = 0x900000
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == -1


def test_prev_token_both_or_neither(m3):
    s = _shape(m3)
    io = _fake_io(m3)
    io.x_prev = 0x900000
    assert _scan(m3, s, io) == -1


@pytest.mark.parametrize("name", ["x", "theta", "y", "dt"])
def test_misaligned_pointer(m3, name):
    assert _scan(m3, _shape(m3), _fake_io(m3, misalign=name)) == -3


def test_unsupported_shapes(m3):
    # too large for the fp32 kernel and not a matrix-core shape
    assert _scan(m3, _shape(m3, io_dtype=m3.M3_F32, dstate=256, headdim=64), _fake_io(m3)) == -2
    assert _scan(m3, _shape(m3, io_dtype=m3.M3_F32, chunk=128), _fake_io(m3)) == -2


def test_decode_validation(m3):
    s = _shape(m3, dstate=48)
    io = m3.DecodeIO()
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == -2
    s = _shape(m3, rank=5)
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == -2
    s = _shape(m3)
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == -1
    assert m3.lib.m3_decode_step(None, ctypes.byref(io), None) == -1


def test_flags_validated(m3):
    """The bf16-state flag is decode only; unknown flag bits are rejected by both calls."""
    assert m3.M3_FLAG_BF16_STATE == 2
    assert _scan(m3, _shape(m3, flags=m3.M3_FLAG_BF16_STATE), _fake_io(m3)) == -1
    assert _scan(m3, _shape(m3, flags=16), _fake_io(m3)) == -1
    io = m3.DecodeIO()
    s = _shape(m3, flags=m3.M3_FLAG_FORCE_GENERIC)
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == -1
    # with the bf16-state flag the decode call gets past the flag check (and stops at the NULL tensors)
    s = _shape(m3, flags=m3.M3_FLAG_BF16_STATE)
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == -1
    s = _shape(m3, batch=0, flags=m3.M3_FLAG_BF16_STATE)
    assert m3.lib.m3_decode_step(ctypes.byref(s), ctypes.byref(io), None) == 0


def test_epilogue_validated(m3):
    """The output-norm gain needs M3_FLAG_OUT_NORM; the after-gate position needs the norm
    and the fused gate; D and the gain are alignment-checked like every other pointer."""
    NORM, AFTER = m3.M3_FLAG_OUT_NORM, m3.M3_FLAG_NORM_AFTER_GATE
    s = _shape(m3, rank=4)
    io = _fake_io(m3)
    io.out_normw = 0x900000
    assert _scan(m3, s, io) == -1
    assert _scan(m3, _shape(m3, rank=4, flags=NORM | AFTER), _fake_io(m3)) == -1
    assert _scan(m3, _shape(m3, rank=4, flags=AFTER), _fake_io(m3, fused=True)) == -1
    io = _fake_io(m3)
    io.D = 0x900004
    assert _scan(m3, s, io) == -3
    io = _fake_io(m3, fused=True)
    io.out_normw = 0x900008
    assert _scan(m3, _shape(m3, rank=4, flags=NORM | AFTER), io) == -3
    d = m3.DecodeIO()
    d.out_normw = 0x900000
    assert m3.lib.m3_decode_step(ctypes.byref(_shape(m3, rank=4, seqlen=1, chunk=1)), ctypes.byref(d), None) == -1
    d = m3.DecodeIO()
    sd = _shape(m3, rank=4, seqlen=1, chunk=1, batch=0, flags=NORM | AFTER)
    assert m3.lib.m3_decode_step(ctypes.byref(sd), ctypes.byref(d), None) == -1
    sd = _shape(m3, rank=4, seqlen=1, chunk=1, batch=0, flags=NORM)
    assert m3.lib.m3_decode_step(ctypes.byref(sd), ctypes.byref(d), None) == 0


def test_plans_for_workloads(m3):
    from state_space_sequence_amd.inputs import WORKLOADS
    for name, w in WORKLOADS.items():
        if w.seqlen == 1:
            continue
        s = m3.make_shape(w.batch, w.seqlen, w.nheads, w.ngroups, w.headdim, w.dstate, w.rank, w.chunk,
                          m3.M3_BF16 if w.io == "bf16" else m3.M3_F32, w.eps)
        p = m3.plan(s)
        assert p.nsegments >= 1
        assert p.workgroups >= w.batch * w.nheads
        assert m3.workspace_bytes(s) == p.workspace_bytes
    tiny = WORKLOADS["tiny_siso_f32"]
    s = m3.make_shape(tiny.batch, tiny.seqlen, tiny.nheads, tiny.ngroups, tiny.headdim, tiny.dstate,
                      tiny.rank, tiny.chunk, m3.M3_F32, tiny.eps)
    assert m3.plan(s).kernel == 0


def _fake_grads(m3, io, base=0x400000, drop=None):
    g = m3.ScanGrads()
    for i, (name, _) in enumerate(m3.ScanGrads._fields_):
        if name in ("dh_final", "dh0"):
            continue
        if name == "dB_normw" and not io.B_normw or name == "dC_normw" and not io.C_normw:
            continue
        if name in ("dx_prev", "dBraw_prev") and not io.x_prev:
            continue
        setattr(g, name, base + 0x1000 * (i + 1))
    if drop:
        setattr(g, drop, None)
    return g


def _bwd(m3, s, io, g, ws=None, wsb=0):
    return m3.lib.m3_scan_bwd(ctypes.byref(s), ctypes.byref(io), ctypes.byref(g), ws, wsb, None)


def test_backward_validated_on_host(m3):
    s = _shape(m3, rank=2, chunk=32)
    io = _fake_io(m3)
    assert m3.lib.m3_scan_bwd_workspace_bytes(ctypes.byref(s)) > 0
    # every required gradient
    for name in ("dy", "dx", "dBraw", "dCraw", "ddt", "dA", "dlam", "dtheta", "dB_bias", "dC_bias"):
        assert _bwd(m3, s, io, _fake_grads(m3, io, drop=name)) == -1, name
    # gain gradients exactly when the gains exist; previous-token gradients likewise
    g = _fake_grads(m3, io)
    g.dB_normw = 0x900000
    assert _bwd(m3, s, io, g) == -1
    io2 = _fake_io(m3)
    io2.x_prev, io2.Braw_prev = 0x910000, 0x920000
    assert _bwd(m3, s, io2, _fake_grads(m3, io)) == -1
    # workspace
    assert _bwd(m3, s, io, _fake_grads(m3, io)) == -4
    # alignment
    g = _fake_grads(m3, io)
    g.dx = g.dx + 4
    assert _bwd(m3, s, io, g) == -3
    # the fused form and the epilogue are not differentiated
    io3 = _fake_io(m3, fused=True)
    assert _bwd(m3, s, io3, _fake_grads(m3, io)) == -2
    io4 = _fake_io(m3)
    io4.D = 0x930000
    assert _bwd(m3, s, io4, _fake_grads(m3, io)) == -2
    assert _bwd(m3, _shape(m3, flags=m3.M3_FLAG_OUT_NORM), io, _fake_grads(m3, io)) == -2
    # shapes beyond the LDS tiles
    assert _bwd(m3, _shape(m3, dstate=256, headdim=16), io, _fake_grads(m3, io)) == -2


# ------------------------------------------------- calibration probes (host) --
def test_probe_copy_validates_before_any_hip_call(m3):
    f = m3.lib.m3_probe_copy
    assert f(0x100000, 0x200000, 17, 0, None) == m3_status(m3, "INVALID_ARG")      # not a multiple of 16
    assert f(None, 0x200000, 64, 0, None) == m3_status(m3, "INVALID_ARG")          # null source
    assert f(0x100000, None, 64, 0, None) == m3_status(m3, "INVALID_ARG")
    assert f(0x100004, 0x200000, 64, 0, None) == m3_status(m3, "MISALIGNED")
    assert f(0x100000, 0x100010, 64, 0, None) == m3_status(m3, "INVALID_ARG")      # overlapping
    assert f(0x100000, 0x200000, 64, -1, None) == m3_status(m3, "INVALID_ARG")
    assert f(None, None, 0, 0, None) == 0                                           # nothing to copy


def test_probe_mfma_and_facts_validate(m3):
    g = m3.lib.m3_probe_mfma_bf16
    assert g(None, None, 4, 4, 1.0, None) == m3_status(m3, "INVALID_ARG")
    assert g(0x100000, None, 0, 4, 1.0, None) == m3_status(m3, "INVALID_ARG")
    assert g(0x100000, None, 4, 0, 1.0, None) == m3_status(m3, "INVALID_ARG")
    assert m3.lib.m3_probe_device_facts(0, None) == m3_status(m3, "INVALID_ARG")


def m3_status(m3, name):
    return {"INVALID_ARG": -1, "UNSUPPORTED": -2, "MISALIGNED": -3, "WORKSPACE_TOO_SMALL": -4, "HIP": -5}[name]


def test_noalloc_rejects_workspace_beyond_its_array(m3):
    # 4 x 262144 tokens need 512 MiB of normalised B and C rows alone, beyond the
    # allocation-free entry point's fixed 256 MiB: refused before any HIP call
    shape = _shape(m3, batch=4, nheads=64, seqlen=1 << 18)
    p = m3.plan(shape)
    assert p.workspace_bytes > m3.noalloc_max_workspace_bytes() == 256 << 20
    io = _fake_io(m3)
    rc = m3.lib.m3_scan_fwd_noalloc(ctypes.byref(shape), ctypes.byref(io), None)
    assert rc == -4  # M3_ERR_WORKSPACE_TOO_SMALL
    # argument errors come first, as in m3_scan_fwd
    assert m3.lib.m3_scan_fwd_noalloc(ctypes.byref(shape), None, None) == -1
    bad = _fake_io(m3, misalign="x")
    assert m3.lib.m3_scan_fwd_noalloc(ctypes.byref(shape), ctypes.byref(bad), None) == -3


def test_matrix_core_workspace_layout(m3):
    # the normalised B and C rows (N/2 f16 pairs each) come first, then the segment records
    for b, L, H, R, C in ((8, 4096, 64, 1, 64), (8, 4096, 64, 4, 16), (2, 32768, 24, 4, 16), (1, 5, 2, 2, 32)):
        p = m3.plan(_shape(m3, batch=b, nheads=H, seqlen=L, rank=R, chunk=C))
        rows = b * L * R
        q = 2 * ((rows * 64 * 4 + 255) // 256 * 256)
        seg = 0
        if p.nsegments > 1:
            ch = b * H * p.nsegments
            seg = sum((n * 4 + 255) // 256 * 256 for n in (ch * 64 * 128, ch, ch * 64))
        assert p.workspace_bytes == q + seg, (b, L, H, R, p.nsegments)


def test_every_automatic_plan_up_to_2pow18_rows_fits_the_noalloc_array(m3):
    cap = m3.noalloc_max_workspace_bytes()
    for b in (1, 2, 3, 4, 8):
        for H in (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 191, 255, 383):
            for L in (1024, 4096, 32768, 1 << 17):
                for R, C in ((1, 64), (2, 32), (4, 16)):
                    if b * L * R > 1 << 18:
                        continue
                    p = m3.plan(_shape(m3, batch=b, nheads=H, seqlen=L, rank=R, chunk=C))
                    assert p.workspace_bytes <= cap, (b, H, L, R, p.workspace_bytes)


def test_projection_steps_validate_before_any_hip_call(m3):
    ok = _shape(m3, batch=2, seqlen=3, nheads=4, headdim=64, rank=4)
    f = m3.lib.m3_expand_ranks
    g = m3.lib.m3_gate_contract
    assert f(ctypes.byref(ok), None, 0x1000, 0x2000, None) == -1                   # missing input
    assert f(ctypes.byref(ok), 0x1004, 0x1000, 0x2000, None) == -3                 # misaligned
    assert f(ctypes.byref(_shape(m3, headdim=60)), 0x1000, 0x2000, 0x3000, None) == -2  # P % 8
    assert f(ctypes.byref(_shape(m3, rank=5)), 0x1000, 0x2000, 0x3000, None) == -2
    assert g(ctypes.byref(ok), 0x1000, None, 0x2000, 0x3000, 0x4000, None) == -1
    assert g(ctypes.byref(ok), 0x1000, 0x2000, 0x3000, 0x4008, 0x5000, None) == -3
    assert g(None, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None) == -1
    empty = _shape(m3, batch=0)
    assert f(ctypes.byref(empty), None, None, None, None) == 0


def test_shapes_beyond_one_launch_grid_are_refused(m3):
    # b * H chains beyond a 32-bit grid: refused on the host, never launched truncated
    big = _shape(m3, batch=1 << 31, nheads=4)
    assert m3.lib.m3_scan_fwd(ctypes.byref(big), ctypes.byref(_fake_io(m3)), None, 0, None) == -2
    assert m3.lib.m3_scan_workspace_bytes(ctypes.byref(big)) == 0
    io = m3.DecodeIO()
    for i, (name, _) in enumerate(m3.DecodeIO._fields_):
        if name in ("x", "Braw", "Craw", "dt", "A", "lam", "theta", "B_bias", "C_bias", "h", "y"):
            setattr(io, name, 0x100000 + 0x1000 * (i + 1))
    dec = _shape(m3, batch=1 << 30, nheads=8, seqlen=1, chunk=1)
    assert m3.lib.m3_decode_step(ctypes.byref(dec), ctypes.byref(io), None) == -2
    # a forced split whose workgroups overflow the grid
    split = _shape(m3, batch=1 << 20, nheads=1024, seqlen=64 * 8, nsegments=8)
    assert m3.lib.m3_scan_fwd(ctypes.byref(split), ctypes.byref(_fake_io(m3)), None, 0, None) == -2
    # tokens beyond 2^40
    toks = _shape(m3, batch=1 << 20, seqlen=1 << 21)
    assert m3.lib.m3_scan_fwd(ctypes.byref(toks), ctypes.byref(_fake_io(m3)), None, 0, None) == -2
    assert m3.lib.m3_expand_ranks(ctypes.byref(_shape(m3, batch=1 << 20, seqlen=1 << 21, rank=4)), 0x1000, 0x2000,
                                  0x3000, None) == -2


def test_backward_low_memory_flag(m3):
    LOW = m3.M3_FLAG_BWD_LOW_MEMORY
    for R, C, cap in ((1, 64, 1.0e9), (4, 16, 1.4e9)):
        full = m3.scan_bwd_workspace_bytes(_shape(m3, batch=8, nheads=64, seqlen=4096, rank=R, chunk=C))
        low = m3.scan_bwd_workspace_bytes(_shape(m3, batch=8, nheads=64, seqlen=4096, rank=R, chunk=C, flags=LOW))
        assert 0 < low < cap < full, (R, low, full)
    # matrix-core chain shapes only
    assert m3.scan_bwd_workspace_bytes(_shape(m3, dstate=64, headdim=32, flags=LOW)) == 0
    io = _fake_io(m3)
    assert _bwd(m3, _shape(m3, dstate=64, headdim=32, flags=LOW), io, _fake_grads(m3, io)) == -2
    # a backward flag: the forward and its plan refuse it
    s = _shape(m3, flags=LOW)
    assert m3.lib.m3_scan_fwd(ctypes.byref(s), ctypes.byref(_fake_io(m3)), None, 0, None) == -1
    assert m3.lib.m3_scan_workspace_bytes(ctypes.byref(s)) == 0
    # still validated like the one-pass call: the workspace is checked
    assert _bwd(m3, _shape(m3, rank=2, chunk=32, flags=LOW), io, _fake_grads(m3, io)) == -4
