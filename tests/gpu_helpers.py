"""Helpers for the GPU parity tests: run the HIP library through its binding on
seeded inputs and compare with the oracle by the max-normalised error
err(T) = max|T_gpu - T_ref| / max|T_ref|."""
from __future__ import annotations

import numpy as np
import torch

TOL_F32 = 1e-4   # fp32 io paths
TOL_BF16 = 2e-2  # bf16-input paths (y is stored in bf16)


def relerr(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(gpu))) if gpu.size else 0.0
    return float(np.max(np.abs(gpu - ref)) / den)


def gpu_scan(inp, shape, **kw):
    from state_space_sequence_amd import m3
    d = m3.to_device(inp, shape.io)
    y, h = m3.scan_fwd(d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"],
                       d["B_bias"], d["C_bias"], chunk=shape.chunk, eps=shape.eps,
                       B_normw=d.get("B_normw"), C_normw=d.get("C_normw"), h0=d.get("h0"),
                       x_prev=d.get("x_prev"), Braw_prev=d.get("Braw_prev"), D=d.get("D"),
                       out_normw=d.get("out_normw"), **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


def gpu_decode(inp, shape, bf16_state=False, **kw):
    """One decode step on the GPU. With bf16_state the state is handed over as bf16
    (the caller passes a state whose values are bf16-exact) and comes back as bf16."""
    from state_space_sequence_amd import m3
    d = m3.to_device(inp, shape.io)
    h = d["h"].clone()
    if bf16_state:
        h = h.to(torch.bfloat16)
    y = m3.decode_step(d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"],
                       d["B_bias"], d["C_bias"], h, eps=shape.eps, B_normw=d.get("B_normw"),
                       C_normw=d.get("C_normw"), x_prev=d.get("x_prev"), Braw_prev=d.get("Braw_prev"),
                       D=d.get("D"), out_normw=d.get("out_normw"), **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), h.float().cpu().numpy().astype(np.float64)


def gpu_scan_fused(inp, shape, **kw):
    """Prefill with the fused projections (inputs from make_fused_scan_inputs)."""
    from state_space_sequence_amd import m3
    d = m3.to_device(inp, shape.io)
    o, h = m3.scan_fused_fwd(d["x_in"], d["z_in"], d["W_X"], d["W_Z"], d["W_O"], d["Braw"], d["Craw"],
                             d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"],
                             chunk=shape.chunk, eps=shape.eps, B_normw=d.get("B_normw"),
                             C_normw=d.get("C_normw"), h0=d.get("h0"), x_prev_in=d.get("x_prev_in"),
                             Braw_prev=d.get("Braw_prev"), D=d.get("D"), out_normw=d.get("out_normw"), **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


def gpu_decode_fused(inp, shape, bf16_state=False, **kw):
    """One fused decode step (inputs from make_fused_decode_inputs)."""
    from state_space_sequence_amd import m3
    d = m3.to_device(inp, shape.io)
    h = d["h"].clone()
    if bf16_state:
        h = h.to(torch.bfloat16)
    o = m3.decode_fused_step(d["x_in"], d["z_in"], d["W_X"], d["W_Z"], d["W_O"], d["Braw"], d["Craw"],
                             d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"], h,
                             eps=shape.eps, B_normw=d.get("B_normw"), C_normw=d.get("C_normw"),
                             x_prev_in=d.get("x_prev_in"), Braw_prev=d.get("Braw_prev"), D=d.get("D"),
                             out_normw=d.get("out_normw"), **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), h.float().cpu().numpy().astype(np.float64)


def gpu_scan_bwd(inp, shape, dy, dh_final=None, **kw):
    """Prefill backward on the GPU; returns a dict of float64 arrays keyed like the inputs."""
    from state_space_sequence_amd import m3
    d = m3.to_device(inp, shape.io)
    dyt = torch.from_numpy(np.ascontiguousarray(dy, dtype=np.float32)).cuda()
    if shape.io == "bf16":
        dyt = dyt.to(torch.bfloat16)
    dhf = None if dh_final is None else torch.from_numpy(np.ascontiguousarray(dh_final, dtype=np.float32)).cuda()
    g = m3.scan_bwd(d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"],
                    d["C_bias"], dyt, eps=shape.eps, B_normw=d.get("B_normw"), C_normw=d.get("C_normw"),
                    h0=d.get("h0"), x_prev=d.get("x_prev"), Braw_prev=d.get("Braw_prev"), dh_final=dhf, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in g.items()}
