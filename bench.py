#!/usr/bin/env python3
"""Benchmark of the Mamba-3 SSM mixer core on one MI355X.

A step is one chunked-scan prefill (m3_scan_fwd) of the 1.5B-scale SISO layer
(batch 8, L 4096, 64 heads x P 64, N 128, chunk 64, bf16 io, fp32 state) over
inputs already resident in HBM; ``value`` is prefill tokens/s. The same JSON
line carries the roofline of that kernel (HIP events on its stream), the CPU
oracle timed on the same workload, and the other hot-path figures: MIMO rank-4
prefill, the long-context MIMO prefill (segment split) followed by 256 decode
steps, and the decode step for N in {128, 64}, SISO and MIMO R=4.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_DENSE_TFLOPS = 2516.6     # MI355X dense bf16 MFMA, TFLOP/s
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_siso_prefill_1p5b.json")
MFMA_BUSY_FILE = os.path.join(ROOT, "profiles", "pmc_mfma_busy_siso_prefill_1p5b.json")
KERNEL_SRC = os.path.join(ROOT, "state_space_sequence_amd", "csrc", "m3_scan_mfma.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------- algorithmic counts --
def prefill_bytes(s) -> int:
    """Bytes a prefill must move at least once: x and y (io dtype), raw B and C,
    dt/A/lam, theta, biases, the final state (fp32)."""
    io = 2 if s.io == "bf16" else 4
    b, L, H, G, P, N, R = s.batch, s.seqlen, s.nheads, s.ngroups, s.headdim, s.dstate, s.rank
    return (2 * b * L * H * R * P * io          # x in, y out
            + 2 * b * L * G * R * N * io        # Braw, Craw
            + 3 * b * L * H * 4                 # dt, A, lam
            + b * L * G * (N // 2) * 4          # theta
            + 2 * H * R * N * 4                 # biases
            + b * H * P * N * 4)                # final state


def prefill_flops(s):
    """Matrix-core flops of the chunked algorithm (dense and causal), per call:
    per chunk-head 2 T^2 N (C B^T) + 2 T^2 P (masked product with X) with
    T = chunk * R rows, plus 2 T N P for the chunk state and 2 T N P for the
    carried-state output."""
    T = s.chunk * s.rank
    nch = -(-s.seqlen // s.chunk) * s.batch * s.nheads
    inter = 4 * T * s.dstate * s.headdim
    dense = 2 * T * T * (s.dstate + s.headdim) + inter
    causal_pairs = s.chunk * (s.chunk + 1) // 2 * s.rank * s.rank
    causal = 2 * causal_pairs * (s.dstate + s.headdim) + inter
    return nch * dense, nch * causal


def decode_bytes(s, state_bytes=4) -> int:
    io = 2 if s.io == "bf16" else 4
    b, H, G, P, N, R = s.batch, s.nheads, s.ngroups, s.headdim, s.dstate, s.rank
    return (2 * b * H * P * N * state_bytes     # state read + write
            + 3 * b * H * R * P * io            # x, x_prev, y
            + 3 * b * G * R * N * io            # Braw, Craw, Braw_prev
            + 3 * b * H * 4 + b * G * (N // 2) * 4 + 2 * H * R * N * 4)


def fused_prefill_bytes(s) -> int:
    """The fused-projection prefill moves X', Z' and O' (one P-row per token)
    instead of x and y (R rows each), plus the three [H,P,R] weights."""
    io = 2 if s.io == "bf16" else 4
    b, L, H, P, R = s.batch, s.seqlen, s.nheads, s.headdim, s.rank
    return prefill_bytes(s) - 2 * b * L * H * R * P * io + 3 * b * L * H * P * io + 3 * H * P * R * 4


def fused_decode_bytes(s, state_bytes=4) -> int:
    io = 2 if s.io == "bf16" else 4
    b, H, P, R = s.batch, s.nheads, s.headdim, s.rank
    return decode_bytes(s, state_bytes) - 3 * b * H * R * P * io + 4 * b * H * P * io + 3 * H * P * R * 4


def bwd_bytes(s) -> int:
    """Bytes the prefill backward must move at least once: the forward's inputs and dy
    (io dtype; dt/A/lam/theta fp32) in, every gradient (fp32) out."""
    io = 2 if s.io == "bf16" else 4
    b, L, H, G, P, N, R = s.batch, s.seqlen, s.nheads, s.ngroups, s.headdim, s.dstate, s.rank
    return (2 * b * L * H * R * P * io + 2 * b * L * G * R * N * io + 3 * b * L * H * 4 + b * L * G * (N // 2) * 4
            + b * L * H * R * P * 4 + 2 * b * L * G * R * N * 4 + 3 * b * L * H * 4 + b * L * G * (N // 2) * 4
            + 4 * H * R * N * 4)


# ----------------------------------------------------------------- helpers --
def scan_args(d, s):
    return (d["x"], d["Braw"], d["Craw"], d["dt"], d["A"], d["lam"], d["theta"], d["B_bias"], d["C_bias"])


def time_prefill(m3, torch, d, s, steps, warmup, y, hf, ws):
    args = scan_args(d, s)
    for _ in range(warmup):
        m3.scan_fwd(*args, chunk=s.chunk, eps=s.eps, y=y, h_final=hf, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for k in range(steps):
        m3.scan_fwd(*args, chunk=s.chunk, eps=s.eps, y=y, h_final=hf, workspace=ws)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]  # ms per launch group
    return wall, per


def settle_clocks(m3, torch, d, s, y, hf, ws, min_s=0.2):
    """Untimed prefill launches until at least min_s seconds of GPU work have run,
    so the timed region starts with the clocks already at their working level
    (20 launches after 5 had varied by up to 20% between runs as clocks settled)."""
    args = scan_args(d, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(20):
            m3.scan_fwd(*args, chunk=s.chunk, eps=s.eps, y=y, h_final=hf, workspace=ws)
        n += 20
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= min_s:
            break
    return {"settle_ms": round(1e3 * (time.perf_counter() - t0), 1), "settle_launches": n}


def measured_ceilings(m3, torch, dev, facts):
    """The HBM and matrix-core ceilings one kernel reaches on this device: the
    library's stream copy over 512 MiB (twice the last-level cache) and its dense
    bf16 matrix-core loop, with the shader clock that loop ran at."""
    nbytes = 512 * 1024 * 1024
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        m3.probe_copy(src, dst)
    torch.cuda.synchronize()
    reps = 10
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for k in range(reps):
        m3.probe_copy(src, dst)
        ev[k + 1].record()
    torch.cuda.synchronize()
    tcopy = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(reps))[reps // 2]
    copy_gbs = 2 * nbytes / (tcopy * 1e-3) / 1e9
    del src, dst
    blocks, iters = 8 * facts["compute_units"], 8192
    out, clk = m3.probe_mfma_bf16(blocks, iters)
    for _ in range(2):
        m3.probe_mfma_bf16(blocks, iters, out=out, clock=clk)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record()
    for k in range(5):
        m3.probe_mfma_bf16(blocks, iters, out=out, clock=clk)
        ev[k + 1].record()
    torch.cuda.synchronize()
    tm = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(5))[2]
    tflops = m3.probe_mfma_flops(blocks, iters) / (tm * 1e-3) / 1e12
    c = clk.cpu().double().reshape(-1, 2)
    mhz = float((c[:, 0] / c[:, 1]).median()) * facts["wall_clock_mhz"] if facts["wall_clock_mhz"] else None
    return {"hbm_copy_GBps": round(copy_gbs, 1), "hbm_copy_frac_of_spec": round(copy_gbs / HBM_PEAK_GBS, 4),
            "hbm_copy_bytes": "512 MiB read + 512 MiB written per launch (m3_probe_copy)",
            "mfma_bf16_TFLOPs": round(tflops, 1), "mfma_frac_of_spec": round(tflops / BF16_DENSE_TFLOPS, 4),
            "mfma_loop": "%d workgroups x 4 waves x %d x 2 v_mfma_f32_16x16x32_bf16 (m3_probe_mfma_bf16)"
                         % (blocks, iters),
            "shader_clock_mhz_in_mfma_loop": None if mhz is None else round(mhz, 1)}


def smi_clocks():
    """Current clocks as rocm-smi reports them (a child process; None if unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    lines = [ln.strip() for ln in r.stdout.splitlines() if "clk" in ln.lower() and "(" in ln]
    return lines[:8] or None


def src_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_counters(bytes_alg):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(PMC_FILE) as f:
            pm = json.load(f)
    except (OSError, ValueError):
        return None
    if pm.get("kernel_src_sha256") != src_digest():
        return None
    return pm.get("hbm_bytes_per_launch")


def mfma_busy_from_counters():
    """MFMA-busy fraction of the headline kernel from the committed counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs and the kernel's cycles), if it was
    taken on the current kernel source; else None."""
    try:
        with open(MFMA_BUSY_FILE) as f:
            pm = json.load(f)
    except (OSError, ValueError):
        return None
    if pm.get("kernel_src_sha256") != src_digest():
        return None
    return pm.get("mfma_busy_frac")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, chains_target):
    """The oracle as it stands, on whole sequences of (batch, head) chains of the
    same workload (all of them by default, a few seconds on a 16-core host),
    scaled to the workload's tokens/s when fewer are run."""
    import numpy as np  # noqa: F401
    import oracle
    from state_space_sequence_amd.inputs import make_scan_inputs
    H = shape.nheads
    nb = max(1, chains_target // H)
    s = shape.replace(batch=nb)
    inp = make_scan_inputs(s, seed=99)
    cores = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.scan(inp, s, nthreads=cores)
    dt = time.perf_counter() - t0
    chains = nb * H
    frac = chains / (shape.batch * shape.nheads)
    full_time = dt / frac
    # one host thread on a smaller sample (the heads of one batch entry)
    s1 = shape.replace(batch=1, nheads=H)
    inp1 = make_scan_inputs(s1, seed=98)
    t1 = time.perf_counter()
    oracle.scan(inp1, s1, nthreads=1)
    dt1 = time.perf_counter() - t1
    full_time1 = dt1 * (shape.batch * shape.nheads) / (s1.batch * s1.nheads)
    return {
        "value": shape.batch * shape.seqlen / full_time,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": ("the whole workload: all %d (batch, head) chains, L=%d, fp64 C oracle with OpenMP over "
                   "chains; %.2f s measured" % (chains, shape.seqlen, dt)) if frac >= 1 else
                  ("%d of %d (batch, head) chains, full L=%d, fp64 C oracle with OpenMP over chains; "
                   "%.2f s measured, scaled by %d/%d" % (chains, shape.batch * shape.nheads, shape.seqlen, dt,
                                                          shape.batch * shape.nheads, chains)),
        "cpu_model": cpu_model(),
        "value_1thread": shape.batch * shape.seqlen / full_time1,
        "sample_1thread": "%d chains on one thread, %.2f s measured, scaled by %d/%d"
                          % (s1.batch * s1.nheads, dt1, shape.batch * shape.nheads, s1.batch * s1.nheads),
    }


# --------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-extra", action="store_true", help="only the headline prefill")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-chains", type=int, default=512)
    ap.add_argument("--pmc-run", action="store_true",
                    help="short run for counter collection: one 512 MiB copy, then 2 prefill steps")
    ap.add_argument("--pmc-decode", action="store_true",
                    help="short run for counter collection: one 512 MiB copy, then 2 decode steps of the "
                         "SISO and MIMO-4 N128 workloads (fp32 state)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only (the work shards over batch and heads, but the library "
              "has no multi-GPU path); got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from state_space_sequence_amd import m3
    from state_space_sequence_amd.inputs import (WORKLOADS, make_decode_inputs, make_fused_decode_inputs,
                                                 make_fused_scan_inputs, make_scan_inputs)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    facts = m3.device_facts(0)
    log("device:", props.name, facts)

    if args.pmc_decode:
        src = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reference copy: reads and writes exactly 512 MiB
        torch.cuda.synchronize()
        del src, dst
        alg = {}
        for nm in ("decode_siso_n128", "decode_mimo4_n128"):
            sd = WORKLOADS[nm]
            de = m3.to_device(make_decode_inputs(sd, seed=3), sd.io)
            ydec = torch.empty_like(de["x"])
            # 8 steps over 4 state buffers (1.07 GB): as in the timed decode, no step
            # finds its state in the 256 MB last-level cache
            states = [de["h"].clone() for _ in range(4)]
            for k in range(8):
                m3.decode_step(de["x"], de["Braw"], de["Craw"], de["dt"], de["A"], de["lam"], de["theta"],
                               de["B_bias"], de["C_bias"], states[k % 4], x_prev=de["x_prev"],
                               Braw_prev=de["Braw_prev"], y=ydec)
            torch.cuda.synchronize()
            alg[nm] = decode_bytes(sd, 4)
            del de, states
        print(json.dumps({"pmc_decode": True, "copy_bytes": 512 * 1024 * 1024, "decode_bytes_alg": alg}))
        return

    name = "siso_prefill_1p5b"
    s = WORKLOADS[name]
    log("generating inputs for", name)
    inp = make_scan_inputs(s, seed=1)
    d = m3.to_device(inp, s.io)
    del inp
    y = torch.empty_like(d["x"])
    hf = torch.empty((s.batch, s.nheads, s.headdim, s.dstate), dtype=torch.float32, device=dev)
    shape_c = m3.scan_shape(d["x"], d["Braw"], s.chunk, s.eps)
    plan = m3.plan(shape_c)
    wsb = m3.workspace_bytes(shape_c)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

    if args.pmc_run:
        src = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reference copy: reads and writes exactly 512 MiB
        torch.cuda.synchronize()
        time_prefill(m3, torch, d, s, 2, 0, y, hf, ws)
        print(json.dumps({"pmc_run": True, "copy_bytes": 512 * 1024 * 1024,
                          "prefill_bytes_alg": prefill_bytes(s)}))
        return

    settle = settle_clocks(m3, torch, d, s, y, hf, ws)
    log("clocks settled: %s" % settle)
    log("timing %s: %d warmup + %d steps (plan: kernel %d, %d segment(s), %d workgroups)"
        % (name, args.warmup, args.steps, plan.kernel, plan.nsegments, plan.workgroups))
    wall, per = time_prefill(m3, torch, d, s, args.steps, args.warmup, y, hf, ws)
    ms_step = 1e3 * wall / args.steps
    tokens = s.batch * s.seqlen
    value = tokens * args.steps / wall
    kern_ms = sum(per) / len(per)
    balg = prefill_bytes(s)
    fl_dense, fl_causal = prefill_flops(s)
    achieved = balg / (kern_ms * 1e-3) / 1e9
    traffic = traffic_from_counters(balg)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "bcnorm_pairs_kernel + scan_mfma_kernel<full, R=1> (one m3_scan_fwd call)",
            "avg_launch_ms": round(kern_ms, 5),
            "alg_bytes_per_launch": balg,
            "mfma_frac_dense": round(fl_dense / (kern_ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 4),
            "mfma_frac_causal": round(fl_causal / (kern_ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 4),
            "mfma_busy_frac_counter": mfma_busy_from_counters()}
    log("prefill: %.4f ms/step, %.3e tokens/s, %.0f GB/s (%.1f%% of HBM peak)"
        % (kern_ms, value, achieved, 100 * achieved / HBM_PEAK_GBS))
    del d, y, hf
    torch.cuda.empty_cache()

    extra = {"timing": dict(settle, protocol="untimed launches until >= 0.2 s of GPU work, then --warmup "
                                              "untimed and --steps timed launches back to back"),
             "device": facts, "rocm_smi_clocks": smi_clocks()}
    ceil = measured_ceilings(m3, torch, dev, facts)
    extra["ceilings"] = ceil
    log("ceilings:", ceil)
    roof["frac_of_measured_copy"] = round(achieved / ceil["hbm_copy_GBps"], 4)
    if not args.no_extra:
        # ---- MIMO rank-4 prefill, same shape
        for nm in ("mimo4_prefill_1p5b", "mimo4_prefill_long"):
            sm_ = WORKLOADS[nm]
            log("generating inputs for", nm)
            inp = make_scan_inputs(sm_, seed=2)
            dd = m3.to_device(inp, sm_.io)
            del inp
            yy = torch.empty_like(dd["x"])
            hh = torch.empty((sm_.batch, sm_.nheads, sm_.headdim, sm_.dstate), dtype=torch.float32, device=dev)
            shp = m3.scan_shape(dd["x"], dd["Braw"], sm_.chunk, sm_.eps)
            pl = m3.plan(shp)
            w2 = m3.workspace_bytes(shp)
            wsp = torch.empty(w2, dtype=torch.uint8, device=dev) if w2 else None
            wl, pr = time_prefill(m3, torch, dd, sm_, 50, 20, yy, hh, wsp)
            ms = sum(pr) / len(pr)
            bb = prefill_bytes(sm_)
            fd, fc = prefill_flops(sm_)
            ent = {"tokens_per_s": round(sm_.batch * sm_.seqlen / (ms * 1e-3), 1), "ms": round(ms, 4),
                   "hbm_frac": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "mfma_frac_dense": round(fd / (ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 4),
                   "mfma_frac_causal": round(fc / (ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 4),
                   "segments": pl.nsegments, "workgroups": pl.workgroups}
            log(nm, ent)
            if nm == "mimo4_prefill_long":
                # 256 decode steps continuing from the prefill's final state: step k
                # takes new token k (its own x, raw B and C, dt, A, lambda, theta) with
                # the prefill's biases, and token k - 1 (the prefill's last token for
                # k = 0) as its previous token
                K = 256
                cont = make_scan_inputs(sm_.replace(seqlen=K), seed=6)
                ct = m3.to_device({k: cont[k] for k in ("x", "Braw", "Craw", "dt", "A", "lam", "theta")}, sm_.io)
                del cont
                h = hh.clone()
                toks = [{k: ct[k][:, i].contiguous() for k in ct} for i in range(K)]
                prevs = [(dd["x"][:, -1].contiguous(), dd["Braw"][:, -1].contiguous())]
                prevs += [(toks[i]["x"], toks[i]["Braw"]) for i in range(K - 1)]
                ydec = torch.empty_like(toks[0]["x"])

                def step(i):
                    t = toks[i]
                    m3.decode_step(t["x"], t["Braw"], t["Craw"], t["dt"], t["A"], t["lam"], t["theta"],
                                   dd["B_bias"], dd["C_bias"], h, eps=sm_.eps, x_prev=prevs[i][0],
                                   Braw_prev=prevs[i][1], y=ydec)

                for i in range(8):
                    step(i)
                h.copy_(hh)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(K):
                    step(i)
                e1.record()
                torch.cuda.synchronize()
                ent["decode_256_steps_us_per_step"] = round(1e3 * e0.elapsed_time(e1) / K, 3)
                log("  then 256 decode steps:", ent["decode_256_steps_us_per_step"], "us/step")
                # the same 256 steps captured once in a HIP graph and replayed: the
                # step is launch-bound at this size (48 workgroups, 3.2 MB)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for i in range(K):
                        step(i)
                h.copy_(hh)
                graph.replay()
                torch.cuda.synchronize()
                h.copy_(hh)
                torch.cuda.synchronize()
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                ent["decode_256_steps_graph_us_per_step"] = round(1e3 * e0.elapsed_time(e1) / K, 3)
                log("  the same from one graph:", ent["decode_256_steps_graph_us_per_step"], "us/step")
                del graph, toks, prevs, ct, h
            extra[nm] = ent
            del dd, yy, hh, wsp
            torch.cuda.empty_cache()
        # ---- decode steps, cycling 4 state buffers so the 256 MB last-level cache
        # cannot hold the state between steps
        # (then the same four with the state stored in bf16)
        decode_runs = [(nm, False) for nm in ("decode_siso_n128", "decode_mimo4_n128", "decode_siso_n64",
                                              "decode_mimo4_n64")]
        decode_runs += [(nm, True) for nm, _ in decode_runs]
        for nm, bf16_state in decode_runs:
            sd = WORKLOADS[nm]
            dinp = make_decode_inputs(sd, seed=3)
            de = m3.to_device(dinp, sd.io)
            h0 = de["h"].to(torch.bfloat16) if bf16_state else de["h"]
            states = [h0.clone() for _ in range(4)]
            ydec = torch.empty_like(de["x"])
            base = (de["x"], de["Braw"], de["Craw"], de["dt"], de["A"], de["lam"], de["theta"],
                    de["B_bias"], de["C_bias"])
            for k in range(40):
                m3.decode_step(*base, states[k % 4], x_prev=de["x_prev"], Braw_prev=de["Braw_prev"], y=ydec)
            torch.cuda.synchronize()
            reps = 200
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            evs[0].record()
            for k in range(reps):
                m3.decode_step(*base, states[k % 4], x_prev=de["x_prev"], Braw_prev=de["Braw_prev"], y=ydec)
                evs[k + 1].record()
            torch.cuda.synchronize()
            tms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(reps))
            med = tms[reps // 2]
            bb = decode_bytes(sd, 2 if bf16_state else 4)
            ent = {"us_per_step": round(1e3 * med, 2), "p10_us": round(1e3 * tms[reps // 10], 2),
                   "p90_us": round(1e3 * tms[(9 * reps) // 10], 2),
                   "hbm_frac": round(bb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": bb}
            key = nm + ("_bf16state" if bf16_state else "")
            log(key, ent)
            extra[key] = ent
            del de, states
            torch.cuda.empty_cache()

        # ---- the fused rank projections and gate (MIMO rank 4): prefill and decode
        nm = "mimo4_prefill_1p5b"
        sf = WORKLOADS[nm]
        inp = make_fused_scan_inputs(sf, seed=8)
        df = m3.to_device(inp, sf.io)
        del inp
        of = torch.empty_like(df["x_in"])
        hf2 = torch.empty((sf.batch, sf.nheads, sf.headdim, sf.dstate), dtype=torch.float32, device=dev)
        fargs = (df["x_in"], df["z_in"], df["W_X"], df["W_Z"], df["W_O"], df["Braw"], df["Craw"], df["dt"],
                 df["A"], df["lam"], df["theta"], df["B_bias"], df["C_bias"])
        for _ in range(10):
            m3.scan_fused_fwd(*fargs, chunk=sf.chunk, eps=sf.eps, o=of, h_final=hf2)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(31)]
        evs[0].record()
        for k in range(30):
            m3.scan_fused_fwd(*fargs, chunk=sf.chunk, eps=sf.eps, o=of, h_final=hf2)
            evs[k + 1].record()
        torch.cuda.synchronize()
        ms = sum(evs[k].elapsed_time(evs[k + 1]) for k in range(30)) / 30
        bb = fused_prefill_bytes(sf)
        ent = {"tokens_per_s": round(sf.batch * sf.seqlen / (ms * 1e-3), 1), "ms": round(ms, 4),
               "hbm_frac": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": bb}
        log(nm + "_fused", ent)
        extra[nm + "_fused"] = ent
        # the same output without the fusion: rank expansion, the core, gate and
        # rank contraction as three launches (X and y round-trip through HBM)
        xe = torch.empty((sf.batch, sf.seqlen, sf.nheads, sf.rank, sf.headdim), dtype=df["x_in"].dtype, device=dev)
        ye = torch.empty_like(xe)
        core = (df["Braw"], df["Craw"], df["dt"], df["A"], df["lam"], df["theta"], df["B_bias"], df["C_bias"])

        def unfused():
            m3.expand_ranks(df["x_in"], df["W_X"], x_out=xe)
            m3.scan_fwd(xe, *core, chunk=sf.chunk, eps=sf.eps, y=ye, h_final=hf2)
            m3.gate_contract(ye, df["z_in"], df["W_Z"], df["W_O"], o=of)

        for _ in range(10):
            unfused()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(31)]
        evs[0].record()
        for k in range(30):
            unfused()
            evs[k + 1].record()
        torch.cuda.synchronize()
        ms_u = sum(evs[k].elapsed_time(evs[k + 1]) for k in range(30)) / 30
        ent_u = {"ms": round(ms_u, 4), "tokens_per_s": round(sf.batch * sf.seqlen / (ms_u * 1e-3), 1),
                 "fused_speedup": round(ms_u / ent["ms"], 3),
                 "steps": "m3_expand_ranks + m3_scan_fwd + m3_gate_contract"}
        log(nm + "_unfused_pipeline", ent_u)
        extra[nm + "_unfused_pipeline"] = ent_u
        del df, of, hf2, xe, ye
        torch.cuda.empty_cache()
        for nm, bf16_state in (("decode_mimo4_n128", False), ("decode_mimo4_n128", True)):
            sd = WORKLOADS[nm]
            de = m3.to_device(make_fused_decode_inputs(sd, seed=9), sd.io)
            h0 = de["h"].to(torch.bfloat16) if bf16_state else de["h"]
            states = [h0.clone() for _ in range(4)]
            od = torch.empty_like(de["x_in"])
            base = (de["x_in"], de["z_in"], de["W_X"], de["W_Z"], de["W_O"], de["Braw"], de["Craw"], de["dt"],
                    de["A"], de["lam"], de["theta"], de["B_bias"], de["C_bias"])
            # the same protocol as the plain decode: 40 untimed steps, then the median of 200
            for k in range(40):
                m3.decode_fused_step(*base, states[k % 4], x_prev_in=de["x_prev_in"], Braw_prev=de["Braw_prev"], o=od)
            torch.cuda.synchronize()
            reps = 200
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            evs[0].record()
            for k in range(reps):
                m3.decode_fused_step(*base, states[k % 4], x_prev_in=de["x_prev_in"], Braw_prev=de["Braw_prev"], o=od)
                evs[k + 1].record()
            torch.cuda.synchronize()
            tms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(reps))
            med = tms[reps // 2]
            bb = fused_decode_bytes(sd, 2 if bf16_state else 4)
            ent = {"us_per_step": round(1e3 * med, 2), "p10_us": round(1e3 * tms[reps // 10], 2),
                   "p90_us": round(1e3 * tms[(9 * reps) // 10], 2),
                   "hbm_frac": round(bb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": bb}
            key = nm + "_fused" + ("_bf16state" if bf16_state else "")
            log(key, ent)
            extra[key] = ent
            # the same step unfused: expansion, the plain decode step, gate
            xe = torch.empty((sd.batch, sd.nheads, sd.rank, sd.headdim), dtype=de["x_in"].dtype, device=dev)
            xpe = torch.empty_like(xe)
            ye = torch.empty_like(xe)
            dcore = (de["Braw"], de["Craw"], de["dt"], de["A"], de["lam"], de["theta"], de["B_bias"], de["C_bias"])

            def unfused(st):
                m3.expand_ranks(de["x_in"], de["W_X"], x_out=xe)
                m3.expand_ranks(de["x_prev_in"], de["W_X"], x_out=xpe)
                m3.decode_step(xe, *dcore, st, x_prev=xpe, Braw_prev=de["Braw_prev"], y=ye)
                m3.gate_contract(ye, de["z_in"], de["W_Z"], de["W_O"], o=od)

            for k in range(40):
                unfused(states[k % 4])
            torch.cuda.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            evs[0].record()
            for k in range(reps):
                unfused(states[k % 4])
                evs[k + 1].record()
            torch.cuda.synchronize()
            tu = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(reps))[reps // 2]
            ent_u = {"us_per_step": round(1e3 * tu, 2), "fused_speedup": round(tu / med, 3),
                     "steps": "2 x m3_expand_ranks + m3_decode_step + m3_gate_contract"}
            log(key.replace("_fused", "_unfused_pipeline"), ent_u)
            extra[key.replace("_fused", "_unfused_pipeline")] = ent_u
            del de, states, xe, xpe, ye
            torch.cuda.empty_cache()

        # ---- prefill backward (training): SISO and MIMO rank-4, b8 L4096
        for nm in ("siso_prefill_1p5b", "mimo4_prefill_1p5b"):
            sb = WORKLOADS[nm]
            inp = make_scan_inputs(sb, seed=10)
            db = m3.to_device(inp, sb.io)
            del inp
            dyb = torch.randn(db["x"].shape, device=dev).to(db["x"].dtype)
            bargs = (db["x"], db["Braw"], db["Craw"], db["dt"], db["A"], db["lam"], db["theta"], db["B_bias"],
                     db["C_bias"], dyb)
            grads = m3.scan_bwd(*bargs, eps=sb.eps)
            shp = m3.make_shape(sb.batch, sb.seqlen, sb.nheads, sb.ngroups, sb.headdim, sb.dstate, sb.rank,
                                sb.chunk, m3.M3_BF16, sb.eps)
            bb = bwd_bytes(sb)
            # one pass, then the windowed low-memory schedule (same gradients, bit for bit)
            for low in (False, True):
                shp = m3.make_shape(sb.batch, sb.seqlen, sb.nheads, sb.ngroups, sb.headdim, sb.dstate, sb.rank,
                                    sb.chunk, m3.M3_BF16, sb.eps, m3.M3_FLAG_BWD_LOW_MEMORY if low else 0)
                wsb = m3.scan_bwd_workspace_bytes(shp)
                wsp = torch.empty(wsb, dtype=torch.uint8, device=dev)
                for _ in range(5):
                    m3.scan_bwd(*bargs, eps=sb.eps, grads=grads, workspace=wsp, low_memory=low)
                torch.cuda.synchronize()
                reps = 15
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
                evs[0].record()
                for k in range(reps):
                    m3.scan_bwd(*bargs, eps=sb.eps, grads=grads, workspace=wsp, low_memory=low)
                    evs[k + 1].record()
                torch.cuda.synchronize()
                ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(reps))[reps // 2]
                ent = {"tokens_per_s": round(sb.batch * sb.seqlen / (ms * 1e-3), 1), "ms": round(ms, 3),
                       "hbm_frac": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": bb,
                       "workspace_bytes": wsb}
                key = nm + ("_backward_low_memory" if low else "_backward")
                log(key, ent)
                extra[key] = ent
                del wsp
                torch.cuda.empty_cache()
            del db, dyb, grads
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(s, args.cpu_chains)
        log("cpu oracle:", cpu)

    out = {
        "metric": "SSM prefill tokens/s (%MFMA peak) + decode us/step (%HBM BW), SISO & MIMO R=4",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": s.batch, "seqlen": s.seqlen, "nheads": s.nheads,
                   "headdim": s.headdim, "dstate": s.dstate, "rank": s.rank, "chunk": s.chunk,
                   "io": s.io, "state": "fp32"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
