#!/usr/bin/env python3
"""Throughput of the Newton-parallel sLSTM forward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input. For the
full-layer workload (B=128, T=2048, d_in=d_h=1024, bf16 x and W_x):
    bf16 MFMA input projection -> Newton forward (warm start, K x [residual + Jacobian,
    block-bidiagonal solve, update], final residual, flags, h and final-state outputs) -> a
    T=1 sequential decode step at B=128 continuing from the final state (its own projection).
For workloads whose solver input is P the step is the Newton forward alone. The Newton
forward runs in the schedule the library picks for the shape (--schedule fused) and writes
the layer's default output, h and the final state (--outputs states writes the state tensor
too); the same step writing the states, the scan form of the fused iteration, the layered
schedule, the backward pass, the same tokens packed as ragged sequences (cu_seqlens), head
mixing (block-diagonal R, its own seeded input), the sigmoid/bf16 and long-context
workloads and the sequential forward are timed after it as context.

Prints ONE JSON line on stdout. Timing: W untimed warm-up steps, then exactly K steps
between two device synchronisations, wall clock. Per-kernel durations come from HIP events
the library records on the launching stream during the timed steps; the dominant kernel's
algorithmic bytes per launch over its mean duration give the roofline figure. The CPU
baseline times the float64 oracle on a bounded lane sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sLSTM Newton forward state-elems/s (B·T·d_h) + % HBM roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
# MI355X fp32 vector peak, published: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed
# dual-rate fp32) x 2.4 GHz = 157.3 TFLOP/s. The library's kernels are built without packed
# fp32 instructions, so 78.6 TFLOP/s is their ceiling for pure FMA streams.
FP32_VECTOR_PEAK_TFLOPS = 157.3
FP32_UNPACKED_PEAK_TFLOPS = 78.6
# vector issue: a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles; 1024 SIMDs at
# 2.4 GHz
SIMDS = 1024
CLOCK_GHZ = 2.4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
VALU_FILE = os.path.join(ROOT, "profiles", "valu.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# algorithmic work per launch
# ---------------------------------------------------------------------------------------
# The solver's Jacobian planes: the 12 entries of each 4x4 block that are not structural
# zeros of the channelwise cell ((c,n'), (n,c'), (m,c'), (m,n') are identically zero).
JAC_BYTES = 12 * 4


def solve_flops_per_elem(K, sigmoid_forget):
    """Floating-point operations of one state element of a whole Newton solve as the one-kernel
    solve forms them (an add, multiply, compare-select or max counts 1, an FMA 2, an exp2, log2
    or reciprocal 1): warm-start step 25 (with the scaling of the z and o pre-activations for
    their exponentials, done once per step), cell step 32, the coefficients of its Jacobian in
    factored form 12, residual and its maximum 8, the Newton step through the factored Jacobian
    22, the update 4; the sigmoid forget gate adds a log-sigmoid to every step (6) and its
    derivative to every linearisation (5)."""
    sig = 1 if sigmoid_forget else 0
    warm = 25 + 6 * sig
    cell = 32 + 6 * sig
    lin = 12 + 5 * sig
    return warm + K * (cell + lin + 8 + 22 + 4) + (cell + 8)


def kernel_work(w, n_e, p_bytes, states_out=True):
    """Algorithmic work per launch of each kernel kind. Bytes: every operand of every state
    element read once and every result written once (per element: P p_bytes, a state 16, a
    right-hand side / Newton step 16, the Jacobian JAC_BYTES, h 4). The one-kernel solve is
    reported against HBM on its bytes (P in; S_K, if the caller asks for the states, and h out;
    the final state's B·4·d_h floats are negligible), with its flop count of
    solve_flops_per_elem and its vector-issue share beside it."""
    return {
        "warm_start": {"bound": "hbm", "bytes": n_e * (p_bytes + 16)},                        # P in, S out
        "residual_jacobian": {"bound": "hbm", "bytes": n_e * (p_bytes + 16 + JAC_BYTES + 16)},  # P, S in; A, rhs out
        "scan_block4": {"bound": "hbm", "bytes": n_e * (JAC_BYTES + 16 + 16)},                # A, rhs in; Delta out
        "update": {"bound": "hbm", "bytes": n_e * 48},                                        # S, Delta in; S out
        "final_residual": {"bound": "hbm", "bytes": n_e * (p_bytes + 16)},                    # P, S in
        "newton_iteration": {"bound": "hbm", "bytes": n_e * (p_bytes + 16 + 16)},             # P, S_k in; S_k+1 out
        "newton_solve": {"bound": "hbm", "bytes": n_e * (p_bytes + (16 if states_out else 0) + 4),  # P in; (S_K,) h out
                         "flops": n_e * solve_flops_per_elem(w.max_iters, w.forget == "sigmoid")},
        "backward": {"bound": "hbm", "bytes": n_e * (p_bytes + 16 + 4 + 8)},                  # P, S, dL/dh in; bf16 dP out
    }


# Head mixing (block-diagonal R, 32 heads of 32 units) at the size of the sigmoid workload's
# batch and width: a context line, not the metric.
HEAD = dict(B=16, T=4096, d=1024, n_heads=32, forget="exp", K=3, seed=20265)
HEAD_WORKLOAD = "head_b16_t4096_d1024_h32"


def head_solve_flops_per_elem(d_head, K, sigmoid_forget):
    """Floating-point operations of one state element (b, t, j) in the one-sweep head-mixing
    Newton solve as the kernel forms them: K + 1 block products (R h' of the warm start, then
    R Delta h' of each iteration) for the four gates, 8 d_head each; the warm-start step 34; per
    iteration the cell step 34, its own-state and gate Jacobians 30, the residual and its maximum
    8, the factored solve (3 own-state and 4 gate FMAs per slot) 56, the update 4 and the
    pre-activation update 4; the final residual 34 + 8. The sigmoid forget gate adds 6 to every
    cell step and 5 to every Jacobian, as in solve_flops_per_elem."""
    sig = 1 if sigmoid_forget else 0
    cell = 34 + 6 * sig
    return 8 * d_head * (K + 1) + cell + K * (cell + 30 + 5 * sig + 8 + 56 + 4 + 4) + cell + 8


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "residual_jacobian": ["recurrent_nets_amd/csrc/k_residual.hip", "recurrent_nets_amd/csrc/cell.h",
                          "recurrent_nets_amd/csrc/common.h"],
    "scan_block4": ["recurrent_nets_amd/csrc/k_scan.hip", "recurrent_nets_amd/csrc/affine4.h",
                    "recurrent_nets_amd/csrc/common.h"],
    "newton_iteration": ["recurrent_nets_amd/csrc/k_newton_fused.hip", "recurrent_nets_amd/csrc/affine4.h",
                         "recurrent_nets_amd/csrc/cell.h", "recurrent_nets_amd/csrc/common.h"],
    "newton_solve": ["recurrent_nets_amd/csrc/k_newton_pipe.hip", "recurrent_nets_amd/csrc/cell.h",
                     "recurrent_nets_amd/csrc/common.h", "recurrent_nets_amd/csrc/kernels.h"],
    "update": ["recurrent_nets_amd/csrc/k_update.hip", "recurrent_nets_amd/csrc/common.h"],
    "final_residual": ["recurrent_nets_amd/csrc/k_residual.hip", "recurrent_nets_amd/csrc/cell.h",
                       "recurrent_nets_amd/csrc/common.h"],
    "warm_start": ["recurrent_nets_amd/csrc/k_warm.hip", "recurrent_nets_amd/csrc/cell.h",
                   "recurrent_nets_amd/csrc/common.h"],
    "input_projection": ["recurrent_nets_amd/csrc/k_gemm.hip", "recurrent_nets_amd/csrc/common.h"],
    "backward": ["recurrent_nets_amd/csrc/k_backward.hip", "recurrent_nets_amd/csrc/affine4.h",
                 "recurrent_nets_amd/csrc/cell.h", "recurrent_nets_amd/csrc/common.h",
                 "recurrent_nets_amd/csrc/kernels.h"],
    "packed_iteration": ["recurrent_nets_amd/csrc/k_newton_fused.hip", "recurrent_nets_amd/csrc/affine4.h",
                         "recurrent_nets_amd/csrc/cell.h", "recurrent_nets_amd/csrc/common.h"],
    "packed_solve": ["recurrent_nets_amd/csrc/k_newton_pipe.hip", "recurrent_nets_amd/csrc/cell.h",
                     "recurrent_nets_amd/csrc/common.h", "recurrent_nets_amd/csrc/kernels.h"],
    "packed_backward": ["recurrent_nets_amd/csrc/k_backward.hip", "recurrent_nets_amd/csrc/affine4.h",
                        "recurrent_nets_amd/csrc/cell.h", "recurrent_nets_amd/csrc/common.h",
                        "recurrent_nets_amd/csrc/kernels.h"],
    "newton_solve_states": ["recurrent_nets_amd/csrc/k_newton_pipe.hip", "recurrent_nets_amd/csrc/cell.h",
                            "recurrent_nets_amd/csrc/common.h", "recurrent_nets_amd/csrc/kernels.h"],
    "head_solve": ["recurrent_nets_amd/csrc/k_head_solve.hip", "recurrent_nets_amd/csrc/head.h",
                   "recurrent_nets_amd/csrc/affine4.h", "recurrent_nets_amd/csrc/cell.h",
                   "recurrent_nets_amd/csrc/common.h", "recurrent_nets_amd/csrc/kernels.h"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when they were
    taken on another workload or on an older version of the kernel's source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        data = json.load(f)
    rec = data.get(f"{kernel}@{workload}") or data.get(kernel)
    if not rec or rec.get("workload") != workload:
        return None
    if rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def measured_valu(kernel, workload):
    """VALU instructions per launch (SQ_INSTS_VALU, summed over the launch's waves) from a
    committed rocprofv3 counter run, or None when it was taken on another workload or on an
    older version of the kernel's source."""
    if not os.path.exists(VALU_FILE):
        return None
    with open(VALU_FILE) as f:
        data = json.load(f)
    rec = data.get(f"{kernel}@{workload}") or data.get(kernel)
    if not rec or rec.get("workload") != workload:
        return None
    if rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("valu_insts_per_launch")


def valu_issue_frac(insts, ms):
    """Share of the GPU's vector issue slots a launch's VALU instructions fill: each wave64
    instruction holds a 16-lane SIMD for 4 cycles."""
    return insts * 4.0 / (SIMDS * CLOCK_GHZ * 1e9 * ms * 1e-3)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def copy_bandwidth(torch, dev, nbytes=4 << 30, reps=5):
    """Device-to-device copy bandwidth on this GPU (torch's copy of nbytes, read + write
    counted), median of reps: the practical ceiling of a kernel that reads and writes HBM."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    times.sort()
    return 2.0 * nbytes / (times[len(times) // 2] * 1e-3) / 1e9


# ---------------------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a lane sample
# ---------------------------------------------------------------------------------------
_CPU = {}


def _cpu_block(args):
    from threadpoolctl import threadpool_limits
    import numpy as np
    from oracle import slstm_ref as ref
    b, j0, j1 = args
    w = _CPU["w"]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if "x" in _CPU:
            x = _CPU["x"][b:b + 1].astype(np.float64)
            P = ref.input_projection(x, _CPU["W"][:, j0:j1], _CPU["bias"][:, j0:j1])
        else:
            P = _CPU["P"][b:b + 1, :, :, j0:j1]
        t1 = time.perf_counter()
        _, st = ref.newton(P, _CPU["R"][:, j0:j1], None, w.forget, w.max_iters, tol=w.tol)
        t2 = time.perf_counter()
        ref.sequential(P, _CPU["R"][:, j0:j1], None, w.forget)
        t3 = time.perf_counter()
    # per block: projection, Newton and sequential seconds
    return t1 - t0, t2 - t1, t3 - t2


def cpu_baseline(w, host, lanes_wanted):
    import multiprocessing as mp
    import numpy as np
    import torch
    workers = max(1, min(16, os.cpu_count() or 1))
    block = 256
    per_b = w.d_h // block if w.d_h >= block else 1
    blk = min(block, w.d_h)
    tasks = []
    for b in range(w.B):
        for k in range(per_b):
            tasks.append((b, k * blk, (k + 1) * blk))
            if len(tasks) * blk >= lanes_wanted:
                break
        if len(tasks) * blk >= lanes_wanted:
            break
    n_lanes = len(tasks) * blk
    _CPU.clear()
    _CPU["w"] = w
    _CPU["R"] = host["R"].double().numpy()
    if "x" in host:
        rows = sorted({t[0] for t in tasks})
        xs = np.zeros((w.B, w.T, w.d_in), dtype=np.float32)
        xs[rows] = host["x"][rows].float().numpy()
        _CPU["x"] = xs
        _CPU["W"] = host["W"].double().numpy()
        _CPU["bias"] = host["bias"].double().numpy()
    else:
        _CPU["P"] = host["P"].double().numpy()
    ctx = mp.get_context("fork")
    n_proc = min(workers, len(tasks))
    with ctx.Pool(processes=n_proc) as pool:
        parts = pool.map(_cpu_block, tasks, chunksize=1)
    _CPU.clear()
    # every process works through its blocks one after another: the wall time of each leg is
    # its summed process time spread over the processes
    t_proj = sum(p[0] for p in parts) / n_proc
    t_newton = sum(p[1] for p in parts) / n_proc
    t_seq = sum(p[2] for p in parts) / n_proc
    elems = n_lanes * w.T
    proj = "input projection + " if "x" in host else ""
    dt = t_proj + t_newton
    return {"value": elems / dt, "unit": "state-elems/s", "cores": n_proc, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n_lanes} of {w.lanes} lanes (b, j) x full T={w.T}: float64 {proj}Newton "
                      f"K={w.max_iters}{' tol=%g' % w.tol if w.tol > 0 else ''}, {elems} state elements, "
                      f"{dt:.2f} s on {n_proc} single-threaded processes",
            "newton_only": {"value": elems / t_newton, "unit": "state-elems/s"},
            "sequential": {"value": elems / t_seq, "unit": "state-elems/s",
                           "sample": f"the float64 step loop on the same lanes, {t_seq:.2f} s"}}


# ---------------------------------------------------------------------------------------
def head_context(slstm, torch, dev, steps):
    """Head mixing: the Newton solve (one sweep over T with the warm start and K pipelined
    iterations, no early stop), the per-head sequential forward and the backward at the
    solution, on one seeded input."""
    from workloads import draw_head_inputs
    B, T, d, nh, K = HEAD["B"], HEAD["T"], HEAD["d"], HEAD["n_heads"], HEAD["K"]
    dh = d // nh
    inp = draw_head_inputs(HEAD["seed"], B, T, d, nh)
    P, R = inp["P"].to(dev), inp["R"].to(dev)
    S = torch.empty((B, T, 4, d), dtype=torch.float32, device=dev)
    H = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    ws = slstm.alloc_workspace(slstm.head_newton_workspace_bytes(B, T, d, nh), dev)

    def solve():
        slstm.head_newton_forward(P, R, None, HEAD["forget"], K, 0.0, "warm", states=S, h_out=H, workspace=ws,
                                  stats=False)

    solve()
    slstm.head_sequential_forward(P, R, None, HEAD["forget"], states=S, h_out=H)  # first launches load code
    torch.cuda.synchronize()
    st = slstm.read_stats(ws)
    reps = max(3, steps // 2)
    slstm.profile_reset()
    slstm.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(reps):
        solve()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / reps
    for _ in range(reps):
        slstm.head_sequential_forward(P, R, None, HEAD["forget"], states=S, h_out=H)
    torch.cuda.synchronize()
    slstm.profile_enable(False)
    sv = slstm.profile_durations("head_solve")
    sq = slstm.profile_durations("head_sequential")
    sv_ms, sq_ms = sum(sv) / len(sv), sum(sq) / len(sq)
    n_e = B * T * d
    sv_bytes = n_e * (16 + 16 + 4)            # P in; S_K, h out
    sv_flops = n_e * head_solve_flops_per_elem(dh, K, HEAD["forget"] == "sigmoid")
    gbs, tfs = sv_bytes / (sv_ms * 1e-3) / 1e9, sv_flops / (sv_ms * 1e-3) / 1e12
    log(f"[bench] head mixing ({nh} heads of {dh}): solve {ms:.3f} ms, one-sweep kernel {sv_ms:.3f} ms "
        f"({sv_ms * 1e3 / T:.3f} us per step), sequential {sq_ms:.3f} ms")
    # the backward at the solution for a loss on h (dL/dh ~ N(0, 1) and a final-state gradient):
    # bf16 dP, dR per head, dbias, dstate0
    from workloads import random_cotangents_device
    _, g_h, g_fin = random_cotangents_device(HEAD["seed"] + 99, B, T, d, dev)
    dP = torch.empty((B, T, 4, d), dtype=torch.bfloat16, device=dev)
    bws = slstm.alloc_workspace(slstm.head_backward_workspace_bytes(B, T, d, nh), dev)

    def bwd():
        slstm.head_backward(P, R, S, None, None, g_h, g_fin, HEAD["forget"], dP=dP, workspace=bws, want_dbias=True)

    bwd()
    torch.cuda.synchronize()
    slstm.profile_reset()
    slstm.profile_enable(True)
    for _ in range(reps):
        bwd()
    torch.cuda.synchronize()
    slstm.profile_enable(False)
    bw = slstm.profile_durations("head_backward")
    bw_ms = sum(bw) / len(bw)
    bw_bytes = n_e * (16 + 16 + 4 + 8)        # P, S, dL/dh in; bf16 dP out
    bw_gbs = bw_bytes / (bw_ms * 1e-3) / 1e9
    log(f"[bench] head mixing backward: {bw_ms:.3f} ms ({bw_ms * 1e3 / T:.3f} us per step), "
        f"{bw_gbs:.0f} GB/s algorithmic")
    del ws, S, H, P, R, dP, bws, g_h, g_fin
    torch.cuda.empty_cache()
    return {
        "B": B, "T": T, "d_h": d, "n_heads": nh, "d_head": dh, "forget_gate": HEAD["forget"], "newton_iters": K,
        "preactivations": "f32", "solve_ms": round(ms, 4), "state_elems_per_s": n_e / (ms * 1e-3),
        "solver": {"iters": st.iters, "max_abs_F": st.max_abs_F[-1], "diverged": st.diverged},
        "form": "one sweep (warm start, K iterations and the final residual pipelined along T, one wave group each)",
        "kernels": {"head_solve": {"avg_ms": round(sv_ms, 4), "us_per_step": round(sv_ms * 1e3 / T, 4),
                                   "bytes_per_launch": sv_bytes, "flops_per_launch": sv_flops},
                    "head_sequential": {"avg_ms": round(sq_ms, 4), "us_per_step": round(sq_ms * 1e3 / T, 4),
                                        "state_elems_per_s": n_e / (sq_ms * 1e-3)},
                    "head_backward": {"avg_ms": round(bw_ms, 4), "us_per_step": round(bw_ms * 1e3 / T, 4),
                                      "gradients_in": "dL/dh, dL/d final state", "dP": "bf16",
                                      "bytes_per_launch": bw_bytes, "hbm_view": {"achieved": round(bw_gbs, 1),
                                                                                  "peak": HBM_PEAK_GBS,
                                                                                  "unit": "GB/s",
                                                                                  "frac": round(bw_gbs / HBM_PEAK_GBS, 4)}}},
        "roofline": {"bound": "latency", "kernel": "head_solve",
                     "note": "one workgroup per (batch row, head) walks T, its stages a tick apart on separate wave groups; the tick's chain and the CU's issue rate bound it",
                     "hbm_view": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)},
                     "alu_view": {"achieved": round(tfs, 2), "peak": FP32_UNPACKED_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tfs / FP32_UNPACKED_PEAK_TFLOPS, 4)},
                     "traffic": measured_traffic("head_solve", HEAD_WORKLOAD)}}


def solver_context(slstm, torch, dev, name, steps, cpu_lanes, no_cpu):
    """One of the workloads whose solver input is P, at its full size, in the schedule the
    library picks for its shape: state-elems/s of the Newton solve, the iteration kernel's HBM
    fraction, the solver's outcome and the float64 oracle on a lane sample. Not the metric."""
    from workloads import by_name, draw_preactivation_inputs
    w = by_name(name)
    t_gen = time.perf_counter()
    host = draw_preactivation_inputs(w, device=dev)
    P = host["P"].to(dev)
    R = host["R"].to(dev)
    log(f"[bench] context {name}: inputs ready in {time.perf_counter() - t_gen:.1f} s")
    p_bytes = 8 if w.p_dtype == "bf16" else 16
    n_e = w.state_elems
    # the library runs a fixed-count solve (K <= 4) on 32 or more lane groups of 256 features
    # as one kernel, and an early stop (K <= 8) as two passes of it; neither needs a state
    # tensor: the layer's default output, h and the final state
    one_kernel = (w.max_iters <= 4 if w.tol == 0.0 else w.max_iters <= 8) and w.B * -(-w.d_h // 256) >= 32
    S = None if one_kernel else torch.empty((w.B, w.T, 4, w.d_h), dtype=torch.float32, device=dev)
    H = torch.empty((w.B, w.T, w.d_h), dtype=torch.float32, device=dev)
    FS = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=dev)
    ws = slstm.alloc_workspace(slstm.newton_workspace_bytes(w.B, w.T, w.d_h, "fused"), dev)

    def solve():
        slstm.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, "warm", states=S, h_out=H, final_state=FS,
                             workspace=ws, stats=False, schedule="fused", output_states=not one_kernel)

    solve()
    torch.cuda.synchronize()
    st = slstm.read_stats(ws)
    reps = max(3, steps // 2)
    t0 = time.perf_counter()
    for _ in range(reps):
        solve()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / reps
    slstm.profile_reset()
    slstm.profile_enable(True)
    for _ in range(reps):
        solve()
    torch.cuda.synchronize()
    slstm.profile_enable(False)
    bytes_of = {"warm_start": n_e * (p_bytes + 16), "newton_iteration": n_e * (p_bytes + 32),
                "final_residual": n_e * (p_bytes + 16 + 4),
                "newton_solve": n_e * (p_bytes + (0 if one_kernel else 16) + 4)}
    kernels = {}
    for kind, nb in bytes_of.items():
        d = slstm.profile_durations(kind)
        if d:
            avg = sum(d) / len(d)
            kernels[kind] = {"launches_per_solve": len(d) // reps, "avg_ms": round(avg, 4),
                             "bytes_per_launch": nb, "GB_s": round(nb / (avg * 1e-3) / 1e9, 1)}
    it = kernels.get("newton_iteration")
    log(f"[bench] context {name}: solve {ms:.3f} ms ({n_e / (ms * 1e-3):.3e} state-elems/s), iters {st.iters}, "
        f"converged {st.converged}, iteration kernel {it['avg_ms'] if it else float('nan'):.3f} ms")
    out = {"B": w.B, "T": w.T, "d_h": w.d_h, "preactivations": w.p_dtype, "forget_gate": w.forget,
           "max_iters": w.max_iters, "tol": w.tol,
           "schedule": ("fused (scan form at this shape)" if not one_kernel else
                        "fused (one-kernel form at this shape)" if w.tol == 0.0 else
                        "fused (one-kernel form at this shape: the budget, the stop test, then the count it chose)"),
           "outputs": "hidden slot and final state" if one_kernel else "states, hidden slot",
           "solve_ms": round(ms, 4), "state_elems_per_s": n_e / (ms * 1e-3),
           "solver": {"iters": st.iters, "converged": st.converged, "diverged": st.diverged,
                      "max_abs_F": st.max_abs_F},
           "kernels": kernels}
    if it:
        out["roofline"] = {"bound": "hbm", "kernel": "newton_iteration", "achieved": it["GB_s"],
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(it["GB_s"] / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("newton_iteration", w.name)}
    sv = kernels.get("newton_solve")
    if sv:
        # few lane groups: the wavefront along T waits on each tile's predecessor in turn; the
        # library's tiles are 15 steps where the lane groups cover the CUs, 24 otherwise
        n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
        n_tt = -(-w.T // (15 if w.B * -(-w.d_h // 256) >= n_cus else 24))
        out["roofline"] = {"bound": "latency", "kernel": "newton_solve", "achieved": sv["GB_s"],
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(sv["GB_s"] / HBM_PEAK_GBS, 4),
                           "tiles_along_T": n_tt, "us_per_tile": round(sv["avg_ms"] * 1e3 / n_tt, 3),
                           "traffic": measured_traffic("newton_solve", w.name)}
    del ws, S, H, FS, P, R
    torch.cuda.empty_cache()
    if not no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, {"P": host["P"], "R": host["R"]}, cpu_lanes)
        log(f"[bench] context {name}: CPU oracle {out['cpu_baseline']['value']:.3e} state-elems/s")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="layer_b128_t2048_d1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-lanes", type=int, default=40960)
    ap.add_argument("--no-copy-bandwidth", action="store_true",
                    help="skip the device-copy bandwidth measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain device copy of 4 GiB (counter calibration runs)")
    ap.add_argument("--no-sequential-context", action="store_true")
    ap.add_argument("--schedule", default="fused", choices=["fused", "fused_scan", "fused_chain", "layered"])
    ap.add_argument("--outputs", default="hidden", choices=["hidden", "states"],
                    help="what the timed forward writes: the layer's default output, the hidden slot and "
                         "the final state (where the solve is the one-kernel form; other forms also write "
                         "the states they iterate on), or the full states beside them")
    ap.add_argument("--no-layered-context", action="store_true",
                    help="skip the context runs of the scan form and the layered schedule")
    ap.add_argument("--no-backward-context", action="store_true",
                    help="skip the context run of the backward pass at the forward solution")
    ap.add_argument("--no-packed-context", action="store_true",
                    help="skip the context run on the same tokens packed as ragged sequences")
    ap.add_argument("--no-head-context", action="store_true",
                    help="skip the context run of head mixing (block-diagonal R)")
    ap.add_argument("--no-workload-contexts", action="store_true",
                    help="skip the sigmoid/bf16 and long-context workloads at their full sizes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library runs the whole Newton solve on a single "
              f"MI355X (requested --gpus {args.gpus}, WORLD_SIZE {world}); it has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_nets_amd import slstm
    from workloads import by_name, draw_decode_inputs, draw_layer_inputs, draw_preactivation_inputs

    w = by_name(args.workload)
    dev = torch.device("cuda:0")
    slstm.load()
    log(f"[bench] workload {w.name}: generating inputs")
    t_gen = time.perf_counter()
    if w.on_gpu_gemm:
        host = draw_layer_inputs(w)
        x = host["x"].to(dev)
        W = host["W"].to(dev)
        bias = host["bias"].to(dev)
        R = host["R"].to(dev)
        P = torch.empty((w.B, w.T, 4, w.d_h), dtype=torch.float32, device=dev)
        x_dec = draw_decode_inputs(w).to(dev)
        P_dec = torch.empty((w.decode_batch, 1, 4, w.d_h), dtype=torch.float32, device=dev)
        S_dec = torch.empty((w.decode_batch, 1, 4, w.d_h), dtype=torch.float32, device=dev)
        H_dec = torch.empty((w.decode_batch, 1, w.d_h), dtype=torch.float32, device=dev)
        p_bytes = 16
    else:
        host = draw_preactivation_inputs(w)
        P = host["P"].to(dev)
        R = host["R"].to(dev)
        p_bytes = 8 if w.p_dtype == "bf16" else 16
    log(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s")
    S = torch.empty((w.B, w.T, 4, w.d_h), dtype=torch.float32, device=dev)
    H = torch.empty((w.B, w.T, w.d_h), dtype=torch.float32, device=dev)
    FS = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=dev)

    if args.copy_calibration:
        src = torch.empty(2**30, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 copies of 4 GiB done")

    n_e = w.state_elems
    work = kernel_work(w, n_e, p_bytes)
    n_cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def one_kernel_form(schedule):
        """Whether the solve resolves to the one-kernel form, which needs no state tensor: under
        fused_chain a fixed count up to 4; under fused up to 8 iterations (an early stop in two
        passes) on 32 or more lane groups of 256 features."""
        lanes = w.B * -(-w.d_h // 256)
        if schedule == "fused_chain":
            return w.tol == 0.0 and w.max_iters <= 4
        return schedule == "fused" and w.max_iters <= 8 and lanes >= 32

    def timed_run(schedule, steps, warmup, states_out=None):
        if states_out is None:
            states_out = args.outputs == "states" or not one_kernel_form(schedule)
        run_work = kernel_work(w, n_e, p_bytes, states_out)
        ws = slstm.alloc_workspace(slstm.newton_workspace_bytes(w.B, w.T, w.d_h, schedule), dev)

        def step():
            if w.on_gpu_gemm:
                slstm.input_projection(x, W, bias, out=P)
            slstm.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, "warm", states=S if states_out else None,
                                 h_out=H, final_state=FS, workspace=ws, stats=False, schedule=schedule,
                                 output_states=states_out)
            if w.on_gpu_gemm:
                slstm.input_projection(x_dec, W, bias, out=P_dec)
                slstm.sequential_forward(P_dec, R, FS, w.forget, states=S_dec, h_out=H_dec)

        for i in range(warmup):
            step()
            torch.cuda.synchronize()
            log(f"[bench] {schedule}: warm-up step {i + 1}/{warmup} done")
        st = slstm.read_stats(ws)
        log(f"[bench] {schedule}: solver iters {st.iters}, max|F| {['%.2e' % e for e in st.max_abs_F]}, "
            f"diverged {st.diverged}; device memory {torch.cuda.memory_allocated() / 2**30:.1f} GiB")
        torch.cuda.synchronize()
        # the metric: exactly `steps` steps between two synchronisations, nothing recorded
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1000.0 / steps
        log(f"[bench] {schedule}: {steps} timed steps, {ms:.3f} ms/step")
        # then the same number of steps again with the library's kernel events and one event
        # pair per step on the stream: per-kernel durations and the spread of step times
        slstm.profile_reset()
        slstm.profile_enable(True)
        evs = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        slstm.profile_enable(False)
        step_ms = sorted(a.elapsed_time(b) for a, b in evs)
        spread = {"median_ms": round(step_ms[len(step_ms) // 2], 4), "min_ms": round(step_ms[0], 4),
                  "max_ms": round(step_ms[-1], 4), "steps": steps, "timing": "HIP events per step, second pass"}
        kernels = {"_work": run_work, "_states_out": states_out}
        for kind, wk in run_work.items():
            d = slstm.profile_durations(kind)
            if not d:
                continue
            avg = sum(d) / len(d)
            kernels[kind] = {"launches": len(d), "avg_ms": avg, "total_ms_per_step": sum(d) / steps,
                             "bytes_per_launch": wk["bytes"], "GB_s": wk["bytes"] / (avg * 1e-3) / 1e9}
            if "flops" in wk:
                kernels[kind]["flops_per_launch"] = wk["flops"]
                kernels[kind]["TFLOP_s"] = wk["flops"] / (avg * 1e-3) / 1e12
        if w.on_gpu_gemm:
            d = slstm.profile_durations("input_projection")
            big = d[0::2]
            small = d[1::2]
            M, N, K = w.B * w.T, 4 * w.d_h, w.d_in
            flops = 2.0 * M * N * K
            avg = sum(big) / len(big)
            kernels["input_projection"] = {"launches": len(big), "avg_ms": avg,
                                           "total_ms_per_step": sum(big) / steps,
                                           "flops_per_launch": flops,
                                           "bytes_per_launch": M * K * 2 + N * K * 2 + M * N * 4,
                                           "TFLOP_s": flops / (avg * 1e-3) / 1e12}
            seqd = slstm.profile_durations("sequential")
            kernels["decode"] = {"launches": len(seqd) + len(small),
                                 "total_ms_per_step": (sum(seqd) + sum(small)) / steps}
        del ws
        torch.cuda.empty_cache()
        kernels["_spread"] = spread
        return ms, kernels, st

    def roofline_of(kernels, steps, ms):
        work = kernels["_work"]
        dominant = max((k for k in kernels if (k in work or k == "input_projection") and not k.startswith("_")),
                       key=lambda k: kernels[k]["total_ms_per_step"])
        k = kernels[dominant]
        if dominant == "input_projection":
            roof = {"bound": "mfma", "kernel": dominant, "achieved": round(k["TFLOP_s"], 1),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(k["TFLOP_s"] / BF16_PEAK_TFLOPS, 4)}
        else:
            roof = {"bound": "hbm", "kernel": dominant, "achieved": round(k["GB_s"], 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(k["GB_s"] / HBM_PEAK_GBS, 4)}
            if copy_gbs:
                roof["copy_ceiling"] = {"achieved": round(copy_gbs, 1), "unit": "GB/s",
                                        "frac_of_copy": round(k["GB_s"] / copy_gbs, 4)}
            if "TFLOP_s" in k:
                # the kernel's arithmetic beside its bytes: flops against the ceiling of the build
                # (no packed fp32), and the share of vector issue its instructions fill; the roof
                # nearer to its peak is the bound, the other its view
                alu = {"achieved": round(k["TFLOP_s"], 2), "peak": FP32_UNPACKED_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(k["TFLOP_s"] / FP32_UNPACKED_PEAK_TFLOPS, 4)}
                if alu["frac"] > roof["frac"]:
                    hbm_view = {kk: roof[kk] for kk in ("achieved", "peak", "unit", "frac", "copy_ceiling") if kk in roof}
                    roof = {"bound": "alu", "kernel": dominant, **alu, "hbm_view": hbm_view}
                else:
                    roof["alu_view"] = alu
            # the one-kernel solve's counters are recorded apart for the step that writes the states
            rec = dominant + ("_states" if dominant == "newton_solve" and kernels.get("_states_out") else "")
            insts = measured_valu(rec, w.name)
            if insts:
                roof["valu_issue"] = {"valu_insts_per_launch": insts,
                                      "frac": round(valu_issue_frac(insts, k["avg_ms"]), 4),
                                      "source": "profiles/valu.json (rocprofv3 SQ_INSTS_VALU)"}
        rec = dominant + ("_states" if dominant == "newton_solve" and kernels.get("_states_out") else "")
        roof["traffic"] = measured_traffic(rec, w.name)
        # whole-step roofline: every kernel at its own bound
        t_roof = 0.0
        for kind, kk in kernels.items():
            if kind.startswith("_"):
                continue
            per_step = kk["launches"] / steps
            if kind == "input_projection":
                t_roof += per_step * max(kk["flops_per_launch"] / (BF16_PEAK_TFLOPS * 1e12),
                                         kk["bytes_per_launch"] / (HBM_PEAK_GBS * 1e9))
            elif kind in work:
                wk = work[kind]
                t = wk["bytes"] / (HBM_PEAK_GBS * 1e9)
                if "flops" in wk:
                    t = max(t, wk["flops"] / (FP32_UNPACKED_PEAK_TFLOPS * 1e12))
                t_roof += per_step * t
        return roof, t_roof / (ms * 1e-3)

    def rounded(kernels):
        return {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                for k, v in kernels.items() if not k.startswith("_")}

    copy_gbs = None
    if not args.no_copy_bandwidth:
        copy_gbs = copy_bandwidth(torch, dev)
        log(f"[bench] device copy of 4 GiB: {copy_gbs:.0f} GB/s (read + write)")

    ms_per_step, kernels, st = timed_run(args.schedule, args.steps, args.warmup)
    roofline, step_frac = roofline_of(kernels, args.steps, ms_per_step)
    value = n_e / (ms_per_step * 1e-3)
    context = {"schedule": args.schedule, "step_roofline_frac": round(step_frac, 4),
               "step_time": kernels["_spread"], "copy_GB_s": round(copy_gbs, 1) if copy_gbs else None,
               "kernels": rounded(kernels),
               "solver": {"iters": st.iters, "max_abs_F": st.max_abs_F, "diverged": st.diverged}}
    if not kernels["_states_out"]:
        # the same step writing the full states beside the hidden slot (output_hidden=False on
        # the pages' layer)
        fsteps = max(2, args.steps // 2)
        fms, fkernels, _ = timed_run(args.schedule, fsteps, 1, states_out=True)
        froof, _ = roofline_of(fkernels, fsteps, fms)
        context["full_states"] = {"ms_per_step": round(fms, 4), "state_elems_per_s": n_e / (fms * 1e-3),
                                  "roofline": froof, "kernels": rounded(fkernels)}
    if w.on_gpu_gemm:
        gk = kernels["input_projection"]
        context["gemm"] = {"TFLOP_s": round(gk["TFLOP_s"], 1), "peak": BF16_PEAK_TFLOPS,
                           "frac": round(gk["TFLOP_s"] / BF16_PEAK_TFLOPS, 4),
                           "traffic": measured_traffic("input_projection", w.name)}
    if not args.no_layered_context and args.schedule not in ("layered", "fused_scan"):
        # the scan form of the fused iteration: residual, Jacobian, 4x4 affine scan with look-back
        # and update in one kernel per iteration
        ssteps = max(2, args.steps // 2)
        sms, skernels, _ = timed_run("fused_scan", ssteps, 1)
        sroof, _ = roofline_of(skernels, ssteps, sms)
        context["fused_scan"] = {"ms_per_step": round(sms, 4), "state_elems_per_s": n_e / (sms * 1e-3),
                                 "roofline": sroof, "kernels": rounded(skernels)}
    if not args.no_layered_context and args.schedule != "layered":
        # the layered schedule: kernels (a) residual + Jacobian, (b) scan, (c) update
        lsteps = max(2, args.steps // 2)
        lms, lkernels, _ = timed_run("layered", lsteps, 1)
        lroof, _ = roofline_of(lkernels, lsteps, lms)
        a, b = lkernels["residual_jacobian"], lkernels["scan_block4"]
        ab_gbs = (a["bytes_per_launch"] + b["bytes_per_launch"]) / ((a["avg_ms"] + b["avg_ms"]) * 1e-3) / 1e9
        context["layered"] = {"ms_per_step": round(lms, 4), "state_elems_per_s": n_e / (lms * 1e-3),
                              "roofline": lroof,
                              "residual_plus_scan": {"achieved": round(ab_gbs, 1), "peak": HBM_PEAK_GBS,
                                                     "unit": "GB/s", "frac": round(ab_gbs / HBM_PEAK_GBS, 4),
                                                     "frac_of_copy": round(ab_gbs / copy_gbs, 4) if copy_gbs else None,
                                                     "traffic": {k: measured_traffic(k, w.name)
                                                                 for k in ("residual_jacobian", "scan_block4", "update")}},
                              "kernels": rounded(lkernels)}

    if not args.no_backward_context:
        # the backward pass at the forward solution for a loss on h (dL/dh ~ N(0, 1) and a
        # final-state gradient): dP (bf16), dR, dbias, dstate0, and for the full layer dW_x and
        # dx from the input projection's backward; not part of the metric
        from workloads import random_cotangents_device
        _, g_h, g_fin = random_cotangents_device(w.seed + 99, w.B, w.T, w.d_h, dev)
        dP = torch.empty((w.B, w.T, 4, w.d_h), dtype=torch.bfloat16, device=dev)
        dR = torch.empty((4, w.d_h), dtype=torch.float32, device=dev)
        db = torch.empty((4, w.d_h), dtype=torch.float32, device=dev)
        d0 = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=dev)
        bws = slstm.alloc_workspace(slstm.backward_workspace_bytes(w.B, w.T, w.d_h), dev)
        if w.on_gpu_gemm:
            dx = torch.empty((w.B, w.T, w.d_in), dtype=torch.float32, device=dev)
            dW = torch.empty((4, w.d_h, w.d_in), dtype=torch.float32, device=dev)
            pws = slstm.alloc_workspace(slstm.input_projection_backward_workspace_bytes(w.B, w.T, w.d_in, w.d_h), dev)

        # the states of the forward solution, which the backward reads
        if w.on_gpu_gemm:
            slstm.input_projection(x, W, bias, out=P)
        slstm.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, "warm", states=S, h_out=H,
                             final_state=FS, stats=False)

        def bwd():
            slstm.backward(P, R, S, None, None, g_h, g_fin, w.forget, dP=dP, dR=dR, dstate0=d0, dbias=db,
                           workspace=bws)
            if w.on_gpu_gemm:
                slstm.input_projection_backward(x, W, dP, dx=dx, dW=dW, workspace=pws)

        bwd()
        torch.cuda.synchronize()
        reps = max(3, args.steps // 2)
        slstm.profile_reset()
        slstm.profile_enable(True)
        tb = time.perf_counter()
        for _ in range(reps):
            bwd()
        torch.cuda.synchronize()
        b_ms = (time.perf_counter() - tb) * 1000.0 / reps
        slstm.profile_enable(False)
        bd = slstm.profile_durations("backward")
        bk = sum(bd) / len(bd)
        gbs = work["backward"]["bytes"] / (bk * 1e-3) / 1e9
        log(f"[bench] backward: {b_ms:.3f} ms per call, recurrence kernels {bk:.3f} ms, {gbs:.0f} GB/s algorithmic")
        context["backward"] = {"ms": round(b_ms, 4), "state_elems_per_s": n_e / (b_ms * 1e-3),
                               "gradients_in": "dL/dh, dL/d final state", "form": "scan",
                               "recurrence": {"kernel_avg_ms": round(bk, 4),
                                              "bytes_per_launch": work["backward"]["bytes"],
                                              "roofline": {"bound": "hbm", "kernel": "backward",
                                                           "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                                           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                                           "traffic": measured_traffic("backward", w.name)}}}
        if w.on_gpu_gemm:
            flops = 2.0 * w.B * w.T * 4 * w.d_h * w.d_in
            for kind in ("weight_gradient", "input_gradient"):
                kd = slstm.profile_durations(kind)
                kavg = sum(kd) / len(kd)
                tf = flops / (kavg * 1e-3) / 1e12
                context["backward"][kind] = {"ms": round(kavg, 4), "flops_per_launch": flops,
                                             "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                                          "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                                          "frac": round(tf / BF16_PEAK_TFLOPS, 4)}}
                log(f"[bench] backward {kind}: {kavg:.3f} ms, {tf:.0f} TFLOP/s (operand transposes included)")
            del dx, dW, pws
        del dP, dR, db, d0, bws, g_h, g_fin
        torch.cuda.empty_cache()

    if not args.no_packed_context:
        # the same B*T tokens as ragged sequences packed end to end in one row (cu_seqlens:
        # log-uniform lengths up to 8192 steps with empty and length-1 sequences mixed in), each
        # from a zero state: the Newton solve (the one-kernel form on tiles aligned to the
        # sequences, and the scan form) and the backward, not the metric
        from workloads import packed_offsets, random_cotangents_device
        cu_host = packed_offsets(w.seed, w.B * w.T, 8192)
        n_seq = len(cu_host) - 1
        cu = torch.as_tensor(cu_host, dtype=torch.int32, device=dev)
        BT = w.B * w.T
        Pp, Sp, Hp = P.view(1, BT, 4, w.d_h), S.view(1, BT, 4, w.d_h), H.view(1, BT, w.d_h)
        fin = torch.empty((n_seq, 4, w.d_h), dtype=torch.float32, device=dev)
        pws = slstm.alloc_workspace(slstm.newton_workspace_bytes(1, BT, w.d_h, "fused"), dev)
        reps = max(3, args.steps // 2)

        def time_packed(schedule):
            def fwd():
                slstm.newton_forward(Pp, R, None, w.forget, w.max_iters, w.tol, "warm", states=Sp, h_out=Hp,
                                     final_state=fin, workspace=pws, stats=False, cu_seqlens=cu, schedule=schedule)
            fwd()
            torch.cuda.synchronize()
            stp = slstm.read_stats(pws)
            slstm.profile_reset()
            slstm.profile_enable(True)
            tp = time.perf_counter()
            for _ in range(reps):
                fwd()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - tp) * 1000.0 / reps
            slstm.profile_enable(False)
            kk = {}
            for kind in ("newton_solve", "warm_start", "newton_iteration", "final_residual"):
                d = slstm.profile_durations(kind)
                if d:
                    avg = sum(d) / len(d)
                    nb = work["newton_solve" if kind == "newton_solve" else kind]["bytes"]
                    kk[kind] = {"launches_per_solve": len(d) // reps, "avg_ms": round(avg, 4),
                                "GB_s": round(nb / (avg * 1e-3) / 1e9, 1)}
            return ms, kk, stp

        # the scan form on tiles aligned to the sequences, then the library's choice for a pack
        # this size: the one-kernel solve on aligned tiles (it also writes the states, which the
        # backward below reads)
        s_ms, sk, _ = time_packed("fused_scan")
        p_ms, pk, pst = time_packed("fused")
        sv = pk["newton_solve"]
        it = sk["newton_iteration"]
        log(f"[bench] packed ({n_seq} sequences): solve {p_ms:.3f} ms (one kernel on aligned tiles, "
            f"{sv['GB_s']:.0f} GB/s algorithmic); scan form {s_ms:.3f} ms, iteration kernel {it['avg_ms']:.3f} ms, "
            f"{it['GB_s']:.0f} GB/s algorithmic")
        _, g_hp, _ = random_cotangents_device(w.seed + 98, 1, BT, w.d_h, dev)
        g_fp = torch.randn((n_seq, 4, w.d_h), generator=torch.Generator(device=dev).manual_seed(w.seed + 97),
                           device=dev)
        dPp = torch.empty((1, BT, 4, w.d_h), dtype=torch.bfloat16, device=dev)
        dRp = torch.empty((4, w.d_h), dtype=torch.float32, device=dev)
        d0p = torch.empty((n_seq, 4, w.d_h), dtype=torch.float32, device=dev)
        pbws = slstm.alloc_workspace(slstm.backward_workspace_bytes(1, BT, w.d_h), dev)

        def packed_bwd():
            slstm.backward(Pp, R, Sp, None, None, g_hp, g_fp, w.forget, dP=dPp, dR=dRp, dstate0=d0p,
                           workspace=pbws, cu_seqlens=cu)

        packed_bwd()
        torch.cuda.synchronize()
        slstm.profile_reset()
        slstm.profile_enable(True)
        for _ in range(reps):
            packed_bwd()
        torch.cuda.synchronize()
        slstm.profile_enable(False)
        bd = slstm.profile_durations("backward")
        pb = sum(bd) / len(bd)
        pb_gbs = work["backward"]["bytes"] / (pb * 1e-3) / 1e9
        log(f"[bench] packed backward: recurrence kernels {pb:.3f} ms, {pb_gbs:.0f} GB/s algorithmic")
        context["packed"] = {
            "sequences": n_seq, "tokens": BT, "max_len": int(max(cu_host[1:] - cu_host[:-1])),
            "form": "one kernel on tiles aligned to the sequences", "solve_ms": round(p_ms, 4),
            "state_elems_per_s": n_e / (p_ms * 1e-3),
            "solver": {"iters": pst.iters, "max_abs_F": pst.max_abs_F[-1], "diverged": pst.diverged},
            "kernels": pk,
            "roofline": {"bound": "latency", "kernel": "newton_solve", "achieved": sv["GB_s"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(sv["GB_s"] / HBM_PEAK_GBS, 4),
                         "note": "each sequence's tiles wait on each other along its steps; the longest sequence's chain bounds the solve",
                         "traffic": measured_traffic("packed_solve", w.name)},
            "scan_form": {"solve_ms": round(s_ms, 4), "kernels": sk,
                          "roofline": {"bound": "hbm", "kernel": "newton_iteration", "achieved": it["GB_s"],
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(it["GB_s"] / HBM_PEAK_GBS, 4),
                                       "traffic": measured_traffic("packed_iteration", w.name)}},
            "backward": {"kernel_avg_ms": round(pb, 4), "gradients_in": "dL/dh, dL/d final states",
                         "roofline": {"bound": "hbm", "kernel": "backward", "achieved": round(pb_gbs, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(pb_gbs / HBM_PEAK_GBS, 4),
                                      "traffic": measured_traffic("packed_backward", w.name)}}}
        del pws, pbws, dPp, dRp, d0p, g_hp, g_fp, fin
        torch.cuda.empty_cache()

    if not args.no_head_context:
        context["head"] = head_context(slstm, torch, dev, args.steps)

    if not args.no_workload_contexts and w.on_gpu_gemm:
        # the sigmoid/bf16 workload (early stop) and the long-context workload at full size,
        # where lanes are few and the scan form's parallelism along T carries the solve
        context["workloads"] = {}
        for name, lanes_n in (("sigmoid_bf16p_b16_t4096_d1024", 4096), ("long_b4_t16384_d2048", 1024)):
            context["workloads"][name] = solver_context(slstm, torch, dev, name, args.steps, lanes_n,
                                                        args.no_cpu_baseline)

    if not args.no_sequential_context:
        # the lane-parallel sequential forward on the same P, for context (not the metric): the
        # layer's default output (h and the final state) like the timed step, then with the states
        def seq_ms_of(states_out):
            run = lambda: slstm.sequential_forward(P, R, None, w.forget, states=S if states_out else None,  # noqa: E731
                                                   h_out=H, final_state=FS, output_states=states_out)
            run()
            torch.cuda.synchronize()
            reps = 5
            ts = time.perf_counter()
            for _ in range(reps):
                run()
            torch.cuda.synchronize()
            return (time.perf_counter() - ts) * 1000.0 / reps
        seq_ms = seq_ms_of(False)
        seq_ms_states = seq_ms_of(True)
        context["sequential_forward"] = {"ms": round(seq_ms, 3), "state_elems_per_s": n_e / (seq_ms * 1e-3),
                                         "outputs": "hidden slot and final state",
                                         "with_states": {"ms": round(seq_ms_states, 3),
                                                         "state_elems_per_s": n_e / (seq_ms_states * 1e-3)}}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: float64 oracle on {args.cpu_lanes} lanes")
        cpu = cpu_baseline(w, host, args.cpu_lanes)
        log(f"[bench] CPU baseline: {cpu['value']:.3e} state-elems/s on {cpu['cores']} cores")

    config = {"workload": w.name, "B": w.B, "T": w.T, "d_in": w.d_in, "d_h": w.d_h,
              "newton_iters": w.max_iters, "tol": w.tol, "forget_gate": w.forget,
              "preactivations": ("bf16 x, W_x -> float32 P on MFMA" if w.on_gpu_gemm else w.p_dtype),
              "decode_batch": w.decode_batch, "init": "warm", "state_dtype": "f32",
              "outputs": ("states (B,T,4,d_h), hidden slot (B,T,d_h), final state" if kernels["_states_out"]
                          else "hidden slot (B,T,d_h) and final state (the layer's default output)")}
    line = {"metric": METRIC, "value": value, "unit": "state-elems/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded; shapes and distributions of the workload)",
            "config": config, "roofline": roofline, "cpu_baseline": cpu, "context": context}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
