"""Run the float64 oracle over lane subsets, optionally in parallel processes.

TEST INFRASTRUCTURE (same rule as ``oracle.slstm_ref``: only the tests, the smoke check and
the benchmark's CPU-baseline leg use it).

Under channelwise mixing (mix='diag', "sLSTM in this library", section "Cell") every
(batch b, feature j) pair is an independent recurrence, so the oracle can be run on any set
of lanes and its per-lane results are exactly those of the full problem. The only coupling
across lanes is the early-stop decision, which uses the maximum of |F| over all lanes; it is
reproduced here by first collecting each lane block's residual history with a fixed
iteration count and then taking the per-iteration maximum.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from . import slstm_ref as ref

_SHARED = {}


def as_f64(a):
    """torch tensor (any float dtype) or array -> float64 numpy array."""
    if hasattr(a, "detach"):
        import torch
        return a.detach().cpu().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def lane_subproblem(P, R, state0, lane_b, lane_j):
    """Gather lanes (lane_b[k], lane_j[k]) into a B=1 problem with d = len(lanes)."""
    lane_b = np.asarray(lane_b)
    lane_j = np.asarray(lane_j)
    Ps = P[lane_b, :, :, lane_j]            # (n, T, 4)
    Ps = np.transpose(Ps, (1, 2, 0))[None]  # (1, T, 4, n)
    Rs = R[:, lane_j]
    s0 = None if state0 is None else np.transpose(state0[lane_b, :, lane_j], (1, 0))[None]
    return np.ascontiguousarray(Ps), np.ascontiguousarray(Rs), s0


def scatter_states(S_sub):
    """(1, T, 4, n) sub-problem states -> (n, T, 4) per-lane states."""
    return np.transpose(S_sub[0], (2, 0, 1))


def _newton_block(args):
    lane_b, lane_j, forget, K, init, keep = args
    P, R, state0 = _SHARED["P"], _SHARED["R"], _SHARED["state0"]
    Ps, Rs, s0 = lane_subproblem(P, R, state0, lane_b, lane_j)
    S, st = ref.newton(Ps, Rs, s0, forget, K, tol=0.0, init=init)
    return st.max_abs_F, (scatter_states(S) if keep else None)


def _sequential_block(args):
    lane_b, lane_j, forget = args
    P, R, state0 = _SHARED["P"], _SHARED["R"], _SHARED["state0"]
    Ps, Rs, s0 = lane_subproblem(P, R, state0, lane_b, lane_j)
    return scatter_states(ref.sequential(Ps, Rs, s0, forget))


def default_workers():
    return max(1, min(16, os.cpu_count() or 1))


def _blocks(lane_b, lane_j, block):
    n = len(lane_b)
    return [(lane_b[i:i + block], lane_j[i:i + block]) for i in range(0, n, block)]


def _run(fn, tasks, workers):
    if workers <= 1 or len(tasks) == 1:
        return [fn(t) for t in tasks]
    ctx = mp.get_context("fork")
    with ctx.Pool(processes=min(workers, len(tasks))) as pool:
        return pool.map(fn, tasks, chunksize=1)


def all_lanes(B, d):
    bb, jj = np.meshgrid(np.arange(B), np.arange(d), indexing="ij")
    return bb.reshape(-1), jj.reshape(-1)


def newton_lanes(P, R, state0, forget, max_iters, tol, init=ref.INIT_WARM, lanes=None,
                 history_lanes=None, workers=None, block=512):
    """Oracle Newton on lane subsets.

    P (B, T, 4, d) float64, R (4, d), state0 (B, 4, d) or None.
    lanes          : (lane_b, lane_j) whose final states are returned (default: all lanes)
    history_lanes  : lanes whose residuals decide the early stop and the flags (default:
                     all lanes -- the exact global decision)
    Returns (states (n, T, 4) for ``lanes``, NewtonStats).
    """
    P = as_f64(P)
    R = as_f64(R)
    state0 = None if state0 is None else as_f64(state0)
    B, T, _, d = P.shape
    workers = default_workers() if workers is None else workers
    if lanes is None:
        lanes = all_lanes(B, d)
    if history_lanes is None:
        history_lanes = all_lanes(B, d)
    _SHARED.update(P=P, R=R, state0=state0)
    try:
        # pass 1: residual history of every lane block at a fixed iteration count
        tasks = [(b, j, forget, max_iters, init, False) for b, j in _blocks(*history_lanes, block)]
        hists = [h for h, _ in _run(_newton_block, tasks, workers)]
        glob = [max(h[k] for h in hists) for k in range(max_iters + 1)]
        stop = max_iters
        if tol > 0:
            for k in range(max_iters):
                if glob[k] < tol:
                    stop = k
                    break
        # pass 2: the requested lanes at the decided iteration count
        tasks = [(b, j, forget, stop, init, True) for b, j in _blocks(*lanes, block)]
        outs = [s for _, s in _run(_newton_block, tasks, workers)]
    finally:
        _SHARED.clear()
    st = ref.NewtonStats(iters=stop, max_abs_F=glob[:stop + 1])
    st.converged, st.diverged, st.nonfinite = ref.newton_flags(glob[stop], tol)
    return np.concatenate(outs, axis=0), st


def sequential_lanes(P, R, state0, forget, lanes=None, workers=None, block=2048):
    """Oracle sequential forward on lane subsets -> states (n, T, 4)."""
    P = as_f64(P)
    R = as_f64(R)
    state0 = None if state0 is None else as_f64(state0)
    B, T, _, d = P.shape
    workers = default_workers() if workers is None else workers
    if lanes is None:
        lanes = all_lanes(B, d)
    _SHARED.update(P=P, R=R, state0=state0)
    try:
        tasks = [(b, j, forget) for b, j in _blocks(*lanes, block)]
        outs = _run(_sequential_block, tasks, workers)
    finally:
        _SHARED.clear()
    return np.concatenate(outs, axis=0)
