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


# ---- packed sequences by groups of whole sequences --------------------------------------------
# Packed sequences ("sLSTM in this library", "Packed sequences") are independent problems: each
# starts from its own state0 and nothing crosses a boundary, forward or backward. A long pack is
# therefore cut into runs of whole sequences, each run solved by the oracle as a pack of its own
# in a worker process, and the results laid back end to end (dR summed over the runs). Without
# an early stop the Newton iterates are per lane and per sequence too.

def packed_groups(cu_seqlens, n_groups):
    """Cut S packed sequences into at most n_groups runs (s_begin, s_end) of whole sequences
    with about equal step counts; every run holds at least one step."""
    cu = [int(v) for v in cu_seqlens]
    S, T = len(cu) - 1, cu[-1]
    target = max(1, -(-T // max(1, n_groups)))
    groups, a = [], 0
    for s in range(S):
        if cu[s + 1] - cu[a] >= target:
            groups.append([a, s + 1])
            a = s + 1
    if a < S:
        if groups and cu[S] == cu[a]:
            groups[-1][1] = S    # trailing empty sequences join the run before them
        else:
            groups.append([a, S])
    return [tuple(g) for g in groups]


def _packed_part(s_a, s_b):
    cu = _SHARED["cu"]
    t0, t1 = cu[s_a], cu[s_b]
    state0 = _SHARED["state0"]
    s0 = None if state0 is None else state0[s_a:s_b]
    return t0, t1, np.asarray(cu[s_a:s_b + 1]) - t0, s0


def _packed_sequential_part(args):
    s_a, s_b, forget = args
    t0, t1, cu, s0 = _packed_part(s_a, s_b)
    return ref.sequential(_SHARED["P"][:, t0:t1], _SHARED["R"], s0, forget, cu_seqlens=cu)


def _packed_newton_part(args):
    s_a, s_b, forget, K, init = args
    t0, t1, cu, s0 = _packed_part(s_a, s_b)
    S, st = ref.newton(_SHARED["P"][:, t0:t1], _SHARED["R"], s0, forget, K, tol=0.0, init=init, cu_seqlens=cu)
    return S, st.max_abs_F


def _packed_backward_part(args):
    s_a, s_b, forget = args
    t0, t1, cu, s0 = _packed_part(s_a, s_b)
    gf = _SHARED["g_final"]
    return ref.backward(_SHARED["P"][:, t0:t1], _SHARED["R"], s0, _SHARED["S"][:, t0:t1], _SHARED["g"][:, t0:t1],
                        forget, cu_seqlens=cu, g_final=None if gf is None else gf[s_a:s_b])


def _packed_run(fn, cu_seqlens, extra, workers, **arrays):
    workers = default_workers() if workers is None else workers
    groups = packed_groups(cu_seqlens, 4 * workers)
    _SHARED.update(cu=[int(v) for v in cu_seqlens], **{k: (None if v is None else as_f64(v)) for k, v in arrays.items()})
    try:
        return groups, _run(fn, [(a, b, *extra) for a, b in groups], workers)
    finally:
        _SHARED.clear()


def packed_sequential(P, R, state0, forget, cu_seqlens, workers=None):
    """ref.sequential(P, R, state0, forget, cu_seqlens=...) computed by runs of sequences."""
    _, outs = _packed_run(_packed_sequential_part, cu_seqlens, (forget,), workers, P=P, R=R, state0=state0)
    return np.concatenate(outs, axis=1)


def packed_newton(P, R, state0, forget, max_iters, cu_seqlens, init=ref.INIT_WARM, workers=None):
    """ref.newton(..., tol=0, cu_seqlens=...) (fixed iteration count) computed by runs of
    sequences; max|F| of each iterate is the largest over the runs."""
    _, outs = _packed_run(_packed_newton_part, cu_seqlens, (forget, max_iters, init), workers,
                          P=P, R=R, state0=state0)
    hist = [max(h[k] for _, h in outs) for k in range(max_iters + 1)]
    st = ref.NewtonStats(iters=max_iters, max_abs_F=hist)
    st.converged, st.diverged, st.nonfinite = ref.newton_flags(hist[-1], 0.0)
    return np.concatenate([S for S, _ in outs], axis=1), st


def packed_backward(P, R, state0, S, g, forget, cu_seqlens, g_final=None, workers=None):
    """ref.backward(..., cu_seqlens=..., g_final=...) computed by runs of sequences -> (dP, dR,
    dstate0); dR is the sum of the runs' sums."""
    groups, outs = _packed_run(_packed_backward_part, cu_seqlens, (forget,), workers, P=P, R=R, state0=state0,
                               S=S, g=g, g_final=g_final)
    dP = np.concatenate([o[0] for o in outs], axis=1)
    dR = np.sum([o[1] for o in outs], axis=0)
    dstate0 = np.concatenate([o[2] for o in outs], axis=0)
    return dP, dR, dstate0
