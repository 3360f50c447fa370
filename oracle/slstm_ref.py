"""Float64 CPU oracle for the sLSTM forward (channelwise mix='diag') and its Newton solve.

TEST INFRASTRUCTURE. This module is the parity reference and the CPU baseline. Only the
test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of the
benchmark may import it; the product path (the HIP library and its binding) never does.
It shares no code with the HIP path: nothing here is generated from, or feeds, the kernels.

What it computes, and where each step is stated:

* the cell f -- "xLSTM: Extended Long Short-Term Memory" (summary card), sLSTM step
  pseudocode under "Key equations" (paper section 2.2, appendix A.2); the stabiliser,
  stabilised gates and running-max recurrence from the educational reimplementation page
  ("xLSTM -- a from-scratch, educational reimplementation"), section "Exponential gating +
  the stabilizer (the crux)". Read-out h = o * c / n as in the paper's sLSTM step; the
  floored read-out of the educational page is a declared deviation and is not used.
* channelwise recurrence (mix='diag'): one recurrent weight per gate and feature, R of
  shape (4, d_h), so each feature is an independent 4-state recurrence with a 4x4
  Jacobian -- "sLSTM in this library", section "Cell" (mix table).
* state layout (B, T, 4, d_h) with slots (c, n, m, h), hidden slot 3 -- same section.
* gate order (z, i, f, o) in P, R and W_x -- order of the pre-activations in the paper's
  sLSTM step pseudocode.
* Newton ("Alg. 1"): residual F_t = s_t - f(s_{t-1}), linearise, solve the
  block-bidiagonal system, update; K iterations; the initial state is prepended as s_0;
  residual early stop and the divergence rule max|F| > 1 after K -- "Layout" page
  (pararnn-torch structure), "Current surface (0.17)"; "sLSTM in this library", "API
  notes".
* the block-bidiagonal solve: Delta_1 = -F_1, Delta_t = A_t Delta_{t-1} - F_t, done here by
  plain block forward substitution (a sequential loop), and on tiny inputs by a dense
  LAPACK solve of the assembled system.
* input projection P = W_x x + b ("W_x is a GEMM" -- "sLSTM in this library", "API
  notes"), and its gradients dW_x = dP^T x, dx = dP W_x, dbias = sum of dP.
* packed sequences ("sLSTM in this library", "Packed sequences"): with cu_seqlens (S + 1
  exclusive prefix offsets) the time axis of a (1, N, ...) problem holds S sequences one after
  the other, each started from its own state0[s] (state0 is (S, 4, d)); at a sequence start the
  previous state is that state0 and the step's Jacobian with respect to the state before it is
  zero (the head flag of the segmented scan), so no value crosses a sequence boundary.
* backward ("sLSTM in this library", section "Backward": the adjoint is one reverse scan of
  the transposed Jacobians, then the cell's vector-Jacobian product for the gradients of R
  and W_x): lam_T = g_T, lam_t = g_t + A_{t+1}^T lam_{t+1}; per step the gate Jacobian
  G_t = d s_t / d x~_t gives dP_t = G_t^T lam_t, dR = sum dP_t * h_{t-1}, dstate0 = A_1^T lam_1.
  Written here as a plain reverse loop, and on tiny inputs as a dense LAPACK solve of the
  transposed system.

Readings where the pages are silent (each listed in the design notes):

* initial Newton iterate: the exact trajectory of the cell with the recurrent term
  R * h_{t-1} removed from the pre-activations ("warm start"); a zero iterate is kept as
  an option.
* max tie-break: a >= i_tilde takes the forget branch; the Jacobian uses that branch.
* early stop: stop before solving when max|F| < tol; ``iters`` counts applied updates.

All arithmetic is float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FORGET_EXP = "exp"
FORGET_SIGMOID = "sigmoid"
# A forget-gate name may carry the read-out variant after a slash: "exp/floored",
# "sigmoid/floored" select h = o c / max(|n|, e^{-m}, READOUT_FLOOR) (the educational page,
# "Exponential gating + the stabilizer (the crux)" and "Implementation notes / deviations"
# item 1) instead of the paper's h = o c / n.
FLOORED = "/floored"
READOUT_FLOOR = 1e-6
INIT_WARM = "warm"
INIT_ZERO = "zero"

# slot indices of the state (c, n, m, h) and gate indices of P and R (z, i, f, o)
C, N, M, H = 0, 1, 2, 3
GZ, GI, GF, GO = 0, 1, 2, 3


# ---------------------------------------------------------------------------------------
# scalar nonlinearities (float64, written to stay finite for any finite argument)
# ---------------------------------------------------------------------------------------
def _softplus(x):
    return np.logaddexp(0.0, x)


def sigmoid(x):
    """sigma(x) = 1 / (1 + e^{-x}), computed as exp(-softplus(-x))."""
    return np.exp(-_softplus(-x))


def cell_mode(forget):
    """(forget-gate form, floored read-out?) of a cell-mode name such as "sigmoid/floored"."""
    base, _, variant = forget.partition("/")
    if variant not in ("", "floored"):
        raise ValueError(f"unknown read-out variant {variant!r}")
    return base, variant == "floored"


def log_forget(f_tilde, forget):
    """log f_t and its derivative d log f / d f_tilde.

    Exponential forget gate: log f = f_tilde. Sigmoid forget gate: log f = log sigma(f_tilde)
    = -softplus(-f_tilde), derivative sigma(-f_tilde). Both forms are allowed by the paper
    (summary card, "Method" item 1; the educational page writes the stabiliser in terms of
    log f so it covers both).
    """
    forget, _ = cell_mode(forget)
    if forget == FORGET_EXP:
        return f_tilde, np.ones_like(f_tilde)
    if forget == FORGET_SIGMOID:
        return -_softplus(-f_tilde), sigmoid(-f_tilde)
    raise ValueError(f"unknown forget mode {forget!r}")


# ---------------------------------------------------------------------------------------
# the cell f and its 4x4 Jacobian
# ---------------------------------------------------------------------------------------
def preactivations(prev, p, r):
    """Gate pre-activations x~ = p_x + r_x h' for x in (z, i, f, o) (channelwise R)."""
    h0 = prev[..., H, :]
    zt = p[..., GZ, :] + r[GZ] * h0
    it = p[..., GI, :] + r[GI] * h0
    ft = p[..., GF, :] + r[GF] * h0
    ot = p[..., GO, :] + r[GO] * h0
    return zt, it, ft, ot


def _step(prev, p, r, forget):
    """The intermediate values of one step, shared by the state, its Jacobian and the gate
    Jacobian (equations in ``cell``)."""
    c0, n0, m0 = prev[..., C, :], prev[..., N, :], prev[..., M, :]
    zt, it, ft, ot = preactivations(prev, p, r)
    z = np.tanh(zt)
    o = sigmoid(ot)
    lf, dlf = log_forget(ft, forget)
    a = lf + m0
    beta = a >= it  # tie -> forget branch
    m = np.where(beta, a, it)
    ig = np.exp(it - m)
    fg = np.exp(a - m)
    c = fg * c0 + ig * z
    n = fg * n0 + ig
    D, dD_dn, dD_dm = _readout_denominator(n, m, cell_mode(forget)[1])
    h = o * c / D  # read-out
    return {"z": z, "o": o, "dlf": dlf, "beta": beta, "m": m, "ig": ig, "fg": fg, "c": c, "n": n, "h": h,
            "D": D, "dD_dn": dD_dn, "dD_dm": dD_dm}


def _readout_denominator(n, m, floored):
    """D of the read-out h = o c / D and its derivatives in n and m: D = n (the paper's sLSTM
    step), or D = max(|n|, e^{-m}, READOUT_FLOOR) with the derivative of the branch the max
    takes (ties go to |n|, then to e^{-m})."""
    if not floored:
        return n, np.ones_like(n), np.zeros_like(n)
    an = np.abs(n)
    em = np.exp(-m)
    on_n = (an >= em) & (an >= READOUT_FLOOR)
    on_m = ~on_n & (em >= READOUT_FLOOR)
    D = np.where(on_n, an, np.where(on_m, em, READOUT_FLOOR))
    return D, np.where(on_n, np.sign(n), 0.0), np.where(on_m, -em, 0.0)


def _readout_row(v, dc, dn, dm):
    """Derivatives of h = o c / D(n, m) through c, n and m (quotient rule), one per column."""
    o, c, D = v["o"], v["c"], v["D"]
    q = o * c / (D * D)
    return [(o / D) * dc[k] - q * (v["dD_dn"] * dn[k] + v["dD_dm"] * dm[k]) for k in range(len(dc))]


def cell(prev, p, r, forget, with_jacobian=False):
    """One stabilised sLSTM step per feature (mix='diag').

    prev : (..., 4, d) previous state (c', n', m', h')
    p    : (..., 4, d) gate pre-activations from the input, gates (z, i, f, o)
    r    : (4, d) channelwise recurrent weights
    returns next state (..., 4, d) and, if asked, A = d next / d prev of shape (..., 4, 4, d)
    with A[..., row, col, :] = d next[row] / d prev[col].

    Equations (sLSTM step pseudocode, summary card; stabiliser from the educational page):
      pre-activation  x~ = p_x + r_x h'                 for x in (z, i, f, o)
      z = tanh z~,  o = sigma(o~),  l = log f(f~)
      a = l + m',  m = max(a, i~)                         (stabiliser, running max)
      i' = exp(i~ - m),  f' = exp(a - m)                  (both in (0, 1])
      c = f' c' + i' z,  n = f' n' + i',  h = o c / n
    (h = o c / max(|n|, e^{-m}, READOUT_FLOOR) for a "/floored" cell mode).
    """
    v = _step(prev, p, r, forget)
    c0, n0 = prev[..., C, :], prev[..., N, :]
    z, o, dlf, beta, ig, fg, c, n = v["z"], v["o"], v["dlf"], v["beta"], v["ig"], v["fg"], v["c"], v["n"]
    nxt = np.stack([c, n, v["m"], v["h"]], axis=-2)
    if not with_jacobian:
        return nxt

    b = beta.astype(np.float64)
    # derivatives of the stabiliser and of the two stabilised gates
    dm_dm = b
    dm_dh = b * dlf * r[GF] + (1.0 - b) * r[GI]
    dig_dm = -b * ig
    dig_dh = ig * (r[GI] - dm_dh)
    dfg_dm = (1.0 - b) * fg
    dfg_dh = fg * (dlf * r[GF] - dm_dh)
    dz_dh = (1.0 - z * z) * r[GZ]
    do_dh = o * (1.0 - o) * r[GO]

    zero = np.zeros_like(c)
    # rows c and n (c' and n' do not enter the gates)
    dc = [fg, zero, c0 * dfg_dm + z * dig_dm, c0 * dfg_dh + z * dig_dh + ig * dz_dh]
    dn = [zero, fg, n0 * dfg_dm + dig_dm, n0 * dfg_dh + dig_dh]
    dmr = [zero, zero, dm_dm, dm_dh]
    # row h = o c / D by the quotient rule, plus the output-gate term on h'
    dh = _readout_row(v, dc, dn, dmr)
    dh[H] = dh[H] + (c / v["D"]) * do_dh
    A = np.stack([np.stack(row, axis=-2) for row in (dc, dn, dmr, dh)], axis=-3)
    return nxt, A


def gate_jacobian(prev, p, r, forget):
    """G = d next / d x~ of one step, x~ = p + r h' the gate pre-activations (z, i, f, o).

    Shape (..., 4, 4, d) with G[..., slot, gate, :] = d next[slot] / d x~[gate]. The state
    enters the gates only through h', so the h' column of the state Jacobian is G r. Same
    equations as ``cell``, differentiated in the pre-activations on the branch the max takes:
      m = max(l(f~) + m', i~):  dm/di~ = 1 - beta,  dm/df~ = beta l'(f~)
      i' = exp(i~ - m):         di'/di~ = i' (1 - dm/di~),  di'/df~ = -i' dm/df~
      f' = exp(l + m' - m):     df'/di~ = -f' dm/di~,       df'/df~ = f' (l' - dm/df~)
      c = f' c' + i' z,  n = f' n' + i',  h = o c / n,  z = tanh z~,  o = sigma(o~)
    """
    v = _step(prev, p, r, forget)
    c0, n0 = prev[..., C, :], prev[..., N, :]
    z, o, dlf, beta, ig, fg, c, n = v["z"], v["o"], v["dlf"], v["beta"], v["ig"], v["fg"], v["c"], v["n"]
    b = beta.astype(np.float64)
    dm_di = 1.0 - b
    dm_df = b * dlf
    dig_di = ig * (1.0 - dm_di)
    dig_df = -ig * dm_df
    dfg_di = -fg * dm_di
    dfg_df = fg * (dlf - dm_df)
    zero = np.zeros_like(c)
    dc = [ig * (1.0 - z * z), c0 * dfg_di + z * dig_di, c0 * dfg_df + z * dig_df, zero]
    dn = [zero, n0 * dfg_di + dig_di, n0 * dfg_df + dig_df, zero]
    dmr = [zero, dm_di, dm_df, zero]
    dh = _readout_row(v, dc, dn, dmr)
    dh[GO] = dh[GO] + (c / v["D"]) * o * (1.0 - o)
    return np.stack([np.stack(row, axis=-2) for row in (dc, dn, dmr, dh)], axis=-3)


def gate_values(prev, p, r, forget):
    """Stabilised gates (i', f') and the stabiliser m of one step, for invariant checks."""
    h0, m0 = prev[..., H, :], prev[..., M, :]
    it = p[..., GI, :] + r[GI] * h0
    ft = p[..., GF, :] + r[GF] * h0
    lf, _ = log_forget(ft, forget)
    a = lf + m0
    m = np.where(a >= it, a, it)
    return np.exp(it - m), np.exp(a - m), m, a, it


# ---------------------------------------------------------------------------------------
# sequential forward and the unstabilised form
# ---------------------------------------------------------------------------------------
def _state0(state0, B, d):
    if state0 is None:
        return np.zeros((B, 4, d))
    return np.asarray(state0, dtype=np.float64)


def sequence_starts(cu_seqlens, T):
    """{t: s} for the first step t of every non-empty packed sequence s (cu_seqlens: S + 1
    non-decreasing offsets from 0 to T)."""
    cu = [int(v) for v in cu_seqlens]
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to T")
    return {cu[s]: s for s in range(len(cu) - 1) if cu[s] < cu[s + 1]}


def final_states(S, state0, cu_seqlens):
    """Last state of every packed sequence (S_seq, 4, d); an empty sequence keeps its state0."""
    cu = [int(v) for v in cu_seqlens]
    n_seq, d = len(cu) - 1, S.shape[-1]
    s0 = _state0(state0, n_seq, d)
    return np.stack([S[0, cu[s + 1] - 1] if cu[s + 1] > cu[s] else s0[s] for s in range(n_seq)])


def sequential(P, R, state0, forget, cu_seqlens=None):
    """s_t = f(s_{t-1}) for t = 1..T from s_0 = state0 (zeros when None).

    P (B, T, 4, d), R (4, d), state0 (B, 4, d) -> states (B, T, 4, d).
    The step loop the 'sequential' solver runs ("sLSTM in this library", "API notes").
    Packed (cu_seqlens given, B = 1, state0 (S, 4, d)): the state restarts from state0[s] at
    the first step of sequence s.
    """
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    B, T, _, d = P.shape
    out = np.empty((B, T, 4, d))
    if cu_seqlens is None:
        s = _state0(state0, B, d)
        starts = {}
    else:
        starts = sequence_starts(cu_seqlens, T)
        s0 = _state0(state0, len(cu_seqlens) - 1, d)
        s = np.zeros((B, 4, d))
    for t in range(T):
        if t in starts:
            s = s0[starts[t]][None]
        s = cell(s, P[:, t], R, forget)
        out[:, t] = s
    return out


def unstabilised_hidden(P, R, forget, floored=False):
    """h from the unstabilised recurrence, zero initial state.

    c_t = f_t c_{t-1} + i_t z_t, n_t = f_t n_{t-1} + i_t, h_t = o_t c_t / n_t with
    i_t = exp(i~), f_t = exp(f~) or sigma(f~). The paper states that the stabilised and
    unstabilised forms give identical outputs (summary card, "Method" item 1). With floored,
    h_t = o_t c_t / max(|n_t|, 1): the floor e^{-m} of the stabilised read-out is 1 in the
    unstabilised domain (educational page, "Implementation notes / deviations" item 1).
    Overflows for long sequences; used only on short ones.
    """
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    B, T, _, d = P.shape
    c = np.zeros((B, d))
    n = np.zeros((B, d))
    h = np.zeros((B, d))
    hs = np.empty((B, T, d))
    cs = np.empty((B, T, d))
    ns = np.empty((B, T, d))
    for t in range(T):
        pt = P[:, t]
        z = np.tanh(pt[:, GZ] + R[GZ] * h)
        i = np.exp(pt[:, GI] + R[GI] * h)
        ft = pt[:, GF] + R[GF] * h
        f = np.exp(ft) if cell_mode(forget)[0] == FORGET_EXP else sigmoid(ft)
        o = sigmoid(pt[:, GO] + R[GO] * h)
        c = f * c + i * z
        n = f * n + i
        h = o * c / (np.maximum(np.abs(n), 1.0) if floored else n)
        hs[:, t], cs[:, t], ns[:, t] = h, c, n
    return hs, cs, ns


# ---------------------------------------------------------------------------------------
# Newton
# ---------------------------------------------------------------------------------------
def warm_start(P, state0, forget, cu_seqlens=None):
    """Initial Newton iterate: the exact trajectory with R * h_{t-1} dropped.

    Reading (the pages give no initial guess): with the recurrent term removed every
    pre-activation is known up front, so the trajectory is the sequential recurrence with
    R = 0, started from state0's (c, n, m). The h slot is o c / n with o = sigma(p_o).
    """
    P = np.asarray(P, dtype=np.float64)
    return sequential(P, np.zeros((4, P.shape[-1])), state0, forget, cu_seqlens)


def _shifted(S, state0, cu_seqlens=None):
    """Previous states s_{t-1} for t = 1..T, with state0 prepended as s_0 (packed: state0[s]
    at the first step of sequence s)."""
    B, T, _, d = S.shape
    prev = np.empty_like(S)
    prev[:, 1:] = S[:, :-1]
    if cu_seqlens is None:
        prev[:, 0] = _state0(state0, B, d)
    else:
        s0 = _state0(state0, len(cu_seqlens) - 1, d)
        for t, s in sequence_starts(cu_seqlens, T).items():
            prev[:, t] = s0[s]
    return prev


def residual(S, P, R, state0, forget, with_jacobian=True, cu_seqlens=None):
    """F_t = s_t - f(s_{t-1}) and A_t = df/ds' at s_{t-1}, for t = 1..T.

    S, P (B, T, 4, d) -> F (B, T, 4, d), A (B, T, 4, 4, d)  (the scan_block4 layout)
    Packed: A is zero at every sequence start (the state before it is data).
    """
    prev = _shifted(S, state0, cu_seqlens)
    if with_jacobian:
        fs, A = cell(prev, P, R, forget, with_jacobian=True)
        if cu_seqlens is not None:
            for t in sequence_starts(cu_seqlens, S.shape[1]):
                A[:, t] = 0.0
        return S - fs, A
    return S - cell(prev, P, R, forget), None


def max_abs(F):
    """max |F| over all entries; a non-finite entry counts as +inf."""
    F = np.asarray(F)
    if F.size == 0:
        return 0.0
    a = np.abs(F)
    return float(np.max(np.where(np.isfinite(a), a, np.inf)))


def forward_substitution(A, rhs):
    """Solve the lower block-bidiagonal system by block forward substitution.

    x_1 = rhs_1,  x_t = A_t x_{t-1} + rhs_t  (A_1 is not used: s_0 is fixed).
    A (B, T, 4, 4, d), rhs (B, T, 4, d) -> x (B, T, 4, d).
    """
    B, T, _, d = rhs.shape
    x = np.empty_like(rhs)
    x[:, 0] = rhs[:, 0]
    for t in range(1, T):
        x[:, t] = np.einsum("bijd,bjd->bid", A[:, t], x[:, t - 1]) + rhs[:, t]
    return x


def dense_solve_lane(A_lane, F_lane):
    """Dense LAPACK solve of one lane's Newton system (tiny inputs only).

    A_lane (T, 4, 4), F_lane (T, 4). Assembles the 4T x 4T matrix with identity blocks on
    the diagonal and -A_t below it, and solves  J Delta = -F.
    """
    T = F_lane.shape[0]
    J = np.eye(4 * T)
    for t in range(1, T):
        J[4 * t:4 * t + 4, 4 * (t - 1):4 * t] = -A_lane[t]
    return np.linalg.solve(J, -F_lane.reshape(-1)).reshape(T, 4)


def backward(P, R, state0, S, g, forget, return_adjoint=False, cu_seqlens=None, g_final=None):
    """Gradients through the recurrence of a loss L whose direct derivative with respect to the
    states is g = dL/dS.

    P, S, g (B, T, 4, d): pre-activations, the forward states s_1..s_T (the solution) and the
    direct gradient; R (4, d); state0 (B, 4, d) or None. Returns dP (B, T, 4, d), dR (4, d),
    dstate0 (B, 4, d), and with return_adjoint the adjoint lam (B, T, 4, d), lam_t = dL/ds_t.

    "sLSTM in this library", section "Backward": the reverse recurrence
      lam_T = g_T,  lam_t = g_t + A_{t+1}^T lam_{t+1}     (A_{t+1} = d s_{t+1} / d s_t)
    then per step the cell's vector-Jacobian product with the gate Jacobian G_t:
      dP_t = G_t^T lam_t,  dR = sum over b and t of dP_t * h_{t-1},  dstate0 = A_1^T lam_1.
    g_final (B, 4, d), or (S, 4, d) when packed, is a gradient with respect to the final
    state(s), added at the last step (of each sequence). Packed (cu_seqlens, B = 1): the
    adjoint of the step before a sequence start takes nothing from that start, whose A^T lam
    is dstate0[s] instead; an empty sequence passes g_final[s] to dstate0[s].
    """
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    g = np.array(g, dtype=np.float64)
    B, T, _, d = P.shape
    prev = _shifted(S, state0, cu_seqlens)
    starts = {} if cu_seqlens is None else sequence_starts(cu_seqlens, T)
    n_seq = B if cu_seqlens is None else len(cu_seqlens) - 1
    dstate0 = np.zeros((n_seq, 4, d))
    if g_final is not None:
        g_final = np.asarray(g_final, dtype=np.float64)
        if cu_seqlens is None:
            g[:, T - 1] += g_final
        else:
            cu = [int(v) for v in cu_seqlens]
            for s in range(n_seq):
                if cu[s + 1] > cu[s]:
                    g[0, cu[s + 1] - 1] += g_final[s]
                else:
                    dstate0[s] += g_final[s]
    dP = np.empty_like(P)
    dR = np.zeros((4, d))
    lam_all = np.empty_like(S)
    lam = g[:, T - 1].copy()
    for t in range(T - 1, -1, -1):
        lam_all[:, t] = lam
        _, A = cell(prev[:, t], P[:, t], R, forget, with_jacobian=True)
        G = gate_jacobian(prev[:, t], P[:, t], R, forget)
        delta = np.einsum("bsgd,bsd->bgd", G, lam)
        dP[:, t] = delta
        dR += np.sum(delta * prev[:, t, H][:, None, :], axis=0)
        lam_prev = np.einsum("bsjd,bsd->bjd", A, lam)
        if cu_seqlens is None:
            if t == 0:
                dstate0 += lam_prev
            lam = g[:, t - 1] + lam_prev if t > 0 else lam_prev
        else:
            if t in starts:
                dstate0[starts[t]] += lam_prev[0]
                lam_prev = np.zeros_like(lam_prev)
            if t > 0:
                lam = g[:, t - 1] + lam_prev
    if return_adjoint:
        return dP, dR, dstate0, lam_all
    return dP, dR, dstate0


def branch_margin(P, R, state0, S, forget, cu_seqlens=None):
    """Distance |a - i~| of every step from the tie of the running maximum m = max(a, i~), and
    the scale |l| + |m'| + |i~| of the operands that form it (a = l + m'), at the states S;
    each (B, T, d).

    The state is continuous where the maximum switches branch but its derivatives are not, so
    a backward computed in another precision agrees with this one only on lanes whose margins
    all exceed that precision's rounding of a and i~ (the tie reading: a >= i~ takes the
    forget branch).
    """
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    prev = _shifted(np.asarray(S, dtype=np.float64), state0, cu_seqlens)
    _, it, ft, _ = preactivations(prev, P, R)
    lf, _ = log_forget(ft, forget)
    a = lf + prev[..., M, :]
    return np.abs(a - it), np.abs(lf) + np.abs(prev[..., M, :]) + np.abs(it)


def dense_adjoint_lane(A_lane, g_lane):
    """Dense LAPACK solve of one lane's adjoint system (tiny inputs only).

    A_lane (T, 4, 4) with A_lane[t] = d s_t / d s_{t-1}, g_lane (T, 4). The forward Newton
    system J x = r has identity blocks on the diagonal and -A_t below it; the adjoint solves
    J^T lam = g.
    """
    T = g_lane.shape[0]
    J = np.eye(4 * T)
    for t in range(1, T):
        J[4 * t:4 * t + 4, 4 * (t - 1):4 * t] = -A_lane[t]
    return np.linalg.solve(J.T, g_lane.reshape(-1)).reshape(T, 4)


@dataclass
class NewtonStats:
    iters: int = 0
    converged: bool = False
    diverged: bool = False
    nonfinite: bool = False
    max_abs_F: list = field(default_factory=list)  # entry k: max|F| after k updates


def newton_flags(e_final, tol):
    """Divergence when max|F| > 1 (or non-finite) after the last iterate; convergence
    when an early-stop tolerance is set and met ("Layout", "Current surface (0.17)")."""
    nonfinite = not np.isfinite(e_final)
    diverged = nonfinite or e_final > 1.0
    converged = (tol > 0) and (not nonfinite) and e_final < tol
    return converged, diverged, nonfinite


def newton(P, R, state0, forget, max_iters, tol=0.0, init=INIT_WARM, return_history=False,
           cu_seqlens=None):
    """Newton solve of the sLSTM recurrence over all T steps at once.

    For k = 0 .. max_iters-1: F, A at the current iterate; e_k = max|F|; stop before the
    solve when tol > 0 and e_k < tol; Delta from the block-bidiagonal system; S += Delta.
    Finally e = max|F| at the last iterate and the flags.
    Returns (S, NewtonStats) and, with return_history, the list of iterates S^0..S^iters.
    Packed sequences (cu_seqlens) share one residual norm, so one stop decision and one set of
    flags cover the whole pack.
    """
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    B, T, _, d = P.shape
    if init == INIT_WARM:
        S = warm_start(P, state0, forget, cu_seqlens)
    elif init == INIT_ZERO:
        S = np.zeros((B, T, 4, d))
    else:
        raise ValueError(f"unknown init {init!r}")
    stats = NewtonStats()
    hist = [S.copy()] if return_history else None
    with np.errstate(all="ignore"):
        stopped = False
        for _ in range(max_iters):
            F, A = residual(S, P, R, state0, forget, cu_seqlens=cu_seqlens)
            e = max_abs(F)
            stats.max_abs_F.append(e)
            if tol > 0 and e < tol:
                stopped = True
                break
            S = S + forward_substitution(A, -F)
            stats.iters += 1
            if return_history:
                hist.append(S.copy())
        if not stopped:
            F, _ = residual(S, P, R, state0, forget, with_jacobian=False, cu_seqlens=cu_seqlens)
            stats.max_abs_F.append(max_abs(F))
    e_final = stats.max_abs_F[-1]
    stats.converged, stats.diverged, stats.nonfinite = newton_flags(e_final, tol)
    if return_history:
        return S, stats, hist
    return S, stats


# ---------------------------------------------------------------------------------------
# input projection
# ---------------------------------------------------------------------------------------
def input_projection(x, W, bias):
    """P[b, t, g, j] = sum_k x[b, t, k] W[g, j, k] + bias[g, j]   (gates g = z, i, f, o).

    x (B, T, d_in), W (4, d_h, d_in), bias (4, d_h) -> P (B, T, 4, d_h), float64.
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    B, T, d_in = x.shape
    g, d_h, _ = W.shape
    P = x.reshape(B * T, d_in) @ W.reshape(g * d_h, d_in).T
    return P.reshape(B, T, g, d_h) + bias


def input_projection_backward(x, W, dP):
    """Gradients of a loss L through P = x W^T + bias, given dP = dL/dP (B, T, 4, d_h):
    dW[g, j, k] = sum_{b,t} dP[b, t, g, j] x[b, t, k], dx[b, t, k] = sum_{g,j} dP[b, t, g, j]
    W[g, j, k], dbias[g, j] = sum_{b,t} dP[b, t, g, j]. ("sLSTM in this library", "Backward":
    the gradient of W_x follows from the cell's VJP by a GEMM.) Returns (dW, dx, dbias), float64.
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    dP = np.asarray(dP, dtype=np.float64)
    B, T, d_in = x.shape
    g, d_h, _ = W.shape
    dP2 = dP.reshape(B * T, g * d_h)
    dW = (dP2.T @ x.reshape(B * T, d_in)).reshape(g, d_h, d_in)
    dx = (dP2 @ W.reshape(g * d_h, d_in)).reshape(B, T, d_in)
    dbias = dP2.sum(axis=0).reshape(g, d_h)
    return dW, dx, dbias


def hidden(S):
    """The hidden slot (B, T, d_h) of a state tensor (hidden slot 3)."""
    return np.asarray(S)[..., H, :]


# ---------------------------------------------------------------------------------------
# head mixing (mix='head'): block-diagonal recurrent matrices, one block per head and gate
# ---------------------------------------------------------------------------------------
# "sLSTM in this library", section "Cell" (mix table, row 'head'): R of shape
# (4, n_heads, d_head, d_head), n_heads dividing d_h; the paper's sLSTM (summary card, "Method"
# item 2 and the one-head step pseudocode under "Key equations") mixes memory through
# recurrent matrices from the previous hidden state to every gate pre-activation, block-diagonal
# with one block per head, so no mixing across heads. Feature j = a d_head + i is unit i of head
# a; its pre-activation for gate g is p[g, j] + sum_k R[g, a, i, k] h'[a d_head + k] (R_g h' with
# the row for unit i). Everything after the pre-activations is the channelwise cell: this
# section calls ``cell`` with the full pre-activation as input and a zero channelwise weight.
# The dense (4 d_head) x (4 d_head) Jacobian per head is assembled here (the dense-J oracle the
# pages keep for this mode); state vectors of a head are ordered unit-major, index 4 i + slot.

def head_recurrent(h, R):
    """R_g h' per gate: h (..., d), R (4, n_heads, d_head, d_head) -> (..., 4, d) with
    [..., g, a d_head + i] = sum_k R[g, a, i, k] h[..., a d_head + k]."""
    R = np.asarray(R, dtype=np.float64)
    _, nh, dh, _ = R.shape
    hh = np.asarray(h, dtype=np.float64).reshape(h.shape[:-1] + (nh, dh))
    y = np.einsum("gaik,...ak->...gai", R, hh)
    return y.reshape(h.shape[:-1] + (4, nh * dh))


def _head_shape(R, d):
    R = np.asarray(R, dtype=np.float64)
    if R.ndim != 4 or R.shape[0] != 4 or R.shape[2] != R.shape[3] or R.shape[1] * R.shape[2] != d:
        raise ValueError(f"head-mixing R must be (4, n_heads, d_head, d_head) with n_heads * d_head = {d}")
    return R, R.shape[1], R.shape[2]


def head_vectors(X, nh):
    """(..., 4, d) -> (..., nh, 4 dh) with index 4 i + slot for unit i of each head."""
    d = X.shape[-1]
    dh = d // nh
    Y = np.moveaxis(X, -2, -1)                   # (..., d, 4)
    return Y.reshape(X.shape[:-2] + (nh, dh * 4))


def from_head_vectors(Y, nh):
    """Inverse of head_vectors: (..., nh, 4 dh) -> (..., 4, d)."""
    dh = Y.shape[-1] // 4
    X = Y.reshape(Y.shape[:-2] + (nh * dh, 4))
    return np.moveaxis(X, -1, -2)


def cell_head(prev, p, R, forget, with_jacobian=False):
    """One sLSTM step under head mixing.

    prev, p (..., 4, d); R (4, n_heads, d_head, d_head). Returns the next state (..., 4, d)
    and, if asked, the dense Jacobian J (..., n_heads, 4 d_head, 4 d_head) of the next state of
    each head with respect to that head's previous state (unit-major ordering):
      J[(i, slot), (i, col)] = d next[slot, i] / d prev[col, i] through the unit's own c', n', m'
      J[(i, slot), (k, h)]  += sum_g G[slot, g, i] R[g, a, i, k]   (h' enters every gate of the
    head), with G = d next / d x~ the gate Jacobian of the step.
    """
    p = np.asarray(p, dtype=np.float64)
    d = p.shape[-1]
    R, nh, dh = _head_shape(R, d)
    pre = p + head_recurrent(prev[..., H, :], R)
    zero_r = np.zeros((4, d))
    if not with_jacobian:
        return cell(prev, pre, zero_r, forget)
    nxt, A0 = cell(prev, pre, zero_r, forget, with_jacobian=True)  # zero h' column
    G = gate_jacobian(prev, pre, zero_r, forget)                     # (..., slot, gate, d)
    lead = p.shape[:-2]
    J = np.zeros(lead + (nh, dh, 4, dh, 4))
    A0h = A0.reshape(lead + (4, 4, nh, dh))      # slot, col, a, i
    Gh = G.reshape(lead + (4, 4, nh, dh))        # slot, gate, a, i
    # own columns: unit i's next state from its own previous state
    for i in range(dh):
        J[..., :, i, :, i, :] = np.moveaxis(A0h[..., i], (-3, -2, -1), (-2, -1, -3))
    # h' columns: sum over gates of G[slot, gate] R[gate, a, i, k]
    J[..., :, :, :, :, H] += np.einsum("...sgai,gaik->...aisk", Gh, R)
    return nxt, J.reshape(lead + (nh, 4 * dh, 4 * dh))


def sequential_head(P, R, state0, forget, cu_seqlens=None):
    """s_t = f(s_{t-1}) under head mixing, t = 1..T, from state0 (zeros when None). Packed
    (cu_seqlens, B = 1, state0 (S, 4, d)): the state restarts from state0[s] at the first step
    of sequence s, as in ``sequential``."""
    P = np.asarray(P, dtype=np.float64)
    B, T, _, d = P.shape
    S = np.empty((B, T, 4, d))
    if cu_seqlens is None:
        starts, s0 = {}, None
        prev = _state0(state0, B, d)
    else:
        starts = sequence_starts(cu_seqlens, T)
        s0 = _state0(state0, len(cu_seqlens) - 1, d)
        prev = np.zeros((B, 4, d))
    with np.errstate(all="ignore"):
        for t in range(T):
            if t in starts:
                prev = s0[starts[t]][None]
            prev = cell_head(prev, P[:, t], R, forget)
            S[:, t] = prev
    return S


def residual_head(S, P, R, state0, forget, with_jacobian=True, cu_seqlens=None):
    """F_t = s_t - f(s_{t-1}) and the dense per-head Jacobians J_t, t = 1..T. Packed: the state
    before a sequence start is that sequence's state0 (data, not an unknown), so J is zero there
    (the head flag of the segmented scan)."""
    prev = _shifted(S, state0, cu_seqlens)
    if with_jacobian:
        fs, J = cell_head(prev, P, R, forget, with_jacobian=True)
        if cu_seqlens is not None:
            for t in sequence_starts(cu_seqlens, S.shape[1]):
                J[:, t] = 0.0
        return S - fs, J
    return S - cell_head(prev, P, R, forget), None


def forward_substitution_head(J, rhs, nh):
    """x_1 = rhs_1, x_t = J_t x_{t-1} + rhs_t with dense per-head blocks (J_1 unused).
    J (B, T, nh, 4 dh, 4 dh), rhs (B, T, 4, d) -> x (B, T, 4, d)."""
    r = head_vectors(rhs, nh)
    x = np.empty_like(r)
    x[:, 0] = r[:, 0]
    for t in range(1, r.shape[1]):
        x[:, t] = np.einsum("bauv,bav->bau", J[:, t], x[:, t - 1]) + r[:, t]
    return from_head_vectors(x, nh)


def newton_head(P, R, state0, forget, max_iters, tol=0.0, init=INIT_WARM, cu_seqlens=None):
    """Newton solve under head mixing: the steps of ``newton`` with the dense per-head
    Jacobians (the warm start drops R h' and is the channelwise one). Packed: cu_seqlens as in
    ``sequential_head``; one residual maximum over the whole pack decides the stop."""
    P = np.asarray(P, dtype=np.float64)
    B, T, _, d = P.shape
    R, nh, _ = _head_shape(R, d)
    if init == INIT_WARM:
        S = warm_start(P, state0, forget, cu_seqlens)
    elif init == INIT_ZERO:
        S = np.zeros((B, T, 4, d))
    else:
        raise ValueError(f"unknown init {init!r}")
    stats = NewtonStats()
    with np.errstate(all="ignore"):
        stopped = False
        for _ in range(max_iters):
            F, J = residual_head(S, P, R, state0, forget, cu_seqlens=cu_seqlens)
            e = max_abs(F)
            stats.max_abs_F.append(e)
            stopped = tol > 0.0 and e < tol  # the stop rule of ``newton``
            if stopped:
                break
            S = S + forward_substitution_head(J, -F, nh)
            stats.iters += 1
        if not stopped:
            F, _ = residual_head(S, P, R, state0, forget, with_jacobian=False, cu_seqlens=cu_seqlens)
            stats.max_abs_F.append(max_abs(F))
    stats.converged, stats.diverged, stats.nonfinite = newton_flags(stats.max_abs_F[-1], tol)
    return S, stats


def backward_head(P, R, state0, S, g, forget, g_final=None, return_adjoint=False, cu_seqlens=None):
    """Gradients through the recurrence under head mixing, for a loss whose direct derivative
    with respect to the states is g = dL/dS (and g_final = dL/d(final state), added at the last
    step). P, S, g (B, T, 4, d); R (4, n_heads, d_head, d_head); state0 (B, 4, d) or None.
    Returns dP (B, T, 4, d), dR (4, n_heads, d_head, d_head), dstate0 (B, 4, d) and, with
    return_adjoint, the adjoint lam (B, T, 4, d).

    The reverse recurrence of ``backward`` with the dense per-head Jacobians of ``cell_head``:
      lam_T = g_T,  lam_t = g_t + J_{t+1}^T lam_{t+1}   (per head, unit-major vectors)
    and per step the gate vector-Jacobian product dP_t = G_t^T lam_t (G_t = d s_t / d x~_t, the
    same for every mixing, since x~ enters the cell the same way); h' enters x~ through R_g h',
    so dR[g, a, i, k] = sum over b and t of dP_t[g, a d_head + i] h_{t-1}[a d_head + k], and
    dstate0 = J_1^T lam_1. Packed (cu_seqlens, B = 1): as ``backward``, the adjoint of the state
    before a sequence start is dstate0[s] and nothing crosses the start; g_final (S, 4, d) is
    added at each sequence's last step, or passed to dstate0 by an empty sequence.
    """
    P = np.asarray(P, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    g = np.array(g, dtype=np.float64)
    B, T, _, d = P.shape
    R, nh, dh = _head_shape(R, d)
    prev = _shifted(S, state0, cu_seqlens)
    starts = {} if cu_seqlens is None else sequence_starts(cu_seqlens, T)
    dstate0 = np.zeros((B if cu_seqlens is None else len(cu_seqlens) - 1, 4, d))
    if g_final is not None:
        g_final = np.asarray(g_final, dtype=np.float64)
        if cu_seqlens is None:
            g[:, T - 1] += g_final
        else:
            cu = [int(v) for v in cu_seqlens]
            for q in range(len(cu) - 1):
                if cu[q + 1] > cu[q]:
                    g[0, cu[q + 1] - 1] += g_final[q]
                else:
                    dstate0[q] += g_final[q]
    zero_r = np.zeros((4, d))
    dP = np.empty_like(P)
    dR = np.zeros((4, nh, dh, dh))
    lam_all = np.empty_like(S)
    lam = g[:, T - 1].copy()
    for t in range(T - 1, -1, -1):
        lam_all[:, t] = lam
        _, J = cell_head(prev[:, t], P[:, t], R, forget, with_jacobian=True)
        pre = P[:, t] + head_recurrent(prev[:, t, H], R)
        G = gate_jacobian(prev[:, t], pre, zero_r, forget)
        delta = (G * lam[:, :, None, :]).sum(axis=1)  # G^T lam: sum over the state slots
        dP[:, t] = delta
        dR += np.einsum("bgai,bak->gaik", delta.reshape(B, 4, nh, dh), prev[:, t, H].reshape(B, nh, dh))
        lam_prev = from_head_vectors(np.einsum("bauv,bau->bav", J, head_vectors(lam, nh)), nh)
        if cu_seqlens is None:
            if t == 0:
                dstate0 += lam_prev
        elif t in starts:
            dstate0[starts[t]] += lam_prev[0]
            lam_prev = np.zeros_like(lam_prev)
        if t > 0:
            lam = g[:, t - 1] + lam_prev
    if return_adjoint:
        return dP, dR, dstate0, lam_all
    return dP, dR, dstate0
