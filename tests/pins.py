"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each pin takes the oracle module as an argument so that the mutation test can run the same
pins against copies of the oracle with planted mistakes. A pin returns nothing and raises
AssertionError when the oracle disagrees.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------
# golden worked examples
# ---------------------------------------------------------------------------------------
def _value(expr: str) -> float:
    """Evaluate a golden-file entry: rationals, ln(), atanh() and + - * /."""
    ns = {"ln": lambda v: math.log(float(v)), "atanh": lambda v: math.atanh(float(v)),
          "__builtins__": {}}
    expr = expr.strip()
    try:
        return float(Fraction(expr))
    except ValueError:
        pass
    # rationals inside function calls are evaluated as floats
    return float(eval(expr, ns, {}))  # noqa: S307 -- our own fixture files


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    conv = lambda a: np.vectorize(_value, otypes=[float])(np.array(a, dtype=object))  # noqa: E731
    P = conv(g["P"])[None]           # (1, T, 4, 1)
    R = conv(g["R"])                 # (4, 1)
    S = conv(g["expected_states"])[None]
    gates = conv(g["expected_gates_i_f"])
    return g, P, R, S, gates


GOLDEN_FILES = ["slstm_exp_forget_r0.json", "slstm_sigmoid_forget_r0.json",
                "slstm_exp_forget_recurrent.json"]


def pin_golden_sequential(ref):
    for name in GOLDEN_FILES:
        g, P, R, S, _ = load_golden(name)
        got = ref.sequential(P, R, None, g["forget"])
        np.testing.assert_allclose(got, S, rtol=1e-13, atol=1e-14, err_msg=name)


def pin_golden_gates(ref):
    for name in GOLDEN_FILES:
        g, P, R, S, gates = load_golden(name)
        prev = np.concatenate([np.zeros((1, 1, 4, 1)), S[:, :-1]], axis=1)
        ig, fg, m, _, _ = ref.gate_values(prev, P, R, g["forget"])
        np.testing.assert_allclose(ig[0, :, 0], gates[:, 0], rtol=1e-13, err_msg=name)
        np.testing.assert_allclose(fg[0, :, 0], gates[:, 1], rtol=1e-13, err_msg=name)
        np.testing.assert_allclose(m[0, :, 0], S[0, :, 2, 0], rtol=1e-13, atol=1e-15, err_msg=name)


# ---------------------------------------------------------------------------------------
# small seeded problems (drawn here so the pins do not depend on the workload module)
# ---------------------------------------------------------------------------------------
def small_problem(seed, B=2, T=64, d=16, forget="exp", forget_bias=3.0, r_scale=0.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, T, d))
    W = rng.standard_normal((4, d, d)) / np.sqrt(d)
    R = rng.uniform(-r_scale, r_scale, size=(4, d))
    P = np.einsum("btk,gjk->btgj", x, W)
    P[:, :, 2, :] += forget_bias
    return P, R


def pin_unstabilised_equivalence(ref):
    """Stabilised and unstabilised forms give the same h (summary card, 'Method' item 1)."""
    for forget, seed in (("exp", 1), ("sigmoid", 2)):
        P, R = small_problem(seed, forget=forget)
        h_stab = ref.hidden(ref.sequential(P, R, None, forget))
        h_raw, c_raw, n_raw = ref.unstabilised_hidden(P, R, forget)
        assert np.all(np.isfinite(h_raw))
        np.testing.assert_allclose(h_stab, h_raw, rtol=1e-11, atol=1e-13, err_msg=forget)
        # the stabilised c, n are the unstabilised ones scaled by exp(-m)
        S = ref.sequential(P, R, None, forget)
        np.testing.assert_allclose(S[..., 0, :], c_raw * np.exp(-S[..., 2, :]), rtol=1e-10,
                                   atol=1e-300, err_msg=forget)
        np.testing.assert_allclose(S[..., 1, :], n_raw * np.exp(-S[..., 2, :]), rtol=1e-10,
                                   err_msg=forget)


def pin_floored_readout_unstabilised(ref):
    """The floored read-out h = o c / max(|n|, e^{-m}) is the unstabilised o c / max(|n|, 1)
    (the floor e^{-m} is 1 in the unstabilised domain), recurrent term included; on inputs
    where the floor is active (input pre-activations shifted down, so n < e^{-m} early on),
    and there it differs from the paper's o c / n."""
    for forget, seed in (("exp", 61), ("sigmoid", 62)):
        P, R = small_problem(seed, T=24, forget=forget)
        P[:, :, 1, :] -= 2.0
        S = ref.sequential(P, R, None, forget + ref.FLOORED)
        h_raw, _, _ = ref.unstabilised_hidden(P, R, forget, floored=True)
        np.testing.assert_allclose(ref.hidden(S), h_raw, rtol=1e-11, atol=1e-13, err_msg=forget)
        active = np.abs(S[..., 1, :]) < np.exp(-S[..., 2, :])
        assert active.mean() > 0.02, forget
        h_exact = ref.hidden(ref.sequential(P, R, None, forget))
        assert np.max(np.abs(h_exact - ref.hidden(S))) > 1e-3, forget


def pin_stabiliser_invariants(ref):
    """Along a sequential trajectory: i', f' in (0, 1], max(i', f') = 1 exactly, n > 0,
    |c| <= n, |h| < 1 (educational page, stabiliser section; the exponent arguments stay
    at or below zero)."""
    for forget, seed, fb in (("exp", 3, 3.0), ("sigmoid", 4, 3.0), ("exp", 5, -2.0)):
        P, R = small_problem(seed, T=96, forget=forget, forget_bias=fb)
        P[:, ::7, 1, :] *= 8.0  # input-gate spikes so both branches are taken
        S = ref.sequential(P, R, None, forget)
        prev = np.concatenate([np.zeros_like(S[:, :1]), S[:, :-1]], axis=1)
        ig, fg, m, a, it = ref.gate_values(prev, P, R, forget)
        assert np.all(ig > 0) and np.all(ig <= 1) and np.all(fg > 0) and np.all(fg <= 1)
        assert np.all(np.maximum(ig, fg) == 1.0)
        np.testing.assert_array_equal(m, np.maximum(a, it))
        assert np.any(it > a) and np.any(a > it), "both branches should be exercised"
        c, n, h = S[..., 0, :], S[..., 1, :], S[..., 3, :]
        assert np.all(n > 0) and np.all(np.abs(c) <= n * (1 + 1e-15)) and np.all(np.abs(h) < 1)


def pin_zero_state_closed_forms(ref):
    """With z constant over time and zero initial state, c_t = z n_t for all t, so
    h_t = o_t z whatever the gates do."""
    P, R = small_problem(6, T=40)
    R[0] = 0.0  # r_z = 0 keeps z constant
    P[:, :, 0, :] = P[:, :1, 0, :]
    S = ref.sequential(P, R, None, "exp")
    z = np.tanh(P[:, 0, 0, :])
    hprev = np.concatenate([np.zeros_like(S[:, :1, 3]), S[:, :-1, 3]], axis=1)
    o = 1.0 / (1.0 + np.exp(-(P[:, :, 3, :] + R[3] * hprev)))
    np.testing.assert_allclose(S[..., 3, :], o * z[:, None, :], rtol=1e-12, atol=1e-15)


def pin_maxplus_closed_form(ref):
    """The stabiliser of the R-free trajectory solves m_t = max(l_t + m_{t-1}, i~_t), whose
    closed form is max(m_0 + sum_{u<=t} l_u, max_s (i~_s + sum_{s<u<=t} l_u))."""
    for forget, seed in (("exp", 7), ("sigmoid", 8)):
        P, R = small_problem(seed, T=50, forget=forget, forget_bias=0.5)
        state0 = np.zeros((2, 4, 16))
        state0[:, 2, :] = np.linspace(-3, 3, 16)
        S0 = ref.warm_start(P, state0, forget)
        lf, _ = ref.log_forget(P[:, :, 2, :], forget)
        it = P[:, :, 1, :]
        T = P.shape[1]
        for t in range(T):
            cand = [state0[:, 2, :] + lf[:, :t + 1].sum(axis=1)]
            for s in range(t + 1):
                cand.append(it[:, s] + lf[:, s + 1:t + 1].sum(axis=1))
            np.testing.assert_allclose(S0[:, t, 2, :], np.max(cand, axis=0), rtol=1e-12,
                                       atol=1e-12)


def pin_warm_start_is_solution_when_r_zero(ref):
    """With R = 0 the warm start is the sequential solution: F^0 = 0 up to rounding."""
    P, R = small_problem(9)
    R0 = np.zeros_like(R)
    S0 = ref.warm_start(P, None, "exp")
    np.testing.assert_allclose(S0, ref.sequential(P, R0, None, "exp"), rtol=0, atol=0)
    F, _ = ref.residual(S0, P, R0, None, "exp", with_jacobian=False)
    assert ref.max_abs(F) == 0.0


def pin_jacobian_finite_differences(ref):
    """Analytic 4x4 Jacobian against central differences, away from branch ties."""
    for forget, seed in (("exp", 10), ("sigmoid", 11), ("exp/floored", 12), ("sigmoid/floored", 13)):
        rng = np.random.Generator(np.random.PCG64(seed))
        d = 64
        prev = np.stack([rng.uniform(-2, 2, d), np.exp(rng.uniform(-1, 2, d)),
                         rng.uniform(-3, 3, d), rng.uniform(-0.9, 0.9, d)])[None]
        prev[0, 0] = np.clip(prev[0, 0], -prev[0, 1], prev[0, 1])
        p = rng.standard_normal((1, 4, d)) * 2.0
        r = rng.uniform(-0.5, 0.5, (4, d))
        _, A = ref.cell(prev, p, r, forget, with_jacobian=True)
        _, _, _, a, it = ref.gate_values(prev, p, r, forget)
        ok = np.abs(a - it)[0] > 1e-3
        if forget.endswith(ref.FLOORED):
            # away from the read-out's own branch switch |n| = e^{-m}, and with the floor active
            # on some features
            nxt = ref.cell(prev, p, r, forget)[0]
            gap = np.abs(np.abs(nxt[1]) - np.exp(-nxt[2]))
            ok &= gap > 1e-3
            assert np.sum(ok & (np.abs(nxt[1]) < np.exp(-nxt[2]))) > 4, forget
        assert ok.sum() > d // 2
        eps = 1e-6
        for col in range(4):
            e = np.zeros_like(prev)
            e[0, col] = eps
            num = (ref.cell(prev + e, p, r, forget) - ref.cell(prev - e, p, r, forget)) / (2 * eps)
            np.testing.assert_allclose(A[0, :, col][:, ok], num[0][:, ok], rtol=1e-6, atol=1e-8,
                                       err_msg=f"{forget} column {col}")
        # structural zeros of the channelwise cell
        for row, col in ((0, 1), (1, 0), (2, 0), (2, 1)):
            assert np.all(A[0, row, col] == 0)


def pin_jacobian_at_ties(ref):
    """At an exact tie a = i~ the forget branch is taken, and the Jacobian is that branch's
    one-sided derivative: the forward difference in m' (which moves a above i~)."""
    for forget in ("exp", "sigmoid"):
        rng = np.random.Generator(np.random.PCG64(21))
        d = 16
        prev = np.stack([rng.uniform(-1, 1, d), np.exp(rng.uniform(0, 1, d)),
                         rng.uniform(-3, 3, d), rng.uniform(-0.9, 0.9, d)])[None]
        r = rng.uniform(-0.5, 0.5, (4, d))
        r[1] = 0.0  # i~ = p_i exactly
        p = rng.standard_normal((1, 4, d))
        lf, _ = ref.log_forget(p[:, 2] + r[2] * prev[:, 3], forget)
        p[:, 1] = lf + prev[:, 2]  # a == i~ bit for bit
        _, A = ref.cell(prev, p, r, forget, with_jacobian=True)
        eps = 1e-7
        e = np.zeros_like(prev)
        e[0, 2] = eps
        fwd = (ref.cell(prev + e, p, r, forget) - ref.cell(prev, p, r, forget)) / eps
        np.testing.assert_allclose(A[0, :, 2], fwd[0], rtol=1e-5, atol=1e-6, err_msg=forget)
        np.testing.assert_array_equal(A[0, 2, 2], 1.0)


def pin_forward_substitution_closed_form(ref):
    """x_t = a x_{t-1} + 1 with scalar-times-identity A_t: x_t = (1 - a^t) / (1 - a)."""
    T, d = 30, 3
    a = np.array([0.5, -0.8, 0.9])
    A = np.zeros((1, T, 4, 4, d))
    for i in range(4):
        A[0, :, i, i, :] = a
    rhs = np.ones((1, T, 4, d))
    x = ref.forward_substitution(A, rhs)
    t = np.arange(1, T + 1)[:, None]
    expect = (1 - a[None, :] ** t) / (1 - a[None, :])
    for i in range(4):
        np.testing.assert_allclose(x[0, :, i, :], expect, rtol=1e-13)


def pin_forward_substitution_vs_dense_lu(ref):
    """Block forward substitution against a dense LAPACK solve of the assembled system,
    at Jacobians of a real iterate (tiny workload shape)."""
    P, R = small_problem(12)
    S = ref.warm_start(P, None, "exp")
    F, A = ref.residual(S, P, R, None, "exp")
    D = ref.forward_substitution(A, -F)
    for b in range(2):
        for j in (0, 5, 15):
            dense = ref.dense_solve_lane(A[b, :, :, :, j], F[b, :, :, j])
            np.testing.assert_allclose(D[b, :, :, j], dense, rtol=1e-10, atol=1e-12)


def pin_scan_bracketing(ref):
    """The affine maps compose associatively: a tree-ordered reduction of (A_t, r_t) gives
    the same final x_T as forward substitution."""
    rng = np.random.Generator(np.random.PCG64(13))
    T, d = 37, 5
    A = rng.uniform(-0.5, 0.5, (1, T, 4, 4, d))
    r = rng.standard_normal((1, T, 4, d))
    x = ref.forward_substitution(A, r)

    def compose(first, second):  # apply first, then second
        A1, b1 = first
        A2, b2 = second
        return np.einsum("ijd,jkd->ikd", A2, A1), np.einsum("ijd,jd->id", A2, b1) + b2

    maps = [(np.zeros((4, 4, d)), r[0, 0])] + [(A[0, t], r[0, t]) for t in range(1, T)]
    while len(maps) > 1:  # pairwise tree reduction
        nxt = [compose(maps[i], maps[i + 1]) for i in range(0, len(maps) - 1, 2)]
        if len(maps) % 2:
            nxt.append(maps[-1])
        maps = nxt
    np.testing.assert_allclose(maps[0][1], x[0, -1], rtol=1e-12, atol=1e-12)


def pin_newton_prefix_exactness(ref):
    """From the zero iterate, k Newton updates make the first k steps exact (s_0 is fixed
    and a step is exact once its predecessor is)."""
    P, R = small_problem(14, T=24, d=8)
    seq = ref.sequential(P, R, None, "exp")
    for k in (1, 2, 3, 5):
        S, st = ref.newton(P, R, None, "exp", k, init="zero")
        assert st.iters == k
        np.testing.assert_allclose(S[:, :k], seq[:, :k], rtol=1e-9, atol=1e-12, err_msg=f"k={k}")


def pin_newton_k_equals_t(ref):
    """K = T Newton iterations reproduce the sequential recurrence (same forward either
    way: 'sLSTM in this library', 'API notes', solver modes)."""
    P, R = small_problem(15, T=16, d=8)
    S, st = ref.newton(P, R, None, "exp", 16, init="zero")
    seq = ref.sequential(P, R, None, "exp")
    np.testing.assert_allclose(S, seq, rtol=1e-9, atol=1e-12)
    S, st = ref.newton(P, R, None, "exp", 16, init="warm")
    np.testing.assert_allclose(S, seq, rtol=1e-12, atol=1e-13)


def pin_newton_quadratic(ref):
    """Near the solution max|F| roughly squares per iteration, and the warm-started solve
    converges to the sequential trajectory."""
    P, R = small_problem(16, B=2, T=256, d=16)
    S, st = ref.newton(P, R, None, "exp", 4)
    e = st.max_abs_F
    floor = 16 * np.finfo(np.float64).eps * np.max(np.abs(S))  # rounding floor of |F|
    assert len(e) == 5 and e[0] < 1.0
    for k in range(3):
        assert e[k + 1] < 10 * e[k] ** 2 + floor, e
    assert e[2] > floor and e[-1] <= floor
    np.testing.assert_allclose(S, ref.sequential(P, R, None, "exp"), rtol=1e-10, atol=1e-12)


def pin_early_stop_and_flags(ref):
    """Early stop before the solve once max|F| < tol; divergence when max|F| > 1 or
    non-finite after the last iterate ('Layout', 'Current surface (0.17)')."""
    P, R = small_problem(17, T=128, forget="sigmoid")
    S, st = ref.newton(P, R, None, "sigmoid", 8, tol=1e-5)
    assert st.converged and not st.diverged
    assert st.max_abs_F[st.iters] < 1e-5 and all(e >= 1e-5 for e in st.max_abs_F[:st.iters])
    assert len(st.max_abs_F) == st.iters + 1
    # the divergence rule itself: max|F| > 1 after the last iterate, or non-finite
    for e, tol, want in ((0.5, 0.0, (False, False, False)), (1.0, 0.0, (False, False, False)),
                         (1.5, 0.0, (False, True, False)), (3e-6, 1e-5, (True, False, False)),
                         (2e-5, 1e-5, (False, False, False)), (np.inf, 0.0, (False, True, True)),
                         (np.nan, 1e-5, (False, True, True))):
        assert tuple(ref.newton_flags(e, tol)) == want, (e, tol)
    # a NaN in the inputs gives a non-finite residual and the divergence flag
    Pn = P.copy()
    Pn[0, 5, 1, 3] = np.nan
    _, st = ref.newton(Pn, R, None, "sigmoid", 3)
    assert st.diverged and st.nonfinite
    # the zero iterate overflows on a long exponential-forget sequence
    P2, R2 = small_problem(18, B=2, T=1024, d=32)
    _, st = ref.newton(P2, R2, None, "exp", 3, init="zero")
    assert st.diverged


def pin_input_projection(ref):
    """P = W_x x + b: one-hot weight rows pick single input features into the right gate
    and feature slots; small sizes against an explicit triple loop."""
    B, T, d_in, d_h = 2, 3, 5, 4
    rng = np.random.Generator(np.random.PCG64(19))
    x = rng.standard_normal((B, T, d_in))
    W = np.zeros((4, d_h, d_in))
    picks = {}
    for g in range(4):
        for j in range(d_h):
            k = (3 * g + j) % d_in
            W[g, j, k] = g + 1.0
            picks[g, j] = k
    bias = rng.standard_normal((4, d_h))
    P = ref.input_projection(x, W, bias)
    assert P.shape == (B, T, 4, d_h)
    for (g, j), k in picks.items():
        np.testing.assert_allclose(P[:, :, g, j], (g + 1.0) * x[:, :, k] + bias[g, j], rtol=1e-15)
    W = rng.standard_normal((4, d_h, d_in))
    P = ref.input_projection(x, W, bias)
    for b in range(B):
        for t in range(T):
            for g in range(4):
                for j in range(d_h):
                    acc = bias[g, j]
                    for k in range(d_in):
                        acc += x[b, t, k] * W[g, j, k]
                    assert abs(P[b, t, g, j] - acc) < 1e-12


def pin_input_projection_backward(ref):
    """dW, dx, dbias of L = sum dP * input_projection(x, W, b): L is linear in each of W, x and
    b, so a central difference along any direction E equals <grad, E> up to rounding; and an
    explicit loop on one entry of each."""
    B, T, d_in, d_h = 2, 3, 5, 4
    rng = np.random.Generator(np.random.PCG64(23))
    x = rng.standard_normal((B, T, d_in))
    W = rng.standard_normal((4, d_h, d_in))
    b = rng.standard_normal((4, d_h))
    dP = rng.standard_normal((B, T, 4, d_h))
    dW, dx, db = ref.input_projection_backward(x, W, dP)
    assert dW.shape == W.shape and dx.shape == x.shape and db.shape == b.shape
    L = lambda x_, W_, b_: float(np.sum(dP * ref.input_projection(x_, W_, b_)))  # noqa: E731
    for grad, arg in ((dW, 1), (dx, 0), (db, 2)):
        E = rng.standard_normal(grad.shape)
        args_p = [x, W, b]
        args_m = [x, W, b]
        args_p[arg] = args_p[arg] + 0.5 * E
        args_m[arg] = args_m[arg] - 0.5 * E
        fd = L(*args_p) - L(*args_m)
        assert abs(fd - float(np.sum(grad * E))) < 1e-10 * (1.0 + abs(fd))
    g, j, k, bb, t = 2, 3, 4, 1, 2
    assert abs(dW[g, j, k] - sum(dP[p, s, g, j] * x[p, s, k] for p in range(B) for s in range(T))) < 1e-12
    assert abs(dx[bb, t, k] - sum(dP[bb, t, q, i] * W[q, i, k] for q in range(4) for i in range(d_h))) < 1e-12
    assert abs(db[g, j] - sum(dP[p, s, g, j] for p in range(B) for s in range(T))) < 1e-12


def pin_state0_chunking(ref):
    """The final state carries a sequence: forward(T) = forward(T/2) then forward(T/2)
    from the carried state ('fused kernels prepend h0', 'Layout' page)."""
    P, R = small_problem(20, T=64)
    full = ref.sequential(P, R, None, "exp")
    first = ref.sequential(P[:, :32], R, None, "exp")
    second = ref.sequential(P[:, 32:], R, first[:, -1], "exp")
    np.testing.assert_allclose(np.concatenate([first, second], axis=1), full, rtol=0, atol=0)
    S, st = ref.newton(P[:, 32:], R, first[:, -1], "exp", 6)
    np.testing.assert_allclose(S, full[:, 32:], rtol=1e-11, atol=1e-13)


def _backward_problem(seed, forget, B=2, T=10, d=3, n_range=(0.5, 2.0)):
    P, R = small_problem(seed, B=B, T=T, d=d, forget=forget.split("/")[0])
    rng = np.random.default_rng(seed + 1)
    s0 = np.stack([rng.uniform(-0.5, 0.5, (B, d)), rng.uniform(*n_range, (B, d)),
                   rng.uniform(-2.0, 2.0, (B, d)), rng.uniform(-0.9, 0.9, (B, d))], axis=1)
    g = rng.standard_normal((B, T, 4, d))
    return P, R, s0, g


def pin_backward_finite_differences(ref):
    """The backward is the gradient of L = sum(g * S(P, R, state0)) with S the sequential
    solution: central differences in float64 on entries of P, every entry of R, and entries of
    state0, for both forget-gate forms ("sLSTM in this library", "Backward")."""
    for seed, forget in ((41, "exp"), (43, "sigmoid"), (45, "exp/floored"), (46, "sigmoid/floored")):
        P, R, s0, g = _backward_problem(seed, forget, n_range=(0.02, 0.3) if "/" in forget else (0.5, 2.0))
        if "/" in forget:
            P[:, :, 1, :] -= 1.5  # small input gates keep the floor active on some steps
        S = ref.sequential(P, R, s0, forget)
        if "/" in forget:
            assert np.any(np.abs(S[..., 1, :]) < np.exp(-S[..., 2, :])), forget
        dP, dR, ds0 = ref.backward(P, R, s0, S, g, forget)

        def loss(P_, R_, s_):
            return float(np.sum(g * ref.sequential(P_, R_, s_, forget)))

        eps = 1e-6
        scale = max(1.0, float(np.max(np.abs(dP))), float(np.max(np.abs(dR))))

        def fd(which, idx):
            args_p = [P.copy(), R.copy(), s0.copy()]
            args_m = [P.copy(), R.copy(), s0.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            return (loss(*args_p) - loss(*args_m)) / (2 * eps)

        for idx in [(0, 0, 0, 0), (1, 5, 2, 1), (0, 9, 3, 2), (1, 3, 1, 0), (0, 7, 0, 2)]:
            assert abs(fd(0, idx) - dP[idx]) < 1e-6 * scale, (forget, "P", idx)
        for gi in range(4):
            for j in range(R.shape[1]):
                assert abs(fd(1, (gi, j)) - dR[gi, j]) < 1e-6 * scale, (forget, "R", gi, j)
        for idx in [(0, 0, 1), (1, 2, 2), (0, 3, 0), (1, 1, 2)]:
            assert abs(fd(2, idx) - ds0[idx]) < 1e-6 * scale, (forget, "state0", idx)


def _packed_problem(seed, lengths, d=5, forget="exp"):
    """A packed problem: sequences of the given lengths (empty and length-1 ones included) one
    after the other along T, each with its own state0."""
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(int)
    T = int(cu[-1])
    P, R = small_problem(seed, B=1, T=T, d=d, forget=forget)
    rng = np.random.default_rng(seed + 3)
    n = len(lengths)
    s0 = np.stack([rng.uniform(-0.5, 0.5, (n, d)), rng.uniform(0.5, 2.0, (n, d)),
                   rng.uniform(-2.0, 2.0, (n, d)), rng.uniform(-0.9, 0.9, (n, d))], axis=1)
    return P, R, s0, cu


PACKED_LENGTHS = [7, 0, 1, 12, 3, 0, 9]


def pin_packed_equals_separate(ref):
    """Packed sequences ("sLSTM in this library", "Packed sequences") are independent problems:
    the sequential forward, the warm start and a fixed-count Newton solve of the pack equal those
    of each sequence alone from its own state0, concatenated; final states are each sequence's
    last state (state0 for an empty one)."""
    for forget in ("exp", "sigmoid"):
        P, R, s0, cu = _packed_problem(71, PACKED_LENGTHS, forget=forget)
        seq = ref.sequential(P, R, s0, forget, cu_seqlens=cu)
        warm = ref.warm_start(P, s0, forget, cu_seqlens=cu)
        newt, st = ref.newton(P, R, s0, forget, 3, cu_seqlens=cu)
        fin = ref.final_states(seq, s0, cu)
        for s in range(len(PACKED_LENGTHS)):
            a, b = cu[s], cu[s + 1]
            if a == b:
                np.testing.assert_array_equal(fin[s], s0[s])
                continue
            one = ref.sequential(P[:, a:b], R, s0[s:s + 1], forget)
            np.testing.assert_allclose(seq[:, a:b], one, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(warm[:, a:b], ref.warm_start(P[:, a:b], s0[s:s + 1], forget),
                                       rtol=1e-13, atol=1e-15)
            S1, _ = ref.newton(P[:, a:b], R, s0[s:s + 1], forget, 3)
            np.testing.assert_allclose(newt[:, a:b], S1, rtol=1e-12, atol=1e-14)
            np.testing.assert_array_equal(fin[s], seq[0, b - 1])


def pin_packed_early_stop_is_global(ref):
    """One residual norm covers the pack: each iterate's max|F| is the largest over the
    sequences solved alone, and the stop comes when that maximum meets the tolerance."""
    P, R, s0, cu = _packed_problem(73, [30, 5, 40], forget="sigmoid")
    tol = 1e-6
    _, st = ref.newton(P, R, s0, "sigmoid", 8, tol=tol, cu_seqlens=cu)
    alone = [ref.newton(P[:, cu[s]:cu[s + 1]], R, s0[s:s + 1], "sigmoid", 8)[1].max_abs_F for s in range(3)]
    glob = [max(h[k] for h in alone) for k in range(9)]
    stop = next((k for k in range(9) if glob[k] < tol), None)
    assert stop is not None and st.iters == stop and st.converged
    np.testing.assert_allclose(st.max_abs_F, glob[:stop + 1], rtol=1e-6, atol=1e-15)


def pin_packed_backward(ref):
    """The packed backward is the backward of each sequence alone: dP concatenated, dR summed,
    dstate0 per sequence (an empty sequence passes its final-state gradient to its state0),
    with the final-state gradients added at each sequence's last step."""
    P, R, s0, cu = _packed_problem(75, PACKED_LENGTHS)
    S = ref.sequential(P, R, s0, "exp", cu_seqlens=cu)
    rng = np.random.default_rng(76)
    g = rng.standard_normal(S.shape)
    gf = rng.standard_normal(s0.shape)
    dP, dR, ds0 = ref.backward(P, R, s0, S, g, "exp", cu_seqlens=cu, g_final=gf)
    dR_sum = np.zeros_like(dR)
    for s in range(len(PACKED_LENGTHS)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            np.testing.assert_array_equal(ds0[s], gf[s])
            continue
        d1, r1, s1 = ref.backward(P[:, a:b], R, s0[s:s + 1], S[:, a:b], g[:, a:b], "exp", g_final=gf[s:s + 1])
        np.testing.assert_allclose(dP[:, a:b], d1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ds0[s], s1[0], rtol=1e-12, atol=1e-14)
        dR_sum += r1
    np.testing.assert_allclose(dR, dR_sum, rtol=1e-12, atol=1e-13)


def pin_backward_adjoint_dense(ref):
    """The reverse recurrence solves the transposed block-bidiagonal system: its adjoint equals a
    dense LAPACK solve of J^T lam = g for every lane (J the forward Newton matrix)."""
    P, R, s0, g = _backward_problem(47, "exp", T=12)
    S = ref.sequential(P, R, s0, "exp")
    _, A = ref.residual(S, P, R, s0, "exp")
    _, _, _, lam = ref.backward(P, R, s0, S, g, "exp", return_adjoint=True)
    for b in range(P.shape[0]):
        for j in range(P.shape[-1]):
            dense = ref.dense_adjoint_lane(A[b, :, :, :, j], g[b, :, :, j])
            np.testing.assert_allclose(lam[b, :, :, j], dense, rtol=1e-10, atol=1e-12)


def pin_gate_jacobian_h_column(ref):
    """h' enters the cell only through the gate pre-activations x~ = p + r h', so the h' column
    of the state Jacobian is G r (G = d next / d x~), to rounding."""
    for forget in ("exp", "sigmoid", "exp/floored", "sigmoid/floored"):
        P, R = small_problem(53, T=8, forget=forget.split("/")[0])
        P[:, :, 1, :] -= 1.5
        S = ref.sequential(P, R, None, forget)
        prev = S[:, :-1]
        _, A = ref.cell(prev, P[:, 1:], R, forget, with_jacobian=True)
        G = ref.gate_jacobian(prev, P[:, 1:], R, forget)
        np.testing.assert_allclose(A[..., :, 3, :], np.einsum("btsgd,gd->btsd", G, R), rtol=1e-12, atol=1e-14)


# ---- head mixing ("sLSTM in this library", "Cell": mix='head'; summary card "Method" item 2) ----
def _head_problem(seed, B=2, T=7, nh=2, dh=3, forget="sigmoid"):
    rng = np.random.default_rng(seed)
    d = nh * dh
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += 2.0
    R = rng.uniform(-0.4, 0.4, (4, nh, dh, dh))
    s0 = np.zeros((B, 4, d))
    s0[:, 0] = rng.uniform(-0.5, 0.5, (B, d))
    s0[:, 1] = rng.uniform(0.5, 2.0, (B, d))
    s0[:, 2] = rng.uniform(-1.0, 1.0, (B, d))
    s0[:, 3] = rng.uniform(-0.5, 0.5, (B, d))
    return P, R, s0


def pin_head_recurrent_worked_example(ref):
    """R_g h' by hand for two heads of two units: row i of block (g, a) meets unit k of head a."""
    R = np.zeros((4, 2, 2, 2))
    R[0, 0, 0, 1] = 2.0    # gate z, head 0: unit 0 reads unit 1
    R[2, 1, 1, 0] = -1.0   # gate f, head 1: unit 1 reads unit 0 (feature 2)
    h = np.array([0.5, 3.0, 7.0, 11.0])
    y = ref.head_recurrent(h, R)
    want = np.zeros((4, 4))
    want[0, 0] = 6.0
    want[2, 3] = -7.0
    np.testing.assert_array_equal(y, want)


def pin_head_width_one_is_channelwise(ref):
    """d_head = 1: block (g, j) is the channelwise weight r[g, j]; the step, its Jacobian and the
    Newton solve are the channelwise ones."""
    rng = np.random.default_rng(91)
    B, T, d = 2, 6, 5
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += 2.0
    r = rng.uniform(-0.5, 0.5, (4, d))
    Rh = r.reshape(4, d, 1, 1).copy()
    np.testing.assert_array_equal(ref.sequential_head(P, Rh, None, "exp"), ref.sequential(P, r, None, "exp"))
    S = ref.sequential(P, r, None, "exp")
    _, A = ref.cell(S[:, 2], P[:, 3], r, "exp", with_jacobian=True)
    _, J = ref.cell_head(S[:, 2], P[:, 3], Rh, "exp", with_jacobian=True)
    np.testing.assert_allclose(J, np.moveaxis(A, -1, 1), rtol=1e-14, atol=1e-15)
    Sd, _ = ref.newton(P, r, None, "exp", 3)
    Sh, _ = ref.newton_head(P, Rh, None, "exp", 3)
    np.testing.assert_allclose(Sh, Sd, rtol=1e-12, atol=1e-13)


def pin_head_diagonal_blocks_are_channelwise(ref):
    """Blocks that are diagonal (unit i reads only itself) give the channelwise recurrence."""
    rng = np.random.default_rng(92)
    B, T, nh, dh = 2, 6, 2, 3
    d = nh * dh
    P = rng.standard_normal((B, T, 4, d))
    r = rng.uniform(-0.5, 0.5, (4, d))
    R = np.zeros((4, nh, dh, dh))
    for a in range(nh):
        for i in range(dh):
            R[:, a, i, i] = r[:, a * dh + i]
    np.testing.assert_array_equal(ref.sequential_head(P, R, None, "sigmoid"), ref.sequential(P, r, None, "sigmoid"))


def pin_head_jacobian_finite_differences(ref):
    """Dense per-head Jacobian against central differences of the step, column by column; a
    perturbation in one head leaves the other heads' next states unchanged."""
    P, R, s0 = _head_problem(93)
    B, T, _, d = P.shape
    nh, dh = R.shape[1], R.shape[2]
    S = ref.sequential_head(P, R, s0, "sigmoid")
    prev, p = S[:, 2], P[:, 3]
    _, J = ref.cell_head(prev, p, R, "sigmoid", with_jacobian=True)
    eps = 1e-6
    for col in range(4):
        for j in range(d):
            dp = np.zeros_like(prev)
            dp[:, col, j] = eps
            fd = (ref.cell_head(prev + dp, p, R, "sigmoid") - ref.cell_head(prev - dp, p, R, "sigmoid")) / (2 * eps)
            a, k = divmod(j, dh)
            got = J[:, a, :, 4 * k + col].reshape(B, dh, 4)
            np.testing.assert_allclose(got, np.moveaxis(fd[:, :, a * dh:(a + 1) * dh], 1, 2), rtol=1e-6, atol=1e-8)
            for o in range(nh):
                if o != a:
                    assert np.max(np.abs(fd[:, :, o * dh:(o + 1) * dh])) == 0.0


def pin_head_newton_exact_at_k_equals_t(ref):
    """From the zero iterate, T Newton steps give the sequential solution exactly (the first k
    steps are exact after k iterations), and near the solution the residual falls
    quadratically."""
    P, R, s0 = _head_problem(94, T=5)
    T = P.shape[1]
    S, st = ref.newton_head(P, R, s0, "sigmoid", T, init=ref.INIT_ZERO)
    np.testing.assert_allclose(S, ref.sequential_head(P, R, s0, "sigmoid"), rtol=1e-13, atol=1e-14)
    _, st = ref.newton_head(P, R, s0, "sigmoid", 4)
    e = st.max_abs_F
    assert e[2] < 0.1 and e[3] < 4.0 * e[2] ** 2 and e[4] < 4.0 * e[3] ** 2 + 1e-14, e


def pin_head_forward_substitution_vs_dense(ref):
    """The block solve with dense per-head blocks against a LAPACK solve of the assembled
    (T 4 d_head) system of one head."""
    rng = np.random.default_rng(95)
    B, T, nh, dh = 1, 5, 2, 2
    J = rng.uniform(-0.5, 0.5, (B, T, nh, 4 * dh, 4 * dh))
    rhs = rng.standard_normal((B, T, 4, nh * dh))
    x = ref.forward_substitution_head(J, rhs, nh)
    for a in range(nh):
        n = 4 * dh
        M = np.eye(T * n)
        for t in range(1, T):
            M[t * n:(t + 1) * n, (t - 1) * n:t * n] = -J[0, t, a]
        rv = ref.head_vectors(rhs, nh)[0, :, a].reshape(-1)
        want = np.linalg.solve(M, rv).reshape(T, n)
        np.testing.assert_allclose(ref.head_vectors(x, nh)[0, :, a], want, rtol=1e-12, atol=1e-13)


def pin_head_units_permute(ref):
    """Renumbering the units of a head (columns of P and state0, rows and columns of its blocks)
    renumbers the solution."""
    P, R, s0 = _head_problem(96, T=6)
    dh = R.shape[2]
    perm = np.array([2, 0, 1])
    full = np.concatenate([perm, dh + np.arange(dh)])      # permute head 0 only
    Rp = R.copy()
    Rp[:, 0] = R[:, 0][:, perm][:, :, perm]
    S = ref.sequential_head(P, R, s0, "sigmoid")
    Sp = ref.sequential_head(P[..., full], Rp, s0[..., full], "sigmoid")
    np.testing.assert_allclose(Sp, S[..., full], rtol=1e-14, atol=1e-15)
    Sn, _ = ref.newton_head(P, R, s0, "sigmoid", 2)
    Snp, _ = ref.newton_head(P[..., full], Rp, s0[..., full], "sigmoid", 2)
    np.testing.assert_allclose(Snp, Sn[..., full], rtol=1e-12, atol=1e-13)


def pin_head_backward_finite_differences(ref):
    """dP, dR and dstate0 of a loss L = sum g S + sum g_final S_T through the sequential head
    recurrence, against central differences along random directions (both forget gates and the
    floored read-out)."""
    P, R, s0 = _head_problem(97, T=6)
    rng = np.random.default_rng(98)
    g = rng.standard_normal(P.shape)
    gf = rng.standard_normal(s0.shape)
    eps = 1e-6
    for forget in ("exp", "sigmoid", "sigmoid" + ref.FLOORED):
        S = ref.sequential_head(P, R, s0, forget)
        dP, dR, d0 = ref.backward_head(P, R, s0, S, g, forget, g_final=gf)

        def loss(P_, R_, s_):
            S_ = ref.sequential_head(P_, R_, s_, forget)
            return float(np.sum(g * S_) + np.sum(gf * S_[:, -1]))

        for which, X, grad in (("P", P, dP), ("R", R, dR), ("state0", s0, d0)):
            E = rng.standard_normal(X.shape)
            plus = [P, R, s0]
            minus = [P, R, s0]
            k = ("P", "R", "state0").index(which)
            plus[k], minus[k] = X + eps * E, X - eps * E
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - float(np.sum(grad * E))) <= 1e-6 * max(1.0, abs(fd)), (forget, which)


def pin_head_backward_diagonal_blocks_are_channelwise(ref):
    """Diagonal blocks: dP and dstate0 are the channelwise backward's, and the diagonal of dR is
    its dR (the off-diagonal entries are the gradients of weights that happen to be zero)."""
    P, R, s0 = _head_problem(99, T=7)
    nh, dh = R.shape[1], R.shape[2]
    r = np.concatenate([np.stack([np.diag(R[q, a]) for a in range(nh)]).reshape(-1)[None] for q in range(4)])
    Rd = np.zeros_like(R)
    for q in range(4):
        for a in range(nh):
            Rd[q, a] = np.diag(r[q, a * dh:(a + 1) * dh])
    rng = np.random.default_rng(100)
    g = rng.standard_normal(P.shape)
    for forget in ("exp", "sigmoid"):
        S = ref.sequential_head(P, Rd, s0, forget)
        dP, dR, d0 = ref.backward_head(P, Rd, s0, S, g, forget)
        cP, cR, c0 = ref.backward(P, r, s0, S, g, forget)
        np.testing.assert_allclose(dP, cP, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(d0, c0, rtol=1e-12, atol=1e-13)
        diag = np.stack([np.concatenate([np.diag(dR[q, a]) for a in range(nh)]) for q in range(4)])
        np.testing.assert_allclose(diag, cR, rtol=1e-12, atol=1e-13)


def pin_head_backward_width_one_is_channelwise(ref):
    """d_head = 1: every output of the head backward is the channelwise backward's."""
    rng = np.random.default_rng(101)
    B, T, d = 2, 8, 5
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += 2.0
    r = rng.uniform(-0.5, 0.5, (4, d))
    g = rng.standard_normal(P.shape)
    gf = rng.standard_normal((B, 4, d))
    S = ref.sequential(P, r, None, "sigmoid")
    dP, dR, d0 = ref.backward_head(P, r.reshape(4, d, 1, 1), None, S, g, "sigmoid", g_final=gf)
    cP, cR, c0 = ref.backward(P, r, None, S, g, "sigmoid", g_final=gf)
    np.testing.assert_allclose(dP, cP, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dR.reshape(4, d), cR, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(d0, c0, rtol=1e-12, atol=1e-13)


def _head_pack(seed, lengths, nh=2, dh=3):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, n, d = int(cu[-1]), len(lengths), nh * dh
    P = rng.standard_normal((1, T, 4, d))
    P[:, :, 2] += 2.0
    R = rng.uniform(-0.4, 0.4, (4, nh, dh, dh))
    s0 = np.zeros((n, 4, d))
    s0[:, 0] = rng.uniform(-0.5, 0.5, (n, d))
    s0[:, 1] = rng.uniform(0.5, 2.0, (n, d))
    s0[:, 2] = rng.uniform(-1.0, 1.0, (n, d))
    s0[:, 3] = rng.uniform(-0.5, 0.5, (n, d))
    return P, R, s0, cu


def pin_head_packed_equals_separate(ref):
    """Packed head mixing is the sequences solved one by one: the sequential forward, Newton at
    a fixed count, final states; with an early stop the pack stops once for all, at the
    iterate each sequence reaches in that many iterations."""
    lengths = [3, 0, 5, 1, 4]
    P, R, s0, cu = _head_pack(102, lengths)
    for forget in ("exp", "sigmoid"):
        S = ref.sequential_head(P, R, s0, forget, cu_seqlens=cu)
        Sn, st = ref.newton_head(P, R, s0, forget, 3, cu_seqlens=cu)
        Se, ste = ref.newton_head(P, R, s0, forget, 8, tol=1e-6, cu_seqlens=cu)
        assert ste.converged and ste.iters < 8
        for q in range(len(lengths)):
            a, b = int(cu[q]), int(cu[q + 1])
            if a == b:
                continue
            Pq = P[:, a:b]
            np.testing.assert_allclose(S[:, a:b], ref.sequential_head(Pq, R, s0[q:q + 1], forget), rtol=1e-13, atol=1e-14)
            Sq, _ = ref.newton_head(Pq, R, s0[q:q + 1], forget, 3)
            np.testing.assert_allclose(Sn[:, a:b], Sq, rtol=1e-11, atol=1e-12)
            Sq, _ = ref.newton_head(Pq, R, s0[q:q + 1], forget, ste.iters)
            np.testing.assert_allclose(Se[:, a:b], Sq, rtol=1e-11, atol=1e-12)
        fin = ref.final_states(S, s0, cu)
        np.testing.assert_array_equal(fin[1], s0[1])   # the empty sequence keeps its state0


def pin_head_packed_backward(ref):
    """The packed head backward is the per-sequence backwards: dP and dstate0 per sequence, dR
    summed; an empty sequence passes its final-state gradient to dstate0."""
    lengths = [4, 0, 3, 6]
    P, R, s0, cu = _head_pack(103, lengths)
    rng = np.random.default_rng(104)
    g = rng.standard_normal(P.shape)
    gf = rng.standard_normal(s0.shape)
    S = ref.sequential_head(P, R, s0, "sigmoid", cu_seqlens=cu)
    dP, dR, d0 = ref.backward_head(P, R, s0, S, g, "sigmoid", g_final=gf, cu_seqlens=cu)
    dR_sum = np.zeros_like(dR)
    for q in range(len(lengths)):
        a, b = int(cu[q]), int(cu[q + 1])
        if a == b:
            np.testing.assert_array_equal(d0[q], gf[q])
            continue
        pq, rq, dq = ref.backward_head(P[:, a:b], R, s0[q:q + 1], S[:, a:b], g[:, a:b], "sigmoid", g_final=gf[q:q + 1])
        np.testing.assert_allclose(dP[:, a:b], pq, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(d0[q], dq[0], rtol=1e-12, atol=1e-13)
        dR_sum += rq
    np.testing.assert_allclose(dR, dR_sum, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------------------
# branch margin (chooses the lanes the backward's parity compares)
# ---------------------------------------------------------------------------------------
def pin_branch_margin_worked_example(ref):
    """|a - i~| and |l| + |m'| + |i~| at the state BEFORE each step, worked by hand.

    One lane, two steps, R = (0.2, 0.5, -0.5, 0.1), state0 = (c, n, m, h) = (0.5, 1, 0.25, 0.5),
    S_1 = (0.1, 2, -1.5, -0.25) (any S: the margin is defined at every iterate).
      t = 1 (previous state = state0): i~ = 0.5 + 0.5*0.5 = 0.75, f~ = 1.5 - 0.5*0.5 = 1.25;
        exponential gate: l = 1.25, a = l + m' = 1.5, margin 0.75, scale 1.25 + 0.25 + 0.75 = 2.25
      t = 2 (previous state = S_1): i~ = 2 + 0.5*(-0.25) = 1.875, f~ = 1 + (-0.5)(-0.25) = 1.125;
        a = 1.125 - 1.5 = -0.375, margin 2.25, scale 1.125 + 1.5 + 1.875 = 4.5
    With the sigmoid gate l = -ln(1 + e^{-f~}) (log of the logistic function) at the same f~.
    """
    R = np.array([0.2, 0.5, -0.5, 0.1])[:, None]
    s0 = np.array([0.5, 1.0, 0.25, 0.5])[None, :, None]
    S = np.zeros((1, 2, 4, 1))
    S[0, 0, :, 0] = [0.1, 2.0, -1.5, -0.25]
    S[0, 1, :, 0] = [0.3, 0.7, 9.0, 0.9]
    P = np.zeros((1, 2, 4, 1))
    P[0, 0, :, 0] = [0.0, 0.5, 1.5, 0.0]
    P[0, 1, :, 0] = [0.0, 2.0, 1.0, 0.0]
    margin, scale = ref.branch_margin(P, R, s0, S, "exp")
    np.testing.assert_allclose(margin[0, :, 0], [0.75, 2.25], rtol=0, atol=1e-15)
    np.testing.assert_allclose(scale[0, :, 0], [2.25, 4.5], rtol=0, atol=1e-15)
    margin, scale = ref.branch_margin(P, R, s0, S, "sigmoid")
    l1 = -math.log1p(math.exp(-1.25))
    l2 = -math.log1p(math.exp(-1.125))
    np.testing.assert_allclose(margin[0, :, 0], [abs(l1 + 0.25 - 0.75), abs(l2 - 1.5 - 1.875)],
                               rtol=1e-14)
    np.testing.assert_allclose(scale[0, :, 0], [abs(l1) + 0.25 + 0.75, abs(l2) + 1.5 + 1.875],
                               rtol=1e-14)
    # packed: a sequence starting at the second step takes its own state0 as the state before
    # it, here state0[1] = (0, 1, -2, 0): i~ = 2, f~ = 1, a = 1 - 2 = -1, margin 3, scale 5
    s0p = np.concatenate([s0, np.array([0.0, 1.0, -2.0, 0.0])[None, :, None]])
    margin, scale = ref.branch_margin(P, R, s0p, S, "exp", cu_seqlens=np.array([0, 1, 2]))
    np.testing.assert_allclose(margin[0, :, 0], [0.75, 3.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(scale[0, :, 0], [2.25, 5.0], rtol=0, atol=1e-15)


def pin_branch_margin_zero_at_ties(ref):
    """An exact tie a = i~ has margin 0, and a step moved off the tie by a known amount in m'
    has exactly that margin (a = l + m' moves with m', i~ does not)."""
    for forget in ("exp", "sigmoid"):
        rng = np.random.Generator(np.random.PCG64(31))
        d = 16
        s0 = np.stack([rng.uniform(-1, 1, d), np.exp(rng.uniform(0, 1, d)),
                       rng.uniform(-3, 3, d), rng.uniform(-0.9, 0.9, d)])[None]
        R = rng.uniform(-0.5, 0.5, (4, d))
        R[1] = 0.0                      # i~ = p_i exactly
        P = rng.standard_normal((1, 1, 4, d))
        lf, _ = ref.log_forget(P[:, 0, 2] + R[2] * s0[:, 3], forget)
        P[:, 0, 1] = lf + s0[:, 2]      # a == i~ bit for bit
        S = np.zeros((1, 1, 4, d))
        margin, _ = ref.branch_margin(P, R, s0, S, forget)
        np.testing.assert_array_equal(margin, 0.0)
        shift = 0.25 * np.arange(1, d + 1)      # exact in binary
        s1 = s0.copy()
        s1[:, 2] += shift
        margin, _ = ref.branch_margin(P, R, s1, S, forget)
        np.testing.assert_allclose(margin[0, 0], shift, rtol=1e-12, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
