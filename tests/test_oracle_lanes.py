"""The lane-block oracle runner against the whole-problem oracle, and the input recipe."""
import numpy as np
import torch

from oracle import lanes, slstm_ref as ref
from workloads import WORKLOADS, by_name, draw_preactivation_inputs, draw_layer_inputs
from workloads import gen


def _problem(seed, B=3, T=200, d=12, forget="sigmoid"):
    rng = np.random.Generator(np.random.PCG64(seed))
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d))
    s0 = np.zeros((B, 4, d))
    s0[:, 0] = rng.uniform(-0.5, 0.5, (B, d))
    s0[:, 1] = 1.0
    s0[:, 2] = rng.uniform(-1, 1, (B, d))
    s0[:, 3] = rng.uniform(-0.5, 0.5, (B, d))
    return P, R, s0


def test_newton_lanes_matches_whole_problem():
    P, R, s0 = _problem(1)
    S, st = ref.newton(P, R, s0, "sigmoid", 8, tol=1e-9)
    lb, lj = lanes.all_lanes(3, 12)
    got, st2 = lanes.newton_lanes(P, R, s0, "sigmoid", 8, 1e-9, lanes=(lb, lj), workers=2, block=7)
    assert st2.iters == st.iters and st2.converged == st.converged
    np.testing.assert_allclose(st2.max_abs_F, st.max_abs_F, rtol=1e-12)
    np.testing.assert_allclose(got, np.transpose(S, (0, 3, 1, 2)).reshape(-1, 200, 4),
                               rtol=1e-13, atol=1e-14)


def test_sequential_lanes_subset():
    P, R, s0 = _problem(2, forget="exp")
    full = ref.sequential(P, R, s0, "exp")
    lb = np.array([0, 2, 1])
    lj = np.array([11, 0, 5])
    got = lanes.sequential_lanes(P, R, s0, "exp", lanes=(lb, lj), workers=1)
    for k in range(3):
        np.testing.assert_array_equal(got[k], full[lb[k], :, :, lj[k]])


def test_packed_groups_cover_every_sequence():
    cu = [0, 0, 5, 5, 6, 20, 20, 21, 21]
    for n in (1, 2, 3, 5, 50):
        groups = lanes.packed_groups(cu, n)
        assert groups[0][0] == 0 and groups[-1][1] == len(cu) - 1
        assert all(a[1] == b[0] for a, b in zip(groups, groups[1:]))
        assert all(cu[b] > cu[a] for a, b in groups)  # at least one step per run
        assert len(groups) <= n


def test_packed_runs_match_one_call():
    """Runs of whole sequences solved apart reproduce the one-call packed oracle: forward,
    fixed-count Newton (states and residual history) and backward (dR summed over the runs)."""
    cu = gen.packed_offsets(5, 700, 60)
    T, n, d = int(cu[-1]), len(cu) - 1, 5
    rng = np.random.Generator(np.random.PCG64(9))
    P = rng.standard_normal((1, T, 4, d))
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d))
    s0 = np.stack([rng.uniform(-0.5, 0.5, (n, d)), rng.uniform(0.5, 2.0, (n, d)),
                   rng.uniform(-2.0, 2.0, (n, d)), rng.uniform(-0.9, 0.9, (n, d))], axis=1)
    for forget in ("exp", "sigmoid"):
        seq = ref.sequential(P, R, s0, forget, cu_seqlens=cu)
        np.testing.assert_array_equal(lanes.packed_sequential(P, R, s0, forget, cu, workers=3), seq)
        S, st = ref.newton(P, R, s0, forget, 3, cu_seqlens=cu)
        S2, st2 = lanes.packed_newton(P, R, s0, forget, 3, cu, workers=3)
        np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(st2.max_abs_F, st.max_abs_F, rtol=1e-12, atol=1e-300)
        g = rng.standard_normal(seq.shape)
        gf = rng.standard_normal((n, 4, d))
        want = ref.backward(P, R, s0, seq, g, forget, cu_seqlens=cu, g_final=gf)
        got = lanes.packed_backward(P, R, s0, seq, g, forget, cu, g_final=gf, workers=3)
        np.testing.assert_allclose(got[0], want[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(got[1], want[1], rtol=1e-11)
        np.testing.assert_allclose(got[2], want[2], rtol=1e-13, atol=1e-14)


def test_workload_recipe():
    names = [w.name for w in WORKLOADS]
    assert len(set(names)) == 5
    w = by_name("long_b4_t16384_d2048")
    x, W, R = gen._draw_x_w_r(w, B=1, T=1100)
    x0, _, _ = gen._draw_x_w_r(by_name("tiny_b2_t64_d16"), B=1, T=1100)
    assert x.shape == (1, 1100, 2048) and W.shape == (4, 2048, 2048)
    # 1-based every 512th step is scaled by 8: 0-based steps 511 and 1023
    big = np.abs(x).mean(axis=(0, 2))
    assert set(np.nonzero(big > 3.0)[0]) == {511, 1023}
    assert abs(W.var() - 1.0 / 2048) < 1e-5 and R.min() >= -0.5 and R.max() <= 0.5
    # same seed, same draw
    x2, _, _ = gen._draw_x_w_r(w, B=1, T=1100)
    np.testing.assert_array_equal(x, x2)


def test_preactivations_and_layer_inputs():
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    d = draw_preactivation_inputs(w, B=1, T=8)
    assert d["P"].dtype == torch.bfloat16 and tuple(d["P"].shape) == (1, 8, 4, 1024)
    # forget-gate row carries the +3 bias
    assert abs(d["P"][:, :, 2].float().mean().item() - 3.0) < 0.2
    assert abs(d["P"][:, :, 0].float().mean().item()) < 0.2
    lw = by_name("layer_b128_t2048_d1024")
    li = draw_layer_inputs(lw, B=2, T=4)
    assert li["x"].dtype == torch.bfloat16 and tuple(li["W"].shape) == (4, 1024, 1024)
    assert li["bias"][2].eq(3.0).all() and li["bias"][[0, 1, 3]].eq(0).all()
