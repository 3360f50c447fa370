"""Calibration of the h error metric against plain float32 arithmetic (CPU only).

The bar on h is a relative error of 1e-4 for float32 state. Element-wise relative error needs
a floor, since h crosses zero. These tests run the sLSTM recurrence as a plain float32 step
loop -- the most direct float32 evaluation there is -- against the float64 oracle. With the
exponential forget gate float32 meets the bar at the default floor 1e-3 with margin; with the
sigmoid forget gate a floor of 1e-3 asks for more than float32 can deliver, while 1e-2 leaves
a margin of several times under 1e-4.
"""
import numpy as np
import pytest

from oracle import slstm_ref as ref
from parity import H_FLOOR, H_FLOOR_SIGMOID, H_TOL_F32, h_floor
from workloads import by_name, draw_preactivation_inputs

f32 = np.float32


def _float32_step_loop(P, R, forget):
    P = P.astype(f32)
    R = R.astype(f32)
    B, T, _, d = P.shape
    c = np.zeros((B, d), f32)
    n = np.zeros((B, d), f32)
    m = np.zeros((B, d), f32)
    h = np.zeros((B, d), f32)
    hs = np.empty((B, T, d), f32)
    for t in range(T):
        p = P[:, t]
        z = np.tanh(p[:, 0] + R[0] * h)
        it = p[:, 1] + R[1] * h
        ft = p[:, 2] + R[2] * h
        o = f32(1) / (f32(1) + np.exp(-(p[:, 3] + R[3] * h)))
        lf = ft if forget == "exp" else (-np.logaddexp(f32(0), -ft)).astype(f32)
        a = lf + m
        mn = np.where(a >= it, a, it)
        ig = np.exp(it - mn)
        fg = np.exp(a - mn)
        c = fg * c + ig * z
        n = fg * n + ig
        m = mn
        h = o * c / n
        hs[:, t] = h
    return hs


def _rel(a, b, floor):
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor)))


@pytest.mark.parametrize("name,B,T,d", [("tiny_b2_t64_d16", None, None, 16),
                                        ("mid_b8_t1024_d256", None, None, 256),
                                        ("long_b4_t16384_d2048", 1, 4096, 64)])
def test_float32_meets_the_bar_at_the_default_floor(name, B, T, d):
    """Exponential forget gate (the tiny, mid and long-context workloads): float32 is inside
    1e-4 at the floor 1e-3 (measured 5.6e-7, 2.1e-5 and 7e-6)."""
    w = by_name(name)
    assert h_floor(w.forget, H_TOL_F32) == H_FLOOR == 1e-3
    inp = draw_preactivation_inputs(w, B=B, T=T)
    P = inp["P"].double().numpy()[..., :d]
    R = inp["R"].double().numpy()[:, :d]
    h64 = ref.hidden(ref.sequential(P, R, None, w.forget))
    with np.errstate(all="ignore"):
        h32 = _float32_step_loop(P, R, w.forget)
    assert _rel(h32, h64, H_FLOOR) < 0.5 * H_TOL_F32


def test_sigmoid_forget_needs_the_wider_floor():
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    assert h_floor(w.forget, H_TOL_F32) == H_FLOOR_SIGMOID
    inp = draw_preactivation_inputs(w, B=2, T=4096)
    P = inp["P"].double().numpy()[..., :256]
    R = inp["R"].double().numpy()[:, :256]
    h64 = ref.hidden(ref.sequential(P, R, None, w.forget))
    with np.errstate(all="ignore"):
        h32 = _float32_step_loop(P, R, w.forget)
    assert _rel(h32, h64, H_FLOOR) > 1e-4           # a 1e-3 floor is beyond float32 here
    assert _rel(h32, h64, H_FLOOR_SIGMOID) < 3e-5   # the wider floor: float32 passes with margin
    assert float(np.max(np.abs(h32 - h64))) < 1e-6
