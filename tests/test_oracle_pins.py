"""The float64 oracle against golden worked examples, closed forms, invariants, textbook
routines and brute force (CPU only). Also checks that planted mistakes in a copy of the
oracle are caught by at least one pin."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import pins
from oracle import slstm_ref

ORACLE_SRC = os.path.join(os.path.dirname(slstm_ref.__file__), "slstm_ref.py")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(slstm_ref)


# Each mutation: (label, original text, replacement). A mutation that no pin notices would
# mean the pins leave that part of the oracle unchecked.
MUTATIONS = [
    ("gate order i<->f", "it = p[..., GI, :] + r[GI] * h0\n    ft = p[..., GF, :] + r[GF] * h0\n    ot",
     "it = p[..., GF, :] + r[GF] * h0\n    ft = p[..., GI, :] + r[GI] * h0\n    ot"),
    ("dropped input term in c", "c = fg * c0 + ig * z\n", "c = fg * c0\n"),
    ("wrong sign in stabiliser gate", "ig = np.exp(it - m)\n    fg = np.exp(a - m)\n    c =",
     "ig = np.exp(m - it)\n    fg = np.exp(a - m)\n    c ="),
    ("tie to input branch", "beta = a >= it  # tie", "beta = a > it  # tie"),
    ("read-out floor variant", "return n, np.ones_like(n), np.zeros_like(n)",
     "return np.maximum(np.abs(n), 1.0), np.ones_like(n), np.zeros_like(n)"),
    ("quotient rule sign", "- q * (v[\"dD_dn\"] * dn[k]", "+ q * (v[\"dD_dn\"] * dn[k]"),
    ("missing output-gate term", "dh[H] = dh[H] + (c / v[\"D\"]) * do_dh", "dh[H] = dh[H]"),
    ("sigmoid-forget derivative", "return -_softplus(-f_tilde), sigmoid(-f_tilde)",
     "return -_softplus(-f_tilde), sigmoid(f_tilde)"),
    ("transposed Jacobian in the solve", 'np.einsum("bijd,bjd->bid", A[:, t], x[:, t - 1])',
     'np.einsum("bjid,bjd->bid", A[:, t], x[:, t - 1])'),
    ("off-by-one state shift", "prev[:, 1:] = S[:, :-1]", "prev[:, 1:] = S[:, 1:]"),
    ("transposed weight", "P = x.reshape(B * T, d_in) @ W.reshape(g * d_h, d_in).T",
     "P = x.reshape(B * T, d_in) @ W.transpose(0, 2, 1).reshape(g * d_h, d_in).T"),
    ("early stop after the solve", "if tol > 0 and e < tol:\n                stopped = True",
     "if tol > 0 and e < tol * 1e-30:\n                stopped = True"),
    ("divergence threshold", "diverged = nonfinite or e_final > 1.0", "diverged = nonfinite or e_final > 10.0"),
    ("backward: transposed gate Jacobian", 'np.einsum("bsgd,bsd->bgd", G, lam)', 'np.einsum("bgsd,bsd->bgd", G, lam)'),
    ("backward: dropped direct gradient", "lam = g[:, t - 1] + lam_prev if t > 0 else lam_prev",
     "lam = lam_prev"),
    ("backward: dR against h_t", "dR += np.sum(delta * prev[:, t, H][:, None, :], axis=0)",
     "dR += np.sum(delta * S[:, t, H][:, None, :], axis=0)"),
    ("floored read-out: floor e^{+m}", "    em = np.exp(-m)\n", "    em = np.exp(m)\n"),
    ("floored read-out: m derivative dropped", "np.where(on_m, -em, 0.0)", "np.where(on_m, 0.0 * em, 0.0)"),
    ("floored read-out: n branch without the floor", "on_n = (an >= em) & (an >= READOUT_FLOOR)",
     "on_n = an >= READOUT_FLOOR"),
    ("packed: no restart from state0", "            prev[:, t] = s0[s]\n", "            pass\n"),
    ("packed: Jacobian not cut at starts", "                A[:, t] = 0.0\n", "                pass\n"),
    ("packed backward: adjoint leaks across a start", "                lam_prev = np.zeros_like(lam_prev)\n",
     "                pass\n"),
    ("weight gradient: transposed operand", "dW = (dP2.T @ x.reshape(B * T, d_in)).reshape(g, d_h, d_in)",
     "dW = (dP2.T @ x.reshape(B * T, d_in)[::-1]).reshape(g, d_h, d_in)"),
    ("input gradient: gate rows swapped", "dx = (dP2 @ W.reshape(g * d_h, d_in)).reshape(B, T, d_in)",
     "dx = (dP2 @ W[::-1].reshape(g * d_h, d_in)).reshape(B, T, d_in)"),
    ("gate Jacobian: forget derivative", "dfg_df = fg * (dlf - dm_df)", "dfg_df = fg * (1.0 - dm_df)"),
    ("gate Jacobian: output-gate term", "dh[GO] = dh[GO] + (c / v[\"D\"]) * o * (1.0 - o)", "dh[GO] = dh[GO]"),
    ("head mixing: transposed block", 'np.einsum("gaik,...ak->...gai", R, hh)', 'np.einsum("gaki,...ak->...gai", R, hh)'),
    ("head Jacobian: transposed coupling", 'np.einsum("...sgai,gaik->...aisk", Gh, R)',
     'np.einsum("...sgai,gaki->...aisk", Gh, R)'),
    ("head backward: transposed gate Jacobian", "(G * lam[:, :, None, :]).sum(axis=1)",
     "(G * lam[:, None, :, :]).sum(axis=2)"),
    ("head backward: untransposed Jacobian", 'np.einsum("bauv,bau->bav", J, head_vectors(lam, nh))',
     'np.einsum("bauv,bav->bau", J, head_vectors(lam, nh))'),
    ("head backward: transposed dR", 'np.einsum("bgai,bak->gaik", delta.reshape', 'np.einsum("bgai,bak->gaki", delta.reshape'),
    ("head backward: dR against h_t", "prev[:, t, H].reshape(B, nh, dh))", "S[:, t, H].reshape(B, nh, dh))"),
    ('head packed: no restart at a start', '            if t in starts:\n                prev = s0[starts[t]][None]\n', ''),
    ('head packed: Jacobian not cut at a start', '                J[:, t] = 0.0\n', '                pass\n'),
    ('head packed backward: adjoint leaks across a start', '        elif t in starts:\n            dstate0[starts[t]] += lam_prev[0]\n            lam_prev = np.zeros_like(lam_prev)\n', '        elif t in starts:\n            dstate0[starts[t]] += lam_prev[0]\n'),
    ("branch margin at s_t instead of s_{t-1}", "prev = _shifted(np.asarray(S, dtype=np.float64), state0, cu_seqlens)\n    _, it, ft, _ = preactivations(prev, P, R)",
     "prev = np.asarray(S, dtype=np.float64)\n    _, it, ft, _ = preactivations(prev, P, R)"),
    ("branch margin without the stabiliser", "a = lf + prev[..., M, :]\n    return np.abs(a - it)",
     "a = lf\n    return np.abs(a - it)"),
    ("head solve: transposed block", 'np.einsum("bauv,bav->bau", J[:, t], x[:, t - 1])',
     'np.einsum("bavu,bav->bau", J[:, t], x[:, t - 1])'),
]


def _mutant(label, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {label!r} not found exactly once"
    spec = importlib.util.spec_from_loader(f"mutant_{abs(hash(label))}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    exec(compile(src.replace(old, new), f"<mutant {label}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(label, old, new):
    mod = _mutant(label, old, new)
    caught = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"no pin notices the planted mistake {label!r}"
