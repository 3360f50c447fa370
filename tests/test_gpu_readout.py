"""GPU parity of the floored read-out variant, h = o c / max(|n|, e^{-m}, 1e-6), against the
float64 oracle in the same cell mode: the residual and Jacobian, the warm start, the Newton
solve in every kernel layout (the one-kernel solve included), the sequential forward and the
backward. Inputs shift the input-gate pre-activations down so that the floor is active on a
share of the steps (checked on the oracle's trajectory), where the two read-outs differ."""
import numpy as np
import pytest
import torch

from oracle import slstm_ref as ref
from parity import GRAD_TOL, H_TOL_F32, case, grad_rel_err, h_floor, h_rel_err, to_np
from workloads import random_cotangents, random_states

pytestmark = pytest.mark.gpu

DEV = "cuda"
MARGIN = 1e-5


def _problem(seed, B, T, d, forget):
    rng = np.random.Generator(np.random.PCG64(seed))
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 1] -= 2.0
    # forget bias +1 for the exponential gate: the stabiliser grows slowly enough that the
    # floor is active past the first steps, and Newton still converges from the warm start
    P[:, :, 2] += 3.0 if forget == "sigmoid" else 1.0
    R = rng.uniform(-0.5, 0.5, (4, d))
    s0 = np.zeros((B, 4, d))
    s0[:, 0] = rng.uniform(-0.05, 0.05, (B, d))
    s0[:, 1] = rng.uniform(0.05, 0.3, (B, d))
    s0[:, 2] = rng.uniform(-0.5, 1.0, (B, d))
    s0[:, 3] = rng.uniform(-0.5, 0.5, (B, d))
    f32 = lambda a: torch.from_numpy(a.astype(np.float32))  # noqa: E731
    return f32(P), f32(R), f32(s0)


def _floor_share(S):
    """Share of (b, t, j) where the floored read-out's denominator is e^{-m} (floor active)."""
    return float(np.mean(np.abs(S[..., 1, :]) < np.exp(-S[..., 2, :])))


@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_residual_jacobian_floored(gpu_lib, forget):
    B, T, d = 2, 37, 70
    mode = forget + ref.FLOORED
    case(f"residual_jacobian {mode} B={B} T={T} d={d}")
    rng = np.random.Generator(np.random.PCG64(300))
    P = (rng.standard_normal((B, T, 4, d)) * 1.5).astype(np.float32)
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d)).astype(np.float32)
    S = random_states(31, B, T, d).astype(np.float32)
    s0 = random_states(32, B, 1, d)[:, 0].astype(np.float32)
    A, rhs, _ = gpu_lib.residual_jacobian(torch.from_numpy(P).to(DEV), torch.from_numpy(R).to(DEV),
                                          torch.from_numpy(S).to(DEV), torch.from_numpy(s0).to(DEV),
                                          forget, readout="floored")
    torch.cuda.synchronize()
    F, A_ref = ref.residual(S.astype(np.float64), P.astype(np.float64), R.astype(np.float64),
                            s0.astype(np.float64), mode)
    f_next = S.astype(np.float64) - F
    assert _floor_share(f_next) > 0.005
    # compare away from the read-out's own branch switch |n| = e^{-m}
    gap = np.abs(np.abs(f_next[..., 1, :]) - np.exp(-f_next[..., 2, :])) > 1e-4 * np.exp(-f_next[..., 2, :])
    f_gpu = to_np(rhs) + S
    assert float(np.max(np.abs(f_gpu - f_next)[:, :, :, :] / np.maximum(np.abs(f_next), 1.0))) < 5e-6
    A_gpu = to_np(A)
    scale = np.maximum(np.max(np.abs(A_ref), axis=3, keepdims=True), 1e-3)
    err = np.abs(A_gpu - A_ref) / scale
    assert float(np.max(err[:, :, 3][np.broadcast_to(gap[:, :, None, :], err[:, :, 3].shape)])) < 5e-5
    assert float(np.max(err[:, :, :3])) < 5e-5


@pytest.mark.parametrize("schedule", ["fused_scan", "fused_chain", "layered"])
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("K", [3, 6])
def test_newton_floored(gpu_lib, schedule, forget, K):
    """K = 3 on the chain layout runs the one-kernel solve; K = 6 the per-iteration kernels."""
    B, T, d = 3, 300, 72
    mode = forget + ref.FLOORED
    case(f"newton {mode} {schedule} K={K} B={B} T={T} d={d}")
    P, R, s0 = _problem(400 + K, B, T, d, forget)
    S, h, st = gpu_lib.newton_forward(P.to(DEV), R.to(DEV), s0.to(DEV), forget, K, 0.0,
                                      raise_on_divergence=False, schedule=schedule, readout="floored")
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton(to_np(P), to_np(R), to_np(s0), mode, K)
    seq = ref.sequential(to_np(P), to_np(R), to_np(s0), mode)
    assert _floor_share(seq) > 0.001
    assert np.max(np.abs(seq[..., 3, :] - ref.sequential(to_np(P), to_np(R), to_np(s0), forget)[..., 3, :])) > 1e-3
    err = h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32))
    print(f"floored newton {schedule} {forget} K={K}: h rel err {err:.2e}, iters {st.iters}")
    assert err < H_TOL_F32
    assert st.iters == st_ref.iters and st.diverged == st_ref.diverged


@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_sequential_and_warm_start_floored(gpu_lib, forget):
    B, T, d = 2, 129, 40
    mode = forget + ref.FLOORED
    case(f"sequential and warm start {mode}")
    P, R, s0 = _problem(500, B, T, d, forget)
    _, hs = gpu_lib.sequential_forward(P.to(DEV), R.to(DEV), s0.to(DEV), forget, readout="floored")
    torch.cuda.synchronize()
    seq = ref.sequential(to_np(P), to_np(R), to_np(s0), mode)
    assert h_rel_err(hs, seq[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32
    warm_ref = ref.warm_start(to_np(P), to_np(s0), mode)
    for form in ("fused_scan", "fused_chain"):
        W = gpu_lib.warm_start(P.to(DEV), s0.to(DEV), forget, schedule=form, readout="floored")
        torch.cuda.synchronize()
        assert h_rel_err(W[..., 3, :], warm_ref[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32, form


@pytest.mark.parametrize("schedule", ["fused_scan", "fused_chain"])
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_backward_floored(gpu_lib, schedule, forget):
    B, T, d = 2, 90, 48
    mode = forget + ref.FLOORED
    case(f"backward {mode} {schedule}")
    P, R, s0 = _problem(600, B, T, d, forget)
    S = torch.from_numpy(ref.sequential(to_np(P), to_np(R), to_np(s0), mode).astype(np.float32))
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(601, B, T, d))
    dP, dR, ds0 = gpu_lib.backward(P.to(DEV), R.to(DEV), S.to(DEV), s0.to(DEV), gs.to(DEV), gh.to(DEV),
                                   gf.to(DEV), forget, schedule=schedule, readout="floored")
    torch.cuda.synchronize()
    g = to_np(gs)
    g[:, :, 3] += to_np(gh)
    g[:, T - 1] += to_np(gf)
    dP_ref, dR_ref, ds0_ref = ref.backward(to_np(P), to_np(R), to_np(s0), to_np(S), g, mode)
    # lanes clear of both branch switches: the stabiliser's (a = i~) and the read-out's
    margin, scale = ref.branch_margin(to_np(P), to_np(R), to_np(s0), to_np(S), mode)
    Sn = to_np(S)
    ro_gap = np.abs(np.abs(Sn[..., 1, :]) - np.exp(-Sn[..., 2, :])) > 1e-4 * np.exp(-Sn[..., 2, :])
    keep = np.all((margin > MARGIN * (1.0 + scale)) & ro_gap, axis=1)
    assert keep.mean() > 0.8
    errs = [grad_rel_err(dP, dP_ref, keep[:, None, None, :]), grad_rel_err(ds0, ds0_ref, keep[:, None, :]),
            grad_rel_err(dR, dR_ref, np.all(keep, axis=0)[None, :])]
    print(f"floored backward {schedule} {forget}: rel err {['%.2e' % e for e in errs]}")
    assert max(errs) < GRAD_TOL
