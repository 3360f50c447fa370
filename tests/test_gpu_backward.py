"""GPU parity of the backward pass (adjoint recurrence and cell vector-Jacobian product)
against the float64 oracle at the same inputs: dP, dR and dstate0 within GRAD_TOL.

The states fed to both sides are the oracle's own sequential trajectory (rounded to float32),
or plausible random states at the full layer size. The derivatives of the running maximum
m = max(a, i~) jump where it switches branch, so a lane is compared only where every step's
|a - i~| clears float32 rounding by a wide margin (oracle.branch_margin); on the other lanes both
branches are valid derivatives and the GPU result is only checked to be finite."""
import numpy as np
import pytest
import torch

from oracle import slstm_ref as ref
from parity import GRAD_TOL, case, grad_rel_err, sample_lanes, to_np
from workloads import by_name, draw_preactivation_inputs, random_cotangents, random_cotangents_device

pytestmark = pytest.mark.gpu

DEV = "cuda"
# a lane is decided when |a - i~| > MARGIN * (1 + |l| + |m'| + |i~|) at every step: float32
# forms a = l + m' and i~ to within a few units in the last place (1.2e-7) of that scale
MARGIN = 1e-5


def _decided_lanes(P, R, state0, S, forget):
    margin, scale = ref.branch_margin(P, R, state0, S, forget)
    return np.all(margin > MARGIN * (1.0 + scale), axis=1)  # (B, d)


def _problem(seed, B, T, d, forget, p_dtype, with_state0):
    """P, R, state0 and the oracle trajectory, as float32 torch tensors (P possibly bf16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d))
    s0 = None
    if with_state0:
        s0 = np.zeros((B, 4, d))
        s0[:, 0] = rng.uniform(-0.3, 0.3, (B, d))
        s0[:, 1] = rng.uniform(0.5, 1.5, (B, d))
        s0[:, 2] = rng.uniform(-1, 1, (B, d))
        s0[:, 3] = rng.uniform(-0.5, 0.5, (B, d))
        s0 = torch.from_numpy(s0.astype(np.float32))
    Pt = torch.from_numpy(P.astype(np.float32))
    if p_dtype == "bf16":
        Pt = Pt.to(torch.bfloat16)
    Rt = torch.from_numpy(R.astype(np.float32))
    S = ref.sequential(to_np(Pt), to_np(Rt), None if s0 is None else to_np(s0), forget)
    St = torch.from_numpy(S.astype(np.float32))
    return Pt, Rt, s0, St


def _oracle(P, R, s0, S, g_states, g_h, g_final, forget):
    """The oracle's backward with the three direct gradients folded into one g (B, T, 4, d)."""
    B, T, _, d = S.shape
    g = np.zeros((B, T, 4, d))
    if g_states is not None:
        g += to_np(g_states)
    if g_h is not None:
        g[:, :, 3] += to_np(g_h)
    if g_final is not None:
        g[:, T - 1] += to_np(g_final)
    return ref.backward(to_np(P), to_np(R), None if s0 is None else to_np(s0), to_np(S), g, forget)


def _gpu(gpu_lib, P, R, s0, S, g_states, g_h, g_final, forget, **kw):
    on = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    dP, dR, ds0 = gpu_lib.backward(on(P), on(R), on(S), on(s0), on(g_states), on(g_h), on(g_final),
                                   forget, **kw)
    torch.cuda.synchronize()
    return dP, dR, ds0


def _compare(P, R, s0, S, forget, got, want, tol=GRAD_TOL, max_undecided=0.05):
    dP, dR, ds0 = got
    dP_ref, dR_ref, ds0_ref = want
    keep = _decided_lanes(to_np(P), to_np(R), None if s0 is None else to_np(s0), to_np(S), forget)
    assert 1.0 - keep.mean() <= max_undecided, f"{1 - keep.mean():.3f} of the lanes undecided"
    assert torch.isfinite(dP).all() and torch.isfinite(dR).all() and torch.isfinite(ds0).all()
    B, _, _, d = S.shape
    e_dP = grad_rel_err(dP, dP_ref, keep[:, None, None, :])
    e_ds0 = grad_rel_err(ds0, ds0_ref, keep[:, None, :])
    feat = np.all(keep, axis=0)  # features whose every batch row is decided
    e_dR = grad_rel_err(dR, dR_ref, feat[None, :])
    print(f"backward rel err: dP {e_dP:.2e}, dR {e_dR:.2e}, dstate0 {e_ds0:.2e}, "
          f"undecided lanes {int((~keep).sum())}/{keep.size}")
    assert e_dP < tol and e_dR < tol and e_ds0 < tol


SHAPES = [(1, 1, 1), (2, 64, 16), (3, 33, 65), (2, 257, 20), (1, 70, 300), (4, 9, 256)]


@pytest.fixture(params=["fused_scan", "fused_chain"])
def schedule(request):
    """Both kernel forms of the backward must meet the same bar."""
    return request.param


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("p_dtype", ["f32", "bf16"])
def test_backward_matches_oracle(gpu_lib, shape, forget, p_dtype, schedule):
    B, T, d = shape
    case(f"backward {schedule} B={B} T={T} d={d} {forget} P {p_dtype}")
    P, R, s0, S = _problem(B * 7919 + T * 31 + d, B, T, d, forget, p_dtype, with_state0=True)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(B + T + d, B, T, d))
    got = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, forget, schedule=schedule)
    want = _oracle(P, R, s0, S, gs, gh, gf, forget)
    _compare(P, R, s0, S, forget, got, want)


@pytest.mark.parametrize("which", ["states", "h", "final", "none"])
def test_backward_optional_gradients(gpu_lib, which, schedule):
    B, T, d = 2, 40, 48
    case(f"backward {schedule} with only the {which} gradient")
    P, R, s0, S = _problem(5, B, T, d, "exp", "f32", with_state0=False)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(6, B, T, d))
    gs = gs if which == "states" else None
    gh = gh if which == "h" else None
    gf = gf if which == "final" else None
    got = _gpu(gpu_lib, P, R, None, S, gs, gh, gf, "exp", schedule=schedule)
    if which == "none":
        assert all(bool((t == 0).all()) for t in got)
        return
    want = _oracle(P, R, None, S, gs, gh, gf, "exp")
    _compare(P, R, None, S, "exp", got, want)


def test_backward_without_dstate0(gpu_lib):
    B, T, d = 2, 20, 32
    case("backward without dstate0")
    P, R, s0, S = _problem(8, B, T, d, "sigmoid", "f32", with_state0=True)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(9, B, T, d))
    dP, dR, ds0 = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "sigmoid", want_dstate0=False)
    assert ds0 is None
    dP2, dR2, _ = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "sigmoid")
    assert torch.equal(dP, dP2) and torch.equal(dR, dR2)


def test_backward_bitwise_reproducible(gpu_lib, schedule):
    B, T, d = 16, 300, 512
    case(f"backward {schedule} reproducibility B={B} T={T} d={d}")
    P, R, s0, S = _problem(11, B, T, d, "exp", "f32", with_state0=True)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(12, B, T, d))
    ws = gpu_lib.alloc_workspace(gpu_lib.backward_workspace_bytes(B, T, d, schedule))
    a = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "exp", workspace=ws, schedule=schedule)
    b = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "exp", workspace=ws, schedule=schedule)
    c = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "exp", schedule=schedule)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_backward_forms_agree(gpu_lib):
    """The two forms order their float32 sums differently but agree to rounding."""
    B, T, d = 3, 200, 96
    case(f"backward forms agree B={B} T={T} d={d}")
    P, R, s0, S = _problem(13, B, T, d, "sigmoid", "f32", with_state0=True)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(14, B, T, d))
    a = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "sigmoid", schedule="fused_scan")
    b = _gpu(gpu_lib, P, R, s0, S, gs, gh, gf, "sigmoid", schedule="fused_chain")
    for x, y in zip(a, b):
        assert grad_rel_err(x, y) < 1e-5


def test_backward_fused_picks_a_form(gpu_lib):
    B, T, d = 2, 64, 128
    P, R, s0, S = _problem(15, B, T, d, "exp", "f32", with_state0=False)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(16, B, T, d))
    a = _gpu(gpu_lib, P, R, None, S, gs, gh, gf, "exp", schedule="fused")
    # the default form of the backward is the scan
    b = _gpu(gpu_lib, P, R, None, S, gs, gh, gf, "exp", schedule="fused_scan")
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("sched", ["fused_scan", "fused_chain"])
def test_backward_mid_workload_full_size(gpu_lib, sched):
    """The mid workload (B=8, T=1024, d=256) at its full size on its own trajectory."""
    w = by_name("mid_b8_t1024_d256")
    case(f"backward {sched} {w.name} full size")
    inp = draw_preactivation_inputs(w)
    P, R = inp["P"], inp["R"]
    S = torch.from_numpy(ref.sequential(to_np(P), to_np(R), None, w.forget).astype(np.float32))
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(w.seed + 7, w.B, w.T, w.d_h))
    got = _gpu(gpu_lib, P, R, None, S, gs, gh, gf, w.forget, schedule=sched)
    want = _oracle(P, R, None, S, gs, gh, gf, w.forget)
    _compare(P, R, None, S, w.forget, got, want)


def test_backward_rejects_bad_arguments(gpu_lib):
    P = torch.zeros((1, 4, 4, 8), device=DEV)
    R = torch.zeros((4, 8), device=DEV)
    S = torch.zeros((1, 4, 4, 8), device=DEV)
    with pytest.raises(gpu_lib.SlstmError):
        gpu_lib.backward(P, R, S, schedule="layered")
    with pytest.raises(gpu_lib.SlstmError):
        gpu_lib.backward(P, R, S, workspace=gpu_lib.alloc_workspace(64))
    assert gpu_lib.backward_workspace_bytes(1, 4, 8, "layered") == 0


@pytest.mark.parametrize("name", ["layer_b128_t2048_d1024", "sigmoid_bf16p_b16_t4096_d1024",
                                  "long_b4_t16384_d2048"])
def test_backward_workload_full_size(gpu_lib, name):
    """Full workload sizes in the default (scan) form, and chains at the layer's size. The states are the GPU's Newton solve, with the
    oracle's own trajectory written over the lanes the oracle checks: every batch row of three
    features (which fixes dR there) and 64 sampled lanes."""
    w = by_name(name)
    B, T, d = w.B, w.T, w.d_h
    case(f"backward {w.name} full size, sampled lanes")
    inp = draw_preactivation_inputs(w, device=DEV)
    P, R = inp["P"].to(DEV), inp["R"].to(DEV)
    S, _, _ = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, want_hidden=False)
    js = [0, 517, d - 1]
    lb, lj = sample_lanes(B, d, 64, seed=3)
    apart = ~np.isin(lj, js)  # lanes outside the three features
    ib = torch.as_tensor(lb[apart], device=DEV)
    ij = torch.as_tensor(lj[apart], device=DEV)

    # sub-problems: (B, T, 4, 3) for the features, (1, T, 4, n) for the lanes
    feat = lambda t: t[..., js].cpu()  # noqa: E731
    lane4 = lambda t: t[ib, :, :, ij].permute(1, 2, 0).unsqueeze(0).cpu()  # noqa: E731
    subs = {"features": (feat(P), R[:, js].cpu()), "lanes": (lane4(P), R[:, ij].cpu())}
    S_ref = {}
    for part, (Ps, Rs) in subs.items():
        S_ref[part] = torch.from_numpy(ref.sequential(to_np(Ps), to_np(Rs), None, w.forget).astype(np.float32))
    S[..., js] = S_ref["features"].to(DEV)
    S[ib, :, :, ij] = S_ref["lanes"][0].permute(2, 0, 1).to(DEV)

    gs, gh, gf = random_cotangents_device(w.seed + 12, B, T, d, DEV)
    dP, dR, ds0 = gpu_lib.backward(P, R, S, None, gs, gh, gf, w.forget)
    torch.cuda.synchronize()
    assert torch.isfinite(dP).all() and torch.isfinite(dR).all() and torch.isfinite(ds0).all()
    if B >= 128:
        # chains agree with the scan to rounding
        cP, cR, c0 = gpu_lib.backward(P, R, S, None, gs, gh, gf, w.forget, schedule="fused_chain")
        torch.cuda.synchronize()
        assert grad_rel_err(cP, dP) < 1e-5 and grad_rel_err(cR, dR) < 1e-5 and grad_rel_err(c0, ds0) < 1e-5
        del cP, cR, c0

    grads = {"features": (feat(gs), gh[:, :, js].cpu(), gf[:, :, js].cpu()),
             "lanes": (lane4(gs), gh[ib, :, ij].T.unsqueeze(0).cpu(), gf[ib, :, ij].T.unsqueeze(0).cpu())}
    got = {"features": (feat(dP), dR[:, js].cpu(), ds0[:, :, js].cpu()),
           "lanes": (lane4(dP), None, ds0[ib, :, ij].T.unsqueeze(0).cpu())}
    for part, (Ps, Rs) in subs.items():
        want = _oracle(Ps, Rs, None, S_ref[part], *grads[part], w.forget)
        keep = _decided_lanes(to_np(Ps), to_np(Rs), None, to_np(S_ref[part]), w.forget)
        assert 1.0 - keep.mean() <= 0.05
        dP_g, dR_g, ds0_g = got[part]
        errs = [grad_rel_err(dP_g, want[0], keep[:, None, None, :]),
                grad_rel_err(ds0_g, want[2], keep[:, None, :])]
        if dR_g is not None:
            errs.append(grad_rel_err(dR_g, want[1], np.all(keep, axis=0)[None, :]))
        print(f"{w.name} full size backward ({part}): rel err {['%.2e' % e for e in errs]}, "
              f"undecided {int((~keep).sum())}/{keep.size}")
        assert max(errs) < GRAD_TOL


# ---- dbias, bf16 dP and the input projection's gradients ----------------------------------------
def test_backward_dbias_and_bf16_dP(gpu_lib, schedule):
    B, T, d = 3, 75, 40
    case(f"backward {schedule} dbias and bf16 dP B={B} T={T} d={d}")
    P, R, s0, S = _problem(17, B, T, d, "exp", "f32", with_state0=True)
    gs, gh, gf = (torch.from_numpy(a) for a in random_cotangents(18, B, T, d))
    on = lambda t: t.to(DEV)  # noqa: E731
    dP, dR, ds0, db = gpu_lib.backward(on(P), on(R), on(S), on(s0), on(gs), on(gh), on(gf), "exp",
                                       schedule=schedule, want_dbias=True)
    dPb, dRb, ds0b, dbb = gpu_lib.backward(on(P), on(R), on(S), on(s0), on(gs), on(gh), on(gf), "exp",
                                           schedule=schedule, dP_dtype=torch.bfloat16, want_dbias=True)
    torch.cuda.synchronize()
    want = _oracle(P, R, s0, S, gs, gh, gf, "exp")
    keep = _decided_lanes(to_np(P), to_np(R), to_np(s0), to_np(S), "exp")
    _, _, db_ref = ref.input_projection_backward(np.zeros((B, T, 8)), np.zeros((4, d, 8)), want[0])
    assert grad_rel_err(db, db_ref, np.all(keep, axis=0)[None, :]) < GRAD_TOL
    # the bf16 output is the float32 dP rounded to nearest even; everything else is unchanged
    assert torch.equal(dPb, dP.to(torch.bfloat16))
    assert torch.equal(dRb, dR) and torch.equal(ds0b, ds0) and torch.equal(dbb, db)


PROJ_SHAPES = [(2, 5, 8, 4), (3, 7, 24, 5), (1, 130, 40, 20), (2, 300, 72, 66)]


@pytest.mark.parametrize("shape", PROJ_SHAPES)
@pytest.mark.parametrize("dp_dtype", ["bf16", "f32"])
def test_input_projection_backward_matches_oracle(gpu_lib, shape, dp_dtype):
    """dW_x = dP^T x and dx = dP W_x. With bf16 dP both sides multiply the same bf16 values and
    only the float32 accumulation differs (bar 1e-4); float32 dP is rounded to bf16 on the GPU
    (the bf16 bar, 2e-2)."""
    B, T, d_in, d_h = shape
    case(f"input projection backward B={B} T={T} d_in={d_in} d_h={d_h} dP {dp_dtype}")
    rng = np.random.Generator(np.random.PCG64(B * 1000 + T + d_in + d_h))
    x = torch.from_numpy(rng.standard_normal((B, T, d_in)).astype(np.float32)).to(torch.bfloat16)
    W = torch.from_numpy((rng.standard_normal((4, d_h, d_in)) / np.sqrt(d_in)).astype(np.float32)).to(torch.bfloat16)
    dP = torch.from_numpy(rng.standard_normal((B, T, 4, d_h)).astype(np.float32))
    if dp_dtype == "bf16":
        dP = dP.to(torch.bfloat16)
    dx, dW = gpu_lib.input_projection_backward(x.to(DEV), W.to(DEV), dP.to(DEV))
    torch.cuda.synchronize()
    dW_ref, dx_ref, _ = ref.input_projection_backward(to_np(x), to_np(W), to_np(dP))
    tol = GRAD_TOL if dp_dtype == "bf16" else 2e-2
    e_w, e_x = grad_rel_err(dW, dW_ref), grad_rel_err(dx, dx_ref)
    print(f"input projection backward rel err: dW {e_w:.2e}, dx {e_x:.2e}")
    assert e_w < tol and e_x < tol
    # each output alone, and reproducible
    dx2, none = gpu_lib.input_projection_backward(x.to(DEV), W.to(DEV), dP.to(DEV), want_dW=False)
    none2, dW2 = gpu_lib.input_projection_backward(x.to(DEV), W.to(DEV), dP.to(DEV), want_dx=False)
    torch.cuda.synchronize()
    assert none is None and none2 is None
    assert torch.equal(dx, dx2) and torch.equal(dW, dW2)


def test_input_projection_backward_layer_full_size(gpu_lib):
    """x (128, 2048, 1024), W_x (4, 1024, 1024), bf16 dP: sampled entries of dW_x (each a sum
    over all 262,144 rows) and sampled rows of dx against the oracle on those entries."""
    w = by_name("layer_b128_t2048_d1024")
    B, T, d_in, d = w.B, w.T, w.d_in, w.d_h
    case(f"input projection backward {w.name} full size")
    from workloads import draw_layer_inputs
    inp = draw_layer_inputs(w)
    x, W = inp["x"].to(DEV), inp["W"].to(DEV)
    dP = random_cotangents_device(w.seed + 21, B, T, d, DEV)[0].to(torch.bfloat16)
    dx, dW = gpu_lib.input_projection_backward(x, W, dP)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(5))
    gj = [(int(rng.integers(4)), int(rng.integers(d))) for _ in range(24)] + [(0, 0), (3, d - 1)]
    ks = rng.integers(0, d_in, size=8).tolist() + [0, d_in - 1]
    # the oracle on sub-problems: one (gate, feature) column of dP against the sampled columns of
    # x gives dW[g, j, ks]; one row of dP against all of W_x gives dx[b, t]
    xs = to_np(x[:, :, ks].cpu())
    errs = []
    for g, j in gj:
        col = to_np(dP[:, :, g:g + 1, j:j + 1].cpu())
        want, _, _ = ref.input_projection_backward(xs, np.zeros((1, 1, len(ks))), col)
        got = to_np(dW[g, j, ks])
        errs.append(grad_rel_err(got, want[0, 0]))
    rows = [(int(rng.integers(B)), int(rng.integers(T))) for _ in range(12)] + [(0, 0), (B - 1, T - 1)]
    Wn = to_np(W.cpu())
    for b, t in rows:
        _, want, _ = ref.input_projection_backward(np.zeros((1, 1, d_in)), Wn, to_np(dP[b:b + 1, t:t + 1].cpu()))
        errs.append(grad_rel_err(dx[b, t], want[0, 0]))
    print(f"input projection backward full size: max rel err {max(errs):.2e}")
    assert max(errs) < GRAD_TOL
