"""GPU parity of head mixing (mix='head'): block-diagonal recurrent matrices R of shape
(4, n_heads, d_head, d_head), h' of a head feeding every gate of that head ("sLSTM in this
library", "Cell", the mix table; the paper's sLSTM memory mixing, summary card "Method"), against
the float64 oracle's dense per-head forms.

Covered: the sequential forward and the Newton solve (warm and zero start, fixed count and early
stop, state0 and final state; the one-sweep kernel for a fixed count of up to 4 iterations and
the per-iteration kernels otherwise, and always for heads of 128 units) for every supported
head width, both forget-gate forms, the
floored read-out and bf16 pre-activations; T = 1 and T not a multiple of the kernels' 8-step
prefetch; many narrow heads; diagonal blocks against the channelwise solver at a larger size;
and the head-mixing benchmark workload at full size on sampled (batch row, head) pairs: each
head is its own recurrence, so the oracle solves one head alone."""
import numpy as np
import pytest
import torch

from oracle import slstm_ref as ref
from parity import H_TOL_BF16, H_TOL_F32, case, h_floor, h_rel_err, to_np
from workloads import draw_head_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
WIDTHS = [8, 16, 32, 64, 128]


def _dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _state_err(gpu, ref_states):
    """Largest error per slot (c, n, m, h) relative to the slot's largest value."""
    g, r = to_np(gpu), np.asarray(ref_states)
    return max(float(np.max(np.abs(g[..., k, :] - r[..., k, :])) / max(float(np.max(np.abs(r[..., k, :]))), 1e-30))
               for k in range(4))


def _inputs(seed, B, T, dh, nh, p_dtype="f32", state0=True):
    x = draw_head_inputs(seed, B, T, nh * dh, nh, p_dtype=p_dtype, with_state0=state0)
    return x["P"], x["R"], x["state0"]


@pytest.mark.parametrize("dh", WIDTHS)
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_head_sequential(gpu_lib, dh, forget):
    P, R, s0 = _inputs(900 + dh, 3, 45, dh, 2)
    case(f"head sequential d_head={dh} {forget}")
    fin = torch.empty_like(s0).to(DEV)
    S, h = gpu_lib.head_sequential_forward(*_dev(P, R, s0), forget, final_state=fin)
    torch.cuda.synchronize()
    seq = ref.sequential_head(to_np(P), to_np(R), to_np(s0), forget)
    assert h_rel_err(h, seq[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32
    assert _state_err(S, seq) < 1e-5
    assert _state_err(fin, seq[:, -1]) < 1e-5


@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_head_sequential_bf16_floored(gpu_lib, forget):
    P, R, s0 = _inputs(910, 2, 77, 16, 4, p_dtype="bf16")
    case(f"head sequential bf16 P, floored read-out, {forget}")
    _, h = gpu_lib.head_sequential_forward(*_dev(P, R, s0), forget, readout="floored")
    torch.cuda.synchronize()
    seq = ref.sequential_head(to_np(P), to_np(R), to_np(s0), forget + ref.FLOORED)
    assert h_rel_err(h, seq[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32


@pytest.mark.parametrize("dh", WIDTHS)
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("K", [3, 6])
def test_head_newton(gpu_lib, dh, forget, K):
    P, R, s0 = _inputs(920 + dh + K, 2, 45, dh, 2)
    case(f"head newton d_head={dh} {forget} K={K}")
    fin = torch.empty_like(s0).to(DEV)
    S, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), forget, K, 0.0, final_state=fin,
                                           raise_on_divergence=False)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), forget, K)
    err = h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32))
    print(f"head newton d_head={dh} {forget} K={K}: h rel err {err:.2e}, max|F| {st.max_abs_F[-1]:.2e} "
          f"(oracle {st_ref.max_abs_F[-1]:.2e})")
    assert err < H_TOL_F32
    assert _state_err(S, S_ref) < 1e-4
    assert _state_err(fin, S_ref[:, -1]) < 1e-4
    assert st.iters == st_ref.iters == K
    assert st.diverged == st_ref.diverged and st.nonfinite == st_ref.nonfinite
    # every recorded residual maximum but the converged tail agrees with the oracle's
    for e_gpu, e_ref in zip(st.max_abs_F, st_ref.max_abs_F):
        if e_ref > 1e-3:
            assert abs(e_gpu - e_ref) <= 1e-3 * e_ref


@pytest.mark.parametrize("dh", [8, 32])
def test_head_newton_zero_init(gpu_lib, dh):
    """From a zero iterate the early iterates wander far (residuals up to 1e5); after K = T
    iterations the iterate is the exact solution whatever the path, on both sides."""
    T = 12
    P, R, s0 = _inputs(930 + dh, 2, T, dh, 3)
    case(f"head newton zero init d_head={dh} K=T={T}")
    _, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), "sigmoid", T, 0.0, init="zero",
                                           raise_on_divergence=False)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "sigmoid", T, init=ref.INIT_ZERO)
    seq = ref.sequential_head(to_np(P), to_np(R), to_np(s0), "sigmoid")
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32
    assert h_rel_err(h, seq[..., 3, :]) < H_TOL_F32
    assert st.iters == st_ref.iters == T and not st.diverged


@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_head_newton_floored(gpu_lib, forget):
    P, R, s0 = _inputs(940, 2, 61, 32, 2)
    case(f"head newton floored read-out {forget}")
    _, h, _ = gpu_lib.head_newton_forward(*_dev(P, R, s0), forget, 4, 0.0, readout="floored")
    torch.cuda.synchronize()
    S_ref, _ = ref.newton_head(to_np(P), to_np(R), to_np(s0), forget + ref.FLOORED, 4)
    assert h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32


@pytest.mark.parametrize("dh", [16, 64, 128])
def test_head_newton_early_stop(gpu_lib, dh):
    """tol > 0: the solve stops at the first iterate whose residual maximum is below tol; the
    stop is global over every (batch row, head)."""
    P, R, s0 = _inputs(950 + dh, 3, 70, dh, 2, p_dtype="bf16")
    case(f"head newton early stop d_head={dh}")
    _, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), "sigmoid", 8, 1e-5)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "sigmoid", 8, tol=1e-5)
    assert st_ref.converged and st.converged
    assert st.iters == st_ref.iters < 8
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16


def test_head_newton_stop_after_last_iterate(gpu_lib):
    """A tolerance met only by the final iterate: iters = max_iters, converged."""
    P, R, s0 = _inputs(955, 2, 40, 16, 2)
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", 2)
    tol = float(np.sqrt(st_ref.max_abs_F[1] * 1e-5))   # between the residual of S^1 and the floor
    case("head newton stop at the last iterate")
    _, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), "exp", 2, tol)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", 2, tol=tol)
    assert st_ref.iters == 2 and st_ref.converged
    assert st.iters == 2 and st.converged
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("dh", [8, 64])
def test_head_one_sweep_solve(gpu_lib, K, dh):
    """tol = 0 and K <= 4: the whole solve is one launch of the one-sweep kernel (no iteration
    kernel); a tolerance that is never met forces one iteration kernel per iteration instead.
    Both match the oracle's iterate, residual maxima and flags."""
    P, R, s0 = _inputs(1000 + K + dh, 2, 45, dh, 2)
    Pd, Rd, s0d = _dev(P, R, s0)
    case(f"head one-sweep solve vs iteration kernels d_head={dh} K={K}")
    gpu_lib.profile_reset()
    gpu_lib.profile_enable(True)
    _, h1, st1 = gpu_lib.head_newton_forward(Pd, Rd, s0d, "exp", K, 0.0)
    n_sweep = len(gpu_lib.profile_durations("head_solve"))
    n_iter1 = len(gpu_lib.profile_durations("head_iteration"))
    gpu_lib.profile_reset()
    _, h2, st2 = gpu_lib.head_newton_forward(Pd, Rd, s0d, "exp", K, 1e-30)
    n_iter2 = len(gpu_lib.profile_durations("head_iteration"))
    gpu_lib.profile_enable(False)
    torch.cuda.synchronize()
    assert (n_sweep, n_iter1, n_iter2) == (1, 0, K)
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", K)
    for h, st in ((h1, st1), (h2, st2)):
        assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32
        assert st.iters == K and st.diverged == st_ref.diverged and not st.converged
        assert len(st.max_abs_F) == K + 1
        for e_gpu, e_ref in zip(st.max_abs_F, st_ref.max_abs_F):
            if e_ref > 1e-3:
                assert abs(e_gpu - e_ref) <= 1e-3 * e_ref
    assert h_rel_err(h1, to_np(h2)) < H_TOL_F32


@pytest.mark.parametrize("K", [1, 3])
@pytest.mark.parametrize("B,nh,dh", [(1, 3, 32), (2, 150, 8), (2, 300, 8)])
def test_head_one_sweep_forms(gpu_lib, B, nh, dh, K):
    """The one-sweep solve picks its kernel by the number of (batch row, head) workgroups per CU:
    its stages on separate wave groups at one (3 heads) and two (300: with the register cut from
    K = 2), the single-group sweep from three (600). Every form matches the oracle's states and
    residual maxima."""
    P, R, s0 = _inputs(1020 + nh + K, B, 21, dh, nh)
    case(f"head one-sweep form B={B} heads={nh} d_head={dh} K={K}")
    S, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), "exp", K, 0.0)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", K)
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32
    assert _state_err(S, S_ref) < 1e-4
    assert st.iters == K and st.diverged == st_ref.diverged
    for e_gpu, e_ref in zip(st.max_abs_F, st_ref.max_abs_F):
        if e_ref > 1e-3:
            assert abs(e_gpu - e_ref) <= 1e-3 * e_ref


@pytest.mark.parametrize("K", [2, 3])
@pytest.mark.parametrize("forget,p_dtype", [("sigmoid", "f32"), ("exp", "bf16"), ("sigmoid", "bf16")])
@pytest.mark.parametrize("B,nh,dh", [(1, 3, 32), (2, 100, 16), (3, 200, 16), (17, 32, 32), (2, 300, 8)])
def test_head_one_sweep_forms_gates(gpu_lib, B, nh, dh, forget, p_dtype, K):
    """Both one-sweep forms with the sigmoid forget gate and bf16 pre-activations: the wave-group
    form (3 and 200 workgroups: one per CU) and the single-group sweep (600, 544 and 600
    workgroups: three a CU, d_head 8, 16 and 32), on sampled (batch row, head) pairs, each solved
    alone by the oracle (heads are independent recurrences)."""
    T = 33
    x = draw_head_inputs(1100 + B + nh + dh + K, B, T, nh * dh, nh, p_dtype=p_dtype, with_state0=True)
    P, R, s0 = x["P"], x["R"], x["state0"]
    case(f"head one-sweep B={B} heads={nh} d_head={dh} {forget} {p_dtype} K={K}")
    gpu_lib.profile_reset()
    gpu_lib.profile_enable(True)
    S, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), forget, K, 0.0, raise_on_divergence=False)
    n_sweep = len(gpu_lib.profile_durations("head_solve"))
    gpu_lib.profile_enable(False)
    torch.cuda.synchronize()
    assert n_sweep == 1 and st.iters == K
    S, h = S.cpu(), h.cpu()
    bar = H_TOL_BF16 if p_dtype == "bf16" else H_TOL_F32
    pairs = sorted({(0, 0), (B - 1, nh - 1), (B // 2, nh // 2)})
    for b, a in pairs:
        cols = slice(a * dh, (a + 1) * dh)
        Pa = to_np(P[b:b + 1, :, :, cols])
        Ra = to_np(R[:, a:a + 1])
        s0a = to_np(s0[b:b + 1, :, cols])
        S_ref, st_ref = ref.newton_head(Pa, Ra, s0a, forget, K)
        err = h_rel_err(h[b:b + 1, :, cols], S_ref[..., 3, :], h_floor(forget, bar))
        assert err < bar, (b, a, err)
        assert _state_err(S[b:b + 1, :, :, cols], S_ref) < (2e-2 if p_dtype == "bf16" else 1e-4)


def test_head_one_sweep_zero_init_exact(gpu_lib):
    """The one-sweep kernel from a zero iterate: after K = T iterations the iterate is the exact
    solution (the sequential one). Sigmoid forget gate: with the exponential one, this zero
    start's intermediate iterates reach residuals of 3e3 and float32 keeps h only to 8e-4 of
    it, on the one-sweep and the per-iteration kernels alike."""
    T = 4
    P, R, s0 = _inputs(1010, 3, T, 16, 2)
    case(f"head one-sweep zero init K=T={T}")
    _, h, st = gpu_lib.head_newton_forward(*_dev(P, R, s0), "sigmoid", T, 0.0, init="zero")
    torch.cuda.synchronize()
    seq = ref.sequential_head(to_np(P), to_np(R), to_np(s0), "sigmoid")
    S_ref, _ = ref.newton_head(to_np(P), to_np(R), to_np(s0), "sigmoid", T, init=ref.INIT_ZERO)
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32
    assert h_rel_err(h, seq[..., 3, :]) < H_TOL_F32
    assert st.iters == T


@pytest.mark.parametrize("T", [1, 7, 8, 9])
def test_head_short_sequences(gpu_lib, T):
    """T below, at and just above the 8-step prefetch; T = 1 is the decode step."""
    P, R, s0 = _inputs(960 + T, 4, T, 32, 2)
    case(f"head short T={T}")
    _, hq = gpu_lib.head_sequential_forward(*_dev(P, R, s0), "exp")
    _, hn, _ = gpu_lib.head_newton_forward(*_dev(P, R, s0), "exp", 3, 0.0)
    torch.cuda.synchronize()
    seq = ref.sequential_head(to_np(P), to_np(R), to_np(s0), "exp")
    S_ref, _ = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", 3)
    assert h_rel_err(hq, seq[..., 3, :]) < H_TOL_F32
    assert h_rel_err(hn, S_ref[..., 3, :]) < H_TOL_F32


def test_head_many_narrow_heads_no_state0(gpu_lib):
    P, R, _ = _inputs(970, 2, 33, 8, 32, state0=False)
    case("head newton 32 heads of 8 units, no state0")
    _, h, _ = gpu_lib.head_newton_forward(*_dev(P, R), None, "exp", 3, 0.0)
    _, hq = gpu_lib.head_sequential_forward(*_dev(P, R), None, "exp")
    torch.cuda.synchronize()
    S_ref, _ = ref.newton_head(to_np(P), to_np(R), None, "exp", 3)
    seq = ref.sequential_head(to_np(P), to_np(R), None, "exp")
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32
    assert h_rel_err(hq, seq[..., 3, :]) < H_TOL_F32


@pytest.mark.parametrize("dh", [16, 64])
def test_head_diagonal_blocks_match_channelwise(gpu_lib, dh):
    """Diagonal blocks R[g, a] = diag(r_g[a d_head : (a+1) d_head]) make head mixing the
    channelwise cell: at a larger size than the oracle cases, the head solver matches the
    channelwise solver's result."""
    B, T, d = 4, 1000, 256
    nh = d // dh
    x = draw_head_inputs(980 + dh, B, T, d, nh, with_state0=True)
    P, s0 = x["P"], x["state0"]
    r = torch.from_numpy(np.random.Generator(np.random.PCG64(981)).uniform(-0.5, 0.5, (4, d)).astype(np.float32))
    R = torch.zeros(4, nh, dh, dh)
    for a in range(nh):
        R[:, a] = torch.diag_embed(r[:, a * dh:(a + 1) * dh])
    case(f"head diagonal blocks vs channelwise d_head={dh}")
    _, h_head, st_head = gpu_lib.head_newton_forward(*_dev(P, R, s0), "exp", 3, 0.0)
    _, h_diag, st_diag = gpu_lib.newton_forward(*_dev(P, r, s0), "exp", 3, 0.0)
    _, hq_head = gpu_lib.head_sequential_forward(*_dev(P, R, s0), "exp")
    _, hq_diag = gpu_lib.sequential_forward(*_dev(P, r, s0), "exp")
    torch.cuda.synchronize()
    assert h_rel_err(h_head, to_np(h_diag)) < H_TOL_F32
    assert h_rel_err(hq_head, to_np(hq_diag)) < 1e-5
    assert st_head.iters == st_diag.iters


def test_head_rejects_bad_shapes(gpu_lib):
    P, R, s0 = _inputs(990, 1, 8, 16, 2)
    with pytest.raises(ValueError):
        gpu_lib.head_newton_forward(*_dev(P, R[:, :1], s0), "exp", 3, 0.0)   # n_heads d_head != d_h
    Rbad = torch.zeros(4, 8, 4, 4)                                           # heads of 4 units
    with pytest.raises(gpu_lib.SlstmError, match="heads"):
        gpu_lib.head_sequential_forward(*_dev(P[..., :32].contiguous(), Rbad), None, "exp")


FULL = dict(B=16, T=4096, d=1024, nh=32, K=3, seed=20265)


def test_head_full_size_sampled(gpu_lib):
    """The head-mixing benchmark workload (B=16, T=4096, d_h=1024, 32 heads of 32, exp forget,
    K=3) in the launch configuration the benchmark times, checked on sampled (batch row, head)
    pairs: the corners and one inside, each solved alone by the oracle over all T."""
    B, T, d, nh, K = FULL["B"], FULL["T"], FULL["d"], FULL["nh"], FULL["K"]
    dh = d // nh
    x = draw_head_inputs(FULL["seed"], B, T, d, nh)
    P, R = x["P"], x["R"]
    case("head full size B=16 T=4096 d=1024 n_heads=32")
    Pd, Rd = _dev(P, R)
    S, h, st = gpu_lib.head_newton_forward(Pd, Rd, None, "exp", K, 0.0)
    _, hq = gpu_lib.head_sequential_forward(Pd, Rd, None, "exp")
    torch.cuda.synchronize()
    assert st.iters == K and not st.diverged
    h, hq = h.cpu(), hq.cpu()
    for b, a in [(0, 0), (B - 1, nh - 1), (7, 13)]:
        cols = slice(a * dh, (a + 1) * dh)
        Pa = to_np(P[b:b + 1, :, :, cols])
        Ra = to_np(R[:, a:a + 1])
        S_ref, _ = ref.newton_head(Pa, Ra, None, "exp", K)
        seq = ref.sequential_head(Pa, Ra, None, "exp")
        e_n = h_rel_err(h[b:b + 1, :, cols], S_ref[..., 3, :])
        e_q = h_rel_err(hq[b:b + 1, :, cols], seq[..., 3, :])
        print(f"head full size (b={b}, head={a}): newton h rel err {e_n:.2e}, sequential {e_q:.2e}")
        assert e_n < H_TOL_F32 and e_q < H_TOL_F32
