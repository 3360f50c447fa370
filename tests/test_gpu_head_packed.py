"""GPU parity of packed sequences under head mixing: ragged sequences laid end to end in one row,
each from its own state0 ("sLSTM in this library", "Packed sequences"; the head-mixing cell of the
"Cell" section's mix table), against the float64 oracle's packed head forms. Covered: the
sequential forward with per-sequence final states, the Newton solve at a fixed count (up to 4
iterations in the single-group one-sweep kernel, more by the warm start and one kernel per
iteration) and with an early stop, and the backward with a gradient at each sequence's final
state. Lengths mix empty and length-1 sequences with
ones that cross the kernels' 8-step prefetch blocks; one case starts a sequence at every step,
one holds a single sequence."""
import numpy as np
import pytest
import torch

from oracle import slstm_ref as ref
from parity import GRAD_TOL, H_TOL_BF16, H_TOL_F32, case, grad_rel_err, h_floor, h_rel_err, to_np
from workloads import draw_head_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
LAYOUTS = {
    "mixed": [37, 0, 1, 30, 5, 0, 16, 1, 1, 20, 3],
    "all_ones": [1] * 20,
    "empty_ends": [0, 0, 40, 0, 1, 0],
    "single": [50],
}


def _problem(seed, lengths, dh, nh, p_dtype="f32"):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, S, d = int(cu[-1]), len(lengths), nh * dh
    x = draw_head_inputs(seed, 1, T, d, nh, p_dtype=p_dtype)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    s0 = np.stack([rng.uniform(-0.5, 0.5, (S, d)), rng.uniform(0.5, 2.0, (S, d)),
                   rng.uniform(-2.0, 2.0, (S, d)), rng.uniform(-0.9, 0.9, (S, d))], axis=1)
    return x["P"], x["R"], torch.from_numpy(s0.astype(np.float32)), cu


def _on(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _state_err(gpu, want):
    g, r = to_np(gpu), np.asarray(want)
    return max(float(np.max(np.abs(g[..., k, :] - r[..., k, :])) / max(float(np.max(np.abs(r[..., k, :]))), 1e-30))
               for k in range(4))


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("dh", [8, 32])
def test_head_packed_sequential(gpu_lib, layout, forget, dh):
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(1300 + dh, lengths, dh, 2)
    case(f"head packed sequential {layout} {forget} d_head={dh}")
    fin = torch.empty_like(s0).to(DEV)
    S, h = gpu_lib.head_sequential_forward(*_on(P, R, s0), forget, final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    seq = ref.sequential_head(to_np(P), to_np(R), to_np(s0), forget, cu_seqlens=cu)
    assert h_rel_err(h, seq[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32
    assert _state_err(S, seq) < 1e-5
    assert _state_err(fin, ref.final_states(seq, to_np(s0), cu)) < 1e-5
    for q in range(len(lengths)):  # an empty sequence hands its state0 on unchanged
        if cu[q] == cu[q + 1]:
            assert torch.equal(fin[q].cpu(), s0[q])


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("K", [3, 5])
def test_head_packed_newton(gpu_lib, layout, forget, K):
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(1310 + K, lengths, 16, 2)
    case(f"head packed newton {layout} {forget} K={K}")
    fin = torch.empty_like(s0).to(DEV)
    S, h, st = gpu_lib.head_newton_forward(*_on(P, R, s0), forget, K, 0.0, final_state=fin, cu_seqlens=cu,
                                           raise_on_divergence=False)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), forget, K, cu_seqlens=cu)
    err = h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32))
    print(f"head packed newton {layout} {forget} K={K}: h rel err {err:.2e}")
    assert err < H_TOL_F32
    assert st.iters == st_ref.iters == K and st.diverged == st_ref.diverged
    assert _state_err(fin, ref.final_states(S_ref, to_np(s0), cu)) < 1e-4


def test_head_packed_newton_early_stop(gpu_lib):
    """One residual maximum covers the whole pack, so the stop is global."""
    P, R, s0, cu = _problem(1320, LAYOUTS["mixed"], 32, 2, p_dtype="bf16")
    case("head packed newton early stop")
    _, h, st = gpu_lib.head_newton_forward(*_on(P, R, s0), "sigmoid", 8, 1e-5, cu_seqlens=cu)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "sigmoid", 8, tol=1e-5, cu_seqlens=cu)
    assert st_ref.converged and st.converged
    assert st.iters == st_ref.iters < 8
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16


@pytest.mark.parametrize("layout,dh,K,init", [(lay, dh, K, "warm") for lay in ("mixed", "all_ones", "empty_ends")
                                               for dh, K in ((8, 1), (16, 2), (32, 4), (64, 3))]
                         + [("all_ones", 16, 2, "zero")])
def test_head_packed_one_sweep(gpu_lib, layout, dh, K, init):
    """The packed one-sweep solve (fixed K <= 4) against the oracle, and against the same pack run
    iteration by iteration (a tolerance no residual meets keeps the per-iteration kernels)."""
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(1340 + dh + K, lengths, dh, 2)
    case(f"head packed one-sweep {layout} d_head={dh} K={K} {init}")
    fin = torch.empty_like(s0).to(DEV)
    S, h, st = gpu_lib.head_newton_forward(*_on(P, R, s0), "exp", K, 0.0, init=init, final_state=fin,
                                           cu_seqlens=cu, raise_on_divergence=False)
    _, h_it, _ = gpu_lib.head_newton_forward(*_on(P, R, s0), "exp", K, 1e-30, init=init, cu_seqlens=cu,
                                             raise_on_divergence=False)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", K, init=init, cu_seqlens=cu)
    err = h_rel_err(h, S_ref[..., 3, :])
    print(f"head packed one-sweep {layout} d_head={dh} K={K} {init}: h rel err {err:.2e}, "
          f"per-iteration form {h_rel_err(h_it, S_ref[..., 3, :]):.2e}")
    assert not st_ref.diverged and not st.diverged
    assert err < H_TOL_F32
    assert h_rel_err(h_it, to_np(h)) < H_TOL_F32
    assert st.iters == st_ref.iters == K
    assert _state_err(fin, ref.final_states(S_ref, to_np(s0), cu)) < 1e-4


def test_head_packed_single_sequence_matches_unpacked(gpu_lib):
    P, R, s0, cu = _problem(1330, [50], 32, 2)
    case("head packed single sequence vs unpacked call")
    _, hp, _ = gpu_lib.head_newton_forward(*_on(P, R, s0), "exp", 3, 0.0, cu_seqlens=cu)
    _, hu3, _ = gpu_lib.head_newton_forward(*_on(P, R, s0), "exp", 3, 0.0)  # unpacked: the one-sweep kernel
    torch.cuda.synchronize()
    S_ref, _ = ref.newton_head(to_np(P), to_np(R), to_np(s0), "exp", 3)
    assert h_rel_err(hp, S_ref[..., 3, :]) < H_TOL_F32
    assert h_rel_err(hu3, S_ref[..., 3, :]) < H_TOL_F32


@pytest.mark.parametrize("layout,dh", [(lay, dh) for lay in LAYOUTS for dh in (8, 32)] + [("mixed", 128)])
def test_head_packed_backward(gpu_lib, layout, dh):
    """At the oracle's packed trajectory (exponential forget gate: every step clear of the
    running maximum's tie), a loss on the states, h and each sequence's final state."""
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(1340 + dh, lengths, dh, 2)
    T, d, n = P.shape[1], P.shape[3], len(lengths)
    S = torch.from_numpy(ref.sequential_head(to_np(P), to_np(R), to_np(s0), "exp", cu_seqlens=cu).astype(np.float32))
    rng = np.random.Generator(np.random.PCG64(1350 + dh))
    gs = torch.from_numpy(rng.standard_normal((1, T, 4, d)).astype(np.float32))
    gh = torch.from_numpy(rng.standard_normal((1, T, d)).astype(np.float32))
    gf = torch.from_numpy(rng.standard_normal((n, 4, d)).astype(np.float32))
    case(f"head packed backward {layout} d_head={dh}")
    dP, dR, d0, db = gpu_lib.head_backward(*_on(P, R, S, s0, gs, gh, gf), "exp", want_dbias=True, cu_seqlens=cu)
    torch.cuda.synchronize()
    g = to_np(gs).copy()
    g[:, :, 3] += to_np(gh)
    want = ref.backward_head(to_np(P), to_np(R), to_np(s0), to_np(S), g, "exp", g_final=to_np(gf), cu_seqlens=cu)
    errs = [grad_rel_err(dP, want[0]), grad_rel_err(dR, want[1]), grad_rel_err(d0, want[2]),
            grad_rel_err(db, want[0].sum(axis=(0, 1)))]
    print(f"head packed backward {layout} d_head={dh}: rel err {['%.2e' % e for e in errs]}")
    assert max(errs) < GRAD_TOL
    for q in range(n):  # an empty sequence passes its final-state gradient on
        if cu[q] == cu[q + 1]:
            assert torch.equal(d0[q].cpu(), gf[q])
