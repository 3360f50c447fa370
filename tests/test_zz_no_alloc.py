"""The Newton entry point that allocates nothing (slstm_newton_forward_noalloc) against the one
that takes a caller workspace: the same kernels, so the same states, hidden slot, final state
and statistics bit for bit, on consecutive calls of decreasing size that share the library's
fixed scratch; and a problem too large for the scratch is refused before any work."""
import numpy as np
import pytest
import torch

from oracle import slstm_ref as ref
from parity import H_TOL_F32, case, h_rel_err, to_np
from workloads import by_name, draw_preactivation_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(gpu_lib, P, R, s0, forget, K, tol, schedule):
    B, T, _, d = P.shape
    outs = []
    for entry in ("workspace", "noalloc"):
        S = torch.full((B, T, 4, d), float("nan"), dtype=torch.float32, device=DEV)
        H = torch.full((B, T, d), float("nan"), dtype=torch.float32, device=DEV)
        F = torch.full((B, 4, d), float("nan"), dtype=torch.float32, device=DEV)
        if entry == "workspace":
            _, _, st = gpu_lib.newton_forward(P, R, s0, forget, K, tol, states=S, h_out=H, final_state=F,
                                              raise_on_divergence=False, schedule=schedule)
        else:
            _, _, st = gpu_lib.newton_forward_noalloc(P, R, s0, forget, K, tol, states=S, h_out=H,
                                                      final_state=F, raise_on_divergence=False,
                                                      schedule=schedule)
        outs.append((S, H, F, st))
    torch.cuda.synchronize()
    return outs


def _same(a, b):
    (Sa, Ha, Fa, sa), (Sb, Hb, Fb, sb) = a, b
    assert torch.equal(Sa, Sb) and torch.equal(Ha, Hb) and torch.equal(Fa, Fb)
    assert (sa.iters, sa.converged, sa.diverged, sa.nonfinite) == (sb.iters, sb.converged, sb.diverged,
                                                                    sb.nonfinite)
    assert sa.max_abs_F == sb.max_abs_F


def test_noalloc_matches_workspace_entry_on_consecutive_calls(gpu_lib):
    # call 1: the mid workload at full size, scan form (56 MiB of the 64 MiB scratch)
    w = by_name("mid_b8_t1024_d256")
    inp = draw_preactivation_inputs(w)
    P, R = inp["P"].to(DEV), inp["R"].to(DEV)
    case(f"noalloc 1: {w.name} K={w.max_iters} fused")
    a, b = _both(gpu_lib, P, R, None, w.forget, w.max_iters, 0.0, "fused")
    _same(a, b)
    S_ref, st_ref = ref.newton(to_np(inp["P"][:2, :, :, :32]), to_np(inp["R"][:, :32]), None, w.forget, w.max_iters)
    assert h_rel_err(b[1][:2, :, :32], S_ref[..., 3, :]) < H_TOL_F32
    assert b[3].iters == st_ref.iters == w.max_iters

    # call 2, smaller: the sigmoid / bf16 workload's early stop (one kernel per iteration, the
    # stop decided on the device from the scratch's control block)
    w2 = by_name("sigmoid_bf16p_b16_t4096_d1024")
    inp2 = draw_preactivation_inputs(w2, B=2, T=4096)
    P2 = inp2["P"][..., :64].contiguous().to(DEV)
    R2 = inp2["R"][:, :64].contiguous().to(DEV)
    case(f"noalloc 2: early stop B=2 T=4096 d=64 tol={w2.tol}")
    a, b = _both(gpu_lib, P2, R2, None, w2.forget, w2.max_iters, w2.tol, "fused")
    _same(a, b)
    assert b[3].converged and 2 <= b[3].iters < w2.max_iters

    # call 3, smaller again: the tiny workload in every schedule
    w3 = by_name("tiny_b2_t64_d16")
    inp3 = draw_preactivation_inputs(w3)
    for sched in ("fused_scan", "fused_chain", "layered"):
        case(f"noalloc 3: {w3.name} K=3 {sched}")
        a, b = _both(gpu_lib, inp3["P"].to(DEV), inp3["R"].to(DEV), None, w3.forget, 3, 0.0, sched)
        _same(a, b)


def test_noalloc_one_kernel_solve_then_smaller(gpu_lib):
    """Enough lane groups for the chain form: the whole fixed-count solve is one pipelined
    kernel whose look-back words live in the scratch; then a smaller problem of the same form
    with a state0."""
    rng = np.random.Generator(np.random.PCG64(77))
    for B, T, d in ((256, 40, 256), (256, 7, 250)):
        case(f"noalloc one-kernel solve B={B} T={T} d={d}")
        P = rng.standard_normal((B, T, 4, d))
        P[:, :, 2] += 3.0
        P = torch.from_numpy(P.astype(np.float32)).to(DEV)
        R = torch.from_numpy(rng.uniform(-0.5, 0.5, (4, d)).astype(np.float32)).to(DEV)
        s0 = torch.zeros((B, 4, d), dtype=torch.float32)
        s0[:, 1] = 1.0
        s0[:, 3] = torch.from_numpy(rng.uniform(-0.5, 0.5, (B, d)).astype(np.float32))
        a, b = _both(gpu_lib, P, R, s0.to(DEV), "exp", 3, 0.0, "fused")
        _same(a, b)


def test_noalloc_refuses_problems_beyond_the_scratch(gpu_lib):
    w = by_name("mid_b8_t1024_d256")
    inp = draw_preactivation_inputs(w)
    P, R = inp["P"].to(DEV), inp["R"].to(DEV)
    need = gpu_lib.newton_workspace_bytes(w.B, w.T, w.d_h, "layered")
    assert need > gpu_lib.NOALLOC_SCRATCH_BYTES
    case("noalloc: layered mid workload needs more than the scratch")
    S = torch.full((w.B, w.T, 4, w.d_h), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(gpu_lib.SlstmError, match="scratch"):
        gpu_lib.newton_forward_noalloc(P, R, None, w.forget, 3, 0.0, states=S, schedule="layered")
    torch.cuda.synchronize()
    assert bool((S == 7.0).all())
