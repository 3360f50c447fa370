"""End-to-end GPU parity of the Newton and sequential forwards against the float64 oracle:
h within the bar, identical iteration counts and flags; edge shapes; divergence; early stop;
sequence carrying through the final state."""
import numpy as np
import pytest
import torch

from oracle import lanes, slstm_ref as ref
from parity import H_TOL_BF16, H_TOL_F32, case, h_floor, h_rel_err, to_np
from workloads import by_name, draw_preactivation_inputs, random_states

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(params=["fused_scan", "fused_chain", "layered"])
def schedule(request):
    """Every kernel form of a Newton iteration must meet the same bar."""
    return request.param


def _run_both(gpu_lib, P, R, state0, forget, K, tol=0.0, init="warm", schedule="fused"):
    S, h, st = gpu_lib.newton_forward(P.to(DEV), R.to(DEV),
                                      None if state0 is None else state0.to(DEV), forget,
                                      K, tol, init, raise_on_divergence=False, schedule=schedule)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton(to_np(P), to_np(R), None if state0 is None else to_np(state0),
                               forget, K, tol=tol, init=init)
    return S, h, st, S_ref, st_ref


@pytest.mark.parametrize("K", [1, 2, 3, 4, 8, 16, 32, 64])
def test_tiny_fixed_k_sweep(gpu_lib, K, schedule):
    w = by_name("tiny_b2_t64_d16")
    case(f"newton {w.name} K={K}")
    inp = draw_preactivation_inputs(w)
    S, h, st, S_ref, st_ref = _run_both(gpu_lib, inp["P"], inp["R"], None, w.forget, K, schedule=schedule)
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_F32
    assert torch.equal(h, S[..., 3, :])
    assert st.iters == st_ref.iters == K
    assert st.diverged == st_ref.diverged is False
    assert st.converged == st_ref.converged is False
    assert len(st.max_abs_F) == K + 1


def test_mid_workload_full_size(gpu_lib, schedule):
    w = by_name("mid_b8_t1024_d256")
    case(f"newton {w.name} full size K={w.max_iters}")
    inp = draw_preactivation_inputs(w)
    S, h, st = gpu_lib.newton_forward(inp["P"].to(DEV), inp["R"].to(DEV), None, w.forget,
                                      w.max_iters, w.tol, schedule=schedule)
    torch.cuda.synchronize()
    S_ref, st_ref = lanes.newton_lanes(inp["P"], inp["R"], None, w.forget, w.max_iters, w.tol)
    h_ref = S_ref[:, :, 3].reshape(w.B, w.d_h, w.T).transpose(0, 2, 1)
    assert h_rel_err(h, h_ref) < H_TOL_F32
    assert st.iters == st_ref.iters and st.diverged == st_ref.diverged
    # and against the sequential recurrence: the K=3 Newton iterate is converged here
    seq = lanes.sequential_lanes(inp["P"], inp["R"], None, w.forget)
    h_seq = seq[:, :, 3].reshape(w.B, w.d_h, w.T).transpose(0, 2, 1)
    assert h_rel_err(h, h_seq) < H_TOL_F32


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 2, 3), (3, 33, 65), (2, 257, 20), (1, 70, 64)])
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_edge_shapes(gpu_lib, shape, forget, schedule):
    B, T, d = shape
    case(f"newton edge B={B} T={T} d={d} {forget}")
    rng = np.random.Generator(np.random.PCG64(B * 1000 + T * 10 + d))
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d))
    s0 = np.zeros((B, 4, d))
    s0[:, 0] = rng.uniform(-0.3, 0.3, (B, d))
    s0[:, 1] = rng.uniform(0.5, 1.5, (B, d))
    s0[:, 2] = rng.uniform(-1, 1, (B, d))
    s0[:, 3] = rng.uniform(-0.5, 0.5, (B, d))
    Pt = torch.from_numpy(P.astype(np.float32))
    Rt = torch.from_numpy(R.astype(np.float32))
    s0t = torch.from_numpy(s0.astype(np.float32))
    S, h, st, S_ref, st_ref = _run_both(gpu_lib, Pt, Rt, s0t, forget, 6, schedule=schedule)
    assert h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32
    assert st.iters == st_ref.iters and st.diverged == st_ref.diverged
    Ss, hs = gpu_lib.sequential_forward(Pt.to(DEV), Rt.to(DEV), s0t.to(DEV), forget)
    torch.cuda.synchronize()
    seq_ref = ref.sequential(to_np(Pt), to_np(Rt), to_np(s0t), forget)
    assert h_rel_err(hs, seq_ref[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32


@pytest.mark.parametrize("name", ["tiny_b2_t64_d16", "mid_b8_t1024_d256"])
def test_sequential_full_size(gpu_lib, name):
    w = by_name(name)
    case(f"sequential {name}")
    inp = draw_preactivation_inputs(w)
    S, h = gpu_lib.sequential_forward(inp["P"].to(DEV), inp["R"].to(DEV), None, w.forget)
    torch.cuda.synchronize()
    seq = lanes.sequential_lanes(inp["P"], inp["R"], None, w.forget)
    h_seq = seq[:, :, 3].reshape(w.B, w.d_h, w.T).transpose(0, 2, 1)
    assert h_rel_err(h, h_seq) < H_TOL_F32
    assert torch.equal(h, S[..., 3, :])


def test_zero_guess_diverges_on_both_sides(gpu_lib, schedule):
    # the zero iterate overflows on a long exponential-forget sequence
    w = by_name("mid_b8_t1024_d256")
    case("newton zero init B=2 T=1024 d=32 K=3")
    inp = draw_preactivation_inputs(w, B=2)
    P = inp["P"][..., :32].contiguous()
    R = inp["R"][:, :32].contiguous()
    S, h, st, S_ref, st_ref = _run_both(gpu_lib, P, R, None, "exp", 3, init="zero", schedule=schedule)
    assert st_ref.diverged and st.diverged
    assert st.nonfinite == st_ref.nonfinite


def test_nan_input_gives_nonfinite(gpu_lib, schedule):
    w = by_name("tiny_b2_t64_d16")
    case("newton NaN input")
    inp = draw_preactivation_inputs(w)
    P = inp["P"].clone()
    P[1, 17, 1, 5] = float("nan")
    S, h, st, S_ref, st_ref = _run_both(gpu_lib, P, inp["R"], None, w.forget, 3, schedule=schedule)
    assert st.diverged and st.nonfinite and st_ref.diverged and st_ref.nonfinite
    assert st.status == gpu_lib.NONFINITE
    with pytest.raises(gpu_lib.NewtonDivergenceError):
        gpu_lib.newton_forward(P.to(DEV), inp["R"].to(DEV), None, w.forget, 3, schedule=schedule)


@pytest.mark.parametrize("B,T,d", [(2, 4096, 64), (1, 1000, 16)])
def test_early_stop_sigmoid_bf16(gpu_lib, B, T, d, schedule):
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    case(f"newton early stop {w.name} B={B} T={T} d={d}")
    inp = draw_preactivation_inputs(w, B=B, T=T)
    P = inp["P"][..., :d].contiguous()
    R = inp["R"][:, :d].contiguous()
    S, h, st, S_ref, st_ref = _run_both(gpu_lib, P, R, None, w.forget, w.max_iters, w.tol, schedule=schedule)
    assert st_ref.converged and st.converged
    assert st.iters == st_ref.iters
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16
    # the GPU's residual history tracks the oracle's until the rounding floor
    for k in range(st.iters):
        assert st.max_abs_F[k] == pytest.approx(st_ref.max_abs_F[k], rel=0.05, abs=2e-5)


def test_state_carry_across_calls(gpu_lib, schedule):
    w = by_name("tiny_b2_t64_d16")
    case("newton state carry T=64 as 32 + 32")
    inp = draw_preactivation_inputs(w)
    P = inp["P"].to(DEV)
    R = inp["R"].to(DEV)
    S_full, h_full, _ = gpu_lib.newton_forward(P, R, None, w.forget, 8, schedule=schedule)
    fin1 = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=DEV)
    S1, _, _ = gpu_lib.newton_forward(P[:, :32].contiguous(), R, None, w.forget, 8, final_state=fin1,
                                      schedule=schedule)
    S2, h2, _ = gpu_lib.newton_forward(P[:, 32:].contiguous(), R, fin1, w.forget, 8, schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(fin1, S1[:, -1])
    assert h_rel_err(h2, h_full[:, 32:]) < H_TOL_F32
    fq1 = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=DEV)
    Sq1, _ = gpu_lib.sequential_forward(P[:, :32].contiguous(), R, None, w.forget, final_state=fq1)
    Sq2, hq2 = gpu_lib.sequential_forward(P[:, 32:].contiguous(), R, fq1, w.forget)
    Sq, hq = gpu_lib.sequential_forward(P, R, None, w.forget)
    torch.cuda.synchronize()
    assert torch.equal(fq1, Sq1[:, -1])
    assert torch.equal(hq2, hq[:, 32:])


def test_async_stats_readback(gpu_lib, schedule):
    w = by_name("tiny_b2_t64_d16")
    case("newton async + read_stats")
    inp = draw_preactivation_inputs(w)
    ws = torch.empty(gpu_lib.newton_workspace_bytes(w.B, w.T, w.d_h, schedule), dtype=torch.uint8,
                     device=DEV)
    S, h, st = gpu_lib.newton_forward(inp["P"].to(DEV), inp["R"].to(DEV), None, w.forget, 4,
                                      workspace=ws, stats=False, schedule=schedule)
    assert st is None
    st = gpu_lib.read_stats(ws)
    assert st.iters == 4 and not st.diverged and len(st.max_abs_F) == 5


@pytest.mark.parametrize("form", ["fused_scan", "fused_chain"])
def test_schedules_agree(gpu_lib, form):
    """The fused forms and the layered schedule compute the same iterates up to float32
    rounding."""
    w = by_name("mid_b8_t1024_d256")
    case(f"{form} vs layered, mid workload")
    inp = draw_preactivation_inputs(w)
    P = inp["P"].to(DEV)
    R = inp["R"].to(DEV)
    Sf, hf, stf = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, schedule=form)
    Sl, hl, stl = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, schedule="layered")
    torch.cuda.synchronize()
    assert stf.iters == stl.iters
    assert h_rel_err(hf, hl) < H_TOL_F32
    for k in range(stf.iters + 1):
        assert stf.max_abs_F[k] == pytest.approx(stl.max_abs_F[k], rel=1e-3, abs=1e-4)


def test_fused_picks_a_form(gpu_lib):
    """schedule="fused" resolves to one of the two fused forms, bit for bit."""
    w = by_name("mid_b8_t1024_d256")
    case("fused (automatic form) equals fused_scan or fused_chain")
    inp = draw_preactivation_inputs(w)
    P = inp["P"].to(DEV)
    R = inp["R"].to(DEV)
    outs = {s: gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, schedule=s)
            for s in ("fused", "fused_scan", "fused_chain")}
    torch.cuda.synchronize()
    assert any(torch.equal(outs["fused"][0], outs[s][0]) for s in ("fused_scan", "fused_chain"))


@pytest.mark.parametrize("form", ["fused_scan", "fused_chain"])
def test_early_stop_lands_in_either_buffer(gpu_lib, form):
    """Fused forms: an early stop after an odd or even number of updates leaves the result
    in either iterate buffer; the returned states must be the stopped iterate either way."""
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    inp = draw_preactivation_inputs(w, B=1, T=2048)
    P = inp["P"][..., :64].contiguous()
    R = inp["R"][:, :64].contiguous()
    # n: the iteration the oracle stops at. Budgets n and n + 1 make the stop fall on the last
    # launch (the chain form decides it after its last iteration), 7 and 8 well before it.
    n = ref.newton(to_np(P), to_np(R), None, w.forget, 8, tol=w.tol)[1].iters
    assert 2 <= n < 6
    for K in sorted({n, n + 1, n + 2, 7, 8}):
        case(f"{form} early stop at {n}, budget K={K}")
        S, h, st, S_ref, st_ref = _run_both(gpu_lib, P, R, None, w.forget, K, w.tol, schedule=form)
        assert st.converged and st.iters == st_ref.iters == min(n, K)
        assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16
        assert torch.equal(h, S[..., 3, :])


@pytest.mark.parametrize("init", ["warm", "zero"])
def test_one_kernel_solve_matches_iteration_kernels(gpu_lib, init):
    """fused_chain with tol = 0 and K <= 4 runs the whole solve as one pipelined kernel; with a
    tolerance that is never met it runs one kernel per iteration. Both form every value with
    the same float32 operations in the same order, so they agree bit for bit (ragged T and d,
    a random initial state)."""
    w = by_name("mid_b8_t1024_d256")
    inp = draw_preactivation_inputs(w, B=3, T=999)
    P = inp["P"][..., :200].contiguous().to(DEV)
    R = inp["R"][:, :200].contiguous().to(DEV)
    s0 = torch.from_numpy(random_states(w.seed + 7, 3, 1, 200)[:, 0].astype(np.float32)).to(DEV)
    for K in (1, 3, 4, 5):
        case(f"one-kernel solve vs per-iteration chain, init={init}, K={K}")
        gpu_lib.profile_reset()
        gpu_lib.profile_enable(True)
        Sa, ha, sta = gpu_lib.newton_forward(P, R, s0, w.forget, K, 0.0, init, raise_on_divergence=False,
                                             schedule="fused_chain")
        n_solve = len(gpu_lib.profile_durations("newton_solve"))
        gpu_lib.profile_reset()
        Sb, hb, stb = gpu_lib.newton_forward(P, R, s0, w.forget, K, 1e-30, init, raise_on_divergence=False,
                                             schedule="fused_chain")
        n_iter = len(gpu_lib.profile_durations("newton_iteration"))
        gpu_lib.profile_enable(False)
        torch.cuda.synchronize()
        # K = 5 is past the one-kernel solve's limit: both calls iterate kernel by kernel
        assert n_solve == (1 if K <= 4 else 0) and n_iter == K
        assert sta.iters == stb.iters == K
        # the zero guess diverges: NaN in the same places (its payload may come from either
        # operand of a product, which the compiler may order differently), equal elsewhere
        for a, b in ((Sa, Sb), (ha, hb)):
            nan = torch.isnan(a)
            assert torch.equal(nan, torch.isnan(b))
            assert torch.equal(a[~nan], b[~nan])
        assert np.array_equal(np.array(sta.max_abs_F), np.array(stb.max_abs_F), equal_nan=True)


@pytest.mark.parametrize("name,readout", [("mid_b8_t1024_d256", "exact"), ("sigmoid_bf16p_b16_t4096_d1024", "exact"),
                                          ("mid_b8_t1024_d256", "floored")])
def test_hidden_only_output(gpu_lib, name, readout):
    """The layer's default output, the hidden slot and the final state without the state tensor
    ("sLSTM in this library", "Outputs"): the one-kernel solve writes h and the final state
    itself. Both equal, bit for bit, what the same solve writes beside the states, and match the
    oracle (ragged T and d; a random initial state on the float32 workload, none on the
    sigmoid/bf16 one; warm and zero guesses; K = 4 at its limit)."""
    w = by_name(name)
    forget = w.forget
    p_dtype = w.p_dtype
    inp = draw_preactivation_inputs(w, B=3, T=999)
    P = inp["P"][..., :200].contiguous()
    R = inp["R"][:, :200].contiguous()
    s0 = (torch.from_numpy(random_states(w.seed + 11, 3, 1, 200)[:, 0].astype(np.float32))
          if p_dtype == "f32" else None)
    dev = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    for init, K in (("warm", 3), ("warm", 4), ("zero", 2)):
        case(f"hidden-only output {p_dtype}/{forget}/{readout}, init={init}, K={K}")
        fs_a = torch.empty(3, 4, 200, device=DEV)
        fs_b = torch.full((3, 4, 200), float("nan"), device=DEV)
        Sa, ha, sta = gpu_lib.newton_forward(P.to(DEV), R.to(DEV), dev(s0), forget, K, 0.0, init,
                                             final_state=fs_a, raise_on_divergence=False,
                                             schedule="fused_chain", readout=readout)
        Sb, hb, stb = gpu_lib.newton_forward(P.to(DEV), R.to(DEV), dev(s0), forget, K, 0.0, init,
                                             final_state=fs_b, raise_on_divergence=False,
                                             schedule="fused_chain", readout=readout, output_states=False)
        torch.cuda.synchronize()
        assert Sb is None
        # the zero guess diverges: compare NaN positions, values elsewhere
        for a, b in ((fs_a, Sa[:, -1]), (ha, hb), (fs_a, fs_b)):
            nan = torch.isnan(a)
            assert torch.equal(nan, torch.isnan(b))
            assert torch.equal(a[~nan], b[~nan])
        assert sta.iters == stb.iters == K
        assert np.array_equal(np.array(sta.max_abs_F), np.array(stb.max_abs_F), equal_nan=True)
        if init == "warm":
            mode = forget if readout == "exact" else forget + "/floored"
            S_ref, st_ref = ref.newton(to_np(P), to_np(R), None if s0 is None else to_np(s0), mode, K,
                                       init=init)
            bar = H_TOL_BF16 if p_dtype == "bf16" else H_TOL_F32
            fl = h_floor(forget, bar)
            assert h_rel_err(hb, S_ref[..., 3, :], fl) < bar
            assert h_rel_err(fs_b[:, 3], S_ref[:, -1, 3], fl) < bar
            for slot in range(3):  # c, n, m of the final state, normwise per slot
                ref_s = S_ref[:, -1, slot]
                assert np.max(np.abs(to_np(fs_b[:, slot]) - ref_s)) <= bar * np.max(np.abs(ref_s))
            assert stb.diverged == st_ref.diverged


@pytest.mark.parametrize("p_dtype", ["f32", "bf16"])
def test_sequential_hidden_only_output(gpu_lib, p_dtype):
    """The sequential forward writing only h and the final state (no state tensor) gives, bit
    for bit, what it writes beside the states (ragged d, a random initial state)."""
    w = by_name("mid_b8_t1024_d256")
    inp = draw_preactivation_inputs(w, B=3, T=333)
    P = inp["P"][..., :200].contiguous()
    if p_dtype == "bf16":
        P = P.to(torch.bfloat16)
    R = inp["R"][:, :200].contiguous().to(DEV)
    s0 = torch.from_numpy(random_states(w.seed + 13, 3, 1, 200)[:, 0].astype(np.float32)).to(DEV)
    case(f"sequential hidden-only output {p_dtype}")
    fa = torch.empty(3, 4, 200, device=DEV)
    fb = torch.empty(3, 4, 200, device=DEV)
    Sa, ha = gpu_lib.sequential_forward(P.to(DEV), R, s0, w.forget, final_state=fa)
    Sb, hb = gpu_lib.sequential_forward(P.to(DEV), R, s0, w.forget, final_state=fb, output_states=False)
    torch.cuda.synchronize()
    assert Sb is None
    assert torch.equal(ha, hb) and torch.equal(fa, fb) and torch.equal(fa, Sa[:, -1])


def test_early_stop_as_two_one_kernel_passes(gpu_lib):
    """FUSED on 32 lane groups with a tolerance runs the one-kernel solve for the budget, finds
    the first iterate below tol and runs it again for that count. Iteration count, flags, every
    residual maximum, h and the final state equal, bit for bit, those of the per-iteration chain
    kernels with the same early stop (the stop landing before, at and past the budget, and no
    stop), and match the oracle; with no state tensor the same h and final state come out."""
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    inp = draw_preactivation_inputs(w, B=32, T=256)
    P = inp["P"][..., :256].contiguous()
    R = inp["R"][:, :256].contiguous()
    n = ref.newton(to_np(P), to_np(R), None, w.forget, 8, tol=w.tol)[1].iters
    assert 2 <= n < 8
    Pd, Rd = P.to(DEV), R.to(DEV)
    for K in sorted({n - 1, n, n + 1, 8}):
        case(f"early stop at {n} as two one-kernel passes, budget K={K}")
        gpu_lib.profile_reset()
        gpu_lib.profile_enable(True)
        fa = torch.empty(32, 4, 256, device=DEV)
        Sa, ha, sta = gpu_lib.newton_forward(Pd, Rd, None, w.forget, K, w.tol, final_state=fa,
                                             raise_on_divergence=False, schedule="fused")
        n_solve = len(gpu_lib.profile_durations("newton_solve"))
        n_iter = len(gpu_lib.profile_durations("newton_iteration"))
        gpu_lib.profile_enable(False)
        fb = torch.empty(32, 4, 256, device=DEV)
        Sb, hb, stb = gpu_lib.newton_forward(Pd, Rd, None, w.forget, K, w.tol, final_state=fb,
                                             raise_on_divergence=False, schedule="fused_chain")
        fc = torch.empty(32, 4, 256, device=DEV)
        _, hc, stc = gpu_lib.newton_forward(Pd, Rd, None, w.forget, K, w.tol, final_state=fc,
                                            raise_on_divergence=False, schedule="fused", output_states=False)
        torch.cuda.synchronize()
        assert n_solve == 2 and n_iter == 0  # both passes of the one-kernel form, no iteration kernels
        for st in (sta, stc):
            assert (st.iters, st.converged, st.diverged, st.nonfinite) == \
                (stb.iters, stb.converged, stb.diverged, stb.nonfinite)
            assert np.array_equal(np.array(st.max_abs_F), np.array(stb.max_abs_F))
        assert torch.equal(ha, hb) and torch.equal(hc, hb) and torch.equal(Sa, Sb)
        assert torch.equal(fa, fb) and torch.equal(fc, fb)
        S_ref, st_ref = ref.newton(to_np(P), to_np(R), None, w.forget, K, tol=w.tol)
        assert sta.iters == st_ref.iters == min(n, K) and sta.converged == st_ref.converged
        assert h_rel_err(ha, S_ref[..., 3, :]) < H_TOL_BF16
    # a fixed count past the single-pass limit of FUSED_CHAIN (4) but within FUSED's (8): one
    # launch of the one-kernel form, bitwise the per-iteration chain kernels
    case("fused fixed count K=6 as one kernel")
    gpu_lib.profile_reset()
    gpu_lib.profile_enable(True)
    Sa, ha, sta = gpu_lib.newton_forward(Pd, Rd, None, w.forget, 6, 0.0, raise_on_divergence=False, schedule="fused")
    n_solve = len(gpu_lib.profile_durations("newton_solve"))
    gpu_lib.profile_enable(False)
    Sb, hb, stb = gpu_lib.newton_forward(Pd, Rd, None, w.forget, 6, 0.0, raise_on_divergence=False,
                                         schedule="fused_chain")
    torch.cuda.synchronize()
    assert n_solve == 1 and sta.iters == stb.iters == 6
    assert np.array_equal(np.array(sta.max_abs_F), np.array(stb.max_abs_F))
    assert torch.equal(ha, hb) and torch.equal(Sa, Sb)
