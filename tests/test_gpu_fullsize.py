"""Parity at the workloads' full sizes, in the configuration the benchmark times.

The GPU solves the whole workload; the float64 oracle solves sampled lanes (b, j) over the full
T. Lanes are independent under channelwise mixing, so a sampled lane's oracle result is exactly
that lane of the full problem. Iteration counts and flags are global: the early-stop count of
the sigmoid workload is compared against the oracle's residual history over every lane; for the
fixed-K workloads the flags are compared through properties that hold at any size (the sampled
oracle residual bounds nothing globally, so the GPU's own global residual is checked against the
float32 rounding floor of its largest state)."""
import numpy as np
import pytest
import torch

from oracle import lanes, slstm_ref as ref
from parity import H_FLOOR_SIGMOID, H_TOL_BF16, H_TOL_F32, case, h_rel_err, sample_lanes, to_np
from workloads import (by_name, draw_decode_inputs, draw_layer_inputs, draw_preactivation_inputs,
                       random_states, to_bf16)

pytestmark = pytest.mark.gpu

DEV = "cuda"

# Regression guards for the workloads whose contract bar is the bf16 one (2e-2). The float32
# path measures h errors of order 1e-5 there, so a bar of 2e-2 alone would let a thousandfold
# regression pass. Each guard is about ten times the error measured on MI355X, at the same
# floor; exceeding it means the kernels lost accuracy, not that the contract is broken.
GUARD_SIGMOID_BF16 = 1e-3   # measured 8.6e-5 .. 9.1e-5 (all three schedules)
GUARD_LAYER = 1e-4          # measured 1.06e-5
GUARD_DECODE = 1e-4         # measured 1.0e-5 (decode from the forward's final state)


@pytest.fixture(params=["fused_scan", "fused_chain", "layered"])
def schedule(request):
    return request.param


def _gpu_h_at(h, lb, lj):
    """GPU hidden states (B, T, d) at sampled lanes -> (n, T)."""
    idx_b = torch.as_tensor(lb, device=h.device)
    idx_j = torch.as_tensor(lj, device=h.device)
    return h[idx_b, :, idx_j].detach().cpu().double().numpy()


def test_sigmoid_bf16_workload_full_size(gpu_lib, schedule):
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    case(f"full size {w.name}: GPU Newton with early stop, oracle history over all lanes")
    inp = draw_preactivation_inputs(w, device=DEV)
    P = inp["P"].to(DEV)
    R = inp["R"].to(DEV)
    S, h, st = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, schedule=schedule)
    torch.cuda.synchronize()
    assert st.converged and not st.diverged
    lb, lj = sample_lanes(w.B, w.d_h, 96, seed=1)
    # the oracle decides its stop from every lane's residual history (pass 1), then solves the
    # sampled lanes to that iteration (pass 2); one iteration beyond the GPU's count is enough to
    # see whether it would stop at the same place
    S_ref, st_ref = lanes.newton_lanes(inp["P"], inp["R"], None, w.forget, st.iters + 1, w.tol,
                                       lanes=(lb, lj))
    assert st_ref.iters == st.iters and st_ref.converged == st.converged
    for k in range(st.iters):
        assert st.max_abs_F[k] == pytest.approx(st_ref.max_abs_F[k], rel=0.05, abs=2e-5)
    hg = _gpu_h_at(h, lb, lj)
    err = h_rel_err(hg, S_ref[:, :, 3])
    err_sig = h_rel_err(hg, S_ref[:, :, 3], H_FLOOR_SIGMOID)
    print(f"sigmoid bf16 full size: iters {st.iters}, h rel err {err:.2e} (floor 1e-3), "
          f"{err_sig:.2e} (floor 1e-2)")
    assert err < H_TOL_BF16
    assert err < GUARD_SIGMOID_BF16


def test_long_context_workload_full_size(gpu_lib, schedule):
    w = by_name("long_b4_t16384_d2048")
    case(f"full size {w.name}: GPU Newton K={w.max_iters}, oracle on sampled lanes")
    inp = draw_preactivation_inputs(w, device=DEV)
    P = inp["P"].to(DEV)
    R = inp["R"].to(DEV)
    S, h, st = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, schedule=schedule)
    torch.cuda.synchronize()
    assert st.iters == w.max_iters and not st.diverged and not st.nonfinite
    # the residual of the last iterate sits at the float32 rounding floor of m (~ulp of max m)
    m_max = float(S[..., 2, :].abs().max())
    assert st.max_abs_F[-1] <= 64 * np.spacing(np.float32(m_max))
    lb, lj = sample_lanes(w.B, w.d_h, 48, seed=2)
    S_ref, st_ref = lanes.newton_lanes(inp["P"], inp["R"], None, w.forget, w.max_iters, w.tol,
                                       lanes=(lb, lj), history_lanes=(lb, lj))
    assert not st_ref.diverged
    err = h_rel_err(_gpu_h_at(h, lb, lj), S_ref[:, :, 3])
    print(f"long context full size: h rel err {err:.2e}, GPU max|F| {st.max_abs_F}")
    assert err < H_TOL_F32
    # and the sequential forward on the same lanes
    Ss, hs = gpu_lib.sequential_forward(P, R, None, w.forget)
    torch.cuda.synchronize()
    seq = lanes.sequential_lanes(inp["P"], inp["R"], None, w.forget, lanes=(lb, lj))
    assert h_rel_err(_gpu_h_at(hs, lb, lj), seq[:, :, 3]) < H_TOL_F32


def test_full_layer_workload_full_size(gpu_lib, schedule):
    w = by_name("layer_b128_t2048_d1024")
    case(f"full size {w.name}: MFMA projection + Newton K={w.max_iters}, oracle on sampled lanes")
    inp = draw_layer_inputs(w)
    x = inp["x"].to(DEV)
    W = inp["W"].to(DEV)
    bias = inp["bias"].to(DEV)
    R = inp["R"].to(DEV)
    P = gpu_lib.input_projection(x, W, bias)
    fin = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=DEV)
    S, h, st = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, final_state=fin,
                                      schedule=schedule)
    torch.cuda.synchronize()
    assert st.iters == w.max_iters and not st.diverged
    assert torch.equal(fin, S[:, -1])
    m_max = float(S[..., 2, :].abs().max())
    assert st.max_abs_F[-1] <= 64 * np.spacing(np.float32(m_max))
    lb, lj = sample_lanes(w.B, w.d_h, 64, seed=3)
    # oracle: its own float64 projection of the sampled lanes from the same bf16 x and W_x
    x64 = to_np(inp["x"][torch.as_tensor(np.unique(lb))])
    rows = {int(b): k for k, b in enumerate(np.unique(lb))}
    W64 = to_np(inp["W"])
    b64 = to_np(inp["bias"])
    P_lanes = np.empty((1, w.T, 4, len(lb)))
    for k, (b, j) in enumerate(zip(lb, lj)):
        P_lanes[0, :, :, k] = ref.input_projection(x64[rows[int(b)]][None], W64[:, j:j + 1], b64[:, j:j + 1])[0, :, :, 0]
    # GPU projection of the same lanes against the oracle's
    P_gpu = P[torch.as_tensor(lb, device=DEV), :, :, torch.as_tensor(lj, device=DEV)].cpu().double().numpy()
    assert float(np.max(np.abs(P_gpu - np.transpose(P_lanes[0], (2, 0, 1))))) < 2e-5 * np.sqrt(w.d_in)
    S_ref, st_ref = ref.newton(P_lanes, to_np(inp["R"])[:, lj], None, w.forget, w.max_iters, tol=w.tol)
    assert not st_ref.diverged
    err = h_rel_err(_gpu_h_at(h, lb, lj), np.transpose(S_ref[0, :, 3, :], (1, 0)))
    print(f"full layer: h rel err {err:.2e} (bar {H_TOL_BF16}, guard {GUARD_LAYER})")
    assert err < H_TOL_BF16
    assert err < GUARD_LAYER

    # the T = 1 decode step continues each side's own forward: the GPU from the GPU's final
    # state, the oracle from its own K-iteration final state of the sampled lanes, both with
    # the benchmark's fresh bf16 input row projected by the same weights
    case("decode: T=1 step at B=128 from the forward's final state")
    del S, h
    x_dec = draw_decode_inputs(w)
    P_dec = gpu_lib.input_projection(x_dec.to(DEV), W, bias)
    _, h_dec = gpu_lib.sequential_forward(P_dec, R, fin, w.forget)
    torch.cuda.synchronize()
    Pd_ref = ref.input_projection(to_np(x_dec), W64, b64)            # (B, 1, 4, d)
    Pd_lanes = Pd_ref[lb, 0, :, lj].T                               # (4, n) at the sampled lanes
    fin_ref = S_ref[0, -1]                                            # (4, n) at the sampled lanes
    S_dec_ref = ref.sequential(Pd_lanes[None, None], to_np(inp["R"])[:, lj], fin_ref[None], w.forget)
    hd = h_dec[torch.as_tensor(lb, device=DEV), 0, torch.as_tensor(lj, device=DEV)].cpu().double().numpy()
    err_dec = h_rel_err(hd, S_dec_ref[0, 0, 3])
    print(f"full layer decode from the forward's final state: h rel err {err_dec:.2e}")
    assert err_dec < H_TOL_BF16
    assert err_dec < GUARD_DECODE


def test_full_layer_hidden_only_as_benchmarked(gpu_lib):
    """The full-layer forward in the launch the benchmark times: schedule "fused" (the one-kernel
    solve at this shape) writing the layer's default output, h and the final state, without a
    state tensor. h and the final state equal, bit for bit, those of the same solve writing the
    states, and h matches the oracle on sampled lanes."""
    w = by_name("layer_b128_t2048_d1024")
    case(f"full size {w.name}: hidden-only one-kernel solve as the benchmark launches it")
    inp = draw_layer_inputs(w)
    W = inp["W"].to(DEV)
    bias = inp["bias"].to(DEV)
    R = inp["R"].to(DEV)
    P = gpu_lib.input_projection(inp["x"].to(DEV), W, bias)
    ws = gpu_lib.alloc_workspace(gpu_lib.newton_workspace_bytes(w.B, w.T, w.d_h, "fused"), P.device)
    H = torch.empty((w.B, w.T, w.d_h), dtype=torch.float32, device=DEV)
    fin = torch.empty((w.B, 4, w.d_h), dtype=torch.float32, device=DEV)
    gpu_lib.profile_reset()
    gpu_lib.profile_enable(True)
    Sn, _, st = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, "warm", states=None, h_out=H,
                                       final_state=fin, workspace=ws, schedule="fused", output_states=False)
    n_solve = len(gpu_lib.profile_durations("newton_solve"))
    gpu_lib.profile_enable(False)
    torch.cuda.synchronize()
    assert Sn is None and n_solve == 1  # the one-kernel form ran
    assert st.iters == w.max_iters and not st.diverged
    S, h, st2 = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, workspace=ws, schedule="fused")
    torch.cuda.synchronize()
    assert torch.equal(H, h) and torch.equal(fin, S[:, -1])
    assert np.array_equal(np.array(st.max_abs_F), np.array(st2.max_abs_F))
    del S, h
    lb, lj = sample_lanes(w.B, w.d_h, 32, seed=5)
    x64 = to_np(inp["x"][torch.as_tensor(np.unique(lb))])
    rows = {int(b): k for k, b in enumerate(np.unique(lb))}
    W64 = to_np(inp["W"])
    b64 = to_np(inp["bias"])
    P_lanes = np.empty((1, w.T, 4, len(lb)))
    for k, (b, j) in enumerate(zip(lb, lj)):
        P_lanes[0, :, :, k] = ref.input_projection(x64[rows[int(b)]][None], W64[:, j:j + 1], b64[:, j:j + 1])[0, :, :, 0]
    S_ref, st_ref = ref.newton(P_lanes, to_np(inp["R"])[:, lj], None, w.forget, w.max_iters, tol=w.tol)
    err = h_rel_err(_gpu_h_at(H, lb, lj), np.transpose(S_ref[0, :, 3, :], (1, 0)))
    print(f"full layer, hidden-only: h rel err {err:.2e}")
    assert err < H_TOL_BF16 and err < GUARD_LAYER
    fin_gpu = fin[torch.as_tensor(lb, device=DEV), 3, torch.as_tensor(lj, device=DEV)]
    assert h_rel_err(fin_gpu, S_ref[0, -1, 3]) < GUARD_LAYER


def test_full_layer_decode_step(gpu_lib):
    """The decode step on every lane of the batch, from a drawn state (the chained case on
    sampled lanes is part of the full-layer test)."""
    w = by_name("layer_b128_t2048_d1024")
    case("decode: T=1 sequential step at B=128 after the input projection")
    inp = draw_layer_inputs(w, B=1, T=1)
    rng = np.random.Generator(np.random.PCG64(w.seed + 2000))
    x = to_bf16(rng.standard_normal((w.decode_batch, 1, w.d_in)))
    # a plausible state to continue from, drawn here: it is an input of the step
    s0 = random_states(w.seed + 3000, w.decode_batch, 1, w.d_h)[:, 0].astype(np.float32)
    P = gpu_lib.input_projection(x.to(DEV), inp["W"].to(DEV), inp["bias"].to(DEV))
    fin = torch.empty((w.decode_batch, 4, w.d_h), dtype=torch.float32, device=DEV)
    S, h = gpu_lib.sequential_forward(P, inp["R"].to(DEV), torch.from_numpy(s0).to(DEV), w.forget,
                                      final_state=fin)
    torch.cuda.synchronize()
    P_ref = ref.input_projection(to_np(x), to_np(inp["W"]), to_np(inp["bias"]))
    S_ref = ref.sequential(P_ref, to_np(inp["R"]), s0.astype(np.float64), w.forget)
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16
    assert torch.equal(fin, S[:, 0])
