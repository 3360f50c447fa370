"""Per-kernel parity on the GPU, through the C ABI, against the float64 oracle on the same
seeded inputs: residual + Jacobian, the 4x4 scan, the warm start, the input projection."""
import numpy as np
import pytest
import torch

from oracle import slstm_ref as ref
from parity import case, h_floor, h_rel_err, to_np
from workloads import by_name, draw_preactivation_inputs, random_scan_operands, random_states, to_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rel(a, b, floor):
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor)))


@pytest.mark.parametrize("forget,p_dtype", [("exp", "f32"), ("sigmoid", "f32"), ("sigmoid", "bf16")])
@pytest.mark.parametrize("shape", [(2, 64, 16), (3, 37, 70), (1, 1, 1)])
def test_residual_jacobian(gpu_lib, forget, p_dtype, shape):
    B, T, d = shape
    case(f"residual_jacobian {forget} {p_dtype} B={B} T={T} d={d}")
    rng = np.random.Generator(np.random.PCG64(100 + B * T * d))
    P = rng.standard_normal((B, T, 4, d)) * 1.5
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d)).astype(np.float32)
    S = random_states(7, B, T, d).astype(np.float32)
    s0 = random_states(8, B, 1, d)[:, 0].astype(np.float32)
    Pt = torch.from_numpy(P.astype(np.float32))
    if p_dtype == "bf16":
        Pt = Pt.to(torch.bfloat16)
    A, rhs, err = gpu_lib.residual_jacobian(Pt.to(DEV), torch.from_numpy(R).to(DEV),
                                            torch.from_numpy(S).to(DEV),
                                            torch.from_numpy(s0).to(DEV), forget)
    torch.cuda.synchronize()
    P64 = to_np(Pt)
    F, A_ref = ref.residual(S.astype(np.float64), P64, R.astype(np.float64), s0.astype(np.float64), forget)
    # f(s') itself, compared relative to its own scale (rhs = f - s cancels)
    f_gpu = to_np(rhs) + S
    f_ref = S - F
    assert _rel(f_gpu, f_ref, 1.0) < 5e-6
    A_gpu = to_np(A)
    # entries of the h row scale with 1/n; compare relative to each row's magnitude
    scale = np.maximum(np.max(np.abs(A_ref), axis=3, keepdims=True), 1e-3)
    assert float(np.max(np.abs(A_gpu - A_ref) / scale)) < 5e-5
    # structural zeros are exact
    for row, col in ((0, 1), (1, 0), (2, 0), (2, 1)):
        assert np.all(A_gpu[:, :, row, col] == 0)
    assert abs(err.item() - ref.max_abs(F)) <= 5e-6 * max(1.0, ref.max_abs(F))


@pytest.mark.parametrize("shape", [(3, 1000, 70), (2, 64, 16), (1, 1, 1), (1, 33, 1), (2, 4097, 64)])
@pytest.mark.parametrize("inplace", [False, True])
def test_scan_block4(gpu_lib, shape, inplace):
    B, T, d = shape
    case(f"scan_block4 B={B} T={T} d={d} inplace={inplace}")
    A, r = random_scan_operands(11 + T, B, T, d)
    A = A.astype(np.float32)
    r = r.astype(np.float32)
    At = torch.from_numpy(A).to(DEV)
    rt = torch.from_numpy(r).to(DEV)
    out = gpu_lib.scan_block4(At, rt, out=rt if inplace else None)
    torch.cuda.synchronize()
    x_ref = ref.forward_substitution(A.astype(np.float64), r.astype(np.float64))
    x = to_np(out)
    assert np.all(np.isfinite(x))
    assert float(np.max(np.abs(x - x_ref))) < 2e-5 * max(1.0, float(np.max(np.abs(x_ref))))


@pytest.mark.parametrize("shape", [(4, 8192, 96), (64, 256, 512)])
def test_scan_block4_is_deterministic(gpu_lib, shape):
    # few lane groups (anchored look-back) and many (plain chain): bitwise equal reruns
    B, T, d = shape
    case(f"scan_block4 determinism B={B} T={T} d={d}")
    A, r = random_scan_operands(3, B, T, d)
    At = torch.from_numpy(A.astype(np.float32)).to(DEV)
    rt = torch.from_numpy(r.astype(np.float32)).to(DEV)
    first = gpu_lib.scan_block4(At, rt)
    for _ in range(5):
        again = gpu_lib.scan_block4(At, rt)
        assert torch.equal(first, again)
    x_ref = ref.forward_substitution(A[:1, :, :, :, :8].astype(np.float32).astype(np.float64),
                                     r[:1, :, :, :8].astype(np.float32).astype(np.float64))
    assert float(np.max(np.abs(to_np(first[:1, :, :, :8]) - x_ref))) < 2e-5 * max(1.0, float(np.max(np.abs(x_ref))))


@pytest.mark.parametrize("schedule", ["fused_scan", "fused_chain", "layered"])
def test_warm_start_and_newton_are_deterministic(gpu_lib, schedule):
    w = by_name("sigmoid_bf16p_b16_t4096_d1024")
    case(f"warm start / newton determinism B=2 T=4096 d=1024 {schedule}")
    inp = draw_preactivation_inputs(w, B=2, T=4096)
    P = inp["P"].to(DEV)
    R = inp["R"].to(DEV)
    w0 = gpu_lib.warm_start(P, None, w.forget, schedule=schedule)
    S0, h0, st0 = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, schedule=schedule)
    for _ in range(3):
        assert torch.equal(w0, gpu_lib.warm_start(P, None, w.forget, schedule=schedule))
        S1, h1, st1 = gpu_lib.newton_forward(P, R, None, w.forget, w.max_iters, w.tol, schedule=schedule)
        assert torch.equal(S0, S1) and st0.max_abs_F == st1.max_abs_F


@pytest.mark.parametrize("form", ["fused_scan", "fused_chain"])
@pytest.mark.parametrize("name,B,T", [("tiny_b2_t64_d16", None, None), ("mid_b8_t1024_d256", 2, 1024),
                                      ("sigmoid_bf16p_b16_t4096_d1024", 1, 700)])
def test_warm_start(gpu_lib, name, B, T, form):
    w = by_name(name)
    case(f"warm_start {name} B={B} T={T} {form}")
    inp = draw_preactivation_inputs(w, B, T)
    P = inp["P"]
    d = P.shape[-1]
    rng = np.random.Generator(np.random.PCG64(5))
    s0 = np.zeros((P.shape[0], 4, d), dtype=np.float32)
    s0[:, 0] = rng.uniform(-0.5, 0.5, (P.shape[0], d))
    s0[:, 1] = rng.uniform(0.5, 2.0, (P.shape[0], d))
    s0[:, 2] = rng.uniform(-2, 2, (P.shape[0], d))
    out = gpu_lib.warm_start(P.to(DEV), torch.from_numpy(s0).to(DEV), w.forget, schedule=form)
    torch.cuda.synchronize()
    S_ref = ref.warm_start(to_np(P), s0.astype(np.float64), w.forget)
    S = to_np(out)
    assert h_rel_err(S[..., 3, :], S_ref[..., 3, :], h_floor(w.forget, 1e-4)) < 1e-4
    n_ref = S_ref[..., 1, :]
    assert _rel(S[..., 1, :], n_ref, 1e-3) < 1e-4
    # |c| <= n: c is measured against n's scale where it passes through zero
    c_err = np.abs(S[..., 0, :] - S_ref[..., 0, :]) / np.maximum(np.abs(S_ref[..., 0, :]), 1e-2 * n_ref)
    assert float(np.max(c_err)) < 1e-4
    # m is a running sum that grows by about f~ per step: float32 rounding of the sum
    m_ref = S_ref[..., 2, :]
    assert float(np.max(np.abs(S[..., 2, :] - m_ref) / (1 + np.abs(m_ref)))) < 2e-5


@pytest.mark.parametrize("B,T,d_in,d_h", [(2, 64, 64, 16), (3, 50, 1024, 40), (1, 128, 256, 256)])
def test_input_projection(gpu_lib, B, T, d_in, d_h):
    case(f"input_projection B={B} T={T} d_in={d_in} d_h={d_h}")
    rng = np.random.Generator(np.random.PCG64(17))
    x = to_bf16(rng.standard_normal((B, T, d_in)))
    W = to_bf16(rng.standard_normal((4, d_h, d_in)) / np.sqrt(d_in))
    bias = torch.from_numpy(rng.standard_normal((4, d_h)).astype(np.float32))
    P = gpu_lib.input_projection(x.to(DEV), W.to(DEV), bias.to(DEV))
    torch.cuda.synchronize()
    P_ref = ref.input_projection(to_np(x), to_np(W), to_np(bias))
    # float32 accumulation of exact bf16 products: error ~ sqrt(K) * eps32 * |terms|
    assert float(np.max(np.abs(to_np(P) - P_ref))) < 2e-5 * np.sqrt(d_in)
