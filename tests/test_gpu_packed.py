"""GPU parity of packed sequences (cu_seqlens): ragged sequences laid end to end along time in
one row, each from its own initial state ("sLSTM in this library", "Packed sequences"), against
the float64 oracle's packed forms. Covered: the sequential forward, the warm start, the Newton
solve (scan and layered forms, fixed count and early stop) with each sequence's final state,
and the backward with a gradient at each sequence's final state. Lengths mix empty and length-1
sequences, sequences shorter than one tile and ones that span several tiles with ragged tails;
one case starts a sequence at every step, one has a single sequence (the unpacked problem)."""
import numpy as np
import pytest
import torch

from oracle import lanes, slstm_ref as ref
from parity import GRAD_TOL, H_TOL_BF16, H_TOL_F32, case, grad_rel_err, h_floor, h_rel_err, to_np
from workloads import by_name, draw_preactivation_inputs, packed_offsets, random_cotangents

pytestmark = pytest.mark.gpu

DEV = "cuda"
MARGIN = 1e-5
MIXED = [37, 0, 1, 130, 5, 0, 64, 1, 1, 200, 3]     # T = 442: empties, ones, several tiles
LAYOUTS = {
    "mixed": MIXED,
    "all_ones": [1] * 40,                             # every step starts a sequence
    "empty_ends": [0, 0, 150, 0, 1, 0],               # leading and trailing empties
    "single": [333],                                  # the unpacked problem
    "many": list(np.diff(packed_offsets(11, 3000, 40))),  # ~300 short sequences
    # lengths at and around the 32-step tiles of the scan form's aligned tiles (which serve packs
    # of at most about T / 32 sequences: this one, "mixed" and "single")
    "tile_edges": [32, 0, 33, 31, 1, 64, 0, 96, 2, 65, 127, 1, 300],
    # lengths at and around multiples of 96 steps, and so of the 32-step aligned tiles of both the
    # iteration and the backward (the backward's serve packs of at most about T / 96 sequences:
    # this one, "single" and the full-size pack)
    "wide_tile_edges": [96, 0, 97, 95, 1, 192, 0, 288, 2, 193, 383, 1, 4000],
}


def _problem(seed, lengths, d, forget):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, S = int(cu[-1]), len(lengths)
    rng = np.random.Generator(np.random.PCG64(seed))
    P = rng.standard_normal((1, T, 4, d))
    P[:, :, 2] += 3.0
    R = rng.uniform(-0.5, 0.5, (4, d))
    s0 = np.stack([rng.uniform(-0.5, 0.5, (S, d)), rng.uniform(0.5, 2.0, (S, d)),
                   rng.uniform(-2.0, 2.0, (S, d)), rng.uniform(-0.9, 0.9, (S, d))], axis=1)
    f32 = lambda a: torch.from_numpy(a.astype(np.float32))  # noqa: E731
    return f32(P), f32(R), f32(s0), cu


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _state_err(gpu, ref_states):
    """Largest error per slot (c, n, m, h) relative to the slot's largest value (tensors with
    the slot on axis -2)."""
    g, r = to_np(gpu), np.asarray(ref_states)
    return max(float(np.max(np.abs(g[..., k, :] - r[..., k, :])) / max(float(np.max(np.abs(r[..., k, :]))), 1e-30))
               for k in range(4))


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_packed_sequential(gpu_lib, layout, forget):
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(800, lengths, 70, forget)
    case(f"packed sequential {layout} {forget} T={P.shape[1]} S={len(lengths)}")
    fin = torch.empty_like(s0).to(DEV)
    S, h = gpu_lib.sequential_forward(*_dev(P, R, s0), forget, final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    seq = ref.sequential(to_np(P), to_np(R), to_np(s0), forget, cu_seqlens=cu)
    assert h_rel_err(h, seq[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32
    assert _state_err(S, seq) < 1e-5
    assert _state_err(fin, ref.final_states(seq, to_np(s0), cu)) < 1e-5
    for s in range(len(lengths)):  # an empty sequence hands its state0 on unchanged
        if cu[s] == cu[s + 1]:
            assert torch.equal(fin[s].cpu(), s0[s])


def test_packed_sequential_bf16(gpu_lib):
    P, R, s0, cu = _problem(801, MIXED, 130, "exp")
    Pb = P.to(torch.bfloat16)
    case("packed sequential bf16 P")
    _, h = gpu_lib.sequential_forward(*_dev(Pb, R, s0), "exp", cu_seqlens=cu)
    torch.cuda.synchronize()
    seq = ref.sequential(to_np(Pb), to_np(R), to_np(s0), "exp", cu_seqlens=cu)
    assert h_rel_err(h, seq[..., 3, :]) < H_TOL_F32


@pytest.mark.parametrize("schedule", ["fused", "fused_scan", "layered"])
@pytest.mark.parametrize("layout", ["mixed", "all_ones", "empty_ends", "many"])
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_packed_warm_start(gpu_lib, schedule, layout, forget):
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(810, lengths, 70, forget)
    case(f"packed warm start {layout} {forget} {schedule}")
    W = gpu_lib.warm_start(*_dev(P, s0), forget, schedule=schedule, cu_seqlens=cu)
    torch.cuda.synchronize()
    warm = ref.warm_start(to_np(P), to_np(s0), forget, cu_seqlens=cu)
    assert h_rel_err(W[..., 3, :], warm[..., 3, :], h_floor(forget, H_TOL_F32)) < H_TOL_F32
    assert _state_err(W, warm) < 1e-5


@pytest.mark.parametrize("schedule", ["fused", "fused_scan", "layered"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("K", [3, 6])
def test_packed_newton(gpu_lib, schedule, layout, forget, K):
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(820 + K, lengths, 70, forget)
    case(f"packed newton {layout} {forget} {schedule} K={K}")
    fin = torch.empty_like(s0).to(DEV)
    S, h, st = gpu_lib.newton_forward(*_dev(P, R, s0), forget, K, 0.0, final_state=fin,
                                      raise_on_divergence=False, schedule=schedule, cu_seqlens=cu)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton(to_np(P), to_np(R), to_np(s0), forget, K, cu_seqlens=cu)
    err = h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32))
    print(f"packed newton {layout} {forget} {schedule} K={K}: h rel err {err:.2e}, "
          f"max|F| {st.max_abs_F[-1]:.2e} (oracle {st_ref.max_abs_F[-1]:.2e})")
    assert err < H_TOL_F32
    assert st.iters == st_ref.iters and st.diverged == st_ref.diverged
    assert _state_err(fin, ref.final_states(S_ref, to_np(s0), cu)) < 1e-4


@pytest.mark.parametrize("schedule", ["fused_scan", "layered"])
def test_packed_newton_early_stop(gpu_lib, schedule):
    """One residual maximum covers the whole pack, so the stop is global."""
    P, R, s0, cu = _problem(830, MIXED, 70, "sigmoid")
    Pb = P.to(torch.bfloat16)
    case(f"packed newton early stop {schedule}")
    _, h, st = gpu_lib.newton_forward(*_dev(Pb, R, s0), "sigmoid", 8, 1e-5, schedule=schedule, cu_seqlens=cu)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton(to_np(Pb), to_np(R), to_np(s0), "sigmoid", 8, tol=1e-5, cu_seqlens=cu)
    assert st_ref.converged and st.converged
    assert st.iters == st_ref.iters
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16


@pytest.mark.parametrize("layout", ["tile_edges", "wide_tile_edges"])
def test_packed_aligned_tiles_reproducible(gpu_lib, layout):
    """The scan form on tiles aligned to the sequences: two solves give the same bits (the
    tiles of many sequences run at once, in whatever order the hardware schedules them)."""
    P, R, s0, cu = _problem(815, LAYOUTS[layout], 200, "exp")
    case(f"packed aligned tiles reproducible {layout}")
    Pd, Rd, s0d = _dev(P, R, s0)
    a = gpu_lib.newton_forward(Pd, Rd, s0d, "exp", 3, 0.0, schedule="fused_scan", cu_seqlens=cu)[0].clone()
    b = gpu_lib.newton_forward(Pd, Rd, s0d, "exp", 3, 0.0, schedule="fused_scan", cu_seqlens=cu)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_packed_single_sequence_matches_unpacked(gpu_lib):
    P, R, s0, cu = _problem(840, [333], 70, "exp")
    case("packed single sequence vs unpacked call")
    _, hp, _ = gpu_lib.newton_forward(*_dev(P, R, s0), "exp", 3, 0.0, schedule="fused_scan", cu_seqlens=cu)
    _, hu, _ = gpu_lib.newton_forward(*_dev(P, R, s0), "exp", 3, 0.0, schedule="fused_scan")
    torch.cuda.synchronize()
    assert h_rel_err(hp, to_np(hu)) < 1e-6


def test_packed_chain_form_is_rejected(gpu_lib):
    P, R, s0, cu = _problem(841, MIXED, 16, "exp")
    case("packed chain form rejected on the host")
    with pytest.raises(gpu_lib.SlstmError):
        gpu_lib.newton_forward(*_dev(P, R, s0), "exp", 3, 0.0, schedule="fused_chain", cu_seqlens=cu)
    with pytest.raises(gpu_lib.SlstmError):
        gpu_lib.backward(*_dev(P, R), torch.zeros((1, P.shape[1], 4, 16), device=DEV), s0.to(DEV),
                         schedule="fused_chain", cu_seqlens=cu)


def _backward_case(gpu_lib, P, R, s0, cu, forget, schedule, seed, dP_dtype=torch.float32):
    T, d = P.shape[1], P.shape[3]
    n_seq = len(cu) - 1
    S = torch.from_numpy(ref.sequential(to_np(P), to_np(R), to_np(s0), forget, cu_seqlens=cu).astype(np.float32))
    gs, gh, _ = (torch.from_numpy(a) for a in random_cotangents(seed, 1, T, d))
    gf = torch.from_numpy(random_cotangents(seed + 1, n_seq, 1, d)[2])
    dP, dR, ds0, db = gpu_lib.backward(*_dev(P, R, S, s0, gs, gh, gf), forget, schedule=schedule,
                                       want_dbias=True, dP_dtype=dP_dtype, cu_seqlens=cu)
    torch.cuda.synchronize()
    g = to_np(gs)
    g[:, :, 3] += to_np(gh)
    dP_ref, dR_ref, ds0_ref = ref.backward(to_np(P), to_np(R), to_np(s0), to_np(S), g, forget,
                                           cu_seqlens=cu, g_final=to_np(gf))
    margin, scale = ref.branch_margin(to_np(P), to_np(R), to_np(s0), to_np(S), forget, cu_seqlens=cu)
    keep_j = np.all(margin > MARGIN * (1.0 + scale), axis=1)[0]  # (d,): features clear of ties
    assert keep_j.mean() > 0.8
    db_ref = dP_ref.sum(axis=(0, 1))
    errs = [grad_rel_err(dP, dP_ref, keep_j), grad_rel_err(dR, dR_ref, keep_j), grad_rel_err(db, db_ref, keep_j),
            grad_rel_err(ds0, ds0_ref, keep_j)]
    return errs, ds0, ds0_ref, gf


@pytest.mark.parametrize("schedule", ["fused", "fused_scan"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
def test_packed_backward(gpu_lib, schedule, layout, forget):
    lengths = LAYOUTS[layout]
    P, R, s0, cu = _problem(850, lengths, 70, forget)
    case(f"packed backward {layout} {forget} {schedule}")
    errs, ds0, _, gf = _backward_case(gpu_lib, P, R, s0, cu, forget, schedule, 851)
    print(f"packed backward {layout} {forget} {schedule}: rel err dP dR dbias dstate0 {['%.2e' % e for e in errs]}")
    assert max(errs) < GRAD_TOL
    for s in range(len(lengths)):  # an empty sequence passes g_final to its dstate0 unchanged
        if cu[s] == cu[s + 1]:
            assert torch.equal(ds0[s].cpu(), gf[s])


def test_packed_backward_aligned_reproducible(gpu_lib):
    """The backward on sequence-aligned tiles (taken for this pack) forms every value in one
    fixed order: two calls agree bitwise."""
    lengths = LAYOUTS["wide_tile_edges"]
    P, R, s0, cu = _problem(870, lengths, 130, "exp")
    S = torch.from_numpy(ref.sequential(to_np(P), to_np(R), to_np(s0), "exp", cu_seqlens=cu).astype(np.float32))
    gen = torch.Generator().manual_seed(871)
    gh = torch.randn((1, P.shape[1], 130), generator=gen)
    gf = torch.randn((len(lengths), 4, 130), generator=gen)
    case("packed backward on aligned tiles, twice")
    args = _dev(P, R, S, s0) + [None] + _dev(gh, gf)
    a = [t.clone() for t in gpu_lib.backward(*args, "exp", want_dbias=True, cu_seqlens=cu)]
    b = gpu_lib.backward(*args, "exp", want_dbias=True, cu_seqlens=cu)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("layout", ["mixed", "wide_tile_edges"])  # along the row; on aligned tiles
def test_packed_backward_bf16_dp(gpu_lib, layout):
    P, R, s0, cu = _problem(860, LAYOUTS[layout], 70, "exp")
    case(f"packed backward, bf16 dP, {layout}")
    errs, _, _, _ = _backward_case(gpu_lib, P, R, s0, cu, "exp", "fused", 861, dP_dtype=torch.bfloat16)
    assert errs[0] < 1e-2            # dP rounded to bfloat16
    assert max(errs[1:]) < GRAD_TOL  # dR, dbias and dstate0 from the float32 values


def _full_size_packed():
    """The full-layer workload's 128 x 2048 tokens packed as ragged sequences (log-uniform
    lengths up to 8192 steps, empties and ones mixed in) in one row at d_h = 1024, each sequence
    with its own state0."""
    w = by_name("layer_b128_t2048_d1024")
    inp = draw_preactivation_inputs(w, B=w.B, T=w.T, device=DEV)
    P = inp["P"].reshape(1, w.B * w.T, 4, w.d_h).to(DEV)
    R = inp["R"].to(DEV)
    cu = packed_offsets(w.seed, w.B * w.T, 8192)
    n_seq, d = len(cu) - 1, w.d_h
    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    s0 = np.stack([rng.uniform(-0.5, 0.5, (n_seq, d)), rng.uniform(0.5, 2.0, (n_seq, d)),
                   rng.uniform(-2.0, 2.0, (n_seq, d)), rng.uniform(-0.9, 0.9, (n_seq, d))], axis=1)
    return w, P, R, torch.from_numpy(s0.astype(np.float32)).to(DEV), cu


# sampled features: both ends, a 64-feature tile boundary, one inside; channelwise mixing keeps
# every feature an independent problem (dR and dbias of a feature included)
FULL_JS = np.array([0, 1, 63, 64, 517, 1023])


def test_packed_workload_full_size_forward(gpu_lib):
    w, P, R, s0, cu = _full_size_packed()
    case(f"full-size packed forward: T={P.shape[1]} d={w.d_h} S={len(cu) - 1}")
    fin = torch.empty_like(s0)
    S, h, st = gpu_lib.newton_forward(P, R, s0, w.forget, w.max_iters, 0.0, final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert st.iters == w.max_iters and not st.diverged
    jt = torch.as_tensor(FULL_JS, device=DEV)
    Pj, Rj, s0j = to_np(P[..., jt]), to_np(R[:, jt]), to_np(s0[..., jt])
    S_ref, _ = lanes.packed_newton(Pj, Rj, s0j, w.forget, w.max_iters, cu)
    err = h_rel_err(h[..., jt], S_ref[..., 3, :])
    print(f"full-size packed newton: h rel err {err:.2e}")
    assert err < H_TOL_F32
    assert _state_err(fin[..., jt], ref.final_states(S_ref, s0j, cu)) < 1e-4
    del S, h
    _, hs = gpu_lib.sequential_forward(P, R, s0, w.forget, cu_seqlens=cu)
    torch.cuda.synchronize()
    seq = lanes.packed_sequential(Pj, Rj, s0j, w.forget, cu)
    assert h_rel_err(hs[..., jt], seq[..., 3, :]) < H_TOL_F32


def test_packed_workload_full_size_backward(gpu_lib):
    w, P, R, s0, cu = _full_size_packed()
    T, d, n_seq = P.shape[1], w.d_h, len(cu) - 1
    case(f"full-size packed backward: T={T} d={d} S={n_seq}")
    S, _, _ = gpu_lib.newton_forward(P, R, s0, w.forget, w.max_iters, 0.0, want_hidden=False, cu_seqlens=cu)
    jt = torch.as_tensor(FULL_JS, device=DEV)
    Pj, Rj, s0j = to_np(P[..., jt]), to_np(R[:, jt]), to_np(s0[..., jt])
    # the oracle's float32 trajectory over the sampled features, so that both sides
    # differentiate at the same states there
    seq = lanes.packed_sequential(Pj, Rj, s0j, w.forget, cu).astype(np.float32)
    S[..., jt] = torch.from_numpy(seq).to(DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(w.seed + 8)
    gh = torch.randn((1, T, d), generator=gen, device=DEV)
    gf = torch.randn((n_seq, 4, d), generator=gen, device=DEV)
    dP, dR, ds0 = gpu_lib.backward(P, R, S, s0, None, gh, gf, w.forget, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.isfinite(dP).all() and torch.isfinite(dR).all() and torch.isfinite(ds0).all()
    g = np.zeros(seq.shape)
    g[:, :, 3] = to_np(gh[..., jt])
    seq64 = seq.astype(np.float64)
    dP_ref, dR_ref, ds0_ref = lanes.packed_backward(Pj, Rj, s0j, seq64, g, w.forget, cu, g_final=to_np(gf[..., jt]))
    margin, scale = ref.branch_margin(Pj, Rj, s0j, seq64, w.forget, cu_seqlens=cu)
    keep = np.all(margin > MARGIN * (1.0 + scale), axis=1)[0]
    assert keep.sum() >= 4
    errs = [grad_rel_err(dP[..., jt], dP_ref, keep), grad_rel_err(dR[:, jt], dR_ref, keep),
            grad_rel_err(ds0[..., jt], ds0_ref, keep)]
    print(f"full-size packed backward: rel err dP dR dstate0 {['%.2e' % e for e in errs]}, kept {keep.sum()}")
    assert max(errs) < GRAD_TOL


# lengths around the one-kernel solve's 24-step aligned tiles, empties and single steps, enough
# sequences for its chains (two lane groups of 256 features times 40 sequences)
PIPE_LENGTHS = [24, 0, 25, 23, 1, 48, 0, 72, 2, 49, 95, 1, 300, 7, 120, 0, 24, 200, 33, 3,
                96, 17, 0, 250, 64, 1, 47, 180, 5, 90, 26, 140, 0, 71, 9, 160, 24, 13, 110, 55]


@pytest.mark.parametrize("forget", ["exp", "sigmoid"])
@pytest.mark.parametrize("K", [3, 6])
def test_packed_one_kernel_solve(gpu_lib, forget, K):
    """FUSED on a pack with enough sequences runs the one-kernel solve on tiles aligned to the
    sequence starts: h, each sequence's final state (state0 for the empty ones), the iteration
    count and the flags match the oracle; without the state tensor h and the final states are
    bitwise the same."""
    P, R, s0, cu = _problem(870 + K, PIPE_LENGTHS, 300, forget)
    case(f"packed one-kernel solve {forget} K={K} T={P.shape[1]} S={len(PIPE_LENGTHS)}")
    Pd, Rd, s0d = _dev(P, R, s0)
    fin = torch.empty_like(s0).to(DEV)
    gpu_lib.profile_reset()
    gpu_lib.profile_enable(True)
    S, h, st = gpu_lib.newton_forward(Pd, Rd, s0d, forget, K, 0.0, final_state=fin, raise_on_divergence=False,
                                      schedule="fused", cu_seqlens=cu)
    n_solve = len(gpu_lib.profile_durations("newton_solve"))
    n_iter = len(gpu_lib.profile_durations("newton_iteration"))
    gpu_lib.profile_enable(False)
    fin2 = torch.full_like(fin, float("nan"))
    S2, h2, st2 = gpu_lib.newton_forward(Pd, Rd, s0d, forget, K, 0.0, final_state=fin2, raise_on_divergence=False,
                                         schedule="fused", cu_seqlens=cu, output_states=False)
    torch.cuda.synchronize()
    assert n_solve == 1 and n_iter == 0
    assert S2 is None and torch.equal(h, h2) and torch.equal(fin, fin2)
    assert np.array_equal(np.array(st.max_abs_F), np.array(st2.max_abs_F))
    S_ref, st_ref = ref.newton(to_np(P), to_np(R), to_np(s0), forget, K, cu_seqlens=cu)
    err = h_rel_err(h, S_ref[..., 3, :], h_floor(forget, H_TOL_F32))
    print(f"packed one-kernel {forget} K={K}: h rel err {err:.2e}")
    assert err < H_TOL_F32
    assert _state_err(S, S_ref) < 1e-4
    assert st.iters == st_ref.iters and st.diverged == st_ref.diverged
    assert _state_err(fin, ref.final_states(S_ref, to_np(s0), cu)) < 1e-4
    for s in range(len(PIPE_LENGTHS)):
        if cu[s] == cu[s + 1]:
            assert torch.equal(fin[s].cpu(), s0[s])


def test_packed_one_kernel_early_stop(gpu_lib):
    """The early stop on a pack as two one-kernel passes: the stop is global, so the count and
    flags equal the oracle's, and h is within the bf16 bar."""
    P, R, s0, cu = _problem(880, PIPE_LENGTHS, 300, "sigmoid")
    Pb = P.to(torch.bfloat16)
    case("packed one-kernel early stop")
    gpu_lib.profile_reset()
    gpu_lib.profile_enable(True)
    _, h, st = gpu_lib.newton_forward(*_dev(Pb, R, s0), "sigmoid", 8, 1e-5, schedule="fused", cu_seqlens=cu)
    n_solve = len(gpu_lib.profile_durations("newton_solve"))
    gpu_lib.profile_enable(False)
    torch.cuda.synchronize()
    S_ref, st_ref = ref.newton(to_np(Pb), to_np(R), to_np(s0), "sigmoid", 8, tol=1e-5, cu_seqlens=cu)
    assert n_solve == 2
    assert st_ref.converged and st.converged and st.iters == st_ref.iters
    assert h_rel_err(h, S_ref[..., 3, :]) < H_TOL_BF16
