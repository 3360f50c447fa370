"""The C-ABI library on the host: it loads, exports every function include/slstm.h declares,
and its argument checks and workspace sizing behave as documented (no GPU work is done)."""
import ctypes
import os
import re

import pytest

import torch  # noqa: F401  (binds the library to the HIP runtime torch loads)
from recurrent_nets_amd import slstm

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "slstm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slstm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(slstm.lib_path()):
        pytest.fail("library not built: run `python -m recurrent_nets_amd.build`")
    return slstm.load()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert len(declared) >= 15
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared) == set(slstm.EXPORTED)


def test_status_strings(lib):
    for s in (0, 1, 2, -1, -2, -3):
        assert lib.slstm_status_string(s).decode()
    assert lib.slstm_status_string(99).decode() == "unknown status"


def test_workspace_sizes(lib):
    # Jacobians (64 B) + right-hand sides (16 B) per state element, plus look-back words
    B, T, d = 128, 2048, 1024
    n = lib.slstm_newton_workspace_bytes(B, T, d, 1)  # layered
    assert n >= 80 * B * T * d
    assert n < 90 * B * T * d
    # fused forms: a second iterate buffer (16 B) and look-back words, no Jacobians; the chain
    # form publishes 4 tagged words per lane and tile of 8 steps (4 B per state element)
    for sched in (0, 2, 3):
        nf = lib.slstm_newton_workspace_bytes(B, T, d, sched)
        assert 16 * B * T * d <= nf < 32 * B * T * d
    assert lib.slstm_newton_workspace_bytes(B, T, d, 3) < 21 * B * T * d
    assert lib.slstm_newton_workspace_bytes(B, T, d, 7) == 0
    assert lib.slstm_newton_workspace_bytes(0, 1, 1, 0) == 0
    assert lib.slstm_newton_workspace_bytes(1, -1, 1, 0) == 0
    assert lib.slstm_scan_block4_workspace_bytes(2, 64, 16) > 0
    for sched in (0, 1, 2, 3):
        assert lib.slstm_warm_start_workspace_bytes(2, 64, 16, sched) > 0
    assert lib.slstm_warm_start_workspace_bytes(2, 64, 16, 9) == 0
    # tiny shapes still get a control block and one tile of look-back words
    assert lib.slstm_newton_workspace_bytes(1, 1, 1, 0) >= 512
    # backward chains: 4 tagged words per lane and tile of 8 steps (4 B per state element) and a
    # row of 8 sums per lane and tile (4 B); scan: 24 words per lane and tile of 32 steps (6 B)
    # and a row of 8 sums per lane and tile (1 B)
    nb = lib.slstm_backward_workspace_bytes(B, T, d, 3)
    assert 8 * B * T * d <= nb < 9 * B * T * d
    ns = lib.slstm_backward_workspace_bytes(B, T, d, 2)
    assert 7 * B * T * d <= ns < 8 * B * T * d
    assert lib.slstm_backward_workspace_bytes(B, T, d, 0) == ns
    assert lib.slstm_backward_workspace_bytes(B, T, d, 1) == 0
    assert lib.slstm_backward_workspace_bytes(0, T, d, 0) == 0


def _fwd(lib, **kw):
    args = dict(P=ctypes.c_void_p(256), dt=0, R=ctypes.c_void_p(256), s0=None,
                S=ctypes.c_void_p(256), h=None, fin=None, B=2, T=64, d=16, fm=0, K=3, tol=0.0, init=0,
                sched=0, ws=ctypes.c_void_p(4096), wsb=1 << 30, stream=None, stats=None)
    args.update(kw)
    return lib.slstm_newton_forward(*args.values())


def test_argument_checks_return_einval(lib):
    # every call below is rejected on the host before any device work
    assert _fwd(lib, B=0) == slstm.EINVAL
    assert _fwd(lib, K=0) == slstm.EINVAL
    assert _fwd(lib, K=65) == slstm.EINVAL
    assert _fwd(lib, tol=-1.0) == slstm.EINVAL
    assert _fwd(lib, tol=float("nan")) == slstm.EINVAL
    assert _fwd(lib, fm=7) == slstm.EINVAL
    assert _fwd(lib, fm=0x200) == slstm.EINVAL                    # unknown flag bit
    assert _fwd(lib, fm=0x102) == slstm.EINVAL                    # floored flag, unknown gate
    # the floored read-out flag passes the argument checks (then the workspace check fails)
    assert _fwd(lib, fm=0x101, wsb=100) == slstm.EWORKSPACE
    assert _fwd(lib, fm=0x100, wsb=100) == slstm.EWORKSPACE
    assert _fwd(lib, dt=5) == slstm.EINVAL
    assert _fwd(lib, init=3) == slstm.EINVAL
    assert _fwd(lib, sched=9) == slstm.EINVAL
    assert _fwd(lib, P=None) == slstm.EINVAL
    assert _fwd(lib, S=ctypes.c_void_p(260)) == slstm.EINVAL      # states not 16-byte aligned
    assert _fwd(lib, fin=ctypes.c_void_p(264)) == slstm.EINVAL    # final_state not 16-byte aligned
    assert _fwd(lib, ws=ctypes.c_void_p(4096 + 16)) == slstm.EINVAL  # workspace not 256-aligned
    assert "256-byte" in lib.slstm_last_error().decode()
    assert _fwd(lib, wsb=100) == slstm.EWORKSPACE
    assert "needed" in lib.slstm_last_error().decode()
    # no state tensor: only where the solve is the one-kernel form, which keeps its iterate on
    # chip (fixed count, tol = 0, max_iters <= 4, unpacked)
    assert _fwd(lib, S=None, sched=1) == slstm.EINVAL            # layered
    assert "one-kernel" in lib.slstm_last_error().decode()
    assert _fwd(lib, S=None, sched=2) == slstm.EINVAL            # scan form
    assert _fwd(lib, S=None, sched=0) == slstm.EINVAL            # fused on 2 lane groups: scan form
    assert _fwd(lib, S=None, sched=3, tol=1e-5) == slstm.EINVAL  # early stop: per-iteration kernels
    assert _fwd(lib, S=None, sched=3, K=5) == slstm.EINVAL
    assert _fwd(lib, S=None, sched=3, wsb=100) == slstm.EWORKSPACE  # accepted, then sized
    s = lib.slstm_input_projection(ctypes.c_void_p(256), ctypes.c_void_p(256), None,
                                   ctypes.c_void_p(256), 2, 3, 12, 4, 1, None)
    assert s == slstm.EINVAL and "multiple of 8" in lib.slstm_last_error().decode()
    s = lib.slstm_input_projection(ctypes.c_void_p(256), ctypes.c_void_p(256), None,
                                   ctypes.c_void_p(256), 2, 3, 16, 4, 0, None)
    assert s == slstm.EINVAL  # float32 x / W_x are not taken
    s = lib.slstm_scan_block4(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                              2, 64, 16, ctypes.c_void_p(4096), 10, None)
    assert s == slstm.EWORKSPACE
    s = lib.slstm_sequential_forward(None, 0, ctypes.c_void_p(256), None, ctypes.c_void_p(256),
                                     None, None, 2, 64, 16, 0, None)
    assert s == slstm.EINVAL
    # the packed sequential forward gathers its final states from the state tensor
    cu = ctypes.c_void_p(1024)
    s = lib.slstm_sequential_forward_varlen(ctypes.c_void_p(256), 0, ctypes.c_void_p(256), None, cu, 2,
                                            None, None, None, 64, 16, 0, None)
    assert s == slstm.EINVAL and "unpacked" in lib.slstm_last_error().decode()


def _bwd(lib, **kw):
    args = dict(P=ctypes.c_void_p(256), dt=0, R=ctypes.c_void_p(256), s0=None,
                S=ctypes.c_void_p(256), gs=None, gh=None, gf=None, dP=ctypes.c_void_p(256),
                dpt=0, dR=ctypes.c_void_p(256), db=None, ds0=None, B=2, T=64, d=16, fm=0, sched=0,
                ws=ctypes.c_void_p(4096), wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.slstm_backward(*args.values())


def test_backward_argument_checks(lib):
    assert _bwd(lib, T=0) == slstm.EINVAL
    assert _bwd(lib, dP=None) == slstm.EINVAL
    assert _bwd(lib, dR=None) == slstm.EINVAL
    assert _bwd(lib, S=None) == slstm.EINVAL
    assert _bwd(lib, dP=ctypes.c_void_p(264)) == slstm.EINVAL   # dP not 16-byte aligned
    assert _bwd(lib, gh=ctypes.c_void_p(258)) == slstm.EINVAL   # g_h misaligned
    assert _bwd(lib, fm=2) == slstm.EINVAL
    assert _bwd(lib, dpt=3) == slstm.EINVAL
    assert _bwd(lib, db=ctypes.c_void_p(258)) == slstm.EINVAL
    assert _bwd(lib, sched=1) == slstm.EINVAL
    assert "fused forms only" in lib.slstm_last_error().decode()
    assert _bwd(lib, sched=9) == slstm.EINVAL
    assert _bwd(lib, ws=None) == slstm.EINVAL
    assert _bwd(lib, wsb=100) == slstm.EWORKSPACE


def test_binding_refuses_host_tensors():
    P = torch.zeros((1, 2, 4, 3))
    R = torch.zeros((4, 3))
    with pytest.raises(ValueError):
        slstm.newton_forward(P, R)


def _fwd_varlen(lib, **kw):
    args = dict(P=ctypes.c_void_p(256), dt=0, R=ctypes.c_void_p(256), s0=None,
                cu=ctypes.c_void_p(512), n=3, S=ctypes.c_void_p(256), h=None, fin=None, T=64, d=16,
                fm=0, K=3, tol=0.0, init=0, sched=0, ws=ctypes.c_void_p(4096), wsb=1 << 30,
                stream=None, stats=None)
    args.update(kw)
    return lib.slstm_newton_forward_varlen(*args.values())


def _bwd_varlen(lib, **kw):
    args = dict(P=ctypes.c_void_p(256), dt=0, R=ctypes.c_void_p(256), s0=None,
                cu=ctypes.c_void_p(512), n=3, S=ctypes.c_void_p(256), gs=None, gh=None, gf=None,
                dP=ctypes.c_void_p(256), dpt=0, dR=ctypes.c_void_p(256), db=None, ds0=None, T=64,
                d=16, fm=0, sched=0, ws=ctypes.c_void_p(4096), wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.slstm_backward_varlen(*args.values())


def test_varlen_argument_checks(lib):
    # packed sequences: the offsets pointer and count are checked, the chain forms refused;
    # everything here returns on the host before any device work
    assert _fwd_varlen(lib, cu=None) == slstm.EINVAL
    assert "cu_seqlens" in lib.slstm_last_error().decode()
    assert _fwd_varlen(lib, cu=ctypes.c_void_p(514)) == slstm.EINVAL   # not 4-byte aligned
    assert _fwd_varlen(lib, n=0) == slstm.EINVAL
    assert _fwd_varlen(lib, n=-2) == slstm.EINVAL
    assert _fwd_varlen(lib, sched=3) == slstm.EINVAL
    assert "FUSED_CHAIN" in lib.slstm_last_error().decode()
    assert _fwd_varlen(lib, T=0) == slstm.EINVAL
    for sched in (0, 1, 2):
        assert _fwd_varlen(lib, sched=sched, wsb=100) == slstm.EWORKSPACE
    assert _bwd_varlen(lib, cu=None) == slstm.EINVAL
    assert _bwd_varlen(lib, n=0) == slstm.EINVAL
    assert _bwd_varlen(lib, sched=3) == slstm.EINVAL
    assert _bwd_varlen(lib, sched=1) == slstm.EINVAL
    assert _bwd_varlen(lib, wsb=100) == slstm.EWORKSPACE
    s = lib.slstm_warm_start_varlen(ctypes.c_void_p(256), 0, None, ctypes.c_void_p(512), 3,
                                    ctypes.c_void_p(256), 64, 16, 0, 3, ctypes.c_void_p(4096), 1 << 30, None)
    assert s == slstm.EINVAL
    s = lib.slstm_warm_start_varlen(ctypes.c_void_p(256), 0, None, ctypes.c_void_p(512), 3,
                                    ctypes.c_void_p(256), 64, 16, 0, 0, ctypes.c_void_p(4096), 10, None)
    assert s == slstm.EWORKSPACE
    s = lib.slstm_sequential_forward_varlen(ctypes.c_void_p(256), 0, ctypes.c_void_p(256), None, None, 3,
                                            ctypes.c_void_p(256), None, None, 64, 16, 0, None)
    assert s == slstm.EINVAL


def test_binding_checks_offsets():
    P = torch.zeros((1, 10, 4, 3))
    for bad in ([0, 4, 3, 10], [1, 10], [0, 9], [0]):
        with pytest.raises(ValueError):
            slstm._seqs(bad, P)
    with pytest.raises(ValueError):
        slstm._seqs([0, 5, 10], torch.zeros((2, 10, 4, 3)))


def test_head_argument_checks(lib):
    # head mixing: n_heads must split d_h into heads of 8, 16, 32, 64 or 128 units; R 16-byte aligned
    assert lib.slstm_head_newton_workspace_bytes(2, 64, 64, 2) > 0
    assert lib.slstm_head_newton_workspace_bytes(2, 64, 128, 1) > 0       # d_head 128
    assert lib.slstm_head_newton_workspace_bytes(2, 64, 512, 2) == 0      # d_head 256
    for nh in (0, 3, 64, 128):
        assert lib.slstm_head_newton_workspace_bytes(2, 64, 64, nh) == 0
    args = dict(P=ctypes.c_void_p(256), dt=0, R=ctypes.c_void_p(256), s0=None, S=ctypes.c_void_p(256), h=None,
                fin=None, B=2, T=64, d=64, nh=2, fm=0, K=3, tol=0.0, init=0, ws=ctypes.c_void_p(4096),
                wsb=1 << 30, stream=None, stats=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.slstm_head_newton_forward(*a.values())
    assert call(nh=3) == slstm.EINVAL
    assert "heads" in lib.slstm_last_error().decode()
    assert call(nh=16) == slstm.EINVAL            # d_head = 4
    assert call(R=ctypes.c_void_p(260)) == slstm.EINVAL
    assert call(K=0) == slstm.EINVAL
    assert call(wsb=100) == slstm.EWORKSPACE
    assert call(ws=None) == slstm.EINVAL
    s = lib.slstm_head_sequential_forward(ctypes.c_void_p(256), 0, ctypes.c_void_p(256), None, ctypes.c_void_p(256),
                                          None, None, 2, 64, 64, 5, 0, None)
    assert s == slstm.EINVAL


def test_head_backward_argument_checks(lib):
    # widths: 8 to 64 (a lane's block row and dR row must fit in registers, the head's
    # transposed blocks in LDS)
    assert lib.slstm_head_backward_workspace_bytes(2, 64, 64, 2) > 0
    assert lib.slstm_head_backward_workspace_bytes(2, 64, 128, 2) > 0       # d_head 64
    assert lib.slstm_head_backward_workspace_bytes(2, 64, 256, 2) > 0       # d_head 128
    assert lib.slstm_head_backward_workspace_bytes(2, 64, 512, 2) == 0      # d_head 256
    assert lib.slstm_head_backward_workspace_bytes(2, 64, 64, 3) == 0
    args = dict(P=ctypes.c_void_p(256), dt=0, R=ctypes.c_void_p(256), s0=None, S=ctypes.c_void_p(256), gs=None,
                gh=None, gf=None, dP=ctypes.c_void_p(256), dpt=0, dR=ctypes.c_void_p(256), db=None, d0=None, B=2,
                T=64, d=64, nh=2, fm=0, ws=ctypes.c_void_p(4096), wsb=1 << 30, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.slstm_head_backward(*a.values())
    assert call(d=512) == slstm.EINVAL
    assert "8, 16, 32, 64 or 128" in lib.slstm_last_error().decode()
    assert call(nh=3) == slstm.EINVAL
    assert call(dP=None) == slstm.EINVAL
    assert call(dR=None) == slstm.EINVAL
    assert call(dpt=7) == slstm.EINVAL
    assert call(R=ctypes.c_void_p(260)) == slstm.EINVAL
    assert call(ws=None) == slstm.EINVAL
    assert call(wsb=100) == slstm.EWORKSPACE
