"""Python binding of the sLSTM HIP library (ctypes over the C ABI in include/slstm.h).

Argument marshalling only: every step of the computation runs in the library's kernels.
PyTorch supplies device memory and the current stream. Importing torch first makes the
library bind to the HIP runtime torch has already loaded (same SONAME), so torch's streams
are valid handles for it.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

from . import build as _build

# enums of include/slstm.h
OK, DIVERGED, NONFINITE, EINVAL, EWORKSPACE, EHIP = 0, 1, 2, -1, -2, -3
F32, BF16 = 0, 1
FORGET = {"exp": 0, "sigmoid": 1}
READOUT = {"exact": 0, "floored": 0x100}  # OR-ed into the forget argument (SLSTM_READOUT_FLOORED)
INIT = {"warm": 0, "zero": 1}
SCHEDULE = {"fused": 0, "layered": 1, "fused_scan": 2, "fused_chain": 3}
MAX_ITERS = 64
KERNELS = {"warm_start": 0, "residual_jacobian": 1, "scan_block4": 2, "update": 3,
           "final_residual": 4, "input_projection": 5, "sequential": 6, "newton_iteration": 7,
           "newton_solve": 8, "backward": 9, "weight_gradient": 10, "input_gradient": 11,
           "head_iteration": 12, "head_sequential": 13, "head_solve": 14, "head_backward": 15}

EXPORTED = [
    "slstm_status_string", "slstm_last_error", "slstm_newton_workspace_bytes",
    "slstm_newton_forward", "slstm_newton_read_stats", "slstm_sequential_forward",
    "slstm_input_projection", "slstm_residual_jacobian", "slstm_scan_block4_workspace_bytes",
    "slstm_scan_block4", "slstm_warm_start_workspace_bytes", "slstm_warm_start",
    "slstm_profile_enable", "slstm_profile_reset", "slstm_profile_read",
    "slstm_profile_durations", "slstm_backward_workspace_bytes", "slstm_backward",
    "slstm_input_projection_backward_workspace_bytes", "slstm_input_projection_backward",
    "slstm_newton_forward_varlen", "slstm_sequential_forward_varlen", "slstm_warm_start_varlen",
    "slstm_backward_varlen", "slstm_head_newton_workspace_bytes", "slstm_head_newton_forward",
    "slstm_head_sequential_forward", "slstm_head_backward_workspace_bytes", "slstm_head_backward",
    "slstm_head_newton_forward_varlen", "slstm_head_sequential_forward_varlen", "slstm_head_backward_varlen",
    "slstm_newton_forward_noalloc",
]


class NewtonDivergenceError(RuntimeError):
    """Raised when max|F| > 1 (or is not finite) after the last Newton iterate."""


class SlstmError(RuntimeError):
    pass


class _Stats(ctypes.Structure):
    _fields_ = [("iters", ctypes.c_int32), ("converged", ctypes.c_int32),
                ("diverged", ctypes.c_int32), ("nonfinite", ctypes.c_int32),
                ("max_abs_F", ctypes.c_float * (MAX_ITERS + 1))]


@dataclass
class NewtonStats:
    iters: int = 0
    converged: bool = False
    diverged: bool = False
    nonfinite: bool = False
    max_abs_F: list = field(default_factory=list)  # entry k: max|F| after k updates
    status: int = OK

    @classmethod
    def _from(cls, s: _Stats, status: int) -> "NewtonStats":
        return cls(s.iters, bool(s.converged), bool(s.diverged), bool(s.nonfinite),
                   [float(s.max_abs_F[k]) for k in range(s.iters + 1)], status)


_LIB = None
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib_path() -> str:
    return _build.lib_path()


def load(path: str | None = None):
    """Load the built library (once). Raises when it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or lib_path()
    if not os.path.exists(path):
        raise ImportError(f"the HIP library is not built ({path} missing); run "
                          f"`python -m recurrent_nets_amd.build` first")
    L = ctypes.CDLL(path)
    L.slstm_status_string.restype = ctypes.c_char_p
    L.slstm_status_string.argtypes = [_i]
    L.slstm_last_error.restype = ctypes.c_char_p
    L.slstm_scan_block4_workspace_bytes.restype = _sz
    L.slstm_scan_block4_workspace_bytes.argtypes = [_i, _i, _i]
    L.slstm_warm_start_workspace_bytes.restype = _sz
    L.slstm_warm_start_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.slstm_newton_workspace_bytes.restype = _sz
    L.slstm_newton_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.slstm_newton_forward.restype = _i
    L.slstm_newton_forward.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                       _i, _i, _vp, _sz, _vp, ctypes.POINTER(_Stats)]
    L.slstm_newton_forward_noalloc.restype = _i
    L.slstm_newton_forward_noalloc.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                               _i, _i, _vp, ctypes.POINTER(_Stats)]
    L.slstm_newton_read_stats.restype = _i
    L.slstm_newton_read_stats.argtypes = [_vp, _sz, _vp, ctypes.POINTER(_Stats)]
    L.slstm_sequential_forward.restype = _i
    L.slstm_sequential_forward.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
    L.slstm_input_projection.restype = _i
    L.slstm_input_projection.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    L.slstm_residual_jacobian.restype = _i
    L.slstm_residual_jacobian.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
    L.slstm_scan_block4.restype = _i
    L.slstm_scan_block4.argtypes = [_vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]
    L.slstm_warm_start.restype = _i
    L.slstm_warm_start.argtypes = [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]
    L.slstm_backward_workspace_bytes.restype = _sz
    L.slstm_backward_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.slstm_backward.restype = _i
    L.slstm_backward.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp,
                                 _i, _i, _i, _i, _i, _vp, _sz, _vp]
    L.slstm_input_projection_backward_workspace_bytes.restype = _sz
    L.slstm_input_projection_backward_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.slstm_input_projection_backward.restype = _i
    L.slstm_input_projection_backward.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _vp,
                                                  _sz, _vp]
    L.slstm_newton_forward_varlen.restype = _i
    L.slstm_newton_forward_varlen.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i,
                                              _i, _f, _i, _i, _vp, _sz, _vp, ctypes.POINTER(_Stats)]
    L.slstm_sequential_forward_varlen.restype = _i
    L.slstm_sequential_forward_varlen.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i,
                                                  _i, _vp]
    L.slstm_warm_start_varlen.restype = _i
    L.slstm_warm_start_varlen.argtypes = [_vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _vp, _sz, _vp]
    L.slstm_backward_varlen.restype = _i
    L.slstm_backward_varlen.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                                        _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]
    L.slstm_head_newton_workspace_bytes.restype = _sz
    L.slstm_head_newton_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.slstm_head_newton_forward.restype = _i
    L.slstm_head_newton_forward.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                                            _vp, _sz, _vp, ctypes.POINTER(_Stats)]
    L.slstm_head_sequential_forward.restype = _i
    L.slstm_head_sequential_forward.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    L.slstm_head_backward_workspace_bytes.restype = _sz
    L.slstm_head_backward_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.slstm_head_backward.restype = _i
    L.slstm_head_backward.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i,
                                      _i, _vp, _sz, _vp]
    L.slstm_head_newton_forward_varlen.restype = _i
    L.slstm_head_newton_forward_varlen.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                                   _i, _vp, _sz, _vp, ctypes.POINTER(_Stats)]
    L.slstm_head_sequential_forward_varlen.restype = _i
    L.slstm_head_sequential_forward_varlen.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i,
                                                       _vp]
    L.slstm_head_backward_varlen.restype = _i
    L.slstm_head_backward_varlen.argtypes = [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp,
                                             _i, _i, _i, _i, _vp, _sz, _vp]
    L.slstm_profile_enable.restype = _i
    L.slstm_profile_enable.argtypes = [_i]
    L.slstm_profile_reset.restype = _i
    L.slstm_profile_read.restype = _i
    L.slstm_profile_read.argtypes = [_i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i)]
    L.slstm_profile_durations.restype = _i
    L.slstm_profile_durations.argtypes = [_i, ctypes.POINTER(ctypes.c_double), _i, ctypes.POINTER(_i)]
    _LIB = L
    return L


def _check(status: int, what: str) -> int:
    if status < 0:
        L = load()
        raise SlstmError(f"{what}: {L.slstm_status_string(status).decode()}: "
                         f"{L.slstm_last_error().decode()}")
    return status


# ---- marshalling helpers ---------------------------------------------------------------------
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fmode(forget, readout):
    """The C forget argument: the forget-gate form with the read-out variant OR-ed in."""
    return FORGET[forget] | READOUT[readout]


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _p_dtype(P):
    return BF16 if P.dtype == torch.bfloat16 else F32


def _shape_check(P, R, state0, n_states=None):
    """(B, T, d_h) of P; state0 is (n_states, 4, d_h), n_states = B unless given."""
    if P.dim() != 4 or P.shape[2] != 4:
        raise ValueError(f"P must be (B, T, 4, d_h), got {tuple(P.shape)}")
    B, T, _, d = P.shape
    if R is not None and tuple(R.shape) != (4, d):
        raise ValueError(f"R must be (4, {d}), got {tuple(R.shape)}")
    n = B if n_states is None else n_states
    if state0 is not None and tuple(state0.shape) != (n, 4, d):
        raise ValueError(f"state0 must be ({n}, 4, {d}), got {tuple(state0.shape)}")
    return B, T, d


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _seqs(cu_seqlens, P):
    """Packed sequences: (device int32 offsets, S) or (None, None). A list, tuple or host tensor
    is checked (cu[0] = 0, non-decreasing, cu[S] = T) and copied to P's device; a device tensor
    must be int32 and is passed as it is. P must then have B = 1."""
    if cu_seqlens is None:
        return None, None
    if P.shape[0] != 1:
        raise ValueError(f"packed sequences take P of shape (1, T, 4, d_h), got {tuple(P.shape)}")
    T = P.shape[1]
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda):
        cu = [int(v) for v in (cu_seqlens.tolist() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens)]
        if len(cu) < 2 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
            raise ValueError(f"cu_seqlens must run from 0 to T = {T} without decreasing, got {cu}")
        cu_seqlens = torch.tensor(cu, dtype=torch.int32, device=P.device)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise TypeError("cu_seqlens must be a 1-D int32 tensor of S + 1 offsets")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    return cu_seqlens, cu_seqlens.numel() - 1


def newton_workspace_bytes(B: int, T: int, d_h: int, schedule: str = "fused") -> int:
    return int(load().slstm_newton_workspace_bytes(B, T, d_h, SCHEDULE[schedule]))


def alloc_workspace(nbytes: int, device=None) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned well beyond 256 bytes
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device or "cuda")


def newton_forward(P, R, state0=None, forget="exp", max_iters=3, tol=0.0, init="warm",
                   states=None, h_out=None, want_hidden=True, final_state=None, workspace=None,
                   stream=None, stats=True, raise_on_divergence=True, schedule="fused",
                   readout="exact", cu_seqlens=None, output_states=True):
    """Newton-parallel forward. Returns (states (B,T,4,d_h), h (B,T,d_h) or None, NewtonStats
    or None). ``output_states=False`` asks for the hidden slot and the final state only (the
    pages' default layer output): states is then None and the library writes no state tensor,
    which it allows where the solve resolves to the one-kernel form (tol = 0, max_iters <= 4,
    unpacked; "fused_chain", or "fused" on enough lanes). With stats=False the call is asynchronous and returns no stats. A given
    ``final_state`` (B,4,d_h) tensor receives the last step's state. ``schedule`` is "fused"
    ("fused_chain" when the lane groups cover the GPU, or number at least 32 for a fixed-count
    solve that runs as one kernel, else "fused_scan"), "fused_scan", "fused_chain" or "layered" (residual + Jacobian, scan,
    update). ``readout`` is "exact" (h = o c / n) or "floored" (h = o c / max(|n|, e^{-m},
    1e-6)); every function taking ``forget`` takes it too.

    ``cu_seqlens`` (S + 1 offsets) packs S sequences end to end along time in P (1, T, 4, d_h):
    state0 and final_state are then (S, 4, d_h); "fused" runs the one-kernel solve on tiles
    aligned to the sequences where it can (up to 8 iterations; enough sequences), else
    "fused_scan" ("fused_chain" is rejected); sequential_forward, warm_start and backward take
    it the same way."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    cu, S = _seqs(cu_seqlens, P)
    B, T, d = _shape_check(P, R, state0, S)
    if states is None and output_states:
        states = torch.empty((B, T, 4, d), dtype=torch.float32, device=P.device)
    if want_hidden and h_out is None:
        h_out = torch.empty((B, T, d), dtype=torch.float32, device=P.device)
    _dev(states, "states", (torch.float32,))
    _dev(h_out, "h_out", (torch.float32,))
    _dev(final_state, "final_state", (torch.float32,))
    _shape(final_state, "final_state", (B if cu is None else S, 4, d))
    need = L.slstm_newton_workspace_bytes(B, T, d, SCHEDULE[schedule])
    if workspace is None:
        workspace = alloc_workspace(need, P.device)
    st = _Stats() if stats else None
    nbytes = workspace.numel() * workspace.element_size()
    st_ref = ctypes.byref(st) if st is not None else None
    if cu is None:
        status = L.slstm_newton_forward(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states),
                                        _ptr(h_out), _ptr(final_state), B, T, d, _fmode(forget, readout),
                                        int(max_iters), float(tol), INIT[init], SCHEDULE[schedule],
                                        _ptr(workspace), nbytes, _stream(stream), st_ref)
    else:
        status = L.slstm_newton_forward_varlen(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(cu), S,
                                               _ptr(states), _ptr(h_out), _ptr(final_state), T, d,
                                               _fmode(forget, readout), int(max_iters), float(tol),
                                               INIT[init], SCHEDULE[schedule], _ptr(workspace), nbytes,
                                               _stream(stream), st_ref)
    _check(status, "slstm_newton_forward")
    out_stats = NewtonStats._from(st, status) if st is not None else None
    if raise_on_divergence and status in (DIVERGED, NONFINITE):
        raise NewtonDivergenceError(
            f"{L.slstm_status_string(status).decode()} (max|F| = {out_stats.max_abs_F[-1]:.3g})")
    return states, h_out, out_stats


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # SLSTM_NOALLOC_SCRATCH_BYTES


def newton_forward_noalloc(P, R, state0=None, forget="exp", max_iters=3, tol=0.0, init="warm",
                           states=None, h_out=None, final_state=None, stream=None, stats=True,
                           raise_on_divergence=True, schedule="fused", readout="exact"):
    """newton_forward through the entry point that allocates nothing: the solver works in the
    library's fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES), so the caller passes outputs but no
    workspace. ``states`` (and ``h_out`` if wanted) must be given. Calls that overlap on one GPU
    race on the shared scratch. Returns (states, h_out, NewtonStats or None)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    B, T, d = _shape_check(P, R, state0, None)
    if states is None:
        raise ValueError("newton_forward_noalloc needs a preallocated states tensor")
    _dev(states, "states", (torch.float32,))
    _dev(h_out, "h_out", (torch.float32,))
    _dev(final_state, "final_state", (torch.float32,))
    _shape(states, "states", (B, T, 4, d))
    _shape(h_out, "h_out", (B, T, d))
    _shape(final_state, "final_state", (B, 4, d))
    st = _Stats() if stats else None
    status = L.slstm_newton_forward_noalloc(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states),
                                            _ptr(h_out), _ptr(final_state), B, T, d, _fmode(forget, readout),
                                            int(max_iters), float(tol), INIT[init], SCHEDULE[schedule],
                                            _stream(stream), ctypes.byref(st) if st is not None else None)
    _check(status, "slstm_newton_forward_noalloc")
    out_stats = NewtonStats._from(st, status) if st is not None else None
    if raise_on_divergence and status in (DIVERGED, NONFINITE):
        raise NewtonDivergenceError(
            f"{L.slstm_status_string(status).decode()} (max|F| = {out_stats.max_abs_F[-1]:.3g})")
    return states, h_out, out_stats


def read_stats(workspace, stream=None) -> NewtonStats:
    L = load()
    st = _Stats()
    status = L.slstm_newton_read_stats(_ptr(workspace), workspace.numel(), _stream(stream),
                                       ctypes.byref(st))
    _check(status, "slstm_newton_read_stats")
    return NewtonStats._from(st, status)


def sequential_forward(P, R, state0=None, forget="exp", states=None, h_out=None,
                       want_hidden=True, final_state=None, stream=None, readout="exact",
                       cu_seqlens=None, output_states=True):
    """Step-by-step forward (also the T=1 decode step). Returns (states, h or None). A given
    ``final_state`` (B,4,d_h) tensor receives the last step's state. ``output_states=False``
    (unpacked only) writes no state tensor and returns None for it: h and the final state are
    the outputs, as in the layer's default output."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    cu, S = _seqs(cu_seqlens, P)
    B, T, d = _shape_check(P, R, state0, S)
    if states is None and output_states:
        states = torch.empty((B, T, 4, d), dtype=torch.float32, device=P.device)
    if want_hidden and h_out is None:
        h_out = torch.empty((B, T, d), dtype=torch.float32, device=P.device)
    _dev(states, "states", (torch.float32,))
    _dev(h_out, "h_out", (torch.float32,))
    _dev(final_state, "final_state", (torch.float32,))
    _shape(final_state, "final_state", (B if cu is None else S, 4, d))
    if cu is None:
        status = L.slstm_sequential_forward(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states),
                                            _ptr(h_out), _ptr(final_state), B, T, d,
                                            _fmode(forget, readout), _stream(stream))
    else:
        status = L.slstm_sequential_forward_varlen(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(cu),
                                                   S, _ptr(states), _ptr(h_out), _ptr(final_state), T, d,
                                                   _fmode(forget, readout), _stream(stream))
    _check(status, "slstm_sequential_forward")
    return states, h_out


def input_projection(x, W, bias=None, out=None, stream=None):
    """P = x W^T + bias on MFMA. x (B,T,d_in) bf16, W (4,d_h,d_in) bf16, bias (4,d_h) f32."""
    L = load()
    _dev(x, "x", (torch.bfloat16,))
    _dev(W, "W_x", (torch.bfloat16,))
    _dev(bias, "bias", (torch.float32,))
    B, T, d_in = x.shape
    g, d, d_in2 = W.shape
    if g != 4 or d_in2 != d_in:
        raise ValueError(f"W_x must be (4, d_h, {d_in}), got {tuple(W.shape)}")
    if bias is not None and tuple(bias.shape) != (4, d):
        raise ValueError(f"bias must be (4, {d})")
    if out is None:
        out = torch.empty((B, T, 4, d), dtype=torch.float32, device=x.device)
    _dev(out, "P", (torch.float32,))
    status = L.slstm_input_projection(_ptr(x), _ptr(W), _ptr(bias), _ptr(out), B, T, d_in, d,
                                      BF16, _stream(stream))
    _check(status, "slstm_input_projection")
    return out


def residual_jacobian(P, R, states, state0=None, forget="exp", stream=None, readout="exact"):
    """One residual + Jacobian evaluation. Returns (A (B,T,4,4,d), rhs = -F (B,T,4,d),
    max|F| as a 1-element device tensor)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    _dev(states, "states", (torch.float32,))
    B, T, d = _shape_check(P, R, state0)
    A = torch.empty((B, T, 4, 4, d), dtype=torch.float32, device=P.device)
    rhs = torch.empty((B, T, 4, d), dtype=torch.float32, device=P.device)
    err = torch.empty((1,), dtype=torch.float32, device=P.device)
    status = L.slstm_residual_jacobian(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states),
                                       _ptr(A), _ptr(rhs), _ptr(err), B, T, d, _fmode(forget, readout),
                                       _stream(stream))
    _check(status, "slstm_residual_jacobian")
    return A, rhs, err


def scan_block4(A, rhs, out=None, workspace=None, stream=None):
    """x_1 = rhs_1, x_t = A_t x_{t-1} + rhs_t per lane. A (B,T,4,4,d), rhs (B,T,4,d).
    ``out`` may be ``rhs`` itself (in place)."""
    L = load()
    _dev(A, "A", (torch.float32,))
    _dev(rhs, "rhs", (torch.float32,))
    B, T, _, d = rhs.shape
    if tuple(A.shape) != (B, T, 4, 4, d):
        raise ValueError("A must be (B, T, 4, 4, d) matching rhs")
    if out is None:
        out = torch.empty_like(rhs)
    _dev(out, "out", (torch.float32,))
    need = L.slstm_scan_block4_workspace_bytes(B, T, d)
    if workspace is None:
        workspace = alloc_workspace(need, rhs.device)
    status = L.slstm_scan_block4(_ptr(A), _ptr(rhs), _ptr(out), B, T, d, _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check(status, "slstm_scan_block4")
    return out


def warm_start(P, state0=None, forget="exp", out=None, workspace=None, stream=None,
               schedule="fused", readout="exact", cu_seqlens=None):
    """The R-free trajectory used as the initial Newton iterate. Returns states (B,T,4,d).
    ``schedule`` picks the kernel form as in newton_forward ("fused_chain": tile-serial
    recurrences; "fused_scan" / "layered": log-space scan with look-back)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(state0, "state0", (torch.float32,))
    cu, S = _seqs(cu_seqlens, P)
    B, T, d = _shape_check(P, None, state0, S)
    if out is None:
        out = torch.empty((B, T, 4, d), dtype=torch.float32, device=P.device)
    _dev(out, "out", (torch.float32,))
    sched = SCHEDULE["fused_scan" if cu is not None and schedule == "fused" else schedule]
    need = L.slstm_warm_start_workspace_bytes(B, T, d, sched)
    if workspace is None:
        workspace = alloc_workspace(need, P.device)
    if cu is None:
        status = L.slstm_warm_start(_ptr(P), _p_dtype(P), _ptr(state0), _ptr(out), B, T, d,
                                    _fmode(forget, readout), SCHEDULE[schedule], _ptr(workspace),
                                    workspace.numel(), _stream(stream))
    else:
        status = L.slstm_warm_start_varlen(_ptr(P), _p_dtype(P), _ptr(state0), _ptr(cu), S, _ptr(out), T, d,
                                           _fmode(forget, readout), SCHEDULE[schedule], _ptr(workspace),
                                           workspace.numel(), _stream(stream))
    _check(status, "slstm_warm_start")
    return out


def backward_workspace_bytes(B: int, T: int, d_h: int, schedule: str = "fused") -> int:
    return int(load().slstm_backward_workspace_bytes(B, T, d_h, SCHEDULE[schedule]))


def backward(P, R, states, state0=None, g_states=None, g_h=None, g_final=None, forget="exp",
             dP=None, dR=None, dstate0=None, want_dstate0=True, workspace=None, stream=None,
             schedule="fused", dP_dtype=torch.float32, dbias=None, want_dbias=False,
             readout="exact", cu_seqlens=None):
    """Gradients through the recurrence at the forward solution ``states`` (B,T,4,d_h).
    g_states (B,T,4,d_h), g_h (B,T,d_h) and g_final (B,4,d_h) are the loss's direct gradients
    (None: zeros). dP is float32 or bfloat16 (``dP_dtype``). Returns (dP (B,T,4,d_h),
    dR (4,d_h), dstate0 (B,4,d_h) or None), and dbias (4,d_h) last when ``want_dbias`` or a
    ``dbias`` tensor is given. With ``cu_seqlens``, g_final and dstate0 are (S,4,d_h)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    cu, S = _seqs(cu_seqlens, P)
    B, T, d = _shape_check(P, R, state0, S)
    n0 = B if cu is None else S
    for name, t, shape in (("states", states, (B, T, 4, d)), ("g_states", g_states, (B, T, 4, d)),
                           ("g_h", g_h, (B, T, d)), ("g_final", g_final, (n0, 4, d))):
        _dev(t, name, (torch.float32,))
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
    if dP is None:
        dP = torch.empty((B, T, 4, d), dtype=dP_dtype, device=P.device)
    if want_dbias and dbias is None:
        dbias = torch.empty((4, d), dtype=torch.float32, device=P.device)
    if dR is None:
        dR = torch.empty((4, d), dtype=torch.float32, device=P.device)
    if want_dstate0 and dstate0 is None:
        dstate0 = torch.empty((n0, 4, d), dtype=torch.float32, device=P.device)
    _dev(dP, "dP", (torch.float32, torch.bfloat16))
    _dev(dR, "dR", (torch.float32,))
    _dev(dbias, "dbias", (torch.float32,))
    _dev(dstate0, "dstate0", (torch.float32,))
    need = L.slstm_backward_workspace_bytes(B, T, d, SCHEDULE[schedule])
    if workspace is None:
        workspace = alloc_workspace(need, P.device)
    dpt = BF16 if dP.dtype == torch.bfloat16 else F32
    if cu is None:
        status = L.slstm_backward(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states),
                                  _ptr(g_states), _ptr(g_h), _ptr(g_final), _ptr(dP), dpt, _ptr(dR),
                                  _ptr(dbias), _ptr(dstate0), B, T, d, _fmode(forget, readout),
                                  SCHEDULE[schedule], _ptr(workspace), workspace.numel(), _stream(stream))
    else:
        status = L.slstm_backward_varlen(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(cu), S,
                                         _ptr(states), _ptr(g_states), _ptr(g_h), _ptr(g_final), _ptr(dP),
                                         dpt, _ptr(dR), _ptr(dbias), _ptr(dstate0), T, d,
                                         _fmode(forget, readout), SCHEDULE[schedule], _ptr(workspace),
                                         workspace.numel(), _stream(stream))
    _check(status, "slstm_backward")
    if dbias is not None:
        return dP, dR, dstate0, dbias
    return dP, dR, dstate0


# ---- head mixing (R of shape (4, n_heads, d_head, d_head)) ----------------------------------
def _head_check(P, R, state0, n_seq=None):
    """Shapes of a head-mixing call; n_seq (packed) makes state0 (n_seq, 4, d_h)."""
    if P.dim() != 4 or P.shape[2] != 4:
        raise ValueError(f"P must be (B, T, 4, d_h), got {tuple(P.shape)}")
    B, T, _, d = P.shape
    if R.dim() != 4 or R.shape[0] != 4 or R.shape[2] != R.shape[3] or R.shape[1] * R.shape[2] != d:
        raise ValueError(f"R must be (4, n_heads, d_head, d_head) with n_heads * d_head = {d}, got {tuple(R.shape)}")
    _shape(state0, "state0", (B if n_seq is None else n_seq, 4, d))
    return B, T, d, int(R.shape[1])


def head_newton_workspace_bytes(B: int, T: int, d_h: int, n_heads: int) -> int:
    return int(load().slstm_head_newton_workspace_bytes(B, T, d_h, n_heads))


def head_newton_forward(P, R, state0=None, forget="exp", max_iters=3, tol=0.0, init="warm",
                        states=None, h_out=None, want_hidden=True, final_state=None, workspace=None,
                        stream=None, stats=True, raise_on_divergence=True, readout="exact", cu_seqlens=None):
    """Newton-parallel forward under head mixing (block-diagonal R, one block per head and
    gate). Arguments and returns as newton_forward; R (4, n_heads, d_head, d_head) float32 with
    d_head in {8, 16, 32, 64, 128}. With cu_seqlens (packed, B = 1), state0 and final_state are
    (S, 4, d_h)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    cu, n_seq = _seqs(cu_seqlens, P)
    B, T, d, nh = _head_check(P, R, state0, n_seq)
    if states is None:
        states = torch.empty((B, T, 4, d), dtype=torch.float32, device=P.device)
    if want_hidden and h_out is None:
        h_out = torch.empty((B, T, d), dtype=torch.float32, device=P.device)
    _dev(states, "states", (torch.float32,))
    _dev(h_out, "h_out", (torch.float32,))
    _dev(final_state, "final_state", (torch.float32,))
    _shape(final_state, "final_state", (B if cu is None else n_seq, 4, d))
    if workspace is None:
        workspace = alloc_workspace(L.slstm_head_newton_workspace_bytes(B, T, d, nh), P.device)
    st = _Stats() if stats else None
    wsb = workspace.numel() * workspace.element_size()
    sref = ctypes.byref(st) if st is not None else None
    if cu is None:
        status = L.slstm_head_newton_forward(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states), _ptr(h_out),
                                             _ptr(final_state), B, T, d, nh, _fmode(forget, readout),
                                             int(max_iters), float(tol), INIT[init], _ptr(workspace), wsb,
                                             _stream(stream), sref)
    else:
        status = L.slstm_head_newton_forward_varlen(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(cu), n_seq,
                                                    _ptr(states), _ptr(h_out), _ptr(final_state), T, d, nh,
                                                    _fmode(forget, readout), int(max_iters), float(tol), INIT[init],
                                                    _ptr(workspace), wsb, _stream(stream), sref)
    _check(status, "slstm_head_newton_forward")
    out_stats = NewtonStats._from(st, status) if st is not None else None
    if raise_on_divergence and status in (DIVERGED, NONFINITE):
        raise NewtonDivergenceError(
            f"{L.slstm_status_string(status).decode()} (max|F| = {out_stats.max_abs_F[-1]:.3g})")
    return states, h_out, out_stats


def head_sequential_forward(P, R, state0=None, forget="exp", states=None, h_out=None, want_hidden=True,
                            final_state=None, stream=None, readout="exact", cu_seqlens=None):
    """Step-by-step forward under head mixing (also the T=1 decode step). Returns (states, h).
    With cu_seqlens (packed, B = 1), state0 and final_state are (S, 4, d_h)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    cu, n_seq = _seqs(cu_seqlens, P)
    B, T, d, nh = _head_check(P, R, state0, n_seq)
    if states is None:
        states = torch.empty((B, T, 4, d), dtype=torch.float32, device=P.device)
    if want_hidden and h_out is None:
        h_out = torch.empty((B, T, d), dtype=torch.float32, device=P.device)
    _dev(states, "states", (torch.float32,))
    _dev(h_out, "h_out", (torch.float32,))
    _dev(final_state, "final_state", (torch.float32,))
    _shape(final_state, "final_state", (B if cu is None else n_seq, 4, d))
    if cu is None:
        status = L.slstm_head_sequential_forward(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states),
                                                 _ptr(h_out), _ptr(final_state), B, T, d, nh,
                                                 _fmode(forget, readout), _stream(stream))
    else:
        status = L.slstm_head_sequential_forward_varlen(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(cu),
                                                        n_seq, _ptr(states), _ptr(h_out), _ptr(final_state), T, d,
                                                        nh, _fmode(forget, readout), _stream(stream))
    _check(status, "slstm_head_sequential_forward")
    return states, h_out


def head_backward_workspace_bytes(B: int, T: int, d_h: int, n_heads: int) -> int:
    return int(load().slstm_head_backward_workspace_bytes(B, T, d_h, n_heads))


def head_backward(P, R, states, state0=None, g_states=None, g_h=None, g_final=None, forget="exp",
                  dP=None, dR=None, dstate0=None, want_dstate0=True, workspace=None, stream=None,
                  dP_dtype=torch.float32, dbias=None, want_dbias=False, readout="exact", cu_seqlens=None):
    """Gradients through the head-mixing recurrence at the forward solution ``states``
    (B,T,4,d_h); arguments as ``backward``, R (4, n_heads, d_head, d_head) with d_head 8, 16, 32,
    64 or 128. Returns (dP, dR (4, n_heads, d_head, d_head), dstate0 or None), and dbias (4, d_h) last
    when ``want_dbias`` or a ``dbias`` tensor is given. With cu_seqlens (packed, B = 1),
    state0, g_final and dstate0 are (S, 4, d_h)."""
    L = load()
    _dev(P, "P", (torch.float32, torch.bfloat16))
    _dev(R, "R", (torch.float32,))
    _dev(state0, "state0", (torch.float32,))
    cu, n_seq = _seqs(cu_seqlens, P)
    B, T, d, nh = _head_check(P, R, state0, n_seq)
    n0 = B if cu is None else n_seq
    for name, t, shape in (("states", states, (B, T, 4, d)), ("g_states", g_states, (B, T, 4, d)),
                           ("g_h", g_h, (B, T, d)), ("g_final", g_final, (n0, 4, d))):
        _dev(t, name, (torch.float32,))
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
    if dP is None:
        dP = torch.empty((B, T, 4, d), dtype=dP_dtype, device=P.device)
    if dR is None:
        dR = torch.empty(tuple(R.shape), dtype=torch.float32, device=P.device)
    if want_dbias and dbias is None:
        dbias = torch.empty((4, d), dtype=torch.float32, device=P.device)
    if want_dstate0 and dstate0 is None:
        dstate0 = torch.empty((n0, 4, d), dtype=torch.float32, device=P.device)
    _dev(dP, "dP", (torch.float32, torch.bfloat16))
    _dev(dR, "dR", (torch.float32,))
    _dev(dbias, "dbias", (torch.float32,))
    _dev(dstate0, "dstate0", (torch.float32,))
    if workspace is None:
        workspace = alloc_workspace(max(L.slstm_head_backward_workspace_bytes(B, T, d, nh), 256), P.device)
    dpt = BF16 if dP.dtype == torch.bfloat16 else F32
    wsb = workspace.numel() * workspace.element_size()
    if cu is None:
        status = L.slstm_head_backward(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(states), _ptr(g_states),
                                       _ptr(g_h), _ptr(g_final), _ptr(dP), dpt, _ptr(dR), _ptr(dbias), _ptr(dstate0),
                                       B, T, d, nh, _fmode(forget, readout), _ptr(workspace), wsb, _stream(stream))
    else:
        status = L.slstm_head_backward_varlen(_ptr(P), _p_dtype(P), _ptr(R), _ptr(state0), _ptr(cu), n_seq,
                                              _ptr(states), _ptr(g_states), _ptr(g_h), _ptr(g_final), _ptr(dP), dpt,
                                              _ptr(dR), _ptr(dbias), _ptr(dstate0), T, d, nh, _fmode(forget, readout),
                                              _ptr(workspace), wsb, _stream(stream))
    _check(status, "slstm_head_backward")
    if want_dbias or dbias is not None:
        return dP, dR, dstate0, dbias
    return dP, dR, dstate0


def input_projection_backward_workspace_bytes(B: int, T: int, d_in: int, d_h: int) -> int:
    return int(load().slstm_input_projection_backward_workspace_bytes(B, T, d_in, d_h))


def input_projection_backward(x, W, dP, dx=None, dW=None, want_dx=True, want_dW=True,
                              workspace=None, stream=None):
    """dW_x = dP^T x and dx = dP W_x on MFMA (bf16 operands, float32 results). x (B,T,d_in) bf16,
    W (4,d_h,d_in) bf16, dP (B,T,4,d_h) float32 or bf16. Returns (dx or None, dW or None)."""
    L = load()
    _dev(x, "x", (torch.bfloat16,))
    _dev(W, "W_x", (torch.bfloat16,))
    _dev(dP, "dP", (torch.float32, torch.bfloat16))
    B, T, d_in = x.shape
    g, d, d_in2 = W.shape
    if g != 4 or d_in2 != d_in or tuple(dP.shape) != (B, T, 4, d):
        raise ValueError(f"shapes: x {tuple(x.shape)}, W_x {tuple(W.shape)}, dP {tuple(dP.shape)}")
    if want_dx and dx is None:
        dx = torch.empty((B, T, d_in), dtype=torch.float32, device=x.device)
    if want_dW and dW is None:
        dW = torch.empty((4, d, d_in), dtype=torch.float32, device=x.device)
    _dev(dx, "dx", (torch.float32,))
    _dev(dW, "dW", (torch.float32,))
    need = L.slstm_input_projection_backward_workspace_bytes(B, T, d_in, d)
    if workspace is None:
        workspace = alloc_workspace(need, x.device)
    status = L.slstm_input_projection_backward(
        _ptr(x), _ptr(W), _ptr(dP), BF16 if dP.dtype == torch.bfloat16 else F32, _ptr(dx), _ptr(dW),
        B, T, d_in, d, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(status, "slstm_input_projection_backward")
    return dx, dW


def profile_enable(on: bool = True):
    load().slstm_profile_enable(1 if on else 0)


def profile_reset():
    load().slstm_profile_reset()


def profile_read(kind: str):
    """(summed milliseconds, launch count) of one kernel kind since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int()
    _check(load().slstm_profile_read(KERNELS[kind], ctypes.byref(ms), ctypes.byref(n)),
           "slstm_profile_read")
    return ms.value, n.value


def profile_durations(kind: str):
    """Every launch duration (ms, launch order) of one kernel kind since the last reset."""
    L = load()
    n = ctypes.c_int()
    _check(L.slstm_profile_durations(KERNELS[kind], None, 0, ctypes.byref(n)), "slstm_profile_durations")
    buf = (ctypes.c_double * max(n.value, 1))()
    _check(L.slstm_profile_durations(KERNELS[kind], buf, n.value, ctypes.byref(n)),
           "slstm_profile_durations")
    return [buf[i] for i in range(n.value)]
