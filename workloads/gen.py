"""Seeded generators. numpy PCG64, draws in float64, then cast to the workload dtype.

Draw order per workload seed: x, W_x, R. The decode step draws from seed + 1000.
bf16 casts round to nearest even from float32 (the cast torch applies).
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload


def to_bf16(a) -> torch.Tensor:
    """float64/float32 array -> torch.bfloat16 tensor (via float32, round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float32).numpy().astype(np.float64)


def _bias(w: Workload) -> np.ndarray:
    b = np.zeros((4, w.d_h))
    b[2] = w.forget_bias  # forget-gate row
    return b


def _draw_x_w_r(w: Workload, B: int | None = None, T: int | None = None):
    B = w.B if B is None else B
    T = w.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(w.seed))
    x = rng.standard_normal((B, T, w.d_in))
    if w.spike_every:
        x[:, w.spike_every - 1::w.spike_every, :] *= w.spike_scale
    W = rng.standard_normal((4, w.d_h, w.d_in)) * np.sqrt(1.0 / w.d_in)
    R = rng.uniform(-0.5, 0.5, size=(4, w.d_h))
    return x, W, R


def synth_preactivations(x: np.ndarray, W: np.ndarray, bias: np.ndarray, p_dtype: str,
                         device: str = "cpu") -> torch.Tensor:
    """Gate pre-activations with the workload's structure: x W^T + bias in float64, cast.

    This is input synthesis for workloads whose solver input is P; it runs through torch's
    float64 matmul on ``device``.
    """
    B, T, d_in = x.shape
    g, d_h, _ = W.shape
    xt = torch.from_numpy(x.reshape(B * T, d_in)).to(device)
    Wt = torch.from_numpy(W.reshape(g * d_h, d_in)).to(device)
    P = (xt @ Wt.T).reshape(B, T, g, d_h) + torch.from_numpy(bias).to(device)
    P = P.to(torch.float32)
    if p_dtype == "bf16":
        P = P.to(torch.bfloat16)
    return P.cpu().contiguous()


def draw_preactivation_inputs(w: Workload, B: int | None = None, T: int | None = None,
                              device: str = "cpu"):
    """Inputs for workloads whose solver input is P.

    Returns dict(P=torch tensor (B, T, 4, d_h) in the workload's P dtype, R=float32 (4, d_h)
    tensor, state0=None). ``B``/``T`` override the sizes (same seed, smaller draw) for tests.
    """
    x, W, R = _draw_x_w_r(w, B, T)
    x = x.astype(np.float32).astype(np.float64)
    W = W.astype(np.float32).astype(np.float64)
    P = synth_preactivations(x, W, _bias(w), w.p_dtype, device)
    return dict(P=P, R=torch.from_numpy(R.astype(np.float32)), state0=None)


def draw_layer_inputs(w: Workload, B: int | None = None, T: int | None = None):
    """Inputs for the full-layer workload: bf16 x (B, T, d_in), bf16 W_x (4, d_h, d_in),
    float32 bias (4, d_h), float32 R (4, d_h)."""
    x, W, R = _draw_x_w_r(w, B, T)
    return dict(x=to_bf16(x), W=to_bf16(W), bias=torch.from_numpy(_bias(w).astype(np.float32)),
                R=torch.from_numpy(R.astype(np.float32)))


def draw_decode_inputs(w: Workload):
    """A fresh bf16 input row (decode_batch, 1, d_in) ~ N(0, 1) for the T=1 decode step."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    return to_bf16(rng.standard_normal((w.decode_batch, 1, w.d_in)))


def random_states(seed: int, B: int, T: int, d: int) -> np.ndarray:
    """Plausible sLSTM states (B, T, 4, d): n > 0, |c| <= n, m in [-4, 40], |h| < 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = np.exp(rng.uniform(-3.0, 3.0, size=(B, T, d)))
    c = n * rng.uniform(-1.0, 1.0, size=(B, T, d))
    m = rng.uniform(-4.0, 40.0, size=(B, T, d))
    h = rng.uniform(-0.99, 0.99, size=(B, T, d))
    return np.stack([c, n, m, h], axis=2)


def random_scan_operands(seed: int, B: int, T: int, d: int, scale: float = 0.45):
    """Random affine-map operands for the 4x4 scan: A (B, T, 4, 4, d), r (B, T, 4, d).

    Entries of A are U(-scale, scale), so the 4x4 products stay bounded; r ~ N(0, 1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.uniform(-scale, scale, size=(B, T, 4, 4, d))
    r = rng.standard_normal((B, T, 4, d))
    return A, r


def random_cotangents(seed: int, B: int, T: int, d: int):
    """Direct loss gradients for a backward pass, each ~ N(0, 1) in float32: with respect to
    the states (B, T, 4, d), the hidden states (B, T, d) and the final state (B, 4, d)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g_states = rng.standard_normal((B, T, 4, d)).astype(np.float32)
    g_h = rng.standard_normal((B, T, d)).astype(np.float32)
    g_final = rng.standard_normal((B, 4, d)).astype(np.float32)
    return g_states, g_h, g_final


def random_cotangents_device(seed: int, B: int, T: int, d: int, device):
    """random_cotangents' distributions drawn on ``device`` by torch's seeded generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    g_states = torch.randn((B, T, 4, d), generator=gen, device=device)
    g_h = torch.randn((B, T, d), generator=gen, device=device)
    g_final = torch.randn((B, 4, d), generator=gen, device=device)
    return g_states, g_h, g_final


def packed_offsets(seed: int, total: int, max_len: int, share_empty: float = 0.05,
                   share_one: float = 0.05) -> np.ndarray:
    """Offsets cu_seqlens (S + 1 int64, from 0 to ``total``) of ragged sequences packed end to
    end: lengths log-uniform in [1, max_len] (many short sequences, a few long ones), with a
    share of empty and of length-1 sequences mixed in; the last length is cut so that the
    lengths sum to ``total``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = []
    left = total
    while left > 0:
        u = rng.uniform()
        if u < share_empty:
            n = 0
        elif u < share_empty + share_one:
            n = 1
        else:
            n = int(np.exp(rng.uniform(0.0, np.log(max_len))))
        n = min(max(n, 0), left)
        lengths.append(n)
        left -= n
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def draw_head_inputs(seed: int, B: int, T: int, d: int, n_heads: int, p_dtype: str = "f32",
                     forget_bias: float = 3.0, with_state0: bool = False):
    """Inputs for head mixing: P (B, T, 4, d) ~ N(0, 1) with the forget-gate row shifted by
    ``forget_bias`` (the marginal law of x W^T + bias for x ~ N(0, 1), W ~ N(0, 1/d_in)), in
    float32 or bf16; R (4, n_heads, d_head, d_head) ~ U(-0.5, 0.5) / sqrt(d_head), so that
    R_g h' has the spread of the channelwise U(-0.5, 0.5) h'; optionally a plausible state0
    (B, 4, d). Returns float32 torch tensors on the CPU (P in bf16 for p_dtype "bf16")."""
    dh = d // n_heads
    rng = np.random.Generator(np.random.PCG64(seed))
    P = rng.standard_normal((B, T, 4, d))
    P[:, :, 2] += forget_bias
    R = rng.uniform(-0.5, 0.5, (4, n_heads, dh, dh)) / np.sqrt(dh)
    s0 = None
    if with_state0:
        s0 = np.stack([rng.uniform(-0.5, 0.5, (B, d)), rng.uniform(0.5, 2.0, (B, d)),
                       rng.uniform(-2.0, 2.0, (B, d)), rng.uniform(-0.9, 0.9, (B, d))], axis=1)
        s0 = torch.from_numpy(s0.astype(np.float32))
    Pt = torch.from_numpy(P.astype(np.float32))
    if p_dtype == "bf16":
        Pt = Pt.to(torch.bfloat16)
    return dict(P=Pt, R=torch.from_numpy(R.astype(np.float32)), state0=s0)
