"""The five sLSTM (mix='diag') forward workloads, named by what they are.

Distributions follow the workload descriptions: x ~ N(0, 1); W_x (4, d_h, d_in) ~ N(0, 1/d_in)
with the second parameter read as the variance; channelwise R (4, d_h) ~ U(-0.5, 0.5); bias
zero except the forget-gate row, +3. Gate order (z, i, f, o).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    d_in: int
    d_h: int
    p_dtype: str          # dtype of the gate pre-activations handed to the solver: "f32" | "bf16"
    x_dtype: str          # dtype x and W_x are drawn into: "f32" | "bf16"
    forget: str           # "exp" | "sigmoid"
    max_iters: int        # Newton iteration budget
    tol: float            # residual early-stop tolerance (0: fixed number of iterations)
    seed: int
    spike_every: int = 0  # every spike_every-th step (1-based) has x scaled by spike_scale
    spike_scale: float = 1.0
    on_gpu_gemm: bool = False   # P comes from the bf16 MFMA input projection on the GPU
    decode_batch: int = 0       # a T=1 sequential step at this batch follows the forward
    forget_bias: float = 3.0

    @property
    def lanes(self) -> int:
        return self.B * self.d_h

    @property
    def state_elems(self) -> int:
        return self.B * self.T * self.d_h


WORKLOADS = [
    Workload("tiny_b2_t64_d16", B=2, T=64, d_in=16, d_h=16, p_dtype="f32", x_dtype="f32",
             forget="exp", max_iters=64, tol=0.0, seed=20260),
    Workload("mid_b8_t1024_d256", B=8, T=1024, d_in=256, d_h=256, p_dtype="f32", x_dtype="f32",
             forget="exp", max_iters=3, tol=0.0, seed=20261),
    Workload("sigmoid_bf16p_b16_t4096_d1024", B=16, T=4096, d_in=1024, d_h=1024, p_dtype="bf16",
             x_dtype="f32", forget="sigmoid", max_iters=8, tol=1e-5, seed=20262),
    Workload("long_b4_t16384_d2048", B=4, T=16384, d_in=2048, d_h=2048, p_dtype="f32",
             x_dtype="f32", forget="exp", max_iters=4, tol=0.0, seed=20263,
             spike_every=512, spike_scale=8.0),
    Workload("layer_b128_t2048_d1024", B=128, T=2048, d_in=1024, d_h=1024, p_dtype="f32",
             x_dtype="bf16", forget="exp", max_iters=3, tol=0.0, seed=20264,
             on_gpu_gemm=True, decode_batch=128),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)
