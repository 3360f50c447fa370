// Kernel (a): Newton residual and 4x4 Jacobian over all (b, t, j) at once.
//
// For every step t = 1..T of every lane (b, j):  rhs_t = f(s_{t-1}) - s_t = -F_t  and
// A_t = df/ds' at s_{t-1}, with the initial state prepended as s_0 ("Layout" page of the
// pararnn-torch docs, "Current surface (0.17)": fused kernels prepend h0; residual F and
// the per-feature 4x4 Jacobian in the scan_block4 layout (B, T, 4, 4, d), "Naming").
// The maximum of |F| over the launch is folded into one device word (NaN counts as +inf).
//
// Mapping: one thread owns one lane and a chunk of CHUNK consecutive steps; consecutive
// threads are consecutive lanes, so every load and store of a wave covers 64 consecutive
// features of one (b, t, plane) row. The previous state of a chunk's first step is the one
// halo read; after that each state is loaded once and reused as the next step's s'.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kResChunk = 16;
constexpr int kResUnroll = 2;
constexpr int kResBlock = 256;

template <bool BF16, bool JAC>
__global__ __launch_bounds__(kResBlock, 4) void residual_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S, float* __restrict__ A, float* __restrict__ rhs, int B, int T,
    int d, int n_chunks, int sig_forget, const Control* __restrict__ ctl,
    unsigned int* __restrict__ err_dst) {
  if (ctl != nullptr && ctl->stopped) return;
  const i64 n_lanes = static_cast<i64>(B) * d;
  const i64 g = static_cast<i64>(blockIdx.x) * kResBlock + threadIdx.x;
  float fmax_local = 0.0f;
  if (g < n_lanes * n_chunks) {
    const i64 lane = g % n_lanes;
    const int ch = static_cast<int>(g / n_lanes);
    const int b = static_cast<int>(lane / d);
    const int j = static_cast<int>(lane % d);
    const int t0 = ch * kResChunk;
    const int t1 = min(T, t0 + kResChunk);
    const float rz = R[j], ri = R[d + j], rf = R[2 * d + j], ro = R[3 * d + j];
    const bool sig = sig_forget != 0;
    const i64 d4 = 4 * static_cast<i64>(d);
    const i64 lane_base = static_cast<i64>(b) * T * d4 + j;  // (b, t=0, slot 0, j)
    CellIn pv;
    if (t0 == 0) {
      if (state0 != nullptr) {
        const float* s0 = state0 + static_cast<i64>(b) * d4 + j;
        pv = {s0[0], s0[d], s0[2 * d], s0[3 * d]};
      } else {
        pv = {0.0f, 0.0f, 0.0f, 0.0f};
      }
    } else {
      const float* sp = S + lane_base + static_cast<i64>(t0 - 1) * d4;
      pv = {sp[0], sp[d], sp[2 * d], sp[3 * d]};
    }
    for (int tb = t0; tb < t1; tb += kResUnroll) {
      float pg[kResUnroll][4], st[kResUnroll][4];
      // issue every load of the group before any arithmetic
#pragma unroll
      for (int u = 0; u < kResUnroll; ++u) {
        const int t = tb + u;
        const i64 base = lane_base + static_cast<i64>(t) * d4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pg[u][k] = (t < t1) ? load_p<BF16>(P, base + k * d) : 0.0f;
          st[u][k] = (t < t1) ? S[base + k * d] : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < kResUnroll; ++u) {
        const int t = tb + u;
        if (t < t1) {
          float f[4], Aj[16];
          cell_step<JAC>(pv, pg[u][0], pg[u][1], pg[u][2], pg[u][3], rz, ri, rf, ro, sig, f, Aj);
          const i64 base = lane_base + static_cast<i64>(t) * d4;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float F = st[u][k] - f[k];
            fmax_local = fmaxf(fmax_local, abs_nan_inf(F));
            if constexpr (JAC) rhs[base + k * d] = -F;
          }
          if constexpr (JAC) {
            float* Ap = A + (static_cast<i64>(b) * T + t) * 16 * static_cast<i64>(d) + j;
#pragma unroll
            for (int e = 0; e < 16; ++e) Ap[static_cast<i64>(e) * d] = Aj[e];
          }
          pv = {st[u][0], st[u][1], st[u][2], st[u][3]};
        }
      }
    }
  }
  // block maximum, then one device-wide atomic per block
  __shared__ float s_max[kResBlock / kWave];
  const float wm = wave_max(fmax_local);
  if ((threadIdx.x & (kWave - 1)) == 0) s_max[threadIdx.x / kWave] = wm;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = s_max[0];
#pragma unroll
    for (int w = 1; w < kResBlock / kWave; ++w) m = fmaxf(m, s_max[w]);
    atomic_max_nonneg(err_dst, m);
  }
}

hipError_t launch_residual(const void* P, bool p_bf16, const float* R, const float* state0,
                           const float* S, float* A, float* rhs, int B, int T, int d,
                           bool sig_forget, const Control* ctl, unsigned int* err_dst,
                           bool with_jacobian, hipStream_t stream) {
  const int n_chunks = (T + kResChunk - 1) / kResChunk;
  const i64 threads = static_cast<i64>(B) * d * n_chunks;
  const i64 blocks = (threads + kResBlock - 1) / kResBlock;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  const int sig = sig_forget ? 1 : 0;
  if (with_jacobian) {
    if (p_bf16)
      residual_kernel<true, true><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, A, rhs, B, T, d,
                                                                  n_chunks, sig, ctl, err_dst);
    else
      residual_kernel<false, true><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, A, rhs, B, T, d,
                                                                   n_chunks, sig, ctl, err_dst);
  } else {
    if (p_bf16)
      residual_kernel<true, false><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, nullptr, nullptr,
                                                                   B, T, d, n_chunks, sig, ctl, err_dst);
    else
      residual_kernel<false, false><<<grid, kResBlock, 0, stream>>>(
          P, R, state0, S, nullptr, nullptr, B, T, d, n_chunks, sig, ctl, err_dst);
  }
  return hipGetLastError();
}

}  // namespace slstm
