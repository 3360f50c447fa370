// Kernel (a): Newton residual and 4x4 Jacobian over all (b, t, j) at once.
//
// For every step t = 1..T of every lane (b, j):  rhs_t = f(s_{t-1}) - s_t = -F_t  and
// A_t = df/ds' at s_{t-1}, with the initial state prepended as s_0 ("Layout" page of the
// pararnn-torch docs, "Current surface (0.17)": fused kernels prepend h0; residual F and
// the per-feature 4x4 Jacobian in the scan_block4 layout (B, T, 4, 4, d), "Naming").
// The maximum of |F| over the launch is folded into one device word (NaN counts as +inf).
//
// Jacobian planes written:
//   kJacDense   all 16 planes of each 4x4 block;
//   kJacSparse  the 12 planes that are not structural zeros of the channelwise cell
//               ((c, n'), (n, c'), (m, c'), (m, n') are never written); the Newton solver's
//               scan reads exactly these;
//   kJacNone    no Jacobian and no right-hand side: the residual maximum only (the pass over
//               the final iterate, which also writes the hidden slot out when asked).
//
// Mapping: grid (feature tiles of 64, groups of 4 time chunks, batch). Each wave owns 64
// consecutive features of one batch row and one chunk of kResChunk consecutive steps, so
// (b, t) are wave-uniform: every access is a scalar row base plus a 32-bit lane offset, and
// every load or store of a wave covers 256 contiguous bytes of one (b, t, plane) row. The
// previous state of a chunk's first step is the one halo read; after that each state is
// loaded once and reused as the next step's s'.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kResChunk = 16;
constexpr int kResWaves = 4;
constexpr int kResBlock = kResWaves * kWave;

enum { kJacNone = 0, kJacSparse = 1, kJacDense = 2 };

// row-major 4x4 positions written in the sparse form (all but the four structural zeros)
__device__ constexpr int kSparsePlanes[12] = {0, 2, 3, 5, 6, 7, 10, 11, 12, 13, 14, 15};

template <bool BF16, int JMODE>
__global__ __launch_bounds__(kResBlock, 2) void residual_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S, float* __restrict__ A, float* __restrict__ rhs, int T, int d,
    int n_chunks, int cell_mode, Control* __restrict__ ctl, unsigned int* __restrict__ err_base,
    int err_stride, int stop_check_iter, float tol, float* __restrict__ h_out,
    const int* __restrict__ cu, int n_seqs,
    const int* __restrict__ seq_tab) {
  if (ctl != nullptr) {
    if (ctl->stopped) return;
    if (stop_check_iter >= 0 && tol > 0.0f && err_reduced(ctl, stop_check_iter) < tol) {
      if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
        ctl->stopped = 1;
        ctl->iters = stop_check_iter;
      }
      return;
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & (kWave - 1);
  const int b = blockIdx.z;
  const int chunk = blockIdx.y * kResWaves + wave;
  const unsigned j = blockIdx.x * kWave + l;
  float fmax_local = 0.0f;
  if (chunk < n_chunks && j < static_cast<unsigned>(d)) {
    const unsigned ud = static_cast<unsigned>(d);
    const int t0 = chunk * kResChunk;
    const int t1 = min(T, t0 + kResChunk);
    const float rz = R[j], ri = R[ud + j], rf = R[2 * ud + j], ro = R[3 * ud + j];
    const bool sig = (cell_mode & kCellSigmoid) != 0;
    const bool floored = (cell_mode & kCellFloored) != 0;
    const i64 row4 = 4 * static_cast<i64>(d);  // floats per (b, t) row of a state tensor
    const float* Sb = S + static_cast<i64>(b) * T * row4;
    CellIn pv = {0.0f, 0.0f, 0.0f, 0.0f};  // a sequence start replaces it below
    if (t0 > 0) {
      const float* sp = Sb + static_cast<i64>(t0 - 1) * row4;
      pv = {sp[j], sp[ud + j], sp[2 * ud + j], sp[3 * ud + j]};
    }
    SeqCursor seq = seq_cursor(cu, n_seqs, b, t0, seq_tab);
    // next step's operands are loaded one step ahead
    float pn[4], sn[4];
    auto load_step = [&](int t, float (&pg)[4], float (&st)[4]) {
      const i64 row = static_cast<i64>(b) * T + t;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[k] = load_p<BF16>(P, row * row4 + k * ud + j);
        st[k] = Sb[static_cast<i64>(t) * row4 + k * ud + j];
      }
    };
    load_step(t0, pn, sn);
    for (int t = t0; t < t1; ++t) {
      float pg[4], st[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[k] = pn[k];
        st[k] = sn[k];
      }
      if (t + 1 < t1) load_step(t + 1, pn, sn);
      const int sq = seq_begin(seq, t);
      if (sq >= 0) pv = state0_of(state0, sq, ud, j);
      // packed: the step after a sequence boundary does not depend on the state before it
      const bool cut = cu != nullptr && sq >= 0;
      float f[4], Aj[16];
      cell_step<JMODE != kJacNone>(pv, pg[0], pg[1], pg[2], pg[3], rz, ri, rf, ro, sig, floored, f, Aj);
      const i64 row = static_cast<i64>(b) * T + t;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float F = st[k] - f[k];
        fmax_local = fmaxf(fmax_local, abs_nan_inf(F));
        if constexpr (JMODE != kJacNone) rhs[row * row4 + k * ud + j] = -F;
      }
      if constexpr (JMODE == kJacDense) {
        float* Ap = A + row * 16 * static_cast<i64>(d);
#pragma unroll
        for (int e = 0; e < 16; ++e) Ap[e * ud + j] = cut ? 0.0f : Aj[e];
      } else if constexpr (JMODE == kJacSparse) {
        float* Ap = A + row * 16 * static_cast<i64>(d);
#pragma unroll
        for (int q = 0; q < 12; ++q) Ap[kSparsePlanes[q] * ud + j] = cut ? 0.0f : Aj[kSparsePlanes[q]];
      }
      if (h_out != nullptr) h_out[row * static_cast<i64>(d) + j] = st[3];
      pv = {st[0], st[1], st[2], st[3]};
    }
  }
  // block maximum, then one device-wide atomic per block, into a slot of its own
  __shared__ float s_max[kResWaves];
  const float wm = wave_max(fmax_local);
  if (l == 0) s_max[wave] = wm;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = s_max[0];
#pragma unroll
    for (int w = 1; w < kResWaves; ++w) m = fmaxf(m, s_max[w]);
    err_publish(err_base, err_stride, blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), m);
  }
}

template <bool BF16>
static void launch_mode(int mode, dim3 grid, hipStream_t stream, const void* P, const float* R,
                        const float* state0, const float* S, float* A, float* rhs, int T, int d,
                        int n_chunks, int sig, Control* ctl, unsigned int* err_base, int err_stride,
                        int chk, float tol, float* h_out, Seqs seqs) {
  if (mode == kJacDense)
    residual_kernel<BF16, kJacDense><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, A, rhs, T, d,
                                                                      n_chunks, sig, ctl, err_base, err_stride, chk, tol, h_out,
                                                                      seqs.cu, seqs.n, seqs.tab);
  else if (mode == kJacSparse)
    residual_kernel<BF16, kJacSparse><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, A, rhs, T, d,
                                                                       n_chunks, sig, ctl, err_base, err_stride, chk, tol, h_out,
                                                                       seqs.cu, seqs.n, seqs.tab);
  else
    residual_kernel<BF16, kJacNone><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, nullptr, nullptr,
                                                                     T, d, n_chunks, sig, ctl, err_base, err_stride, chk, tol, h_out,
                                                                     seqs.cu, seqs.n, seqs.tab);
}

hipError_t launch_residual(const void* P, bool p_bf16, const float* R, const float* state0,
                           const float* S, float* A, float* rhs, int B, int T, int d,
                           int cell_mode, Control* ctl, unsigned int* err_base, int err_stride,
                           ResidualMode mode, int stop_check_iter, float tol, hipStream_t stream,
                           float* h_out, Seqs seqs) {
  const int n_chunks = (T + kResChunk - 1) / kResChunk;
  const unsigned gx = static_cast<unsigned>((d + kWave - 1) / kWave);
  const unsigned gy = static_cast<unsigned>((n_chunks + kResWaves - 1) / kResWaves);
  if (B > 65535 || gy > 65535u) return hipErrorInvalidValue;
  const dim3 grid(gx, gy, static_cast<unsigned>(B));
  const int sig = cell_mode;
  const int m = mode == ResidualMode::kDense ? kJacDense : (mode == ResidualMode::kSparse ? kJacSparse : kJacNone);
  if (p_bf16)
    launch_mode<true>(m, grid, stream, P, R, state0, S, A, rhs, T, d, n_chunks, sig, ctl, err_base, err_stride,
                      stop_check_iter, tol, h_out, seqs);
  else
    launch_mode<false>(m, grid, stream, P, R, state0, S, A, rhs, T, d, n_chunks, sig, ctl, err_base, err_stride,
                       stop_check_iter, tol, h_out, seqs);
  return hipGetLastError();
}

}  // namespace slstm
