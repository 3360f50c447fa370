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
// Mapping: grid (feature tiles of 64 VEC, groups of 4 time chunks, batch). Each wave owns 64 VEC
// consecutive features of one batch row (VEC = 1 or 2 per thread) and one chunk of kResChunk
// consecutive steps, so (b, t) are wave-uniform and every load or store of a wave covers
// 256 VEC contiguous bytes of one (b, t, plane) row. The
// previous state of a chunk's first step is the one halo read; after that each state is
// loaded once and reused as the next step's s'.
#include <algorithm>

#include "cell.h"
#include "kernels.h"

namespace slstm {

// 8-step chunks and non-temporal stores of the Jacobian and right-hand side (written once,
// read once by the scan) measured fastest on MI355X: 5.01 ms against 5.27 for 16-step chunks and
// plain stores at B = 128, T = 2048, d_h = 1024 (4.9 against 4.7 TB/s of algorithmic traffic).
#ifndef SLSTM_RES_CHUNK
#define SLSTM_RES_CHUNK 8
#endif
#ifndef SLSTM_RES_NT
#define SLSTM_RES_NT 1
#endif
constexpr int kResChunk = SLSTM_RES_CHUNK;
constexpr int kResWaves = 4;
constexpr int kResBlock = kResWaves * kWave;

enum { kJacNone = 0, kJacSparse = 1, kJacDense = 2 };

// row-major 4x4 positions written in the sparse form (all but the four structural zeros)
__device__ constexpr int kSparsePlanes[12] = {0, 2, 3, 5, 6, 7, 10, 11, 12, 13, 14, 15};

// VEC consecutive features per thread (1 or 2): with 2, every load and store of a wave covers
// 512 contiguous bytes, which streams about 7% faster on MI355X than 256; used when d_h is even
// and every row starts 8-byte aligned.
template <bool BF16, int VEC>
__device__ __forceinline__ void load_p_vec(const void* __restrict__ P, i64 idx, float (&out)[VEC]) {
  if constexpr (VEC == 1) {
    out[0] = load_p<BF16>(P, idx);
  } else if constexpr (BF16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(P) + idx);
    out[0] = bf16_to_f32(static_cast<uint16_t>(w & 0xffffu));
    out[1] = bf16_to_f32(static_cast<uint16_t>(w >> 16));
  } else {
    const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(P) + idx);
    out[0] = v.x;
    out[1] = v.y;
  }
}

template <int VEC>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&out)[VEC]) {
  if constexpr (VEC == 1) {
    out[0] = *p;
  } else {
    const float2 v = *reinterpret_cast<const float2*>(p);
    out[0] = v.x;
    out[1] = v.y;
  }
}

template <int VEC>
__device__ __forceinline__ void store_vec(float* __restrict__ p, const float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    if (SLSTM_RES_NT) __builtin_nontemporal_store(v[0], p);
    else *p = v[0];
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 w;
    w[0] = v[0];
    w[1] = v[1];
    if (SLSTM_RES_NT) __builtin_nontemporal_store(w, reinterpret_cast<f32x2*>(p));
    else *reinterpret_cast<f32x2*>(p) = w;
  }
}

template <bool BF16, int JMODE, int VEC>
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
  // the thread's features j0 .. j0 + VEC - 1 (d is a multiple of VEC)
  const unsigned j0 = (blockIdx.x * kWave + l) * VEC;
  float fmax_local = 0.0f;
  // groups of kResWaves chunks, strided over the grid's y extent (which the hardware caps)
  for (int cg = blockIdx.y; cg * kResWaves < n_chunks; cg += gridDim.y) {
    const int chunk = cg * kResWaves + wave;
    if (chunk < n_chunks && j0 < static_cast<unsigned>(d)) {
      const unsigned ud = static_cast<unsigned>(d);
      const int t0 = chunk * kResChunk;
      const int t1 = min(T, t0 + kResChunk);
      float rz[VEC], ri[VEC], rf[VEC], ro[VEC];
      load_vec<VEC>(R + j0, rz);
      load_vec<VEC>(R + ud + j0, ri);
      load_vec<VEC>(R + 2 * ud + j0, rf);
      load_vec<VEC>(R + 3 * ud + j0, ro);
      const bool sig = (cell_mode & kCellSigmoid) != 0;
      const bool floored = (cell_mode & kCellFloored) != 0;
      const i64 row4 = 4 * static_cast<i64>(d);  // floats per (b, t) row of a state tensor
      const float* Sb = S + static_cast<i64>(b) * T * row4;
      CellIn pv[VEC];
  #pragma unroll
      for (int v = 0; v < VEC; ++v) pv[v] = {0.0f, 0.0f, 0.0f, 0.0f};  // a sequence start replaces it below
      if (t0 > 0) {
        const float* sp = Sb + static_cast<i64>(t0 - 1) * row4;
        float sc[4][VEC];
  #pragma unroll
        for (int k = 0; k < 4; ++k) load_vec<VEC>(sp + k * ud + j0, sc[k]);
  #pragma unroll
        for (int v = 0; v < VEC; ++v) pv[v] = {sc[0][v], sc[1][v], sc[2][v], sc[3][v]};
      }
      SeqCursor seq = seq_cursor(cu, n_seqs, b, t0, seq_tab);
      // next step's operands are loaded one step ahead
      float pn[4][VEC], sn[4][VEC];
      auto load_step = [&](int t, float (&pg)[4][VEC], float (&st)[4][VEC]) {
        const i64 row = static_cast<i64>(b) * T + t;
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          load_p_vec<BF16, VEC>(P, row * row4 + k * ud + j0, pg[k]);
          load_vec<VEC>(Sb + static_cast<i64>(t) * row4 + k * ud + j0, st[k]);
        }
      };
      load_step(t0, pn, sn);
      for (int t = t0; t < t1; ++t) {
        float pg[4][VEC], st[4][VEC];
  #pragma unroll
        for (int k = 0; k < 4; ++k)
  #pragma unroll
          for (int v = 0; v < VEC; ++v) {
            pg[k][v] = pn[k][v];
            st[k][v] = sn[k][v];
          }
        if (t + 1 < t1) load_step(t + 1, pn, sn);
        const int sq = seq_begin(seq, t);
        // packed: the step after a sequence boundary does not depend on the state before it
        const bool cut = cu != nullptr && sq >= 0;
        float rr[4][VEC], Aj[16][VEC];
  #pragma unroll
        for (int v = 0; v < VEC; ++v) {
          if (sq >= 0) pv[v] = state0_of(state0, sq, ud, j0 + v);
          float f[4], Av[16];
          cell_step<JMODE != kJacNone>(pv[v], pg[0][v], pg[1][v], pg[2][v], pg[3][v], rz[v], ri[v], rf[v], ro[v],
                                       sig, floored, f, Av);
  #pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float F = st[k][v] - f[k];
            fmax_local = fmaxf(fmax_local, abs_nan_inf(F));
            rr[k][v] = -F;
          }
          if constexpr (JMODE != kJacNone) {
  #pragma unroll
            for (int e = 0; e < 16; ++e) Aj[e][v] = cut ? 0.0f : Av[e];
          }
          pv[v] = {st[0][v], st[1][v], st[2][v], st[3][v]};
        }
        const i64 row = static_cast<i64>(b) * T + t;
        if constexpr (JMODE != kJacNone) {
  #pragma unroll
          for (int k = 0; k < 4; ++k) store_vec<VEC>(rhs + row * row4 + k * ud + j0, rr[k]);
        }
        if constexpr (JMODE == kJacDense) {
          float* Ap = A + row * 16 * static_cast<i64>(d);
  #pragma unroll
          for (int e = 0; e < 16; ++e) store_vec<VEC>(Ap + e * ud + j0, Aj[e]);
        } else if constexpr (JMODE == kJacSparse) {
          float* Ap = A + row * 16 * static_cast<i64>(d);
  #pragma unroll
          for (int q = 0; q < 12; ++q) store_vec<VEC>(Ap + kSparsePlanes[q] * ud + j0, Aj[kSparsePlanes[q]]);
        }
        if (h_out != nullptr) store_vec<VEC>(h_out + row * static_cast<i64>(d) + j0, st[3]);
      }
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

template <bool BF16, int VEC>
static void launch_mode(int mode, dim3 grid, hipStream_t stream, const void* P, const float* R,
                        const float* state0, const float* S, float* A, float* rhs, int T, int d,
                        int n_chunks, int sig, Control* ctl, unsigned int* err_base, int err_stride,
                        int chk, float tol, float* h_out, Seqs seqs) {
  if (mode == kJacDense)
    residual_kernel<BF16, kJacDense, VEC><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, A, rhs, T, d,
                                                                           n_chunks, sig, ctl, err_base, err_stride, chk, tol, h_out,
                                                                           seqs.cu, seqs.n, seqs.tab);
  else if (mode == kJacSparse)
    residual_kernel<BF16, kJacSparse, VEC><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, A, rhs, T, d,
                                                                            n_chunks, sig, ctl, err_base, err_stride, chk, tol, h_out,
                                                                            seqs.cu, seqs.n, seqs.tab);
  else
    residual_kernel<BF16, kJacNone, VEC><<<grid, kResBlock, 0, stream>>>(P, R, state0, S, nullptr, nullptr,
                                                                          T, d, n_chunks, sig, ctl, err_base, err_stride, chk, tol, h_out,
                                                                          seqs.cu, seqs.n, seqs.tab);
}

hipError_t launch_residual(const void* P, bool p_bf16, const float* R, const float* state0,
                           const float* S, float* A, float* rhs, int B, int T, int d,
                           int cell_mode, Control* ctl, unsigned int* err_base, int err_stride,
                           ResidualMode mode, int stop_check_iter, float tol, hipStream_t stream,
                           float* h_out, Seqs seqs) {
  const int n_chunks = (T + kResChunk - 1) / kResChunk;
  // two features per thread when every row of every tensor starts 8-byte aligned
  const bool vec2 = d % 2 == 0 && (reinterpret_cast<uintptr_t>(P) % (p_bf16 ? 4 : 8)) == 0 &&
                    (reinterpret_cast<uintptr_t>(R) % 8) == 0 && (reinterpret_cast<uintptr_t>(S) % 8) == 0 &&
                    (reinterpret_cast<uintptr_t>(A) % 8) == 0 && (reinterpret_cast<uintptr_t>(rhs) % 8) == 0 &&
                    (reinterpret_cast<uintptr_t>(h_out) % 8) == 0;
  const int per_block = kWave * (vec2 ? 2 : 1);
  const unsigned gx = static_cast<unsigned>((d + per_block - 1) / per_block);
  const unsigned gy = static_cast<unsigned>(std::min((n_chunks + kResWaves - 1) / kResWaves, 65535));
  if (B > 65535) return hipErrorInvalidValue;
  const dim3 grid(gx, gy, static_cast<unsigned>(B));
  const int sig = cell_mode;
  const int m = mode == ResidualMode::kDense ? kJacDense : (mode == ResidualMode::kSparse ? kJacSparse : kJacNone);
  if (p_bf16) {
    if (vec2)
      launch_mode<true, 2>(m, grid, stream, P, R, state0, S, A, rhs, T, d, n_chunks, sig, ctl, err_base, err_stride,
                           stop_check_iter, tol, h_out, seqs);
    else
      launch_mode<true, 1>(m, grid, stream, P, R, state0, S, A, rhs, T, d, n_chunks, sig, ctl, err_base, err_stride,
                           stop_check_iter, tol, h_out, seqs);
  } else {
    if (vec2)
      launch_mode<false, 2>(m, grid, stream, P, R, state0, S, A, rhs, T, d, n_chunks, sig, ctl, err_base, err_stride,
                            stop_check_iter, tol, h_out, seqs);
    else
      launch_mode<false, 1>(m, grid, stream, P, R, state0, S, A, rhs, T, d, n_chunks, sig, ctl, err_base, err_stride,
                            stop_check_iter, tol, h_out, seqs);
  }
  return hipGetLastError();
}

}  // namespace slstm
