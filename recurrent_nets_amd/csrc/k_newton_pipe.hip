// A whole fixed-count Newton solve in one pass over HBM: warm start, K iterations and the
// residual of the final iterate, pipelined along T.
//
// The iterations are those of the chain form (the method of the "Layout" page of the
// pararnn-torch docs, "Current surface (0.17)"; cell of the xLSTM summary card's sLSTM step
// pseudocode, channelwise R): per step t of a lane
//   rhs_t = f(s_{t-1}) - s_t,  A_t = df/ds' at s_{t-1}   (s_0 = state0)
//   Delta_1 = rhs_1,  Delta_t = A_t Delta_{t-1} + rhs_t,  s_t <- s_t + Delta_t,
// with the block-bidiagonal system solved tile by tile as a plain recurrence. Iteration k of a
// tile needs the tile's own iterate S_k, which is in its registers, and the Newton step
// entering the tile, which tile tt-1 publishes as soon as its iteration k is done. So a tile
// runs all K iterations on registers: tile tt works on iteration k while tile tt-1 is already on
// iteration k+1, a wavefront along T. P is read once and only S_K (and h) is written: 36 bytes
// per state element for the whole solve instead of 32 + 48 K + 20 for per-iteration passes.
//
// Published per lane and tile, as epoch-tagged words (see tag_store): the initial iterate at
// the tile's last step (c, n, m, h), and the Newton step of each iteration at the last step.
// The state before a tile in iterate k+1 is that of iterate k plus the published step, formed
// with the same float32 addition the tile before used, so every value is bitwise the one the
// per-iteration chain kernels compute. The initial iterate is the trajectory with the
// recurrent term dropped (warm start, formed here the same way as by the chain warm start) or
// zero.
//
// Waits follow tickets as in the other look-back kernels: a tile waits only on tile tt-1 of
// the same lanes, which holds an earlier ticket of the same counter and never waits on tile
// tt. There is no early stop: the residual maxima of every iterate go to the spread slots, and
// the solver uses this kernel only for a fixed iteration count.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kPipeBlock = 256;  // one feature per thread
#ifndef SLSTM_PIPE_STEPS
#define SLSTM_PIPE_STEPS 14
#endif
#ifndef SLSTM_PIPE_MIN_WAVES
#define SLSTM_PIPE_MIN_WAVES 3
#endif
constexpr int kPipeSteps = SLSTM_PIPE_STEPS;  // steps per tile

__host__ __device__ constexpr int pipe_words(int K) { return 4 + 4 * K; }

template <bool BF16, bool WARM, int CM>
__global__ __launch_bounds__(kPipeBlock, SLSTM_PIPE_MIN_WAVES) void newton_pipe_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    float* __restrict__ S_out, float* __restrict__ h_out, int T, int d, int n_jt, int n_lg,
    int n_tt, int K, unsigned long long* __restrict__ carry,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch, Control* __restrict__ ctl) {
  constexpr int TC = kPipeSteps;
  __shared__ int s_tile[2];
  __shared__ unsigned int s_err[kPipeMaxIters + 1];  // block residual maxima per iterate
  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  if (tid <= kPipeMaxIters) s_err[tid] = 0u;
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;

  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * kPipeBlock + tid);
  const bool valid = j < ud;
  const int t0 = tt * TC;
  const bool publish = valid && tt + 1 < n_tt;  // the tile after waits on these words
  const bool wait = valid && tt > 0;
  const int W = pipe_words(K);
  const i64 n_lanes = static_cast<i64>(n_lg) * kPipeBlock;
  const i64 lane = static_cast<i64>(lg) * kPipeBlock + tid;
  auto word = [&](int tile, int w) { return carry + (static_cast<i64>(tile) * W + w) * n_lanes + lane; };
  auto wait_words = [&](int w0, float v[4]) {
    bool ok = false;
    while (true) {
      ok = tag_load(word(tt - 1, w0), epoch, v[0]) & tag_load(word(tt - 1, w0 + 1), epoch, v[1]) &
           tag_load(word(tt - 1, w0 + 2), epoch, v[2]) & tag_load(word(tt - 1, w0 + 3), epoch, v[3]);
      if (ok) break;
      __builtin_amdgcn_s_sleep(2);
    }
  };
  constexpr bool sig = (CM & kCellSigmoid) != 0;   // forget-gate form and read-out,
  constexpr bool floored = (CM & kCellFloored) != 0;  // fixed per instantiation

  // ---- the tile's pre-activations, held for the whole solve ----
  const i64 tile_row = (static_cast<i64>(b) * T + t0) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  float p[TC][4];
#pragma unroll
  for (int u = 0; u < TC; ++u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) p[u][k] = 0.0f;
    if (valid && t0 + u < T) {
      // lane part j in the vector offset, step and gate parts in the scalar offset
#pragma unroll
      for (int k = 0; k < 4; ++k) p[u][k] = buf_ld_p<BF16>(rsP, j, (4u * u + k) * ud);
    }
  }
  float rz = 0.0f, ri = 0.0f, rf = 0.0f, ro = 0.0f;
  float hv[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // the iterate at step t0 - 1 (state0 before the sequence)
  if (valid) {
    rz = R[j];
    ri = R[ud + j];
    rf = R[2 * ud + j];
    ro = R[3 * ud + j];
    if (tt == 0 && state0 != nullptr) {
      const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
      for (int k = 0; k < 4; ++k) hv[k] = s0[k * ud + j];
    }
  }

  // ---- initial iterate S_0 ----
  float s[TC][4];
  if constexpr (WARM) {
    // gate terms first (they need P only): z, l, i~, sigma(p_o) in the slots of s[u]
#pragma unroll
    for (int u = 0; u < TC; ++u) {
      s[u][0] = tanh_fast(p[u][0]);
      s[u][1] = sig ? log_sigmoidf(p[u][2]) : p[u][2];
      s[u][2] = p[u][1];
      s[u][3] = sigmoidf(p[u][3]);
    }
    if (wait) wait_words(0, hv);
    float c = hv[0], n = hv[1], m = hv[2];
#pragma unroll
    for (int u = 0; u < TC; ++u) {
      const float a = s[u][1] + m;
      const float mn = (a >= s[u][2]) ? a : s[u][2];  // a tie takes a
      const float ig = exp_fast(s[u][2] - mn);
      const float fg = exp_fast(a - mn);
      c = fmaf(fg, c, ig * s[u][0]);
      n = fmaf(fg, n, ig);
      m = mn;
      const float h = s[u][3] * c * readout(n, m, floored).rD;
      s[u][0] = c;
      s[u][1] = n;
      s[u][2] = m;
      s[u][3] = h;
    }
    if (publish) {
#pragma unroll
      for (int e = 0; e < 4; ++e) tag_store(word(tt, e), s[TC - 1][e], epoch);
    }
  } else {
    // zero initial iterate: the state before the tile is zero too, except state0 before t = 0
#pragma unroll
    for (int u = 0; u < TC; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[u][e] = 0.0f;
  }

  // ---- K Newton iterations on the registers ----
  const int l = tid & (kWave - 1);
  for (int k = 0; k < K; ++k) {
    CellIn pv = {hv[0], hv[1], hv[2], hv[3]};
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    unsigned int fmax = 0u;
    if (valid) {
#pragma unroll
      for (int u = 0; u < TC; ++u) {
        const int t = t0 + u;
        if (t < T) {
          float f[4], A[16], r[4];
          cell_step<true>(pv, p[u][0], p[u][1], p[u][2], p[u][3], rz, ri, rf, ro, sig, floored, f, A);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = f[e] - s[u][e];
            fmax = res_max(fmax, r[e]);
          }
          if (u == 0 && wait) {
            // the Newton step entering the tile; the state before the tile in iterate k+1
            wait_words(4 + 4 * k, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = hv[e] + x[e];
          }
          if (t == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = r[e];  // s_0 is data: Delta_1 = rhs_1
          } else {
            const float x0 = fmaf(A[0], x[0], fmaf(A[2], x[2], fmaf(A[3], x[3], r[0])));
            const float x1 = fmaf(A[5], x[1], fmaf(A[6], x[2], fmaf(A[7], x[3], r[1])));
            const float x2 = fmaf(A[10], x[2], fmaf(A[11], x[3], r[2]));
            const float x3 = fmaf(A[12], x[0], fmaf(A[13], x[1], fmaf(A[14], x[2], fmaf(A[15], x[3], r[3]))));
            x[0] = x0;
            x[1] = x1;
            x[2] = x2;
            x[3] = x3;
          }
          pv = {s[u][0], s[u][1], s[u][2], s[u][3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) s[u][e] = s[u][e] + x[e];
        }
      }
      if (publish) {
#pragma unroll
        for (int e = 0; e < 4; ++e) tag_store(word(tt, 4 + 4 * k + e), x[e], epoch);
      }
    }
    const unsigned int wm = wave_max_u32(fmax);
    if (l == 0) __hip_atomic_fetch_max(&s_err[k], wm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // ---- residual of S_K, and the outputs ----
  unsigned int fmax = 0u;
  if (valid) {
    const rsrc_t rsO = make_rsrc(S_out + tile_row);
    const rsrc_t rsH = make_rsrc(h_out != nullptr ? h_out + (static_cast<i64>(b) * T + t0) * static_cast<i64>(d) : S_out);
    CellIn pv = {hv[0], hv[1], hv[2], hv[3]};
#pragma unroll
    for (int u = 0; u < TC; ++u) {
      if (t0 + u < T) {
        float f[4];
        cell_step<false>(pv, p[u][0], p[u][1], p[u][2], p[u][3], rz, ri, rf, ro, sig, floored, f, nullptr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fmax = res_max(fmax, s[u][e] - f[e]);
          buf_st(s[u][e], rsO, 4u * j, 4u * (4u * u + e) * ud);
        }
        if (h_out != nullptr) buf_st(s[u][3], rsH, 4u * j, 4u * u * ud);
        pv = {s[u][0], s[u][1], s[u][2], s[u][3]};
      }
    }
  }
  const unsigned int wm = wave_max_u32(fmax);
  if (l == 0) __hip_atomic_fetch_max(&s_err[K], wm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (tid <= K) err_publish(&spread_of(ctl)->err[0][tid], kErrSlotWords, blockIdx.x, res_max_value(s_err[tid]));
  if (blockIdx.x == 0 && tid == 0) ctl->iters = K;
}

static void pipe_grid(int B, int T, int d, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + kPipeBlock - 1) / kPipeBlock;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + kPipeSteps - 1) / kPipeSteps;
}

size_t pipe_desc_words(int B, int T, int d, int K) {
  i64 n_jt, n_lg, n_tt;
  pipe_grid(B, T, d, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * pipe_words(K) * n_lg * kPipeBlock);
}

hipError_t launch_newton_pipe(const void* P, bool p_bf16, const float* R, const float* state0,
                              float* S_out, float* h_out, int B, int T, int d, int cell_mode,
                              bool warm, int K, unsigned long long* carry, unsigned int* tickets,
                              uint32_t epoch, Control* ctl, hipStream_t stream) {
  i64 n_jt, n_lg, n_tt;
  pipe_grid(B, T, d, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL || K < 1 || K > kPipeMaxIters) return hipErrorInvalidValue;
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int a = static_cast<int>(n_jt), c = static_cast<int>(n_lg), e = static_cast<int>(n_tt);
#define SLSTM_PIPE_LAUNCH(BF, WM, CM_)                                                                   \
  newton_pipe_kernel<BF, WM, CM_><<<grid, kPipeBlock, 0, stream>>>(P, R, state0, S_out, h_out, T, d, a, \
                                                                   c, e, K, carry, tickets, n_ctr,      \
                                                                   epoch, ctl)
#define SLSTM_PIPE_TT(CM_) SLSTM_PIPE_LAUNCH(true, true, CM_)
#define SLSTM_PIPE_TF(CM_) SLSTM_PIPE_LAUNCH(true, false, CM_)
#define SLSTM_PIPE_FT(CM_) SLSTM_PIPE_LAUNCH(false, true, CM_)
#define SLSTM_PIPE_FF(CM_) SLSTM_PIPE_LAUNCH(false, false, CM_)
  if (p_bf16) {
    if (warm) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_PIPE_TT) }
    else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_PIPE_TF) }
  } else {
    if (warm) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_PIPE_FT) }
    else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_PIPE_FF) }
  }
#undef SLSTM_PIPE_TT
#undef SLSTM_PIPE_TF
#undef SLSTM_PIPE_FT
#undef SLSTM_PIPE_FF
#undef SLSTM_PIPE_LAUNCH
  return hipGetLastError();
}

}  // namespace slstm
