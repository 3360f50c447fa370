// Head mixing (mix='head'): block-diagonal recurrent matrices, one (d_head x d_head) block per
// head and gate ("sLSTM in this library", section "Cell": the mix table's 'head' row; the
// paper's sLSTM mixes memory through recurrent matrices from h' to every gate, block-diagonal
// per head -- summary card, "Method" item 2 and the one-head step pseudocode under "Key
// equations"). Unit i of head a (feature j = a d_head + i) has the pre-activations
//   x~_g = p_g + sum_k R[g, a, i, k] h'[a d_head + k]        (g = z, i, f, o).
//
// Two kernels, each with one workgroup per (batch row, head) walking T step by step, and one
// thread per (unit, gate): lane 4 i + g holds row i of gate g's block in registers, so the
// block's products are d_head FMAs per lane and step. The head's h (and Delta h) pass from step
// to step through double-buffered LDS; the four lanes of a unit exchange gate values by DPP.
//
// head_seq_kernel: the sequential forward (and the T = 1 decode step).
// head_iter_kernel: one Newton iteration. Residual F_t = s_t - f(s_{t-1}) at the iterate and
//   the linear solve Delta_t = A_t Delta_{t-1} - F_t with the Jacobian applied in factored form,
//     A_t Delta = A_own (Delta c', Delta n', Delta m') + G (R_g Delta h')_g
//   (A_own the unit's own-state columns, G = d s / d x~ the gate Jacobian; see cell_step_lin):
//   the (4 d_head)^2 block is never formed, and the block product costs d_head FMAs per lane.
//   The solve is a recurrence along T for each (batch row, head), like the chain form of the
//   channelwise solver; the iterates are those of the oracle's dense block forward
//   substitution up to float32 rounding. LAST also forms the residual of the new iterate and h.
//
// Per-step operands are prefetched kHeadPrefetch steps ahead; the barrier between steps orders
// LDS only, so those loads stay in flight across it.
#include "cell.h"
#include "head.h"
#include "kernels.h"

namespace slstm {

// Packed sequences (PACKED, one batch row): at the first step of sequence s the state before
// it is state0[s]; the workgroup stages that state's h for the block product behind an extra
// barrier (at sequence starts only) and walks the offsets with a SeqCursor.
template <int DH, bool BF16, int CM, bool PACKED>
__global__ __launch_bounds__(4 * DH) void head_seq_kernel(const void* __restrict__ P, const float* __restrict__ R,
                                                          const float* __restrict__ state0, float* __restrict__ S,
                                                          float* __restrict__ h_out, float* __restrict__ final_state,
                                                          int T, int d, int nh, Seqs seqs) {
  constexpr bool sig = (CM & kCellSigmoid) != 0;
  constexpr bool floored = (CM & kCellFloored) != 0;
  __shared__ __attribute__((aligned(16))) float hbuf[2][DH];
  const int tid = threadIdx.x;
  const int i = tid >> 2, g = tid & 3;
  const int a = blockIdx.x, b = blockIdx.y;
  const int j = a * DH + i;
  const i64 dd = d;
  const GateSel sel(g);
  float row[DH];
  load_block_row<DH>(R, nh, a, i, g, row);
  // previous state of the unit, slot g in this lane
  float prev = state0 != nullptr ? state0[(static_cast<i64>(b) * 4 + g) * dd + j] : 0.0f;
  if (g == 3) hbuf[0][i] = prev;
  const i64 base = static_cast<i64>(b) * T * 4 * dd + g * dd + j;  // (b, t = 0, slot/gate g, j)
  // ring of the next kHeadPrefetch steps' pre-activations; loads past the end re-read step T-1
  float pr[kHeadPrefetch];
#pragma unroll
  for (int u = 0; u < kHeadPrefetch; ++u) pr[u] = load_p<BF16>(P, base + static_cast<i64>(min(u, T - 1)) * 4 * dd);
  head_lds_barrier();
  SeqCursor cur = seq_cursor(seqs.cu, seqs.n, 0, 0, seqs.tab);
  auto step = [&](int t, float p) {
    if constexpr (PACKED) {
      const int sq = seq_begin(cur, t);
      if (sq >= 0) {  // a sequence start (uniform): the state before it is state0[sq]
        prev = state0 != nullptr ? state0[(static_cast<i64>(sq) * 4 + g) * dd + j] : 0.0f;
        if (g == 3) hbuf[t & 1][i] = prev;
        head_lds_barrier();
      }
    }
    const float x = p + block_dot<DH>(row, hbuf[t & 1]);
    float xs[4], ps[4];
    quad_gather(x, xs);
    quad_gather(prev, ps);
    float s[4], A[16];
    cell_step<false>(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs[0], xs[1], xs[2], xs[3], 0.0f, 0.0f, 0.0f, 0.0f, sig,
                     floored, s, A);
    const float v = sel(s);
    S[base + static_cast<i64>(t) * 4 * dd] = v;
    if (g == 3) {
      hbuf[(t + 1) & 1][i] = v;
      if (h_out != nullptr) h_out[(static_cast<i64>(b) * T + t) * dd + j] = v;
    }
    prev = v;
    head_lds_barrier();
  };
  // whole blocks of kHeadPrefetch steps: every ring slot is refilled unconditionally, so no
  // load has to complete before the step kHeadPrefetch later that reads it
  int t0 = 0;
  for (; t0 + kHeadPrefetch <= T; t0 += kHeadPrefetch) {
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) {
      const int t = t0 + u;
      const float p = pr[u];
      pr[u] = load_p<BF16>(P, base + static_cast<i64>(min(t + kHeadPrefetch, T - 1)) * 4 * dd);
      step(t, p);
    }
  }
  // the last T mod kHeadPrefetch steps, whose operands are in the ring
#pragma unroll
  for (int u = 0; u < kHeadPrefetch - 1; ++u)
    if (t0 + u < T) step(t0 + u, pr[u]);
  if (!PACKED && final_state != nullptr) final_state[(static_cast<i64>(b) * 4 + g) * dd + j] = prev;
}

// The residual maximum of iterate k - 1 over the spread slots (read serially by one thread;
// the workgroup may be less than a wave)
__device__ __forceinline__ float head_err_prev(const Control* ctl, int k, float* s_tmp) {
  if (threadIdx.x == 0) {
    float m = 0.0f;
    for (int q = 0; q < kSpreadSlots; ++q) m = fmaxf(m, __uint_as_float(spread_of(ctl)->err[q][k]));
    *s_tmp = m;
  }
  __syncthreads();
  return *s_tmp;
}

template <int DH, bool BF16, int CM, bool LAST, bool PACKED>
__global__ __launch_bounds__(4 * DH) void head_iter_kernel(const void* __restrict__ P, const float* __restrict__ R,
                                                           const float* __restrict__ state0,
                                                           const float* __restrict__ S_in, float* __restrict__ S_out,
                                                           float* __restrict__ h_out, int T, int d, int nh,
                                                           Control* __restrict__ ctl, int k_iter, float tol,
                                                           Seqs seqs) {
  constexpr bool sig = (CM & kCellSigmoid) != 0;
  constexpr bool floored = (CM & kCellFloored) != 0;
  __shared__ __attribute__((aligned(16))) float hbuf[2][DH];   // h of the iterate at t - 1
  __shared__ __attribute__((aligned(16))) float dhbuf[2][DH];  // Delta h at t - 1
  __shared__ unsigned int s_err[2];
  __shared__ float s_tmp;
  if (ctl->stopped) return;
  if (k_iter > 0 && tol > 0.0f) {
    if (head_err_prev(ctl, k_iter - 1, &s_tmp) < tol) {
      // the previous iterate already met the tolerance: it is the result
      if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        ctl->stopped = 1;
        ctl->iters = k_iter - 1;
      }
      return;
    }
  }
  const int tid = threadIdx.x;
  const int i = tid >> 2, g = tid & 3;
  const int a = blockIdx.x, b = blockIdx.y;
  const int j = a * DH + i;
  const i64 dd = d;
  if (tid == 0) {
    s_err[0] = 0u;
    s_err[1] = 0u;
  }
  const GateSel sel(g);
  float row[DH];
  load_block_row<DH>(R, nh, a, i, g, row);
  float prev = state0 != nullptr ? state0[(static_cast<i64>(b) * 4 + g) * dd + j] : 0.0f;  // iterate at t-1
  float dprev = 0.0f;                                                                        // Delta at t-1
  if (g == 3) {
    hbuf[0][i] = prev;
    dhbuf[0][i] = 0.0f;
  }
  const i64 base = static_cast<i64>(b) * T * 4 * dd + g * dd + j;
  // rings of the next kHeadPrefetch steps' operands; loads past the end re-read step T-1
  float pr[kHeadPrefetch], sr[kHeadPrefetch];
#pragma unroll
  for (int u = 0; u < kHeadPrefetch; ++u) {
    const i64 off = base + static_cast<i64>(min(u, T - 1)) * 4 * dd;
    pr[u] = load_p<BF16>(P, off);
    sr[u] = S_in[off];
  }
  unsigned int emax = 0u, emax_new = 0u;
  head_lds_barrier();
  SeqCursor cur = seq_cursor(seqs.cu, seqs.n, 0, 0, seqs.tab);
  auto step = [&](int t, float p, float sin) {
    if constexpr (PACKED) {
      const int sq = seq_begin(cur, t);
      if (sq >= 0) {  // a sequence start: state0[sq] before it, a zero Jacobian (no Delta enters)
        prev = state0 != nullptr ? state0[(static_cast<i64>(sq) * 4 + g) * dd + j] : 0.0f;
        dprev = 0.0f;
        if (g == 3) {
          hbuf[t & 1][i] = prev;
          dhbuf[t & 1][i] = 0.0f;
        }
        head_lds_barrier();
      }
    }
    // residual and factors at the iterate (independent of the solve)
    const float x = p + block_dot<DH>(row, hbuf[t & 1]);
    float xs[4], ps[4];
    quad_gather(x, xs);
    quad_gather(prev, ps);
    float s[4];
    CellLin L;
    cell_step_lin(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs, sig, floored, s, L);
    const float sg = sel(s);
    const float F = sin - sg;
    emax = res_max(emax, F);
    // the solve: Delta_t = A_own Delta_{t-1} + G (R Delta h_{t-1}) - F
    const float y = block_dot<DH>(row, dhbuf[t & 1]);
    float ys[4], ds[4];
    quad_gather(y, ys);
    quad_gather(dprev, ds);
    // slot g of A_own Delta' + G (R Delta h')
    float dv[4];
    cell_jvp(L, ds, ys, dv);
    const float delta = sel(dv) - F;
    const float sout = sin + delta;
    S_out[base + static_cast<i64>(t) * 4 * dd] = sout;
    if constexpr (LAST) {
      // residual of the new iterate: its pre-activations are x~ + R Delta h'
      float sn[4], An[16];
      cell_step<false>(CellIn{ps[0] + ds[0], ps[1] + ds[1], ps[2] + ds[2], 0.0f}, xs[0] + ys[0], xs[1] + ys[1],
                       xs[2] + ys[2], xs[3] + ys[3], 0.0f, 0.0f, 0.0f, 0.0f, sig, floored, sn, An);
      const float sng = sel(sn);
      emax_new = res_max(emax_new, sout - sng);
      if (g == 3 && h_out != nullptr) h_out[(static_cast<i64>(b) * T + t) * dd + j] = sout;
    }
    if (g == 3) {
      hbuf[(t + 1) & 1][i] = sin;
      dhbuf[(t + 1) & 1][i] = delta;
    }
    prev = sin;
    dprev = delta;
    head_lds_barrier();
  };
  // whole blocks of kHeadPrefetch steps with unconditional ring refills (see head_seq_kernel)
  int t0 = 0;
  for (; t0 + kHeadPrefetch <= T; t0 += kHeadPrefetch) {
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) {
      const int t = t0 + u;
      const float p = pr[u], sin = sr[u];
      const i64 off = base + static_cast<i64>(min(t + kHeadPrefetch, T - 1)) * 4 * dd;
      pr[u] = load_p<BF16>(P, off);
      sr[u] = S_in[off];
      step(t, p, sin);
    }
  }
#pragma unroll
  for (int u = 0; u < kHeadPrefetch - 1; ++u)
    if (t0 + u < T) step(t0 + u, pr[u], sr[u]);
  // residual maxima: the workgroup's into LDS, then one device atomic per slot
  __hip_atomic_fetch_max(&s_err[0], emax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (LAST) __hip_atomic_fetch_max(&s_err[1], emax_new, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (tid == 0) {
    const unsigned int slot = blockIdx.x + gridDim.x * blockIdx.y;
    err_publish(&spread_of(ctl)->err[0][k_iter], kErrSlotWords, slot, res_max_value(s_err[0]));
    if (LAST) err_publish(&spread_of(ctl)->err[0][k_iter + 1], kErrSlotWords, slot, res_max_value(s_err[1]));
    if (blockIdx.x == 0 && blockIdx.y == 0) ctl->iters = k_iter + 1;
  }
}

bool head_width_supported(int d_head) {
  return d_head == 8 || d_head == 16 || d_head == 32 || d_head == 64 || d_head == 128;
}

hipError_t launch_head_sequential(const void* P, bool p_bf16, const float* R, const float* state0, float* S,
                                  float* h_out, float* final_state, int B, int T, int d, int n_heads,
                                  int cell_mode, hipStream_t stream, Seqs seqs) {
  if (n_heads < 1 || d % n_heads != 0 || B > 65535) return hipErrorInvalidValue;
  const int dh = d / n_heads;
  const dim3 grid(static_cast<unsigned>(n_heads), static_cast<unsigned>(B));
  const unsigned int lds = head_spread_lds(static_cast<long long>(n_heads) * B, 4096);
  const bool packed = seqs.cu != nullptr;
#define SLSTM_HEAD_SEQ(BF, CM_)                                                                              \
  do {                                                                                                       \
    if (packed)                                                                                              \
      head_seq_kernel<DH, BF, CM_, true><<<grid, 4 * DH, lds, stream>>>(P, R, state0, S, h_out, final_state, T, d, \
                                                                        n_heads, seqs);                      \
    else                                                                                                     \
      head_seq_kernel<DH, BF, CM_, false><<<grid, 4 * DH, lds, stream>>>(P, R, state0, S, h_out, final_state, T, \
                                                                         d, n_heads, seqs);                  \
  } while (0)
#define SLSTM_HEAD_SEQ_T(CM_) SLSTM_HEAD_SEQ(true, CM_)
#define SLSTM_HEAD_SEQ_F(CM_) SLSTM_HEAD_SEQ(false, CM_)
  SLSTM_HEAD_DH_DISPATCH(dh, {
    if (p_bf16) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_SEQ_T) }
    else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_SEQ_F) }
  })
#undef SLSTM_HEAD_SEQ_T
#undef SLSTM_HEAD_SEQ_F
#undef SLSTM_HEAD_SEQ
  return hipGetLastError();
}

hipError_t launch_head_iteration(const void* P, bool p_bf16, const float* R, const float* state0, const float* S_in,
                                 float* S_out, float* h_out, int B, int T, int d, int n_heads, int cell_mode,
                                 Control* ctl, int k_iter, float tol, bool last, hipStream_t stream, Seqs seqs) {
  if (n_heads < 1 || d % n_heads != 0 || B > 65535) return hipErrorInvalidValue;
  const int dh = d / n_heads;
  const dim3 grid(static_cast<unsigned>(n_heads), static_cast<unsigned>(B));
  const unsigned int lds = head_spread_lds(static_cast<long long>(n_heads) * B, 4096);
  const bool packed = seqs.cu != nullptr;
#define SLSTM_HEAD_IT(BF, LS, CM_)                                                                              \
  do {                                                                                                          \
    if (packed)                                                                                                 \
      head_iter_kernel<DH, BF, CM_, LS, true><<<grid, 4 * DH, lds, stream>>>(P, R, state0, S_in, S_out, h_out, T, d, \
                                                                             n_heads, ctl, k_iter, tol, seqs);  \
    else                                                                                                        \
      head_iter_kernel<DH, BF, CM_, LS, false><<<grid, 4 * DH, lds, stream>>>(P, R, state0, S_in, S_out, h_out, T, \
                                                                              d, n_heads, ctl, k_iter, tol, seqs); \
  } while (0)
#define SLSTM_HEAD_IT_TT(CM_) SLSTM_HEAD_IT(true, true, CM_)
#define SLSTM_HEAD_IT_TF(CM_) SLSTM_HEAD_IT(true, false, CM_)
#define SLSTM_HEAD_IT_FT(CM_) SLSTM_HEAD_IT(false, true, CM_)
#define SLSTM_HEAD_IT_FF(CM_) SLSTM_HEAD_IT(false, false, CM_)
  SLSTM_HEAD_DH_DISPATCH(dh, {
    if (p_bf16) {
      if (last) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_IT_TT) }
      else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_IT_TF) }
    } else {
      if (last) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_IT_FT) }
      else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_IT_FF) }
    }
  })
#undef SLSTM_HEAD_IT_TT
#undef SLSTM_HEAD_IT_TF
#undef SLSTM_HEAD_IT_FT
#undef SLSTM_HEAD_IT_FF
#undef SLSTM_HEAD_IT
  return hipGetLastError();
}

}  // namespace slstm
