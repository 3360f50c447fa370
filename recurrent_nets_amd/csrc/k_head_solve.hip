// The whole Newton solve under head mixing in one sweep over T ("sLSTM in this library",
// "Cell", the mix table's 'head' row; Newton's method on the recurrence, "ParaRNN", the
// Newton-iteration section): a fixed count of K iterations (no early stop), pipelined along T.
//
// Iteration k's linear solve Delta^k_t = A^k_t Delta^k_{t-1} - F^k_t is a forward substitution:
// at step t it needs only iterate k at t-1 and t and Delta^k_{t-1}. Iterate k at t is
// S^{k-1}_t + Delta^{k-1}_t, formed by stage k-1 at the same step, and its pre-activations are
// linear in h', so
//   x~^k_t = x~^{k-1}_t + R Delta h^{k-1}_{t-1}        (x~^0_t = p_t + R h^0_{t-1})
// and one block product per stage (R Delta h^k_{t-1}) serves both stage k's solve and stage
// k+1's residual. Stage 0's iterate is the warm start (the channelwise cell with R h' dropped,
// run step by step here) or zero. A step therefore costs K + 1 block products and K + 2 cell
// evaluations (warm start, K residuals with their Jacobians, the final residual); nothing but P
// is read and nothing but S^K and h is written. The iterates are those of one kernel per
// iteration up to float32 rounding.
//
// Layout as in k_head.hip: a workgroup per (batch row, head), lane 4 i + g for unit i and
// gate / state slot g, row i of gate g's block in registers, h of iterate 0 and Delta h of
// every stage passed from step to step through double-buffered LDS.
//
// Packed sequences (PACKED, one batch row, single-group form): at the first step of sequence s
// the state before it is state0[s] in every iterate and no Newton step enters it (a zero
// Jacobian), so every stage restarts there from the same data; the workgroup stages that h
// and zero Delta h for the block products behind an extra barrier (at sequence starts only) and
// walks the offsets with a SeqCursor.
#include "cell.h"
#include "head.h"
#include "kernels.h"

namespace slstm {

// One wave per SIMD is this kernel's occupancy at the sizes it serves (a workgroup per batch
// row and head); saying so lets the scheduler keep a step's LDS reads in flight together
// instead of trading them for registers.
template <int DH, bool BF16, int CM, int K, bool PACKED>
__global__ __launch_bounds__(4 * DH) __attribute__((amdgpu_waves_per_eu(1, 1))) void head_solve_kernel(const void* __restrict__ P, const float* __restrict__ R,
                                                            const float* __restrict__ state0, float* __restrict__ S,
                                                            float* __restrict__ h_out, int T, int d, int nh,
                                                            Control* __restrict__ ctl, int zero_init, Seqs seqs) {
  constexpr bool sig = (CM & kCellSigmoid) != 0;
  constexpr bool floored = (CM & kCellFloored) != 0;
  __shared__ __attribute__((aligned(16))) float h0buf[2][DH];     // h of iterate 0 at t - 1
  __shared__ __attribute__((aligned(16))) float dhbuf[K][2][DH];  // Delta h of stage k at t - 1
  __shared__ unsigned int s_err[K + 1];
  __shared__ float junk[4 * DH];  // the LDS writes of lanes that do not hold h (see h_slot)
  const int tid = threadIdx.x;
  const int i = tid >> 2, g = tid & 3;
  const int a = blockIdx.x, b = blockIdx.y;
  const int j = a * DH + i;
  const i64 dd = d;
  const GateSel sel(g);
  float row[DH];
  load_block_row<DH>(R, nh, a, i, g, row);
  const float s0 = state0 != nullptr ? state0[(static_cast<i64>(b) * 4 + g) * dd + j] : 0.0f;
  // slot g of iterate k at t - 1 (k = 0..K; every iterate starts from state0) and of Delta^k
  float sp[K + 1], dp[K];
  unsigned int emax[K + 1];
#pragma unroll
  for (int k = 0; k <= K; ++k) {
    sp[k] = s0;
    emax[k] = 0u;
  }
#pragma unroll
  for (int k = 0; k < K; ++k) dp[k] = 0.0f;
  if (g == 3) {
    h0buf[0][i] = s0;  // the state before step 0 is state0 for every iterate
#pragma unroll
    for (int k = 0; k < K; ++k) dhbuf[k][0][i] = 0.0f;
  }
  if (tid <= K) s_err[tid] = 0u;
  // where this lane's value goes in an h exchange: the h lane's slot, the others a junk word;
  // an address select keeps the step free of branches, so its stages can be interleaved
  auto h_slot = [&](float* hdst) { return g == 3 ? hdst : &junk[tid]; };
  const i64 base = static_cast<i64>(b) * T * 4 * dd + g * dd + j;  // (b, t = 0, slot/gate g, j)
  float pr[kHeadPrefetch];
#pragma unroll
  for (int u = 0; u < kHeadPrefetch; ++u) pr[u] = load_p<BF16>(P, base + static_cast<i64>(min(u, T - 1)) * 4 * dd);
  head_lds_barrier();

  // a step at t >= T (the rest of the last block of kHeadPrefetch) runs on clamped operands and
  // leaves no trace: no store, no residual maximum; its LDS exchange is never read for a real
  // step. The step returns slot g of iterate K at t; the block stores them after its last step.
  const float warm_scale = zero_init ? 0.0f : 1.0f;  // the warm start's state is finite
  SeqCursor seq = seq_cursor(seqs.cu, seqs.n, 0, 0, seqs.tab);
  auto step = [&](int t, float p, bool real) -> float {
    if constexpr (PACKED) {
      const int sq = real ? seq_begin(seq, t) : -1;
      if (sq >= 0) {  // a sequence start (uniform): every iterate restarts from state0[sq]
        const float v0 = state0 != nullptr ? state0[(static_cast<i64>(sq) * 4 + g) * dd + j] : 0.0f;
#pragma unroll
        for (int k = 0; k <= K; ++k) sp[k] = v0;
#pragma unroll
        for (int k = 0; k < K; ++k) dp[k] = 0.0f;
        if (g == 3) {
          h0buf[t & 1][i] = v0;
#pragma unroll
          for (int k = 0; k < K; ++k) dhbuf[k][t & 1][i] = 0.0f;
        }
        head_lds_barrier();
      }
    }
    // the R Delta h' products of every stage depend on step t - 1 only
    float y[K];
#pragma unroll
    for (int k = 0; k < K; ++k) y[k] = block_dot<DH>(row, dhbuf[k][t & 1]);
    float xs[4], ps[4], pg[4];
    quad_gather(p + block_dot<DH>(row, h0buf[t & 1]), xs);  // x~^0_t
    quad_gather(sp[0], ps);                                  // iterate 0 at t - 1
    // iterate 0 at t (formed also for a zero start, then discarded: no branch in the step)
    float cur;
    {
      quad_gather(p, pg);
      float s[4], A[16];
      cell_step<false>(CellIn{ps[0], ps[1], ps[2], 0.0f}, pg[0], pg[1], pg[2], pg[3], 0.0f, 0.0f, 0.0f, 0.0f, sig,
                       floored, s, A);
      cur = sel(s) * warm_scale;
    }
    *h_slot(&h0buf[(t + 1) & 1][i]) = cur;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k > 0) quad_gather(sp[k], ps);  // iterate k at t - 1
      float s[4];
      CellLin L;
      cell_step_lin(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs, sig, floored, s, L);
      const float F = cur - sel(s);
      const unsigned int em = res_max(emax[k], F);
      emax[k] = real ? em : emax[k];
      float ys[4], ds[4];
      quad_gather(y[k], ys);
      quad_gather(dp[k], ds);
      float dv[4];
      cell_jvp(L, ds, ys, dv);
      const float delta = sel(dv) - F;
      *h_slot(&dhbuf[k][(t + 1) & 1][i]) = delta;
      sp[k] = cur;
      dp[k] = delta;
      cur += delta;  // iterate k + 1 at t
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[q] += ys[q];
    }
    // iterate K at t: the result, and its residual
    quad_gather(sp[K], ps);
    float sn[4], An[16];
    cell_step<false>(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs[0], xs[1], xs[2], xs[3], 0.0f, 0.0f, 0.0f, 0.0f, sig,
                     floored, sn, An);
    const unsigned int em = res_max(emax[K], cur - sel(sn));
    emax[K] = real ? em : emax[K];
    sp[K] = cur;
    head_lds_barrier();
    return cur;
  };
  // blocks of kHeadPrefetch steps; every ring slot is refilled unconditionally (clamped), so no
  // load has to complete before the step kHeadPrefetch later that reads it
  const bool h_lane = g == 3 && h_out != nullptr;
  for (int t0 = 0; t0 < T; t0 += kHeadPrefetch) {
    float out[kHeadPrefetch];
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) {
      const int t = t0 + u;
      const float p = pr[u];
      pr[u] = load_p<BF16>(P, base + static_cast<i64>(min(t + kHeadPrefetch, T - 1)) * 4 * dd);
      out[u] = step(t, p, t < T);
    }
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) {
      const int t = t0 + u;
      if (t < T) {
        S[base + static_cast<i64>(t) * 4 * dd] = out[u];
        if (h_lane) h_out[(static_cast<i64>(b) * T + t) * dd + j] = out[u];
      }
    }
  }

  // residual maxima of iterates 0..K: the workgroup's into LDS, then one device atomic each
#pragma unroll
  for (int k = 0; k <= K; ++k) __hip_atomic_fetch_max(&s_err[k], emax[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (tid == 0) {
    const unsigned int slot = blockIdx.x + gridDim.x * blockIdx.y;
#pragma unroll
    for (int k = 0; k <= K; ++k) err_publish(&spread_of(ctl)->err[0][k], kErrSlotWords, slot, res_max_value(s_err[k]));
    if (blockIdx.x == 0 && blockIdx.y == 0) ctl->iters = K;
  }
}

// The same solve with its stages on separate wave groups of one workgroup: group 0 forms the
// warm start, group k + 1 runs Newton iteration k (its residual, Jacobian and substitution
// step) and group K + 1 the final residual and the stores. At tick tau group r works on step
// tau - r, so the K + 2 stages of a step run one after another on consecutive ticks while the
// groups run side by side; a tick costs about one stage (one block product and one cell
// evaluation) instead of all of them. Stage r hands its iterate at t and its pre-activations
// x~ at t to stage r + 1 through a double-buffered LDS slot, one float of each per lane; every
// group passes one barrier per tick. A group is 4 d_head lanes rounded up to a whole wave (at
// d_head 8 the upper half of the wave repeats the lower: the same values to the same LDS words,
// no global stores), so every branch on the group is uniform over a wave. Heads of up to 32
// units: K + 2 groups of 128 lanes fit a workgroup, and a lane's block row fits its registers.
constexpr int kHeadPipeMaxThreads = 1024;

template <int DH>
constexpr int head_pipe_group() {
  return 4 * DH < 64 ? 64 : 4 * DH;
}

// WAVES: the waves per SIMD the register budget is cut for (1: no cut). Uncut, the kernel takes
// at most 96 VGPRs a lane, so up to 5 waves share a SIMD; the launcher cuts to 6 (80 registers a
// lane) only when two workgroups a CU need more (d_head 32 at K >= 3).
template <int DH, bool BF16, int CM, int WAVES>
__global__ __launch_bounds__(kHeadPipeMaxThreads) __attribute__((amdgpu_waves_per_eu(WAVES))) void head_solve_pipe_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    float* __restrict__ S, float* __restrict__ h_out, int T, int d, int nh, Control* __restrict__ ctl,
    int zero_init, int K) {
  constexpr bool sig = (CM & kCellSigmoid) != 0;
  constexpr bool floored = (CM & kCellFloored) != 0;
  constexpr int GS = head_pipe_group<DH>();
  constexpr int KM = kHeadSolveMaxIters;
  __shared__ __attribute__((aligned(16))) float h0buf[2][DH];      // h of iterate 0 at t - 1
  __shared__ __attribute__((aligned(16))) float dhbuf[KM][2][DH];  // Delta h of iteration k at t - 1
  __shared__ float hand_s[KM + 1][2][GS];  // iterate r at t, slot g: from group r to group r + 1
  __shared__ float hand_x[KM + 1][2][GS];  // x~ of iterate r at t, gate g
  __shared__ unsigned int s_err[KM + 1];
  __shared__ float junk[GS];  // the LDS writes of lanes that do not hold h (see h_slot)
  const int tid = threadIdx.x;
  const int grp = __builtin_amdgcn_readfirstlane(tid / GS);
  const int tg = tid - grp * GS;
  const int i = (tg >> 2) & (DH - 1), g = tg & 3;
  const bool primary = tg < 4 * DH;
  const int a = blockIdx.x, b = blockIdx.y;
  const int j = a * DH + i;
  const i64 dd = d;
  const GateSel sel(g);
  const float s0 = state0 != nullptr ? state0[(static_cast<i64>(b) * 4 + g) * dd + j] : 0.0f;
  if (grp == 0 && g == 3) h0buf[0][i] = s0;  // the state before step 0 is state0 for every iterate
  if (grp >= 1 && grp <= K && g == 3) dhbuf[grp - 1][0][i] = 0.0f;
  if (tid <= K) s_err[tid] = 0u;
  auto h_slot = [&](float* hdst, bool write) { return write ? hdst : &junk[tg]; };
  const i64 base = static_cast<i64>(b) * T * 4 * dd + g * dd + j;  // (b, t = 0, slot/gate g, j)
  // ticks 0 .. T + K, rounded up to whole blocks of kHeadPrefetch: every group passes the same
  // number of barriers
  const int n_ticks = (T + K + 1 + kHeadPrefetch - 1) / kHeadPrefetch * kHeadPrefetch;
  head_lds_barrier();

  if (grp == 0) {
    // the warm start: the channelwise cell with R h' dropped, and x~ of iterate 0
    float row[DH];
    load_block_row<DH>(R, nh, a, i, g, row);
    const float warm_scale = zero_init ? 0.0f : 1.0f;  // the warm start's state is finite
    float sp = s0;
    float pr[kHeadPrefetch];
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) pr[u] = load_p<BF16>(P, base + static_cast<i64>(min(u, T - 1)) * 4 * dd);
    for (int t0 = 0; t0 < n_ticks; t0 += kHeadPrefetch) {
#pragma unroll
      for (int u = 0; u < kHeadPrefetch; ++u) {
        const int t = t0 + u;
        const float p = pr[u];
        pr[u] = load_p<BF16>(P, base + static_cast<i64>(min(t + kHeadPrefetch, T - 1)) * 4 * dd);
        const float x = p + block_dot<DH>(row, h0buf[t & 1]);
        float ps[4], pg[4], s[4], A[16];
        quad_gather(sp, ps);
        quad_gather(p, pg);
        cell_step<false>(CellIn{ps[0], ps[1], ps[2], 0.0f}, pg[0], pg[1], pg[2], pg[3], 0.0f, 0.0f, 0.0f, 0.0f, sig,
                         floored, s, A);
        const float cur = sel(s) * warm_scale;
        *h_slot(&h0buf[(t + 1) & 1][i], g == 3) = cur;
        hand_s[0][t & 1][tg] = cur;
        hand_x[0][t & 1][tg] = x;
        sp = cur;  // past T the values run on unread
        head_lds_barrier();
      }
    }
  } else if (grp <= K) {
    // Newton iteration k at step t: residual and Jacobian at iterate k, Delta^k_t, iterate k + 1
    const int k = grp - 1;
    float row[DH];
    load_block_row<DH>(R, nh, a, i, g, row);
    float sp = s0, dp = 0.0f;  // slot g of iterate k and of Delta^k at t - 1
    unsigned int emax = 0u;
    for (int tau = 0; tau < n_ticks; ++tau) {
      const int t = tau - grp;
      const bool real = t >= 0 && t < T;
      const int rd = (tau - 1) & 1, wr = tau & 1;
      const float cur = hand_s[k][rd][tg];  // iterate k at t
      const float x = hand_x[k][rd][tg];
      const float y = block_dot<DH>(row, dhbuf[k][t & 1]);  // R Delta h^k_{t-1}
      float xs[4], ps[4], ys[4], ds[4], s[4], dv[4];
      quad_gather(x, xs);
      quad_gather(sp, ps);
      CellLin L;
      cell_step_lin(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs, sig, floored, s, L);
      const float F = cur - sel(s);
      const unsigned int em = res_max(emax, F);
      emax = real ? em : emax;
      quad_gather(y, ys);
      quad_gather(dp, ds);
      cell_jvp(L, ds, ys, dv);
      const float delta = sel(dv) - F;
      // before step 0 the slot holds Delta h^k_{-1} = 0: ticks ahead of it write elsewhere
      *h_slot(&dhbuf[k][(t + 1) & 1][i], g == 3 && real) = delta;
      hand_s[grp][wr][tg] = cur + delta;
      hand_x[grp][wr][tg] = x + y;
      sp = real ? cur : sp;
      dp = real ? delta : dp;
      head_lds_barrier();
    }
    __hip_atomic_fetch_max(&s_err[k], emax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    // iterate K at step t: its residual, and the stores
    float sp = s0;
    unsigned int emax = 0u;
    const bool h_lane = g == 3 && h_out != nullptr && primary;
    for (int tau = 0; tau < n_ticks; ++tau) {
      const int t = tau - grp;
      const bool real = t >= 0 && t < T;
      const int rd = (tau - 1) & 1;
      const float cur = hand_s[K][rd][tg];
      const float x = hand_x[K][rd][tg];
      float xs[4], ps[4], sn[4], An[16];
      quad_gather(x, xs);
      quad_gather(sp, ps);
      cell_step<false>(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs[0], xs[1], xs[2], xs[3], 0.0f, 0.0f, 0.0f, 0.0f, sig,
                       floored, sn, An);
      const unsigned int em = res_max(emax, cur - sel(sn));
      emax = real ? em : emax;
      sp = real ? cur : sp;
      if (real && primary) {
        S[base + static_cast<i64>(t) * 4 * dd] = cur;
        if (h_lane) h_out[(static_cast<i64>(b) * T + t) * dd + j] = cur;
      }
      head_lds_barrier();
    }
    __hip_atomic_fetch_max(&s_err[K], emax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (tid == 0) {
    const unsigned int slot = blockIdx.x + gridDim.x * blockIdx.y;
    for (int k = 0; k <= K; ++k) err_publish(&spread_of(ctl)->err[0][k], kErrSlotWords, slot, res_max_value(s_err[k]));
    if (blockIdx.x == 0 && blockIdx.y == 0) ctl->iters = K;
  }
}

hipError_t launch_head_solve(const void* P, bool p_bf16, const float* R, const float* state0, float* S,
                             float* h_out, int B, int T, int d, int n_heads, int cell_mode, int K, bool zero_init,
                             Control* ctl, hipStream_t stream, Seqs seqs) {
  if (n_heads < 1 || d % n_heads != 0 || B > 65535 || K < 1 || K > kHeadSolveMaxIters) return hipErrorInvalidValue;
  const int dh = d / n_heads;
  const dim3 grid(static_cast<unsigned>(n_heads), static_cast<unsigned>(B));
  const unsigned int lds = head_spread_lds(static_cast<long long>(n_heads) * B, 4096);
  const int zi = zero_init ? 1 : 0;
  // Which form: the wave-group form runs a step in about half the single-group sweep's time
  // while each CU holds one workgroup, and with two (at K >= 2 with the register cut that keeps
  // both resident) about 15% faster; from three workgroups a CU on, the CU's issue rate bounds
  // both and the sweep's fewer instructions win (measured at d_head 32, T 4096, K 1 and 3).
  // Heads wider than 32 units always take the sweep.
  const long long cus = head_device_cus();
  const long long wg_per_cu = (static_cast<long long>(n_heads) * B + cus - 1) / cus;
  const bool packed = seqs.cu != nullptr;
  if (packed && B != 1) return hipErrorInvalidValue;
  if (dh <= 32 && wg_per_cu <= 2 && !packed) {
    const unsigned int lds_p = head_spread_lds(static_cast<long long>(n_heads) * B, 24 * 1024);
    // waves a SIMD must hold, counting each workgroup's K + 2 groups of ceil(4 d_head / 64)
    // waves as spread over the 4 SIMDs in whole rounds: uncut (96 VGPRs) a SIMD takes 5
    const long long waves_per_group = (4 * dh + kWave - 1) / kWave;
    const long long waves_per_simd = ((K + 2) * waves_per_group + 3) / 4 * wg_per_cu;
    const bool cut = waves_per_simd > 5;
#define SLSTM_HEAD_PIPE(CM_)                                                                                  \
  if (cut)                                                                                                    \
    head_solve_pipe_kernel<DH, BFV, CM_, 6><<<grid, (K + 2) * head_pipe_group<DH>(), lds_p, stream>>>(      \
        P, R, state0, S, h_out, T, d, n_heads, ctl, zi, K);                                                   \
  else                                                                                                        \
    head_solve_pipe_kernel<DH, BFV, CM_, 1><<<grid, (K + 2) * head_pipe_group<DH>(), lds_p, stream>>>(      \
        P, R, state0, S, h_out, T, d, n_heads, ctl, zi, K);
#define SLSTM_HEAD_PIPE_DH(DHV)                                                              \
  case DHV: {                                                                                \
    constexpr int DH = DHV;                                                                  \
    if (p_bf16) { constexpr bool BFV = true; SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_PIPE) } \
    else { constexpr bool BFV = false; SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_PIPE) }       \
    break;                                                                                   \
  }
    switch (dh) {
      SLSTM_HEAD_PIPE_DH(8)
      SLSTM_HEAD_PIPE_DH(16)
      SLSTM_HEAD_PIPE_DH(32)
      default: return hipErrorInvalidValue;
    }
#undef SLSTM_HEAD_PIPE_DH
#undef SLSTM_HEAD_PIPE
    return hipGetLastError();
  }
#define SLSTM_HEAD_SOLVE(BF, KK, CM_)                                                                           \
  do {                                                                                                          \
    if (packed)                                                                                                 \
      head_solve_kernel<DH, BF, CM_, KK, true><<<grid, 4 * DH, lds, stream>>>(P, R, state0, S, h_out, T, d,    \
                                                                              n_heads, ctl, zi, seqs);          \
    else                                                                                                        \
      head_solve_kernel<DH, BF, CM_, KK, false><<<grid, 4 * DH, lds, stream>>>(P, R, state0, S, h_out, T, d,   \
                                                                               n_heads, ctl, zi, seqs);         \
  } while (0)
#define SLSTM_HEAD_SOLVE_K(BF, CM_)              \
  switch (K) {                                   \
    case 1: SLSTM_HEAD_SOLVE(BF, 1, CM_); break; \
    case 2: SLSTM_HEAD_SOLVE(BF, 2, CM_); break; \
    case 3: SLSTM_HEAD_SOLVE(BF, 3, CM_); break; \
    default: SLSTM_HEAD_SOLVE(BF, 4, CM_); break; \
  }
#define SLSTM_HEAD_SOLVE_T(CM_) SLSTM_HEAD_SOLVE_K(true, CM_)
#define SLSTM_HEAD_SOLVE_F(CM_) SLSTM_HEAD_SOLVE_K(false, CM_)
  SLSTM_HEAD_SWEEP_DH_DISPATCH(dh, {
    if (p_bf16) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_SOLVE_T) }
    else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_SOLVE_F) }
  })
#undef SLSTM_HEAD_SOLVE_T
#undef SLSTM_HEAD_SOLVE_F
#undef SLSTM_HEAD_SOLVE_K
#undef SLSTM_HEAD_SOLVE
  return hipGetLastError();
}

}  // namespace slstm
