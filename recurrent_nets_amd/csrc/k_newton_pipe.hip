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
// iteration k+1, a wavefront along T. P is read once and only S_K (when the caller wants the
// states), h and the final state are written: 36 bytes per state element for the whole solve
// (20 with the hidden slot alone) instead of 32 + 48 K + 20 for per-iteration passes.
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
// tt. There is no early stop inside a launch: the residual maxima of every iterate go to the
// spread slots, and an early stop runs the kernel twice (the budget, then the count the stop
// test chose, read from the control block). Packed sequences (one batch row) run on tiles
// aligned to the sequence starts, from the table of the aligned scan-form tiles: a tile at a
// sequence start begins from that sequence's state0 and waits on nothing, so the sequences'
// chains advance side by side.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kPipeBlock = 256;  // one feature per thread
// Steps per tile. Short tiles (15 steps, P and the iterate in 166 registers, the most that keep
// three workgroups a CU) where the lane groups cover every CU: the solve is bound by vector issue
// there, and more resident waves hide the latency of each step's dependent chain. Long tiles (24
// steps, 238 registers, two workgroups a CU) where they do not: the wavefront along T then waits
// on each tile's predecessor in turn, and longer tiles mean fewer hand-offs. Measured on MI355X
// (K = 3, d_h = 1024): 512 lane groups 2.46 ms at 14 steps against 2.52 at 24 (15 steps: 2.37
// against 2.40 at 14), 256 the same, 128 0.87 against 0.73 ms, 32 (B = 4, T = 16384, d_h = 2048,
// K = 4) 3.91 against 3.21 ms; the results are bitwise equal.
constexpr int kPipeStepsShort = 15;
constexpr int kPipeStepsLong = 24;

__host__ __device__ constexpr int pipe_words(int K) { return 4 + 4 * K; }
__host__ __device__ constexpr int pipe_min_waves(int tc) { return tc <= 15 ? 3 : 2; }

template <bool BF16, bool WARM, int CM, int TC>
__global__ __launch_bounds__(kPipeBlock, pipe_min_waves(TC)) void newton_pipe_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    float* __restrict__ S_out, float* __restrict__ h_out, float* __restrict__ fs_out, int T, int d,
    int n_jt, int n_lg,
    int n_tt, int K, int k_from_ctl, unsigned long long* __restrict__ carry,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch, Control* __restrict__ ctl,
    const int* __restrict__ tiles, int tile_cap) {
  __shared__ int s_tile[2];
  __shared__ unsigned int s_err[kPipeMaxItersStop + 1];  // block residual maxima per iterate
  if (k_from_ctl) {
    // the second pass of an early-stop solve: the iteration count the stop test chose; nothing
    // to redo when no iterate met the tolerance (every workgroup leaves before taking a ticket)
    if (!ctl->stopped) return;
    K = ctl->iters;
  }
  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  if (tid <= kPipeMaxItersStop) s_err[tid] = 0u;
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;
  // The tile: its words' index, its predecessor's, its first step, the end of its sequence (or
  // of the row), whether it starts that sequence and which sequence it is. Packed sequences take
  // tiles aligned to their starts from a table (one batch row; slots ordered by position, then
  // sequence, so a tile's predecessor, the id before it, holds an earlier ticket).
  int wid = tt, pred = tt - 1, t0 = tt * TC, t_end = T, seq = b;
  bool first = tt == 0, has_next = tt + 1 < n_tt;
  if (tiles != nullptr) {
    const int n_real = __builtin_amdgcn_readfirstlane(tiles[0]);
    if (tt >= n_real) {  // a ticket past the last tile
      if (blockIdx.x == 0 && tid == 0) ctl->iters = K;
      return;
    }
    const int id = __builtin_amdgcn_readfirstlane(tiles[1 + tt]);
    const int sq = __builtin_amdgcn_readfirstlane(tiles[1 + tile_cap + tt]);
    const int ps = __builtin_amdgcn_readfirstlane(tiles[1 + 2 * tile_cap + tt]);
    const int a0 = __builtin_amdgcn_readfirstlane(tiles[1 + 3 * tile_cap + tt]);
    const int e0 = __builtin_amdgcn_readfirstlane(tiles[1 + 4 * tile_cap + tt]);
    wid = id;
    pred = id - 1;
    t0 = a0 + ps * TC;
    t_end = e0;
    seq = sq;
    first = ps == 0;
    has_next = t0 + TC < e0;
  }

  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * kPipeBlock + tid);
  const bool valid = j < ud;
  const bool publish = valid && has_next;  // the tile after waits on these words
  const bool wait = valid && !first;
  const int W = pipe_words(K);
  const i64 n_lanes = static_cast<i64>(n_lg) * kPipeBlock;
  const i64 lane = static_cast<i64>(lg) * kPipeBlock + tid;
  auto word = [&](int tile, int w) { return carry + (static_cast<i64>(tile) * W + w) * n_lanes + lane; };
  auto wait_words = [&](int w0, float v[4]) {
    bool ok = false;
    while (true) {
      ok = tag_load(word(pred, w0), epoch, v[0]) & tag_load(word(pred, w0 + 1), epoch, v[1]) &
           tag_load(word(pred, w0 + 2), epoch, v[2]) & tag_load(word(pred, w0 + 3), epoch, v[3]);
      if (ok) break;
      poll_pause();
    }
  };
  constexpr bool sig = (CM & kCellSigmoid) != 0;   // forget-gate form and read-out,
  constexpr bool floored = (CM & kCellFloored) != 0;  // fixed per instantiation

  // ---- the tile's pre-activations, held for the whole solve ----
  const i64 tile_row = (static_cast<i64>(b) * T + t0) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  // lane part j in the vector offset, step and gate parts in the scalar offset; lanes past d_h
  // and steps past the tile's end read the last feature and step (every load in bounds, no zero
  // fill): what they compute is never counted, stored or published
  float p[TC][4];
  const unsigned jc = valid ? j : ud - 1u;
  const int u_last = t_end - 1 - t0;
#pragma unroll
  for (int u = 0; u < TC; ++u) {
    const unsigned uc = static_cast<unsigned>(u < u_last ? u : u_last);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[u][k] = buf_ld_p<BF16>(rsP, jc, (4u * uc + k) * ud);
    // z and o enter only their exponentials: scaled once here for all K + 2 evaluations
    p[u][0] *= kTanhScale;
    p[u][3] *= kSigScale;
  }
  float rz = 0.0f, ri = 0.0f, rf = 0.0f, ro = 0.0f;
  float hv[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // the iterate at step t0 - 1 (state0 before the sequence)
  if (valid) {
    rz = R[j];
    ri = R[ud + j];
    rf = R[2 * ud + j];
    ro = R[3 * ud + j];
    if (first && state0 != nullptr) {
      const float* s0 = state0 + static_cast<i64>(seq) * 4 * static_cast<i64>(d);
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
      s[u][0] = tanh_scaled(p[u][0]);
      s[u][1] = sig ? log_sigmoidf(p[u][2]) : p[u][2];
      s[u][2] = p[u][1];
      s[u][3] = sigmoid_scaled(p[u][3]);
    }
    if (wait) wait_words(0, hv);
    float c = hv[0], n = hv[1], m = hv[2];
#pragma unroll
    for (int u = 0; u < TC; ++u) {
      float mn, ig, fg;
      stab_gates(s[u][1] + m, s[u][2], mn, ig, fg);
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
      for (int e = 0; e < 4; ++e) tag_store(word(wid, e), s[TC - 1][e], epoch);
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
    const CellIn pv0 = {hv[0], hv[1], hv[2], hv[3]};  // iterate k before the tile
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    ResMax2 fmax;
    if (valid) {
      // Step u reads iterate k at step u - 1 as its previous state, then completes that step's
      // update (s[u-1] += Delta_{u-1}): the old value is read in place, never copied.
#pragma unroll
      for (int u = 0; u < TC; ++u) {
        const int t = t0 + u;
        if (t < t_end) {
          float f[4], r[4];
          DiagLin L;
          const CellIn pv = u == 0 ? pv0 : CellIn{s[u - 1][0], s[u - 1][1], s[u - 1][2], s[u - 1][3]};
          cell_step_diag<true>(pv, p[u][0], p[u][1], p[u][2], p[u][3], rz, ri, rf, ro, sig, floored, f, L);
          if (u > 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[u - 1][e] = s[u - 1][e] + x[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = f[e] - s[u][e];
          res_max2(fmax, r[0], r[1]);
          res_max2(fmax, r[2], r[3]);
          if (u == 0 && wait) {
            // the Newton step entering the tile; the state before the tile in iterate k+1
            wait_words(4 + 4 * k, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = hv[e] + x[e];
          }
          if (u == 0 && first) {  // the first step of the sequence
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = r[e];  // s_0 is data: Delta_1 = rhs_1
          } else {
            diag_jvp(L, floored, r, x);  // Delta_t = A_t Delta_t-1 + rhs_t, A_t in factored form
          }
        }
      }
      // the update of the tile's last step
      if (t0 + TC <= t_end) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[TC - 1][e] = s[TC - 1][e] + x[e];
      } else {
#pragma unroll
        for (int u = 0; u < TC - 1; ++u)
          if (u == t_end - 1 - t0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[u][e] = s[u][e] + x[e];
          }
      }
      if (publish) {
#pragma unroll
        for (int e = 0; e < 4; ++e) tag_store(word(wid, 4 + 4 * k + e), x[e], epoch);
      }
    }
    const unsigned int wm = wave_max_u32(res_max2_bits(fmax));
    if (l == 0) __hip_atomic_fetch_max(&s_err[k], wm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // ---- residual of S_K, and the outputs: the states (when asked for), h, the final state ----
  ResMax2 fmax;
  if (valid) {
    // a descriptor over a null base is never used: each store below tests its own pointer
    const rsrc_t rsO = make_rsrc(S_out != nullptr ? S_out + tile_row : nullptr);
    const rsrc_t rsH = make_rsrc(h_out != nullptr ? h_out + (static_cast<i64>(b) * T + t0) * static_cast<i64>(d) : nullptr);
    CellIn pv = {hv[0], hv[1], hv[2], hv[3]};
#pragma unroll
    for (int u = 0; u < TC; ++u) {
      if (t0 + u < t_end) {
        float f[4];
        cell_step<false, true>(pv, p[u][0], p[u][1], p[u][2], p[u][3], rz, ri, rf, ro, sig, floored, f, nullptr);
        res_max2(fmax, s[u][0] - f[0], s[u][1] - f[1]);
        res_max2(fmax, s[u][2] - f[2], s[u][3] - f[3]);
        if (S_out != nullptr) {
#pragma unroll
          for (int e = 0; e < 4; ++e) buf_st(s[u][e], rsO, 4u * j, 4u * (4u * u + e) * ud);
        }
        if (h_out != nullptr) buf_st(s[u][3], rsH, 4u * j, 4u * u * ud);
        if (fs_out != nullptr && t0 + u == t_end - 1) {  // the last step of the row or sequence
          float* fs = fs_out + static_cast<i64>(seq) * 4 * static_cast<i64>(d) + j;
#pragma unroll
          for (int e = 0; e < 4; ++e) fs[e * ud] = s[u][e];
        }
        pv = {s[u][0], s[u][1], s[u][2], s[u][3]};
      }
    }
  }
  const unsigned int wm = wave_max_u32(res_max2_bits(fmax));
  if (l == 0) __hip_atomic_fetch_max(&s_err[K], wm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  if (tid <= K) err_publish(&spread_of(ctl)->err[0][tid], kErrSlotWords, blockIdx.x, res_max_value(s_err[tid]));
  if (blockIdx.x == 0 && tid == 0) ctl->iters = K;
}

static void pipe_grid(int B, int T, int d, int tc, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + kPipeBlock - 1) / kPipeBlock;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + tc - 1) / tc;
}

int pipe_tile_steps(int B, int d, int n_cus) {
  return static_cast<long long>(B) * ((d + kPipeBlock - 1) / kPipeBlock) >= n_cus ? kPipeStepsShort : kPipeStepsLong;
}

// words of the shorter tiles, which are the more: enough for either length
size_t pipe_desc_words(int B, int T, int d, int K) {
  i64 n_jt, n_lg, n_tt;
  pipe_grid(B, T, d, kPipeStepsShort, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * pipe_words(K) * n_lg * kPipeBlock);
}

hipError_t launch_newton_pipe(const void* P, bool p_bf16, const float* R, const float* state0,
                              float* S_out, float* h_out, float* fs_out, int B, int T, int d, int cell_mode,
                              bool warm, int K, bool k_from_ctl, int tile_steps, unsigned long long* carry,
                              unsigned int* tickets, uint32_t epoch, Control* ctl, const int* tiles,
                              int tile_cap, hipStream_t stream) {
  if (tile_steps != kPipeStepsShort && tile_steps != kPipeStepsLong) return hipErrorInvalidValue;
  i64 n_jt, n_lg, n_tt;
  pipe_grid(B, T, d, tile_steps, n_jt, n_lg, n_tt);
  if (tiles != nullptr) {  // aligned tiles of one packed row: a ticket per table slot
    if (B != 1 || tile_cap < 1) return hipErrorInvalidValue;
    n_tt = tile_cap;
  }
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL || K < 1 || K > kPipeMaxItersStop) return hipErrorInvalidValue;
  const int kc = k_from_ctl ? 1 : 0;
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int a = static_cast<int>(n_jt), c = static_cast<int>(n_lg), e = static_cast<int>(n_tt);
#define SLSTM_PIPE_LAUNCH_TC(BF, WM, CM_, TC_)                                                         \
  newton_pipe_kernel<BF, WM, CM_, TC_><<<grid, kPipeBlock, 0, stream>>>(P, R, state0, S_out, h_out, fs_out, T, d, \
                                                                        a, c, e, K, kc, carry, tickets, n_ctr, \
                                                                        epoch, ctl, tiles, tile_cap)
#define SLSTM_PIPE_LAUNCH(BF, WM, CM_)                                                    \
  if (tile_steps == kPipeStepsShort) {                                                    \
    SLSTM_PIPE_LAUNCH_TC(BF, WM, CM_, kPipeStepsShort);                                   \
  } else {                                                                                \
    SLSTM_PIPE_LAUNCH_TC(BF, WM, CM_, kPipeStepsLong);                                    \
  }
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
#undef SLSTM_PIPE_LAUNCH_TC
  return hipGetLastError();
}

// The stop test of an early-stop solve run as two one-kernel passes: after the first pass (a
// fixed count of K iterations, every iterate's residual maximum in the spread slots), the first
// iterate k < K whose max|F| is below tol is where the per-iteration solve would have stopped
// before solving; it is recorded as the stop and the iteration count for the second pass.
__global__ __launch_bounds__(kWave) void pipe_stop_kernel(Control* __restrict__ ctl, int K, float tol) {
  for (int k = 0; k < K; ++k) {
    const float e = err_reduced(ctl, k);  // the whole wave takes part
    if (e < tol) {
      if (threadIdx.x == 0) {
        ctl->stopped = 1;
        ctl->iters = k;
      }
      return;
    }
  }
}

// the one-kernel solve writes each sequence's final state at its last step; an empty sequence
// has none, and its final state is its state0 (zeros without one); cu is read within its
// n_seqs + 1 entries
__global__ __launch_bounds__(256) void empty_seq_final_kernel(const int* __restrict__ cu, int n_seqs, int T,
                                                              const float* __restrict__ state0,
                                                              float* __restrict__ out, int d) {
  const i64 n = static_cast<i64>(n_seqs) * 4 * d;  // (s, slot, j)
  for (i64 i = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<i64>(gridDim.x) * 256) {
    const int s = static_cast<int>(i / (4 * static_cast<i64>(d)));
    // offsets clamped as the tile table clamps them: a sequence with no steps has no tile
    const int a = min(max(cu[s], 0), T);
    const int e = min(max(cu[s + 1], a), T);
    if (e == a) out[i] = state0 != nullptr ? state0[i] : 0.0f;
  }
}

hipError_t launch_empty_seq_final(const int* cu, int n_seqs, int T, const float* state0, float* final_state, int d,
                                  hipStream_t stream) {
  const i64 n = static_cast<i64>(n_seqs) * 4 * d;
  if (n <= 0) return hipSuccess;
  const i64 blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  empty_seq_final_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(cu, n_seqs, T, state0, final_state, d);
  return hipGetLastError();
}

hipError_t launch_pipe_stop(Control* ctl, int K, float tol, hipStream_t stream) {
  pipe_stop_kernel<<<1, kWave, 0, stream>>>(ctl, K, tol);
  return hipGetLastError();
}

}  // namespace slstm
