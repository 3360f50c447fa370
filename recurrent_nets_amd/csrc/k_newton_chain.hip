// One Newton iteration by chains along T, for shapes with many independent lanes.
//
// Same iteration as the scan-based fused kernel (the method of the "Layout" page of the
// pararnn-torch docs, "Current surface (0.17)"; cell of the xLSTM summary card's sLSTM step
// pseudocode, channelwise R): per step t of a lane
//   rhs_t = f(s_{t-1}) - s_t = -F_t,  A_t = df/ds' at s_{t-1}   (s_0 = state0)
//   Delta_1 = rhs_1,  Delta_t = A_t Delta_{t-1} + rhs_t,  s_t <- s_t + Delta_t
// but the block-bidiagonal solve is run as a plain recurrence inside each tile: a thread owns
// one feature and kChainSteps consecutive steps, takes Delta entering its tile from the tile
// before it (published as four epoch-tagged words, see tag_store) and applies A_t and rhs_t
// step by step. No 4x4 maps are composed, which saves about half of the vector instructions of
// the scan form. The price is a dependency chain along T: tile tt waits for tile tt-1 of the
// same lanes. With at least as many lane groups as compute units the predecessor has almost
// always finished (it holds a ticket n_lg places earlier), so the chain costs no waiting; the
// solver picks this kernel only then.
//
// Bitwise reproducible: every value is computed in one fixed order.
//
// The last iteration also evaluates the residual of the iterate it writes, F(S_{k+1}), from the
// same registers (the state before each step of the new iterate is known once Delta entering
// the tile is), and writes the hidden slot of S_{k+1}: no separate pass over S is needed for the
// final residual and h.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kChainBlock = 256;  // one feature per thread: 256 consecutive features per tile
#ifndef SLSTM_CHAIN_STEPS
#define SLSTM_CHAIN_STEPS 16
#endif
constexpr int kChainSteps = SLSTM_CHAIN_STEPS;  // steps per tile
// waves per SIMD the register allocation is bounded for (= workgroups per compute unit)
#ifndef SLSTM_CHAIN_MIN_WAVES
#define SLSTM_CHAIN_MIN_WAVES 3
#endif

template <bool BF16, bool LAST, int CM>
__global__ __launch_bounds__(kChainBlock, SLSTM_CHAIN_MIN_WAVES) void newton_chain_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S_in, float* __restrict__ S_out, float* __restrict__ h_out, int T,
    int d, int n_jt, int n_lg, int n_tt, unsigned long long* __restrict__ carry,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch, Control* __restrict__ ctl,
    int k_iter, float tol) {
  constexpr int TC = kChainSteps;
  if (ctl->stopped) return;
  if (k_iter > 0 && tol > 0.0f && err_reduced(ctl, k_iter - 1) < tol) {
    // the previous iterate already met the tolerance: it is the result
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      ctl->stopped = 1;
      ctl->iters = k_iter - 1;
    }
    return;
  }
  __shared__ int s_tile[2];
  __shared__ unsigned int s_err[2], s_arrived;  // block residual maxima (S_k, S_k+1), waves done
  const int tid = threadIdx.x;
  if (tid == 0) {
    take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
    s_err[0] = 0u;
    s_err[1] = 0u;
    s_arrived = 0u;
  }
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;

  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * kChainBlock + tid);
  const bool valid = j < ud;
  const int t0 = tt * TC;
  const i64 n_lanes = static_cast<i64>(n_lg) * kChainBlock;
  const i64 lane = static_cast<i64>(lg) * kChainBlock + tid;
  auto carry_word = [&](int tile, int e) { return carry + (static_cast<i64>(tile) * 4 + e) * n_lanes + lane; };
  constexpr bool sig = (CM & kCellSigmoid) != 0;   // forget-gate form and read-out,
  constexpr bool floored = (CM & kCellFloored) != 0;  // fixed per instantiation

  // Delta entering the tile, loaded now so that it arrives while the tile's operands do
  unsigned long long pf[4] = {0ull, 0ull, 0ull, 0ull};
  if (valid && tt > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pf[e] = __hip_atomic_load(carry_word(tt - 1, e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // the tile's operands: scalar row bases, 32-bit lane offsets (elements)
  const i64 tile_row = (static_cast<i64>(b) * T + t0) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  const rsrc_t rsS = make_rsrc(S_in + tile_row);
  const rsrc_t rsO = make_rsrc(S_out + tile_row);
  float pg[TC][4], sv[TC][4];
#pragma unroll
  for (int u = 0; u < TC; ++u) {
    if (valid && t0 + u < T) {
      const unsigned o = u * 4u * ud + j;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[u][k] = buf_ld_p<BF16>(rsP, o, k * ud);
        sv[u][k] = buf_ld(rsS, 4u * o, 4u * k * ud);
      }
    }
  }

  float rz = 0.0f, ri = 0.0f, rf = 0.0f, ro = 0.0f;
  CellIn pv = {0.0f, 0.0f, 0.0f, 0.0f};  // S_k before the step
  if (valid) {
    rz = R[j];
    ri = R[ud + j];
    rf = R[2 * ud + j];
    ro = R[3 * ud + j];
    if (t0 == 0) {
      if (state0 != nullptr) {
        const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
        pv = {s0[j], s0[ud + j], s0[2 * ud + j], s0[3 * ud + j]};
      }
    } else {
      const float* sp = S_in + (static_cast<i64>(b) * T + t0 - 1) * 4 * static_cast<i64>(d);
      pv = {sp[j], sp[ud + j], sp[2 * ud + j], sp[3 * ud + j]};
    }
  }

  float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // Delta of the current step
  unsigned int fmax = 0u, fmax_new = 0u;
  CellIn pn = pv;  // S_k+1 before the step (last iteration only)
  float* h_tile = (LAST && h_out != nullptr) ? h_out + (static_cast<i64>(b) * T + t0) * static_cast<i64>(d) : nullptr;
  if (valid) {
#pragma unroll
    for (int u = 0; u < TC; ++u) {
      const int t = t0 + u;
      if (t < T) {
        float f[4];
        DiagLin L;
        cell_step_diag(pv, pg[u][0], pg[u][1], pg[u][2], pg[u][3], rz, ri, rf, ro, sig, floored, f, L);
        float r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          r[k] = f[k] - sv[u][k];
          fmax = res_max(fmax, r[k]);
        }
        if (u == 0 && tt > 0) {
          // Delta entering the tile: the prefetched words, or wait until the tile before
          // publishes them (it holds an earlier ticket of the same counter, so it runs)
          bool ok = true;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = __uint_as_float(static_cast<uint32_t>(pf[e]));
            ok &= static_cast<uint32_t>(pf[e] >> 32) == epoch;
          }
          while (!ok) {
            poll_pause();
            ok = true;
#pragma unroll
            for (int e = 0; e < 4; ++e) ok &= tag_load(carry_word(tt - 1, e), epoch, x[e]);
          }
          if constexpr (LAST) pn = {pv.c + x[0], pv.n + x[1], pv.m + x[2], pv.h + x[3]};
        }
        if (t == 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = r[k];  // s_0 is data: Delta_1 = rhs_1
        } else {
          diag_jvp(L, floored, r, x);  // Delta_t = A_t Delta_t-1 + rhs_t, A_t in factored form
        }
        float sn[4];
        const unsigned o = u * 4u * ud + j;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sn[k] = sv[u][k] + x[k];
          buf_st(sn[k], rsO, 4u * o, 4u * k * ud);
        }
        if constexpr (LAST) {
          float fn[4];
          cell_step<false>(pn, pg[u][0], pg[u][1], pg[u][2], pg[u][3], rz, ri, rf, ro, sig, floored, fn, nullptr);
#pragma unroll
          for (int k = 0; k < 4; ++k) fmax_new = res_max(fmax_new, sn[k] - fn[k]);
          if (h_tile != nullptr) h_tile[static_cast<i64>(u) * d + j] = sn[3];
          pn = {sn[0], sn[1], sn[2], sn[3]};
        }
        pv = {sv[u][0], sv[u][1], sv[u][2], sv[u][3]};
      }
    }
    if (tt + 1 < n_tt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) tag_store(carry_word(tt, e), x[e], epoch);
    }
  }

  // residual maxima: waves fold theirs into the block's in LDS; the last to arrive publishes
  const int l = tid & (kWave - 1);
  const unsigned int w0 = wave_max_u32(fmax);
  const unsigned int w1 = LAST ? wave_max_u32(fmax_new) : 0u;
  if (l == 0) {
    __hip_atomic_fetch_max(&s_err[0], w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (LAST) __hip_atomic_fetch_max(&s_err[1], w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__hip_atomic_fetch_add(&s_arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == kChainBlock / kWave - 1) {
      err_publish(&spread_of(ctl)->err[0][k_iter], kErrSlotWords, blockIdx.x,
                  res_max_value(__hip_atomic_load(&s_err[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)));
      if (LAST)
        err_publish(&spread_of(ctl)->err[0][k_iter + 1], kErrSlotWords, blockIdx.x,
                    res_max_value(__hip_atomic_load(&s_err[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)));
    }
  }
  if (blockIdx.x == 0 && tid == 0) ctl->iters = k_iter + 1;
}

static void chain_grid(int B, int T, int d, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + kChainBlock - 1) / kChainBlock;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + kChainSteps - 1) / kChainSteps;
}

long long chain_lane_groups(int B, int d) {
  return static_cast<long long>(B) * ((d + kChainBlock - 1) / kChainBlock);
}

size_t chain_desc_words(int B, int T, int d) {
  i64 n_jt, n_lg, n_tt;
  chain_grid(B, T, d, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * 4 * n_lg * kChainBlock);
}

hipError_t launch_newton_chain(const void* P, bool p_bf16, const float* R, const float* state0,
                               const float* S_in, float* S_out, float* h_out, int B, int T, int d,
                               int cell_mode, unsigned long long* carry, unsigned int* tickets,
                               uint32_t epoch, Control* ctl, int k_iter, float tol, bool last,
                               hipStream_t stream) {
  i64 n_jt, n_lg, n_tt;
  chain_grid(B, T, d, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int a = static_cast<int>(n_jt), c = static_cast<int>(n_lg), e = static_cast<int>(n_tt);
#define SLSTM_CHAIN_LAUNCH(BF, LS, CM_)                                                                      \
  newton_chain_kernel<BF, LS, CM_><<<grid, kChainBlock, 0, stream>>>(P, R, state0, S_in, S_out, h_out, T, d, \
                                                                     a, c, e, carry, tickets, n_ctr,       \
                                                                     epoch, ctl, k_iter, tol)
#define SLSTM_CHAIN_TT(CM_) SLSTM_CHAIN_LAUNCH(true, true, CM_)
#define SLSTM_CHAIN_TF(CM_) SLSTM_CHAIN_LAUNCH(true, false, CM_)
#define SLSTM_CHAIN_FT(CM_) SLSTM_CHAIN_LAUNCH(false, true, CM_)
#define SLSTM_CHAIN_FF(CM_) SLSTM_CHAIN_LAUNCH(false, false, CM_)
  if (p_bf16) {
    if (last) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_CHAIN_TT) }
    else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_CHAIN_TF) }
  } else {
    if (last) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_CHAIN_FT) }
    else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_CHAIN_FF) }
  }
#undef SLSTM_CHAIN_TT
#undef SLSTM_CHAIN_TF
#undef SLSTM_CHAIN_FT
#undef SLSTM_CHAIN_FF
#undef SLSTM_CHAIN_LAUNCH
  return hipGetLastError();
}

}  // namespace slstm
