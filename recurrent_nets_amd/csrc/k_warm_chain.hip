// Initial Newton iterate by chains along T: the same trajectory as the look-back warm start
// (the sLSTM cell with the recurrent term R h_{t-1} removed from the pre-activations; with R
// dropped step t maps (m, c, n) to
//   m' = max(l_t + m, i~_t),  c' = e^{l_t + m - m'} c + e^{i~_t - m'} z_t,
//   n' = e^{l_t + m - m'} n + e^{i~_t - m'},  h' = sigma(p_o) c' / n'
// with the stabiliser of the educational reimplementation page, "Exponential gating + the
// stabilizer (the crux)"; z = tanh, l = f~ or log sigma(f~)), computed as a plain recurrence.
//
// A thread owns one feature and kWarmChainSteps consecutive steps. The gate terms of all its
// steps (z, sigma(p_o), i~, l) depend on P alone and are formed before the thread needs the
// state entering its tile, which the tile before publishes as three epoch-tagged words
// (m, c, n; see tag_store). The dependent part of a step is then two exponentials and a
// reciprocal. No run aggregates are composed and nothing is re-run, so the kernel reads P once
// and writes the states once; the price is a chain along T, which costs no waiting when there
// are at least as many lane groups as compute units (a tile's predecessor holds a ticket n_lg
// places earlier and has finished). Bitwise reproducible: one fixed order of operations.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kWarmChainBlock = 256;  // one feature per thread
#ifndef SLSTM_WARM_CHAIN_STEPS
#define SLSTM_WARM_CHAIN_STEPS 32
#endif
#ifndef SLSTM_WARM_CHAIN_MIN_WAVES
#define SLSTM_WARM_CHAIN_MIN_WAVES 3
#endif
constexpr int kWarmChainSteps = SLSTM_WARM_CHAIN_STEPS;  // steps per tile

template <bool BF16, int CM>
__global__ __launch_bounds__(kWarmChainBlock, SLSTM_WARM_CHAIN_MIN_WAVES) void warm_chain_kernel(
    const void* __restrict__ P, const float* __restrict__ state0, float* __restrict__ S, int T,
    int d, int n_jt, int n_lg, int n_tt, unsigned long long* __restrict__ carry,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch) {
  constexpr int TC = kWarmChainSteps;
  __shared__ int s_tile[2];
  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;
  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * kWarmChainBlock + tid);
  if (j >= ud) return;  // no other thread waits on this lane
  const int t0 = tt * TC;
  const i64 n_lanes = static_cast<i64>(n_lg) * kWarmChainBlock;
  const i64 lane = static_cast<i64>(lg) * kWarmChainBlock + tid;
  auto carry_word = [&](int tile, int e) { return carry + (static_cast<i64>(tile) * 3 + e) * n_lanes + lane; };
  constexpr bool sig = (CM & kCellSigmoid) != 0;   // forget-gate form and read-out,
  constexpr bool floored = (CM & kCellFloored) != 0;  // fixed per instantiation

  // the state entering the tile: prefetched from the tile before, or state0
  unsigned long long pf[3] = {0ull, 0ull, 0ull};
  if (tt > 0) {
#pragma unroll
    for (int e = 0; e < 3; ++e)
      pf[e] = __hip_atomic_load(carry_word(tt - 1, e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const i64 tile_row = (static_cast<i64>(b) * T + t0) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  const rsrc_t rsS = make_rsrc(S + tile_row);
  float lf[TC], it[TC], zz[TC], oo[TC];
#pragma unroll
  for (int u = 0; u < TC; ++u) {
    if (t0 + u < T) {
      const unsigned o = u * 4u * ud + j;
      const float pz = buf_ld_p<BF16>(rsP, o, 0);
      const float pi = buf_ld_p<BF16>(rsP, o, ud);
      const float pf_ = buf_ld_p<BF16>(rsP, o, 2 * ud);
      const float po = buf_ld_p<BF16>(rsP, o, 3 * ud);
      zz[u] = tanh_fast(pz);
      oo[u] = sigmoidf(po);
      it[u] = pi;
      lf[u] = sig ? log_sigmoidf(pf_) : pf_;
    }
  }

  float m = 0.0f, c = 0.0f, n = 0.0f;
  if (tt == 0) {
    if (state0 != nullptr) {
      const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
      c = s0[j];
      n = s0[ud + j];
      m = s0[2 * ud + j];
    }
  } else {
    bool ok = static_cast<uint32_t>(pf[0] >> 32) == epoch && static_cast<uint32_t>(pf[1] >> 32) == epoch &&
              static_cast<uint32_t>(pf[2] >> 32) == epoch;
    m = __uint_as_float(static_cast<uint32_t>(pf[0]));
    c = __uint_as_float(static_cast<uint32_t>(pf[1]));
    n = __uint_as_float(static_cast<uint32_t>(pf[2]));
    while (!ok) {
      // the tile before holds an earlier ticket of the same counter, so it runs
      poll_pause();
      ok = tag_load(carry_word(tt - 1, 0), epoch, m) & tag_load(carry_word(tt - 1, 1), epoch, c) &
           tag_load(carry_word(tt - 1, 2), epoch, n);
    }
  }

#pragma unroll
  for (int u = 0; u < TC; ++u) {
    if (t0 + u < T) {
      float mn, ig, fg;
      stab_gates(lf[u] + m, it[u], mn, ig, fg);
      c = fmaf(fg, c, ig * zz[u]);
      n = fmaf(fg, n, ig);
      m = mn;
      const unsigned o = 4u * (u * 4u * ud + j);
      buf_st(c, rsS, o, 0);
      buf_st(n, rsS, o, 4u * ud);
      buf_st(m, rsS, o, 8u * ud);
      buf_st(oo[u] * c * readout(n, m, floored).rD, rsS, o, 12u * ud);
    }
  }
  if (tt + 1 < n_tt) {
    tag_store(carry_word(tt, 0), m, epoch);
    tag_store(carry_word(tt, 1), c, epoch);
    tag_store(carry_word(tt, 2), n, epoch);
  }
}

static void warm_chain_grid(int B, int T, int d, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + kWarmChainBlock - 1) / kWarmChainBlock;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + kWarmChainSteps - 1) / kWarmChainSteps;
}

size_t warm_chain_desc_words(int B, int T, int d) {
  i64 n_jt, n_lg, n_tt;
  warm_chain_grid(B, T, d, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * 3 * n_lg * kWarmChainBlock);
}

hipError_t launch_warm_chain(const void* P, bool p_bf16, const float* state0, float* S, int B,
                             int T, int d, int cell_mode, unsigned long long* carry,
                             unsigned int* tickets, uint32_t epoch, hipStream_t stream) {
  i64 n_jt, n_lg, n_tt;
  warm_chain_grid(B, T, d, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  const int n_ctr = ticket_counters(n_lg);
  const int a = static_cast<int>(n_jt), c = static_cast<int>(n_lg), e = static_cast<int>(n_tt);
#define SLSTM_WARM_LAUNCH(BF, CM_)                                                                          \
  warm_chain_kernel<BF, CM_><<<grid, kWarmChainBlock, 0, stream>>>(P, state0, S, T, d, a, c, e, carry, tickets, \
                                                                   n_ctr, epoch)
#define SLSTM_WARM_T(CM_) SLSTM_WARM_LAUNCH(true, CM_)
#define SLSTM_WARM_F(CM_) SLSTM_WARM_LAUNCH(false, CM_)
  if (p_bf16) {
    SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_WARM_T)
  } else {
    SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_WARM_F)
  }
#undef SLSTM_WARM_T
#undef SLSTM_WARM_F
#undef SLSTM_WARM_LAUNCH
  return hipGetLastError();
}

}  // namespace slstm
