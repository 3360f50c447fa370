// Backward of the forward recurrence s_t = f(s_{t-1}, P_t) ("sLSTM in this library", section
// "Backward": one reverse pass of the transposed Jacobians, then the cell's vector-Jacobian
// product for the gradients of R and W_x), chain form.
//
// Per lane (b, j), with g_t the direct gradient of the loss with respect to the state s_t:
//   lam_{T-1} = g_{T-1} (+ the gradient of the final state),  lam_t = g_t + A_{t+1}^T lam_{t+1}
//   dP_t = G_t^T lam_t,  dR = sum over b and t of dP_t * h_{t-1},  dstate0 = A_0^T lam_0
// (A_t = d s_t / d s_{t-1}, G_t = d s_t / d x~_t; cell_vjp forms both products at once from
// the stored state before the step.)
//
// A thread owns one feature and kBackSteps consecutive steps and runs them from the last to the
// first; the adjoint entering its tile from the tile after it (A^T lam of that tile's first
// step) and the running sum of the tile's dR contributions come as epoch-tagged words (see
// tag_store). Tiles take tickets from the last tile along T to the first, so the tile a tile
// waits on holds an earlier ticket of the same counter and runs. The first tile along T holds
// the lane's dR over all of T; it writes it per batch row, and a second kernel sums the batch
// rows in a fixed order. Every value is formed in one fixed order: bitwise reproducible.
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kBackBlock = 256;  // one feature per thread
#ifndef SLSTM_BACK_STEPS
#define SLSTM_BACK_STEPS 8
#endif
#ifndef SLSTM_BACK_MIN_WAVES
#define SLSTM_BACK_MIN_WAVES 3
#endif
constexpr int kBackSteps = SLSTM_BACK_STEPS;  // steps per tile
constexpr int kBackWords = 8;                 // per lane and tile: adjoint (4), running dR (4)

template <bool BF16, bool SIG>
__global__ __launch_bounds__(kBackBlock, SLSTM_BACK_MIN_WAVES) void backward_chain_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S, const float* __restrict__ g, const float* __restrict__ g_h,
    const float* __restrict__ g_final, float* __restrict__ dP, float* __restrict__ dstate0,
    float* __restrict__ dR_rows, int T, int d, int n_jt, int n_lg, int n_tt,
    unsigned long long* __restrict__ carry, unsigned int* __restrict__ tickets, int n_ctr,
    uint32_t epoch) {
  constexpr int TC = kBackSteps;
  constexpr bool sig = SIG;
  __shared__ int s_tile[2];
  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  __syncthreads();
  // tickets run from the last tile along T to the first
  const int tt = n_tt - 1 - __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;
  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * kBackBlock + tid);
  if (j >= ud) return;  // no other thread waits on this lane
  const int t0 = tt * TC;
  const int n_in = min(TC, T - t0);
  const i64 n_lanes = static_cast<i64>(n_lg) * kBackBlock;
  const i64 lane = static_cast<i64>(lg) * kBackBlock + tid;
  auto word = [&](int tile, int e) { return carry + (static_cast<i64>(tile) * kBackWords + e) * n_lanes + lane; };

  // the adjoint entering from the tile after this one, loaded now so that it arrives meanwhile
  unsigned long long pf[kBackWords];
#pragma unroll
  for (int e = 0; e < kBackWords; ++e) pf[e] = 0ull;
  if (tt + 1 < n_tt) {
#pragma unroll
    for (int e = 0; e < kBackWords; ++e)
      pf[e] = __hip_atomic_load(word(tt + 1, e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // the tile's operands: lane part j in the vector offset, step and slot in the scalar offset
  const i64 row = static_cast<i64>(b) * T + t0;
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + row * 4 * static_cast<i64>(d) * (BF16 ? 2 : 4));
  const rsrc_t rsS = make_rsrc(S + row * 4 * static_cast<i64>(d));
  const rsrc_t rsD = make_rsrc(dP + row * 4 * static_cast<i64>(d));
  float p[TC][4], s[TC][4], gs[TC][4];
#pragma unroll
  for (int u = 0; u < TC; ++u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[u][k] = 0.0f;
      s[u][k] = 0.0f;
      gs[u][k] = 0.0f;
    }
    if (u < n_in) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        p[u][k] = buf_ld_p<BF16>(rsP, j, (4u * u + k) * ud);
        s[u][k] = buf_ld(rsS, 4u * j, 4u * (4u * u + k) * ud);
      }
      if (g != nullptr) {
        const float* gr = g + (row + u) * 4 * static_cast<i64>(d);
#pragma unroll
        for (int k = 0; k < 4; ++k) gs[u][k] = gr[k * ud + j];
      }
      if (g_h != nullptr) gs[u][3] += g_h[(row + u) * static_cast<i64>(d) + j];
    }
  }
  // the state before the tile
  CellIn halo = {0.0f, 0.0f, 0.0f, 0.0f};
  if (t0 == 0) {
    if (state0 != nullptr) {
      const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
      halo = {s0[j], s0[ud + j], s0[2 * ud + j], s0[3 * ud + j]};
    }
  } else {
    const float* sp = S + (row - 1) * 4 * static_cast<i64>(d);
    halo = {sp[j], sp[ud + j], sp[2 * ud + j], sp[3 * ud + j]};
  }
  const float rz = R[j], ri = R[ud + j], rf = R[2 * ud + j], ro = R[3 * ud + j];

  // the adjoint contribution entering from after the tile, and the running dR
  float lin[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (tt + 1 < n_tt) {
    bool ok = true;
    float v[kBackWords];
#pragma unroll
    for (int e = 0; e < kBackWords; ++e) {
      v[e] = __uint_as_float(static_cast<uint32_t>(pf[e]));
      ok &= static_cast<uint32_t>(pf[e] >> 32) == epoch;
    }
    while (!ok) {
      // the tile after holds an earlier ticket of the same counter, so it runs
      __builtin_amdgcn_s_sleep(2);
      ok = true;
#pragma unroll
      for (int e = 0; e < kBackWords; ++e) ok &= tag_load(word(tt + 1, e), epoch, v[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lin[e] = v[e];
      dr[e] = v[4 + e];
    }
  } else if (g_final != nullptr) {
    const float* gf = g_final + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
    for (int e = 0; e < 4; ++e) lin[e] = gf[e * ud + j];
  }

  // ---- the steps of the tile, last to first ----
#pragma unroll
  for (int u = TC - 1; u >= 0; --u) {
    if (u < n_in) {
      float lam[4], dx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lam[e] = gs[u][e] + lin[e];
      const CellIn pv = (u == 0) ? halo : CellIn{s[u - 1][0], s[u - 1][1], s[u - 1][2], s[u - 1][3]};
      cell_vjp(pv, p[u][0], p[u][1], p[u][2], p[u][3], rz, ri, rf, ro, sig, lam, dx, lin);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        buf_st(dx[e], rsD, 4u * j, 4u * (4u * u + e) * ud);
        dr[e] = fmaf(dx[e], pv.h, dr[e]);
      }
    }
  }

  if (tt > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tag_store(word(tt, e), lin[e], epoch);
      tag_store(word(tt, 4 + e), dr[e], epoch);
    }
  } else {
    if (dstate0 != nullptr) {
      float* ds = dstate0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[e * ud + j] = lin[e];
    }
    float* rows = dR_rows + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
    for (int e = 0; e < 4; ++e) rows[e * ud + j] = dr[e];
  }
}

// dR[g, j] = sum over batch rows b of dR_rows[b, g, j], in order of b
__global__ __launch_bounds__(256) void sum_rows_kernel(const float* __restrict__ rows, float* __restrict__ out,
                                                       int B, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.0f;
  for (int b = 0; b < B; ++b) acc += rows[static_cast<i64>(b) * n + i];
  out[i] = acc;
}

static void back_grid(int B, int T, int d, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + kBackBlock - 1) / kBackBlock;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + kBackSteps - 1) / kBackSteps;
}

size_t backward_desc_words(int B, int T, int d) {
  i64 n_jt, n_lg, n_tt;
  back_grid(B, T, d, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * kBackWords * n_lg * kBackBlock);
}

hipError_t launch_backward_chain(const void* P, bool p_bf16, const float* R, const float* state0,
                                 const float* S, const float* g, const float* g_h,
                                 const float* g_final, float* dP, float* dR, float* dstate0,
                                 float* dR_rows, int B, int T, int d, bool sig_forget,
                                 unsigned long long* carry, unsigned int* tickets, uint32_t epoch,
                                 hipStream_t stream) {
  i64 n_jt, n_lg, n_tt;
  back_grid(B, T, d, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int a = static_cast<int>(n_jt), c = static_cast<int>(n_lg), e = static_cast<int>(n_tt);
#define SLSTM_BACK_LAUNCH(BF, SG)                                                                         \
  backward_chain_kernel<BF, SG><<<grid, kBackBlock, 0, stream>>>(P, R, state0, S, g, g_h, g_final, dP,    \
                                                                 dstate0, dR_rows, T, d, a, c, e, carry, \
                                                                 tickets, n_ctr, epoch)
  if (p_bf16) {
    if (sig_forget) SLSTM_BACK_LAUNCH(true, true);
    else SLSTM_BACK_LAUNCH(true, false);
  } else {
    if (sig_forget) SLSTM_BACK_LAUNCH(false, true);
    else SLSTM_BACK_LAUNCH(false, false);
  }
#undef SLSTM_BACK_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n = 4 * d;
  sum_rows_kernel<<<(n + 255) / 256, 256, 0, stream>>>(dR_rows, dR, B, n);
  return hipGetLastError();
}

}  // namespace slstm
