// Sequential forward: s_t = f(s_{t-1}) for t = 1..T from s_0 = state0, one thread per lane.
//
// This is the step loop of the sequential solver mode and, at T = 1, the decode step
// ("sLSTM in this library", "API notes": the sequential path in eval mode; at T = 1 one
// launch for the recurrent step, with W_x applied as a separate GEMM). Under channelwise
// mixing each lane (b, j) is an independent recurrence, so lanes run in parallel and each
// thread walks its lane through time. Pre-activations for the next group of steps are loaded
// while the current group is computed. With packed sequences the state restarts from the
// sequence's state0 at each sequence start (see SeqCursor).
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kSeqBlock = 256;
constexpr int kSeqGroup = 4;

template <bool BF16>
__global__ __launch_bounds__(kSeqBlock) void sequential_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    float* __restrict__ S, float* __restrict__ h_out, float* __restrict__ final_state, int B,
    int T, int d, int cell_mode, const int* __restrict__ cu, int n_seqs) {
  const i64 lane = static_cast<i64>(blockIdx.x) * kSeqBlock + threadIdx.x;
  if (lane >= static_cast<i64>(B) * d) return;
  const int b = static_cast<int>(lane / d);
  const int j = static_cast<int>(lane % d);
  const i64 dd = d;
  const i64 d4 = 4 * dd;
  const float rz = R[j], ri = R[dd + j], rf = R[2 * dd + j], ro = R[3 * dd + j];
  const bool sig = (cell_mode & kCellSigmoid) != 0;
  const bool floored = (cell_mode & kCellFloored) != 0;
  CellIn pv = {0.0f, 0.0f, 0.0f, 0.0f};
  SeqCursor cur_seq = seq_cursor(cu, n_seqs, b, 0);
  const i64 lane_base = static_cast<i64>(b) * T * d4 + j;
  float cur[kSeqGroup][4], nxt[kSeqGroup][4];
  auto load_group = [&](int tg, float (&dst)[kSeqGroup][4]) {
#pragma unroll
    for (int u = 0; u < kSeqGroup; ++u) {
      const int t = tg + u;
      const i64 base = lane_base + static_cast<i64>(t) * d4;
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[u][k] = (t < T) ? load_p<BF16>(P, base + k * dd) : 0.0f;
    }
  };
  load_group(0, cur);
  for (int tg = 0; tg < T; tg += kSeqGroup) {
    if (tg + kSeqGroup < T) load_group(tg + kSeqGroup, nxt);
#pragma unroll
    for (int u = 0; u < kSeqGroup; ++u) {
      const int t = tg + u;
      if (t < T) {
        const int sq = seq_begin(cur_seq, t);
        if (sq >= 0) pv = state0_of(state0, sq, static_cast<unsigned>(d), static_cast<unsigned>(j));
        float s[4];
        cell_step<false>(pv, cur[u][0], cur[u][1], cur[u][2], cur[u][3], rz, ri, rf, ro, sig, floored, s,
                         nullptr);
        if (S != nullptr) {  // the states are an output only when asked for
          float* sp = S + lane_base + static_cast<i64>(t) * d4;
          sp[0] = s[0];
          sp[dd] = s[1];
          sp[2 * dd] = s[2];
          sp[3 * dd] = s[3];
        }
        if (h_out != nullptr) h_out[(static_cast<i64>(b) * T + t) * dd + j] = s[3];
        pv = {s[0], s[1], s[2], s[3]};
      }
    }
#pragma unroll
    for (int u = 0; u < kSeqGroup; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) cur[u][k] = nxt[u][k];
  }
  if (final_state != nullptr && cu == nullptr) {  // packed: gathered per sequence afterwards
    float* fs = final_state + static_cast<i64>(b) * d4 + j;
    fs[0] = pv.c;
    fs[dd] = pv.n;
    fs[2 * dd] = pv.m;
    fs[3 * dd] = pv.h;
  }
}

hipError_t launch_sequential(const void* P, bool p_bf16, const float* R, const float* state0,
                             float* S, float* h_out, float* final_state, int B, int T, int d,
                             int cell_mode, hipStream_t stream, Seqs seqs) {
  const i64 lanes = static_cast<i64>(B) * d;
  const i64 blocks = (lanes + kSeqBlock - 1) / kSeqBlock;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int sig = cell_mode;
  if (p_bf16)
    sequential_kernel<true><<<dim3(static_cast<unsigned>(blocks)), kSeqBlock, 0, stream>>>(
        P, R, state0, S, h_out, final_state, B, T, d, sig, seqs.cu, seqs.n);
  else
    sequential_kernel<false><<<dim3(static_cast<unsigned>(blocks)), kSeqBlock, 0, stream>>>(
        P, R, state0, S, h_out, final_state, B, T, d, sig, seqs.cu, seqs.n);
  return hipGetLastError();
}

}  // namespace slstm
