// Backward pass under head mixing ("sLSTM in this library", "Backward": the reverse recurrence
// of the adjoint and the cell's vector-Jacobian product; the head-mixing cell of the "Cell"
// section's mix table). For a loss with direct gradients g_t = dL/ds_t:
//   lam_{T-1} = g_{T-1} (+ dL/d final state),  lam_{t-1} = g_{t-1} + J_t^T lam_t,
//   dP_t = G_t^T lam_t,  dR[g, a, i, k] = sum_{b,t} dP_t[g, a d_head + i] h_{t-1}[a d_head + k],
//   dbias = sum_{b,t} dP_t,  dstate0 = J_0^T lam_0,
// with J_t the per-head Jacobian of step t in factored form: its own-state columns (c', n', m')
// are the channelwise A_own, and its h' column is sum_g R_g^T (G_t^T lam_t)_g, so
//   (J^T lam)[slot] = A_own[:, slot]^T lam  (slot = c, n, m),   (J^T lam)[h'] = sum_g R_g^T dP_g.
//
// Layout as the forward head kernels: a workgroup per (batch row, head) walks T backwards, lane
// 4 i + g for unit i and gate / state slot g. A lane holds row i of gate g's block (for the
// pre-activations, recomputed from the stored states) and column i (for R_g^T dP_g) in
// registers, and its row of dR as running sums over T. Per step: the block product with h' of
// the head (staged in LDS from the states), the cell's gate and own-state Jacobians, dP, then
// one LDS exchange of dP so each lane can form its column's share of R_g^T dP_g, summed over the
// quad. The step is branch-free and the dP stores are batched per 8-step block, as in the
// one-sweep forward. Heads of 64 units keep the block columns in LDS instead (the head's four
// transposed blocks, 64 KiB, rows padded so that the 16 lanes the LDS serves together hit
// distinct banks): a lane's row, column and dR row (192 floats) would not fit the register file.
// Heads of 128 units stream R: the four blocks (256 KiB) fit neither the LDS nor, beside the
// lane's dR row, the registers, so each step reads the lane's row of its block and its column
// (a row of the transposed blocks, written to the workspace first) from memory, as float4
// loads a few at a time (the L2 holds them; every batch row of the head reads the same blocks).
// dR and dbias leave as per-row partial sums that a second kernel adds over the batch in a fixed
// order.
#include "cell.h"
#include "head.h"
#include "kernels.h"

namespace slstm {

// column i of gate g's block of head a: R[g, a, k, i] for k = 0..DH-1
template <int DH>
__device__ __forceinline__ void load_block_col(const float* __restrict__ R, int nh, int a, int i, int g,
                                               float col[DH]) {
  const float* src = R + (static_cast<i64>(g) * nh + a) * DH * DH + i;
#pragma unroll
  for (int k = 0; k < DH; ++k) col[k] = src[k * DH];
}

// Transposed blocks of head a in LDS for heads of 64 units: column i of gate g's block at
// colT[g * kColGate + i * kColRow + k] = R[g, a, k, i]. Rows padded by 4 floats and gates by 16, so
// lane 4 i' + g (i' = 0..3, the 16 lanes served together) reads banks 16 g + 4 i' + (0..3).
template <int DH> struct ColLds {
  static constexpr int kColRow = DH + 4;
  static constexpr int kColGate = DH * kColRow + 16;
  static constexpr int kFloats = 4 * kColGate;
};

template <int DH>
__device__ __forceinline__ void fill_col_lds(const float* __restrict__ R, int nh, int a, float* colT) {
  // thread e of the workgroup copies entries e, e + 4 DH, ...: consecutive threads read
  // consecutive entries of a block row (coalesced) and write them down an LDS column
  for (int e = threadIdx.x; e < 4 * DH * DH; e += 4 * DH) {
    const int g = e / (DH * DH), rest = e - g * DH * DH, k = rest / DH, i = rest - k * DH;
    colT[g * ColLds<DH>::kColGate + i * ColLds<DH>::kColRow + k] = R[(static_cast<i64>(g) * nh + a) * DH * DH + rest];
  }
}

// sum over k of col[k] v[k], col and v both in LDS (float4 reads, two accumulators)
template <int DH>
__device__ __forceinline__ float lds_col_dot(const float* col, const float* v) {
  const float4* c4 = reinterpret_cast<const float4*>(col);
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int k = 0; k < DH / 4; ++k) {
    const float4 c = c4[k], x = v4[k];
    acc0 = fmaf(c.x, x.x, acc0);
    acc1 = fmaf(c.y, x.y, acc1);
    acc0 = fmaf(c.z, x.z, acc0);
    acc1 = fmaf(c.w, x.w, acc1);
  }
  return acc0 + acc1;
}

// Heads of 128 units: row i of gate g's block of M (R, or its transposed blocks) times v (in
// LDS), M read from memory SLSTM_HEAD_STREAM_CHUNK float4 loads at a time
// (4 measured fastest on MI355X, 62 ms for B = 16, T = 4096, 8 heads of 128, against 64 and 67
// for 8 and 16: the walk waits on the L2 for every chunk)
#ifndef SLSTM_HEAD_STREAM_CHUNK
#define SLSTM_HEAD_STREAM_CHUNK 4
#endif
template <int DH>
__device__ __forceinline__ float stream_row_dot(const float* __restrict__ M, int nh, int a, int i, int g,
                                                const float* v) {
  constexpr int kChunk = SLSTM_HEAD_STREAM_CHUNK;
  const float4* src = reinterpret_cast<const float4*>(M + ((static_cast<i64>(g) * nh + a) * DH + i) * DH);
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float acc0 = 0.0f, acc1 = 0.0f;
  // a loop kept rolled: unrolled, the compiler hoists the step-invariant loads out of the walk
  // along T and spills what it hoisted
#pragma unroll 1
  for (int k0 = 0; k0 < DH / 4; k0 += kChunk) {
    float4 r[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) r[k] = src[k0 + k];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float4 x = v4[k0 + k];
      acc0 = fmaf(r[k].x, x.x, acc0);
      acc1 = fmaf(r[k].y, x.y, acc1);
      acc0 = fmaf(r[k].z, x.z, acc0);
      acc1 = fmaf(r[k].w, x.w, acc1);
    }
  }
  return acc0 + acc1;
}

// RT[g, a, i, k] = R[g, a, k, i]: the transposed blocks
__global__ __launch_bounds__(256) void transpose_blocks_kernel(const float* __restrict__ R, float* __restrict__ RT,
                                                               int nh, int dh) {
  const i64 n = static_cast<i64>(4) * nh * dh * dh;
  for (i64 e = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x; e < n; e += static_cast<i64>(gridDim.x) * 256) {
    const i64 blk = e / (static_cast<i64>(dh) * dh);
    const int rest = static_cast<int>(e - blk * dh * dh);
    const int k = rest / dh, i = rest - k * dh;
    RT[blk * dh * dh + static_cast<i64>(i) * dh + k] = R[e];
  }
}

// Packed sequences (PACKED, one batch row): walking T backwards, the kernel follows the sequence
// holding each step; at a sequence's last step its final-state gradient joins the adjoint, and at
// its first step the state before is state0[s] (staged behind an extra barrier), the adjoint
// J^T lam there is dstate0[s], and nothing is carried into the previous sequence.
template <int DH, bool BF16, int CM, bool DP_BF16, bool PACKED>
__global__ __launch_bounds__(4 * DH) void head_backward_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S, const float* __restrict__ g_states, const float* __restrict__ g_h,
    const float* __restrict__ g_final, void* __restrict__ dP, float* __restrict__ dR_part,
    float* __restrict__ db_part, float* __restrict__ dstate0, int T, int d, int nh, Seqs seqs,
    const float* __restrict__ RT) {
  constexpr bool sig = (CM & kCellSigmoid) != 0;
  constexpr bool floored = (CM & kCellFloored) != 0;
  __shared__ __attribute__((aligned(16))) float hbuf[2][DH];      // h of the state before step t
  __shared__ __attribute__((aligned(16))) float dxbuf[2][4][DH];  // dP of step t, per gate
  __shared__ float junk[4 * DH];
  constexpr bool kStream = DH >= 128;  // R read from memory every step
  constexpr bool kColLds = DH == 64;   // block columns in LDS
  __shared__ __attribute__((aligned(16))) float colT[kColLds ? ColLds<DH>::kFloats : 4];
  const int tid = threadIdx.x;
  const int i = tid >> 2, g = tid & 3;
  const int a = blockIdx.x, b = blockIdx.y;
  const int j = a * DH + i;
  const i64 dd = d;
  const GateSel sel(g);
  float row[kStream ? 1 : DH], col[(kColLds || kStream) ? 1 : DH], dr[DH];
  if constexpr (!kStream) load_block_row<DH>(R, nh, a, i, g, row);
  if constexpr (kColLds) fill_col_lds<DH>(R, nh, a, colT);  // visible after the first barrier below
  else if constexpr (!kStream) load_block_col<DH>(R, nh, a, i, g, col);
#pragma unroll
  for (int k = 0; k < DH; ++k) dr[k] = 0.0f;
  float db = 0.0f;
  const i64 base = static_cast<i64>(b) * T * 4 * dd + g * dd + j;  // (b, t = 0, slot/gate g, j)
  const i64 hbase = static_cast<i64>(b) * T * dd + j;              // (b, t = 0, j) of g_h
  const float s0 = state0 != nullptr ? state0[(static_cast<i64>(b) * 4 + g) * dd + j] : 0.0f;
  // optional gradients are read through a valid pointer and selected away when absent
  const bool has_gs = g_states != nullptr, has_gh = g_h != nullptr && g == 3;
  const float* gs_src = has_gs ? g_states : S;
  const float* gh_src = g_h != nullptr ? g_h : S;
  // operands of reverse step r (t = T-1-r, clamped to 0 past the start): p_t, slot g of the state
  // before step t, and the direct gradient at t-1 (none at t = 0)
  auto ld = [&](int r, float& p, float& sp, float& gd) {
    const int t = max(T - 1 - r, 0);
    const i64 tm = static_cast<i64>(max(t - 1, 0));
    p = load_p<BF16>(P, base + static_cast<i64>(t) * 4 * dd);
    const float sv = S[base + tm * 4 * dd];
    const float gsv = gs_src[base + tm * 4 * dd];
    const float ghv = gh_src[hbase + tm * dd];
    sp = t >= 1 ? sv : s0;
    const float gdv = (has_gs ? gsv : 0.0f) + (has_gh ? ghv : 0.0f);
    gd = t >= 1 ? gdv : 0.0f;
  };
  // the adjoint of the last state: direct gradients at T-1 and the final-state gradient
  float lam;
  {
    const i64 tl = static_cast<i64>(T - 1);
    const float gsv = gs_src[base + tl * 4 * dd];
    const float ghv = gh_src[hbase + tl * dd];
    lam = (has_gs ? gsv : 0.0f) + (has_gh ? ghv : 0.0f);
    if (!PACKED && g_final != nullptr) lam += g_final[(static_cast<i64>(b) * 4 + g) * dd + j];
  }
  // the sequence holding the current step (packed), for steps visited in decreasing order
  const SeqCursor c0 = seq_cursor(seqs.cu, seqs.n, 0, T - 1, seqs.tab);
  int rs = c0.s, rstart = c0.start, rend = c0.end;
  float pr[kHeadPrefetch], sr[kHeadPrefetch], gr[kHeadPrefetch];
#pragma unroll
  for (int u = 0; u < kHeadPrefetch; ++u) ld(u, pr[u], sr[u], gr[u]);
  auto h_slot = [&](float* hdst) { return g == 3 ? hdst : &junk[tid]; };
  *h_slot(&hbuf[0][i]) = sr[0];  // h before step T-1
  float d0 = 0.0f;
  head_lds_barrier();

  for (int r0 = 0; r0 < T; r0 += kHeadPrefetch) {
    float out[kHeadPrefetch];
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) {
      const int r = r0 + u;
      const int t = T - 1 - r;
      const bool real = t >= 0;
      const float p = pr[u], gd = gr[u];
      float sp = sr[u];
      ld(r + kHeadPrefetch, pr[u], sr[u], gr[u]);
      const float sp_next = sr[(u + 1) % kHeadPrefetch];  // slot g of the state before step t-1
      const float* hb = hbuf[r & 1];
      bool seq_first = false;
      if constexpr (PACKED) {
        if (real) {
          while (t < rstart && rs > 0) {
            --rs;
            rstart = seqs.cu[rs];
            rend = seqs.cu[rs + 1];
          }
          if (t == rend - 1 && g_final != nullptr) lam += g_final[(static_cast<i64>(rs) * 4 + g) * dd + j];
          seq_first = t == rstart;
          if (seq_first) {  // the state before this step is state0[rs]
            sp = state0 != nullptr ? state0[(static_cast<i64>(rs) * 4 + g) * dd + j] : 0.0f;
            if (g == 3) hbuf[r & 1][i] = sp;
            head_lds_barrier();
          }
        }
      }
      // the step's pre-activations and Jacobians at the stored state before it
      float xs[4], ps[4], ls[4];
      if constexpr (kStream) quad_gather(p + stream_row_dot<DH>(R, nh, a, i, g, hb), xs);
      else quad_gather(p + block_dot<DH>(row, hb), xs);
      quad_gather(sp, ps);
      quad_gather(lam, ls);
      float s[4], dxv[4], dpv[3];
      CellLin L;
      cell_step_lin(CellIn{ps[0], ps[1], ps[2], 0.0f}, xs, sig, floored, s, L);
      cell_vjp_lin(L, ls, dxv, dpv);
      const float dx = sel(dxv);  // dP_t for gate g
      out[u] = dx;
      const float dxm = real ? dx : 0.0f;
      const float4* h4 = reinterpret_cast<const float4*>(hb);
#pragma unroll
      for (int k = 0; k < DH / 4; ++k) {
        const float4 hv = h4[k];
        dr[4 * k] = fmaf(dxm, hv.x, dr[4 * k]);
        dr[4 * k + 1] = fmaf(dxm, hv.y, dr[4 * k + 1]);
        dr[4 * k + 2] = fmaf(dxm, hv.z, dr[4 * k + 2]);
        dr[4 * k + 3] = fmaf(dxm, hv.w, dr[4 * k + 3]);
      }
      if constexpr (DH >= 64) {
        // keep the step's dR update here: left free, the compiler sinks all eight steps' updates
        // to the end of the block and holds their h rows in scratch
#pragma unroll
        for (int k = 0; k < DH; ++k) asm volatile("" : "+v"(dr[k]));
      }
      db += dxm;
      const float la = sel(dpv[0], dpv[1], dpv[2], 0.0f);  // own-state columns of J^T lam (g < 3)
      dxbuf[r & 1][g][i] = dx;
      *h_slot(&hbuf[(r + 1) & 1][i]) = sp_next;
      head_lds_barrier();
      // h' column of J^T lam for unit i: sum over gates of (R_g^T dP_g)[i]
      float ys[4];
      if constexpr (kColLds)
        quad_gather(lds_col_dot<DH>(&colT[g * ColLds<DH>::kColGate + i * ColLds<DH>::kColRow], dxbuf[r & 1][g]), ys);
      else if constexpr (kStream)
        quad_gather(stream_row_dot<DH>(RT, nh, a, i, g, dxbuf[r & 1][g]), ys);
      else
        quad_gather(block_dot<DH>(col, dxbuf[r & 1][g]), ys);
      const float lprev = g == 3 ? (ys[0] + ys[1]) + (ys[2] + ys[3]) : la;
      if constexpr (PACKED) {
        if (seq_first) {  // the adjoint of state0[rs]; nothing crosses into the previous sequence
          if (dstate0 != nullptr) dstate0[(static_cast<i64>(rs) * 4 + g) * dd + j] = lprev;
          lam = gd;
        } else {
          lam = gd + lprev;
        }
      } else {
        d0 = t == 0 ? lprev : d0;
        lam = gd + lprev;
      }
    }
    // this block's dP, in order of the steps
#pragma unroll
    for (int u = 0; u < kHeadPrefetch; ++u) {
      const int t = T - 1 - (r0 + u);
      if (t >= 0) {
        const i64 off = base + static_cast<i64>(t) * 4 * dd;
        if constexpr (DP_BF16) static_cast<uint16_t*>(dP)[off] = f32_to_bf16_rne(out[u]);
        else static_cast<float*>(dP)[off] = out[u];
      }
    }
  }
  // per-row partial sums of dR (this lane's row of block (g, a)) and dbias; dstate0
  float4* dst = reinterpret_cast<float4*>(dR_part + (((static_cast<i64>(b) * 4 + g) * nh + a) * DH + i) * DH);
#pragma unroll
  for (int k = 0; k < DH / 4; ++k) dst[k] = make_float4(dr[4 * k], dr[4 * k + 1], dr[4 * k + 2], dr[4 * k + 3]);
  db_part[(static_cast<i64>(b) * 4 + g) * dd + j] = db;
  if (!PACKED && dstate0 != nullptr) dstate0[(static_cast<i64>(b) * 4 + g) * dd + j] = d0;
}

// packed: an empty sequence passes its final-state gradient (or zero) to dstate0
__global__ __launch_bounds__(256) void head_empty_seq_dstate0_kernel(const int* __restrict__ cu, int n_seqs,
                                                                     const float* __restrict__ g_final,
                                                                     float* __restrict__ dstate0, int d) {
  const i64 n = static_cast<i64>(n_seqs) * 4 * d;
  for (i64 e = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x; e < n; e += static_cast<i64>(gridDim.x) * 256) {
    const int sq = static_cast<int>(e / (4 * static_cast<i64>(d)));
    if (cu[sq] == cu[sq + 1]) dstate0[e] = g_final != nullptr ? g_final[e] : 0.0f;
  }
}

// out[e] = sum over b = 0..B-1 of part[b n + e], added in order of b
__global__ __launch_bounds__(256) void batch_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                       i64 n, int B) {
  const i64 stride = static_cast<i64>(gridDim.x) * 256;
  for (i64 e = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x; e < n; e += stride) {
    float acc = 0.0f;
    for (int bb = 0; bb < B; ++bb) acc += part[static_cast<i64>(bb) * n + e];
    out[e] = acc;
  }
}

size_t head_backward_part_floats(int B, int d, int n_heads) {
  const i64 dh = d / n_heads;
  const size_t rt = dh >= 128 ? static_cast<size_t>(4) * d * dh : 0;  // transposed blocks, streamed heads
  return static_cast<size_t>(B) * 4 * d * dh + static_cast<size_t>(B) * 4 * d + rt;
}

bool head_backward_width_supported(int d_head) {
  return d_head == 8 || d_head == 16 || d_head == 32 || d_head == 64 || d_head == 128;
}

#define SLSTM_HEAD_BWD_DH_DISPATCH(DHV, BODY)        \
  switch (DHV) {                                     \
    case 8: { constexpr int DH = 8; BODY; break; }   \
    case 16: { constexpr int DH = 16; BODY; break; } \
    case 32: { constexpr int DH = 32; BODY; break; } \
    case 64: { constexpr int DH = 64; BODY; break; } \
    case 128: { constexpr int DH = 128; BODY; break; } \
    default: return hipErrorInvalidValue;            \
  }

hipError_t launch_head_backward(const void* P, bool p_bf16, const float* R, const float* state0, const float* S,
                                const float* g_states, const float* g_h, const float* g_final, void* dP,
                                bool dp_bf16, float* dR, float* dbias, float* dstate0, int B, int T, int d,
                                int n_heads, int cell_mode, float* part, hipStream_t stream, Seqs seqs) {
  if (n_heads < 1 || d % n_heads != 0 || B > 65535) return hipErrorInvalidValue;
  const int dh = d / n_heads;
  float* dR_part = part;
  float* db_part = part + static_cast<i64>(B) * 4 * d * dh;
  float* RT = nullptr;
  if (dh >= 128) {  // the transposed blocks the streamed heads read their columns from
    RT = db_part + static_cast<i64>(B) * 4 * d;
    const i64 n = static_cast<i64>(4) * d * dh;
    transpose_blocks_kernel<<<static_cast<unsigned>(std::min<i64>((n + 255) / 256, 4096)), 256, 0, stream>>>(
        R, RT, n_heads, dh);
  }
  const dim3 grid(static_cast<unsigned>(n_heads), static_cast<unsigned>(B));
  // static LDS of a workgroup: the exchange buffers, and for 64-unit heads the transposed blocks
  const unsigned int lds = head_spread_lds(static_cast<long long>(n_heads) * B,
                                           8192 + (dh == 64 ? ColLds<64>::kFloats * 4u : 0u));
  const bool packed = seqs.cu != nullptr;
#define SLSTM_HEAD_BWD(BF, DB, CM_)                                                                             \
  do {                                                                                                          \
    if (packed)                                                                                                 \
      head_backward_kernel<DH, BF, CM_, DB, true><<<grid, 4 * DH, lds, stream>>>(                               \
          P, R, state0, S, g_states, g_h, g_final, dP, dR_part, db_part, dstate0, T, d, n_heads, seqs, RT);     \
    else                                                                                                        \
      head_backward_kernel<DH, BF, CM_, DB, false><<<grid, 4 * DH, lds, stream>>>(                              \
          P, R, state0, S, g_states, g_h, g_final, dP, dR_part, db_part, dstate0, T, d, n_heads, seqs, RT);     \
  } while (0)
#define SLSTM_HEAD_BWD_TT(CM_) SLSTM_HEAD_BWD(true, true, CM_)
#define SLSTM_HEAD_BWD_TF(CM_) SLSTM_HEAD_BWD(true, false, CM_)
#define SLSTM_HEAD_BWD_FT(CM_) SLSTM_HEAD_BWD(false, true, CM_)
#define SLSTM_HEAD_BWD_FF(CM_) SLSTM_HEAD_BWD(false, false, CM_)
  SLSTM_HEAD_BWD_DH_DISPATCH(dh, {
    if (p_bf16) {
      if (dp_bf16) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_BWD_TT) }
      else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_BWD_TF) }
    } else {
      if (dp_bf16) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_BWD_FT) }
      else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_HEAD_BWD_FF) }
    }
  })
#undef SLSTM_HEAD_BWD_TT
#undef SLSTM_HEAD_BWD_TF
#undef SLSTM_HEAD_BWD_FT
#undef SLSTM_HEAD_BWD_FF
#undef SLSTM_HEAD_BWD
#undef SLSTM_HEAD_BWD_DH_DISPATCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const i64 n_dr = static_cast<i64>(4) * d * dh;
  batch_sum_kernel<<<static_cast<unsigned>(std::min<i64>((n_dr + 255) / 256, 2048)), 256, 0, stream>>>(dR_part, dR,
                                                                                                       n_dr, B);
  if (packed && dstate0 != nullptr && seqs.n > 0) {
    const i64 n0 = static_cast<i64>(seqs.n) * 4 * d;
    head_empty_seq_dstate0_kernel<<<static_cast<unsigned>(std::min<i64>((n0 + 255) / 256, 2048)), 256, 0, stream>>>(
        seqs.cu, seqs.n, g_final, dstate0, d);
  }
  if (dbias != nullptr) {
    const i64 n_db = static_cast<i64>(4) * d;
    batch_sum_kernel<<<static_cast<unsigned>(std::min<i64>((n_db + 255) / 256, 2048)), 256, 0, stream>>>(db_part,
                                                                                                         dbias, n_db, B);
  }
  return hipGetLastError();
}

}  // namespace slstm
