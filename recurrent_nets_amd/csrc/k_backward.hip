// Backward of the forward recurrence s_t = f(s_{t-1}, P_t) ("sLSTM in this library", section
// "Backward": the adjoint is one reverse scan of the transposed Jacobians, then the cell's
// vector-Jacobian product gives the gradients of R and W_x).
//
// Per lane (b, j), with g_t the direct gradient of the loss with respect to the state s_t:
//   lam_{T-1} = g_{T-1} (+ the gradient of the final state),  lam_t = g_t + A_{t+1}^T lam_{t+1}
//   dP_t = G_t^T lam_t,  dR = sum over b and t of dP_t * h_{t-1},  dbias = sum of dP_t,
//   dstate0 = A_0^T lam_0
// (A_t = d s_t / d s_{t-1}, G_t = d s_t / d x~_t; cell_vjp forms both products at once from
// the stored state before the step.) The value y_t = A_t^T lam_t handed from step t to step
// t-1 obeys the affine recurrence y_{t-1} = A_t^T (g_t + y_t), run from t = T-1 down to 0.
//
// Two layouts, as for the forward solve:
// * chains: a thread owns one feature and kBackSteps consecutive steps and runs them from the
//   last to the first; y entering its tile (from the tile after it) comes as four epoch-tagged
//   words (see tag_store). Tiles take tickets from the last tile along T to the first, so the
//   tile a tile waits on holds an earlier ticket of the same counter and runs.
// * scan: the four threads of a quad hold four consecutive sub-chunks of one feature (the
//   last in time first), compose their steps' maps y -> A_t^T (g_t + y) into one affine map,
//   scan the maps across the quad and look back across tiles (quad_look_back, tiles in reverse
//   order of time), then run their steps again from the y entering them. Parallel along T at
//   any batch size. With packed sequences (PACKED) the map of a sequence's first step is zero
//   (nothing flows back across the boundary) and its A^T lam is that sequence's dstate0.
// Each tile writes its lane's sums of dP_t h_{t-1} and of dP_t (a row of 8 d floats per batch
// row and tile), and two small kernels add the rows in a fixed order into dR and dbias. dP is
// written as float32 or, for the bf16 weight-gradient GEMMs, rounded to bfloat16. Every value
// is formed in one fixed order: bitwise reproducible.
#include <algorithm>

#include "affine4.h"
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
constexpr int kBackWords = 4;                 // per lane and tile: y entering the tile before

// dP of one step: float32, or bfloat16 rounded to nearest even
__device__ __forceinline__ void store_dp(float v, bool bf16, rsrc_t r, unsigned elem_lane, unsigned elem_uniform) {
  if (bf16)
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), r, 2u * elem_lane, 2u * elem_uniform, 0);
  else
    buf_st(v, r, 4u * elem_lane, 4u * elem_uniform);
}

// GS: a gradient with respect to the states is given (else only dL/dh and the final state's)
template <bool BF16, int CM, bool GS>
__global__ __launch_bounds__(kBackBlock, SLSTM_BACK_MIN_WAVES) void backward_chain_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S, const float* __restrict__ g, const float* __restrict__ g_h,
    const float* __restrict__ g_final, void* __restrict__ dP, int dp_bf16, float* __restrict__ dstate0,
    float* __restrict__ sum_rows, int T, int d, int n_jt, int n_lg, int n_tt,
    unsigned long long* __restrict__ carry, unsigned int* __restrict__ tickets, int n_ctr,
    uint32_t epoch) {
  constexpr int TC = kBackSteps;
  constexpr bool sig = (CM & kCellSigmoid) != 0;   // forget-gate form and read-out,
  constexpr bool floored = (CM & kCellFloored) != 0;  // fixed per instantiation
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
  const bool dpb = dp_bf16 != 0;
  const rsrc_t rsD = make_rsrc(static_cast<char*>(dP) + row * 4 * static_cast<i64>(d) * (dpb ? 2 : 4));
  const rsrc_t rsG = make_rsrc(GS ? g + row * 4 * static_cast<i64>(d) : g);
  const rsrc_t rsH = make_rsrc(g_h != nullptr ? g_h + row * static_cast<i64>(d) : g_h);
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
      if constexpr (GS) {
#pragma unroll
        for (int k = 0; k < 4; ++k) gs[u][k] = buf_ld(rsG, 4u * j, 4u * (4u * u + k) * ud);
      }
      if (g_h != nullptr) gs[u][3] += buf_ld(rsH, 4u * j, 4u * u * ud);
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

  // the adjoint contribution entering from after the tile
  float lin[4] = {0.0f, 0.0f, 0.0f, 0.0f};
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
      poll_pause();
      ok = true;
#pragma unroll
      for (int e = 0; e < kBackWords; ++e) ok &= tag_load(word(tt + 1, e), epoch, v[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) lin[e] = v[e];
  } else if (g_final != nullptr) {
    const float* gf = g_final + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
    for (int e = 0; e < 4; ++e) lin[e] = gf[e * ud + j];
  }

  // ---- the steps of the tile, last to first ----
  float dr[4] = {0.0f, 0.0f, 0.0f, 0.0f}, db[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = TC - 1; u >= 0; --u) {
    if (u < n_in) {
      float lam[4], dx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lam[e] = gs[u][e] + lin[e];
      const CellIn pv = (u == 0) ? halo : CellIn{s[u - 1][0], s[u - 1][1], s[u - 1][2], s[u - 1][3]};
      cell_vjp(pv, p[u][0], p[u][1], p[u][2], p[u][3], rz, ri, rf, ro, sig, floored, lam, dx, lin);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        store_dp(dx[e], dpb, rsD, j, (4u * u + e) * ud);
        dr[e] = fmaf(dx[e], pv.h, dr[e]);
        db[e] += dx[e];
      }
    }
  }
  if (tt > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) tag_store(word(tt, e), lin[e], epoch);
  } else if (dstate0 != nullptr) {
    float* ds = dstate0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[e * ud + j] = lin[e];
  }
  float* rows = sum_rows + (static_cast<i64>(b) * n_tt + tt) * 8 * static_cast<i64>(d);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    rows[e * ud + j] = dr[e];
    rows[(4 + e) * ud + j] = db[e];
  }
}

// ---- scan form ------------------------------------------------------------------------------
// Sub-chunk length and waves per SIMD: the quad scan and look-back cost a fixed number of
// instructions per sub-chunk, so longer sub-chunks spend fewer per step; 8 steps at 2 waves per
// SIMD (the sub-chunk's P, states and gradients in registers, no spills) measured fastest on
// MI355X at every shape tried (4 steps at 3 waves: 5% slower at B=128, 30% at B=4).
#ifndef SLSTM_BACK_SCAN_TSUB
#define SLSTM_BACK_SCAN_TSUB 8
#endif
#ifndef SLSTM_BACK_SCAN_MIN_WAVES
#define SLSTM_BACK_SCAN_MIN_WAVES 2
#endif
constexpr int kBackScanBlock = 256;  // 4 waves x 16 features x 4 sub-chunks
constexpr int kBackScanTSub = SLSTM_BACK_SCAN_TSUB;
// Packed rows on tiles aligned to the sequences (see launch_aligned_tiles): one row's look-back
// words and rows of sums are sized for tiles of kBackAlignedLayoutSteps steps, so that a pack's
// aligned tiles (at most one more per sequence than the row's) fit them. 32-step tiles at three
// workgroups per CU (a few registers spilled), every tile an anchor, measured fastest on MI355X
// (292-sequence pack of 262,144 steps at d_h = 1024: 4.14 ms, against 4.65 at two workgroups per
// CU, 5.13 with 48-step tiles at two, 5.42 with anchors every other tile, 6.56 unaligned)
#ifndef SLSTM_BACK_ALIGNED_TSUB
#define SLSTM_BACK_ALIGNED_TSUB 8
#endif
constexpr int kBackAlignedTSub = SLSTM_BACK_ALIGNED_TSUB;
constexpr int kBackAlignedLayoutSteps = 24;
static_assert(kBackAlignedLayoutSteps < 4 * kBackAlignedTSub, "room for one extra tile per sequence");
static_assert(kBackAlignedLayoutSteps <= 4 * kBackScanTSub, "the row's own tiles fit the layout");
#ifndef SLSTM_BACK_ALIGNED_MIN_WAVES
#define SLSTM_BACK_ALIGNED_MIN_WAVES 3
#endif
#ifndef SLSTM_BACK_ALIGNED_ANCHOR_STRIDE
#define SLSTM_BACK_ALIGNED_ANCHOR_STRIDE 1
#endif

template <bool BF16, int CM, bool GS, int TSUB, bool PACKED, bool ALIGNED>
__global__ __launch_bounds__(kBackScanBlock, (ALIGNED ? SLSTM_BACK_ALIGNED_MIN_WAVES : SLSTM_BACK_SCAN_MIN_WAVES)) void backward_scan_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S, const float* __restrict__ g, const float* __restrict__ g_h,
    const float* __restrict__ g_final, void* __restrict__ dP, int dp_bf16, float* __restrict__ dstate0,
    float* __restrict__ sum_rows, int T, int d, int n_jt, int n_lg, int n_tt, int anchor_stride,
    unsigned long long* __restrict__ desc, unsigned int* __restrict__ tickets, int n_ctr,
    uint32_t epoch, const int* __restrict__ cu, int n_seqs,
    const int* __restrict__ seq_tab, const int* __restrict__ tiles, int tile_cap) {
  constexpr bool sig = (CM & kCellSigmoid) != 0;   // forget-gate form and read-out,
  constexpr bool floored = (CM & kCellFloored) != 0;  // fixed per instantiation
  __shared__ int s_tile[2];
  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  __syncthreads();
  // tickets (and the look-back) run from the last tile along T to the first
  int tr = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;
  // the tile's row of sums, its first step, the end of its steps, the look-back words of its chain
  int tt = n_tt - 1 - tr, row = b * n_tt + tt, t_tile = tt * 4 * TSUB, t_end = T, aseq = -1, a_start = 0;
  unsigned long long* dsc = desc;
  if constexpr (ALIGNED) {
    // slot tr of the table: tile id at position pos of its sequence's chain, counted from the
    // sequence's last tile, so it covers time position nt - 1 - pos of the sequence; the slot's
    // values are read all at once (tr < tile_cap)
    const int n_real = __builtin_amdgcn_readfirstlane(tiles[0]);
    const int id = __builtin_amdgcn_readfirstlane(tiles[1 + tr]);
    const int sq = __builtin_amdgcn_readfirstlane(tiles[1 + tile_cap + tr]);
    const int pos = __builtin_amdgcn_readfirstlane(tiles[1 + 2 * tile_cap + tr]);
    const int a0 = __builtin_amdgcn_readfirstlane(tiles[1 + 3 * tile_cap + tr]);
    const int e0 = __builtin_amdgcn_readfirstlane(tiles[1 + 4 * tile_cap + tr]);
    row = tr;
    if (tr >= n_real) {  // a ticket past the last tile: its row of sums is zero
      const unsigned jz = static_cast<unsigned>(jt * 64) + (threadIdx.x >> 2);
      if ((threadIdx.x & 3) == 0 && jz < static_cast<unsigned>(d)) {
        float* rows = sum_rows + static_cast<i64>(tr) * 8 * static_cast<i64>(d);
#pragma unroll
        for (int e = 0; e < 8; ++e) rows[e * d + jz] = 0.0f;
      }
      return;
    }
    aseq = sq;
    a_start = a0;
    t_end = e0;
    const int nt = (t_end - a_start + 4 * TSUB - 1) / (4 * TSUB);
    t_tile = a_start + (nt - 1 - pos) * 4 * TSUB;
    dsc = desc + static_cast<i64>(id - pos) * kLookBackWords * static_cast<i64>(n_lg) * 64;
    row = id;
    tr = pos;
  }

  // quad position q holds sub-chunk 3 - q: the quad scans in reverse order of time
  const int l = tid & 63;
  const int q = l & 3;
  const int sc = 3 - q;
  const int lane_in_tile = (tid >> 6) * 16 + (l >> 2);
  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * 64 + lane_in_tile);
  const bool valid = j < ud;
  const int t_start = t_tile + sc * TSUB;
  const i64 n_lanes_pad = static_cast<i64>(n_lg) * 64;
  const i64 my_lane = static_cast<i64>(lg) * 64 + lane_in_tile;
  const i64 tile_row = (static_cast<i64>(b) * T + t_tile) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  const rsrc_t rsS = make_rsrc(S + tile_row);
  const bool dpb = dp_bf16 != 0;
  const rsrc_t rsD = make_rsrc(static_cast<char*>(dP) + tile_row * (dpb ? 2 : 4));
  const rsrc_t rsG = make_rsrc(GS ? g + tile_row : g);
  const rsrc_t rsH = make_rsrc(g_h != nullptr ? g_h + (static_cast<i64>(b) * T + t_tile) * static_cast<i64>(d) : g_h);
  const unsigned lane_off = static_cast<unsigned>(sc * TSUB) * 4u * ud + j;  // elements

  const unsigned long long pf = quad_look_back_prefetch(dsc, n_lanes_pad, my_lane, q, tr, anchor_stride);

  // packed: the sequence starting at each step of the sub-chunk and the one ending there (-1: none)
  // (aligned: a tile holds steps of one sequence from a multiple of the tile length on, so only
  // the first step of a sub-chunk can start it and at most one step ends it)
  int sq[PACKED ? TSUB : 1], lq[PACKED ? TSUB : 1];
  bool starts = false;  // aligned: the sub-chunk's first step starts the sequence
  int eu = -1;          // aligned: the sub-chunk's step that ends the sequence
  if constexpr (ALIGNED) {
    starts = t_start == a_start && a_start < t_end;
    if (t_end - 1 >= t_start && t_end - 1 < t_start + TSUB) eu = t_end - 1 - t_start;
  } else if constexpr (PACKED) {
    SeqCursor seq = seq_cursor(cu, n_seqs, b, t_start, seq_tab);
#pragma unroll
    for (int u = 0; u < TSUB; ++u) {
      const int t = t_start + u;
      sq[u] = t < T ? seq_begin(seq, t) : -1;
      lq[u] = (t < T && t + 1 == seq.end) ? seq.s : -1;
    }
  }

  // the sequence starting / ending at step u of the sub-chunk (-1: none)
  auto seq_start = [&](int u) -> int {
    if constexpr (ALIGNED) return (u == 0 && starts) ? aseq : -1;
    else if constexpr (PACKED) return sq[u];
    else return -1;
  };
  auto seq_end = [&](int u) -> int {
    if constexpr (ALIGNED) return u == eu ? aseq : -1;
    else if constexpr (PACKED) return lq[u];
    else return -1;
  };
  float pg[TSUB][4], sv[TSUB][4], gs[TSUB][4];
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pg[u][k] = 0.0f;
      sv[u][k] = 0.0f;
      gs[u][k] = 0.0f;
    }
    const int t = t_start + u;
    if (valid && t < t_end) {
      const unsigned o = lane_off + u * 4u * ud;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[u][k] = buf_ld_p<BF16>(rsP, o, k * ud);
        sv[u][k] = buf_ld(rsS, 4u * o, 4u * k * ud);
      }
      if constexpr (GS) {
#pragma unroll
        for (int k = 0; k < 4; ++k) gs[u][k] = buf_ld(rsG, 4u * o, 4u * k * ud);
      }
      if (g_h != nullptr) gs[u][3] += buf_ld(rsH, 4u * (static_cast<unsigned>(sc * TSUB + u) * ud + j), 0);
      const int fs = (PACKED || ALIGNED) ? seq_end(u) : (t == T - 1 ? b : -1);  // the sequence that ends at t
      if (g_final != nullptr && fs >= 0) {
        const float* gf = g_final + static_cast<i64>(fs) * 4 * static_cast<i64>(d);
#pragma unroll
        for (int k = 0; k < 4; ++k) gs[u][k] += gf[k * ud + j];
      }
    }
  }
  float rz = 0.0f, ri = 0.0f, rf = 0.0f, ro = 0.0f;
  // the state before the sub-chunk: the last step of the sub-chunk before it in time (held by
  // the next thread of the quad), the step before the tile, or the initial state
  CellIn pv0 = {quad_perm<1, 2, 3, 3>(sv[TSUB - 1][0]), quad_perm<1, 2, 3, 3>(sv[TSUB - 1][1]),
                quad_perm<1, 2, 3, 3>(sv[TSUB - 1][2]), quad_perm<1, 2, 3, 3>(sv[TSUB - 1][3])};
  if (valid) {
    rz = R[j];
    ri = R[ud + j];
    rf = R[2 * ud + j];
    ro = R[3 * ud + j];
    if (sc == 0) {
      if (t_start == 0) {
        pv0 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (state0 != nullptr) {
          const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
          pv0 = {s0[j], s0[ud + j], s0[2 * ud + j], s0[3 * ud + j]};
        }
      } else if (t_start < t_end) {
        const float* sp = S + (static_cast<i64>(b) * T + t_start - 1) * 4 * static_cast<i64>(d);
        pv0 = {sp[j], sp[ud + j], sp[2 * ud + j], sp[3 * ud + j]};
      }
    }
  }

  // ---- the sub-chunk's map y -> (M y + v), its steps composed from the last to the first ----
  float M[16], v[4];
#pragma unroll
  for (int e = 0; e < 16; ++e) M[e] = (e % 5 == 0) ? 1.0f : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = 0.0f;
#pragma unroll
  for (int u = TSUB - 1; u >= 0; --u) {
    const int t = t_start + u;
    if (valid && t < t_end) {
      CellIn pv = (u == 0) ? pv0 : CellIn{sv[u - 1][0], sv[u - 1][1], sv[u - 1][2], sv[u - 1][3]};
      if ((PACKED || ALIGNED) && seq_start(u) >= 0) pv = state0_of(state0, seq_start(u), ud, j);
      float f[4], A[16], At[16];
      cell_step<true>(pv, pg[u][0], pg[u][1], pg[u][2], pg[u][3], rz, ri, rf, ro, sig, floored, f, A);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) At[4 * r + c] = A[4 * c + r];
      // (M, v) <- (A^T M, A^T (v + g_t))
      const float w[4] = {v[0] + gs[u][0], v[1] + gs[u][1], v[2] + gs[u][2], v[3] + gs[u][3]};
      const float zero[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      mat4_vec(At, w, zero, v);
      mat4_mul_left(At, M);
    }
    if ((PACKED || ALIGNED) && seq_start(u) >= 0) {
      // a sequence start: nothing flows back to the step before it (padding lanes past d_h
      // too, so that all lanes of a tile agree on where the maps restart)
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = 0.0f;
    }
  }

  // ---- quad scan of the sub-chunk maps, then the look-back across tiles ----
  quad_inclusive_scan(M, v, q);
  float carry[4];
  {
    float arow[4], av;
    quad_row_of_last(M, v, q, arow, av);
    quad_look_back<PACKED>(arow, av, carry, dsc, n_lanes_pad, my_lane, q, tr, anchor_stride, epoch, pf);
  }
  // y entering the sub-chunk: the inclusive value of the thread before in the quad
  float y[4];
  {
    float xe[4];
    mat4_vec(M, carry, v, xe);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = quad_perm<0, 0, 1, 2>(xe[e]);
      if (q == 0) y[e] = carry[e];
    }
  }

  // ---- the steps again, from the last to the first, with the adjoint ----
  float dr[4] = {0.0f, 0.0f, 0.0f, 0.0f}, db[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = TSUB - 1; u >= 0; --u) {
    const int t = t_start + u;
    if (valid && t < t_end) {
      CellIn pv = (u == 0) ? pv0 : CellIn{sv[u - 1][0], sv[u - 1][1], sv[u - 1][2], sv[u - 1][3]};
      if ((PACKED || ALIGNED) && seq_start(u) >= 0) pv = state0_of(state0, seq_start(u), ud, j);
      float lam[4], dx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lam[e] = gs[u][e] + y[e];
      cell_vjp(pv, pg[u][0], pg[u][1], pg[u][2], pg[u][3], rz, ri, rf, ro, sig, floored, lam, dx, y);
      const unsigned o = lane_off + u * 4u * ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        store_dp(dx[e], dpb, rsD, o, e * ud);
        dr[e] = fmaf(dx[e], pv.h, dr[e]);
        db[e] += dx[e];
      }
      if ((PACKED || ALIGNED) && seq_start(u) >= 0) {
        if (dstate0 != nullptr) {
          float* ds = dstate0 + static_cast<i64>(seq_start(u)) * 4 * static_cast<i64>(d);
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[e * ud + j] = y[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = 0.0f;
      }
    }
  }
  // the tile's sums over the quad, in order of time (sub-chunks 3, 2, 1, 0 = q 0..3)
  float tot[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    tot[e] = ((quad_bcast<0>(dr[e]) + quad_bcast<1>(dr[e])) + quad_bcast<2>(dr[e])) + quad_bcast<3>(dr[e]);
    tot[4 + e] = ((quad_bcast<0>(db[e]) + quad_bcast<1>(db[e])) + quad_bcast<2>(db[e])) + quad_bcast<3>(db[e]);
  }
  if (valid && q == 0) {
    float* rows = sum_rows + static_cast<i64>(row) * 8 * static_cast<i64>(d);
#pragma unroll
    for (int e = 0; e < 8; ++e) rows[e * ud + j] = tot[e];
  }
  if (!PACKED && !ALIGNED && valid && t_start == 0 && dstate0 != nullptr) {
    float* ds = dstate0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[e * ud + j] = y[e];
  }

}

// ---- fixed-order sum of the dR rows -------------------------------------------------------------
// rows summed per thread in the first level: about the square root of the row count, so that
// both levels have short loops (a multiple of 8, for the unrolled loads)
static i64 row_chunk(i64 rows) {
  i64 c = 8;
  while (c * c < rows) c += 8;
  return c;
}

// part[c, i] = sum of rows[r, i] over the rows r of chunk c, in order of r
__global__ __launch_bounds__(256) void sum_row_chunks_kernel(const float* __restrict__ rows,
                                                             float* __restrict__ part, int n_rows,
                                                             int chunk, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r0 = blockIdx.y * chunk;
  const int r1 = min(r0 + chunk, n_rows);
  float acc = 0.0f;
#pragma unroll 8
  for (int r = r0; r < r1; ++r) acc += rows[static_cast<i64>(r) * n + i];
  part[static_cast<i64>(blockIdx.y) * n + i] = acc;
}

// sum of part[c, i] over the chunks c, in order of c: into out0[i] for i < n0, else into
// out1[i - n0] (skipped when out1 is null)
__global__ __launch_bounds__(256) void sum_chunks_kernel(const float* __restrict__ part,
                                                         float* __restrict__ out0, float* __restrict__ out1,
                                                         int n_chunks, int n0, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n || (i >= n0 && out1 == nullptr)) return;
  float acc = 0.0f;
#pragma unroll 8
  for (int c = 0; c < n_chunks; ++c) acc += part[static_cast<i64>(c) * n + i];
  if (i < n0) out0[i] = acc;
  else out1[i - n0] = acc;
}

// dstate0 of the empty packed sequences: their final state is state0, so the gradient with
// respect to state0 is g_final (zero without it)
__global__ __launch_bounds__(256) void empty_seq_dstate0_kernel(const int* __restrict__ cu,
                                                                const float* __restrict__ g_final,
                                                                float* __restrict__ dstate0, int n_seqs,
                                                                int d4) {
  const i64 n = static_cast<i64>(n_seqs) * d4;  // (s, slot, j)
  for (i64 o = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x; o < n; o += static_cast<i64>(gridDim.x) * 256) {
    const int s = static_cast<int>(o / d4);
    if (cu[s] == cu[s + 1]) dstate0[o] = g_final != nullptr ? g_final[o] : 0.0f;
  }
}

// ---- sizes and launch ---------------------------------------------------------------------------
struct BackGrid {
  i64 n_jt, n_lg, n_tt, rows;
  i64 layout_tt;  // tiles per row the words and rows of sums hold
};

static BackGrid back_grid(int B, int T, int d, bool scan) {
  BackGrid g;
  if (scan) {
    g.n_jt = (d + 63) / 64;
    g.n_tt = (T + 4 * kBackScanTSub - 1) / (4 * kBackScanTSub);
    g.rows = static_cast<i64>(B) * g.n_tt;
  } else {
    g.n_jt = (d + kBackBlock - 1) / kBackBlock;
    g.n_tt = (T + kBackSteps - 1) / kBackSteps;
    g.rows = static_cast<i64>(B) * g.n_tt;
  }
  g.n_lg = static_cast<i64>(B) * g.n_jt;
  // one row of the scan form (every packed call): room for the aligned tiles
  g.layout_tt = (scan && B == 1) ? (T + kBackAlignedLayoutSteps - 1) / kBackAlignedLayoutSteps : g.n_tt;
  return g;
}

size_t backward_desc_words(int B, int T, int d, bool scan) {
  const BackGrid g = back_grid(B, T, d, scan);
  return static_cast<size_t>(scan ? g.layout_tt * kLookBackWords * g.n_lg * 64 : g.n_tt * kBackWords * g.n_lg * kBackBlock);
}

int backward_aligned_steps() { return 4 * kBackAlignedTSub; }
int backward_aligned_cap(int T) { return static_cast<int>(back_grid(1, T, 1, true).layout_tt); }

size_t backward_row_floats(int B, int T, int d, bool scan) {
  const BackGrid g = back_grid(B, T, d, scan);
  const i64 rows = static_cast<i64>(B) * g.layout_tt;  // at least g.rows
  const i64 chunk = row_chunk(rows);
  const i64 chunks = (rows + chunk - 1) / chunk;
  return static_cast<size_t>((rows + chunks) * 8 * static_cast<i64>(d));
}

hipError_t launch_backward(const void* P, bool p_bf16, const float* R, const float* state0,
                           const float* S, const float* g, const float* g_h, const float* g_final,
                           void* dP, bool dp_bf16, float* dR, float* dbias, float* dstate0,
                           float* rows, int B, int T, int d, int cell_mode, bool scan,
                           unsigned long long* desc, unsigned int* tickets, uint32_t epoch,
                           hipStream_t stream, Seqs seqs) {
  const bool packed = seqs.cu != nullptr;
  if (packed && (!scan || B != 1)) return hipErrorInvalidValue;  // packed: the scan form, one row
  BackGrid gr = back_grid(B, T, d, scan);
  const bool aligned = packed && seqs.tiles != nullptr;
  // aligned: one ticket, and one row of sums, per slot of the tile table (the rows and words
  // hold that many tiles)
  if (aligned) {
    if (seqs.tile_cap != gr.layout_tt) return hipErrorInvalidValue;
    gr.n_tt = gr.layout_tt;
    gr.rows = gr.layout_tt;
  }
  const i64 blocks = gr.n_lg * gr.n_tt;
  const i64 chunk = row_chunk(gr.rows);
  const i64 chunks = (gr.rows + chunk - 1) / chunk;
  if (blocks > 0x7fffffffLL || gr.rows > 0x7fffffffLL) return hipErrorInvalidValue;
  const int n_ctr = ticket_counters(gr.n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int a = static_cast<int>(gr.n_jt), c = static_cast<int>(gr.n_lg), e = static_cast<int>(gr.n_tt);
  const bool gs = g != nullptr;
  const int dpb = dp_bf16 ? 1 : 0;
  // one instantiation per P dtype, cell mode and presence of the state gradient
#define SLSTM_BACK_TT(CM_) SLSTM_BACK_LAUNCH(true, CM_, true)
#define SLSTM_BACK_TF(CM_) SLSTM_BACK_LAUNCH(true, CM_, false)
#define SLSTM_BACK_FT(CM_) SLSTM_BACK_LAUNCH(false, CM_, true)
#define SLSTM_BACK_FF(CM_) SLSTM_BACK_LAUNCH(false, CM_, false)
#define SLSTM_BACK_DISPATCH                                                   \
  do {                                                                        \
    if (p_bf16) {                                                             \
      if (gs) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_BACK_TT) }          \
      else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_BACK_TF) }             \
    } else {                                                                  \
      if (gs) { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_BACK_FT) }          \
      else { SLSTM_CELL_MODE_DISPATCH(cell_mode, SLSTM_BACK_FF) }             \
    }                                                                         \
  } while (0)
  if (scan) {
    const int stride = look_back_anchor_stride(gr.n_lg, SLSTM_BACK_SCAN_MIN_WAVES);
    // packed rows are few lane groups along a long T: anchors every 4 tiles (measured best
    // between 1 and 8 over short and long sequence mixes); on aligned tiles every tile is an
    // anchor, one plain chain per sequence, as in the iteration
    const int stride_used = aligned ? SLSTM_BACK_ALIGNED_ANCHOR_STRIDE : (packed ? kPackedAnchorStride : stride);
    if (aligned) {
#define SLSTM_BACK_LAUNCH(BF, CM_, GS)                                                                        \
  backward_scan_kernel<BF, CM_, GS, kBackAlignedTSub, false, true><<<grid, kBackScanBlock, 0, stream>>>(      \
      P, R, state0, S, g, g_h, g_final, dP, dpb, dstate0, rows, T, d, a, c, e, stride_used, desc, tickets, n_ctr, \
      epoch, seqs.cu, seqs.n, seqs.tab, seqs.tiles, seqs.tile_cap)
      SLSTM_BACK_DISPATCH;
#undef SLSTM_BACK_LAUNCH
    } else if (packed) {
#define SLSTM_BACK_LAUNCH(BF, CM_, GS)                                                                        \
  backward_scan_kernel<BF, CM_, GS, kBackScanTSub, true, false><<<grid, kBackScanBlock, 0, stream>>>(         \
      P, R, state0, S, g, g_h, g_final, dP, dpb, dstate0, rows, T, d, a, c, e, stride_used, desc, tickets, n_ctr, \
      epoch, seqs.cu, seqs.n, seqs.tab, nullptr, 0)
      SLSTM_BACK_DISPATCH;
#undef SLSTM_BACK_LAUNCH
    } else {
#define SLSTM_BACK_LAUNCH(BF, CM_, GS)                                                                        \
  backward_scan_kernel<BF, CM_, GS, kBackScanTSub, false, false><<<grid, kBackScanBlock, 0, stream>>>(        \
      P, R, state0, S, g, g_h, g_final, dP, dpb, dstate0, rows, T, d, a, c, e, stride_used, desc, tickets, n_ctr, \
      epoch, nullptr, 0, nullptr, nullptr, 0)
      SLSTM_BACK_DISPATCH;
#undef SLSTM_BACK_LAUNCH
    }
    if (packed && dstate0 != nullptr && seqs.n > 0) {
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      const i64 n = static_cast<i64>(seqs.n) * 4 * d;
      const unsigned blocks_e = static_cast<unsigned>(std::min<i64>((n + 255) / 256, 4096));
      empty_seq_dstate0_kernel<<<blocks_e, 256, 0, stream>>>(seqs.cu, g_final, dstate0, seqs.n, 4 * d);
    }
  } else {
#define SLSTM_BACK_LAUNCH(BF, CM_, GS)                                                                      \
  backward_chain_kernel<BF, CM_, GS><<<grid, kBackBlock, 0, stream>>>(P, R, state0, S, g, g_h, g_final, dP, \
                                                                      dpb, dstate0, rows, T, d, a, c, e, desc, \
                                                                      tickets, n_ctr, epoch)
    SLSTM_BACK_DISPATCH;
#undef SLSTM_BACK_LAUNCH
  }
#undef SLSTM_BACK_TT
#undef SLSTM_BACK_TF
#undef SLSTM_BACK_FT
#undef SLSTM_BACK_FF
#undef SLSTM_BACK_DISPATCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n = 8 * d;
  float* part = rows + gr.rows * n;
  sum_row_chunks_kernel<<<dim3((n + 255) / 256, static_cast<unsigned>(chunks)), 256, 0, stream>>>(
      rows, part, static_cast<int>(gr.rows), static_cast<int>(chunk), n);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  sum_chunks_kernel<<<(n + 255) / 256, 256, 0, stream>>>(part, dR, dbias, static_cast<int>(chunks), 4 * d, n);
  return hipGetLastError();
}

}  // namespace slstm
