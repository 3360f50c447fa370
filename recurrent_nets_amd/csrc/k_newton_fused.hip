// One Newton iteration in a single pass over HBM: the residual and the 4x4 Jacobian of every
// step are formed in registers, the block-bidiagonal system is solved by the 4x4 affine scan,
// and the updated iterate is written. Reads P and the iterate S_k, writes S_{k+1}; the Jacobian
// and the right-hand side never reach HBM (48 bytes per state element instead of the layered
// kernels' 256 with float32 P).
//
// Per step t of a lane (the method of the "Layout" page of the pararnn-torch docs, "Current
// surface (0.17)"; cell of the xLSTM summary card's sLSTM step pseudocode, channelwise R):
//   rhs_t = f(s_{t-1}) - s_t = -F_t,  A_t = df/ds' at s_{t-1}   (s_0 = state0)
//   Delta_1 = rhs_1,  Delta_t = A_t Delta_{t-1} + rhs_t,  s_t <- s_t + Delta_t
//
// Decomposition: a tile of 64 features of one batch row x 4*TSUB steps per workgroup; the
// four threads of a quad hold the four consecutive sub-chunks of one feature, each its TSUB
// steps' 12 Jacobian entries, right-hand side and iterate in registers. The sub-chunk maps are
// composed and scanned across the quad with DPP; the look-back across tiles (quad_look_back)
// runs in every wave for its own 16 features, so no LDS staging and no barrier sit between
// the residual and the write of the new iterate. The step before a sub-chunk comes from the
// neighbouring thread of the quad or, for the first, from S_k, which this launch never writes.
//
// Packed sequences (PACKED): at the first step of each sequence the state before it is that
// sequence's state0 and its Jacobian is zero, so the composed maps restart there (the head
// flag of the segmented scan); every thread finds the sequences its steps belong to with a
// SeqCursor.
//
// Aligned tiles (ALIGNED, packed sequences with a tile table, see launch_aligned_tiles): a tile
// covers steps of one sequence only, starting at a multiple of the tile length from its first
// step, so the look-back chains are per sequence (position p of sequence s takes the look-back
// words of tile id - p + 0..p) and only position 0 starts a sequence. Tiles are handed out by
// position, then sequence: the tiles in flight at once belong to many sequences, which advance
// side by side instead of one after another.
//
// The residual maximum of S_k goes to the spread slots. Early stop is exact although the
// update of iteration k is formed together with F_k: the next launch (or the final residual
// pass) finds max|F_k| < tol and declares S_k final; S_k is still intact in the other buffer.
#include "affine4.h"
#include "cell.h"
#include "kernels.h"

namespace slstm {

// Sub-chunk length and the occupancy the register allocation is bounded for (waves per SIMD,
// which is also workgroups per compute unit). The kernel issues about 300 VALU instructions per
// step and lane, so it is bound by the vector units as much as by HBM: 4 steps per sub-chunk
// at 3 workgroups per compute unit keep the Jacobians, right-hand sides and iterates of the
// sub-chunk in registers (149 VGPRs, no spills), which measured fastest on MI355X.
#ifndef SLSTM_FUSED_TSUB
#define SLSTM_FUSED_TSUB 4
#endif
#ifndef SLSTM_FUSED_MIN_WAVES
#define SLSTM_FUSED_MIN_WAVES 3
#endif
constexpr int kFusedBlock = 256;
constexpr int kFusedTSub = SLSTM_FUSED_TSUB;
// Rows with few lane groups (packed sequences, or B * d_h up to a few tens of thousands of
// lanes) have long look-back chains along T: the scan advances one anchor per memory round trip,
// and a tile of 4 * TSUB steps sets how far. There the sub-chunks are twice as long (the
// registers then allow 2 workgroups per compute unit), which halves the chain: below 512 lane
// groups this measured faster on MI355X (B = 4, T = 16384, d_h = 2048: 1.82 against 2.72 ms per
// iteration; B = 16, T = 4096, d_h = 1024: 8.2 against 9.3 ms per early-stopped solve).
#ifndef SLSTM_FUSED_LONG_TSUB
#define SLSTM_FUSED_LONG_TSUB 8
#endif
constexpr int kFusedLongTSub = SLSTM_FUSED_LONG_TSUB;
#ifndef SLSTM_FEW_LANE_GROUPS
#define SLSTM_FEW_LANE_GROUPS 512
#endif
constexpr int kFewLaneGroups = SLSTM_FEW_LANE_GROUPS;
static_assert(kFusedLongTSub >= kFusedTSub, "look-back words are sized for the shorter tiles");

template <int TSUB>
constexpr int fused_wgs_per_cu() { return TSUB > 4 ? 2 : SLSTM_FUSED_MIN_WAVES; }

template <bool BF16, int TSUB>
__device__ __forceinline__ void load_sub_chunk(rsrc_t rsP, rsrc_t rsS, unsigned lane_off, unsigned ud,
                                               int t_start, int T, bool valid, float pg[][4],
                                               float sv[][4]) {
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    if (valid && t_start + u < T) {
      const unsigned o = lane_off + u * 4u * ud;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[u][k] = buf_ld_p<BF16>(rsP, o, k * ud);
        sv[u][k] = buf_ld(rsS, 4u * o, 4u * k * ud);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[u][k] = 0.0f;
        sv[u][k] = 0.0f;
      }
    }
  }
}

// residual r = f(s') - s and the 12 Jacobian entries of one step (zero map at a sequence
// start: the state before it is data, not an unknown)
__device__ __forceinline__ void step_terms(const CellIn& pv, const float pg[4], const float sv[4],
                                           float rz, float ri, float rf, float ro, bool sig, bool floored,
                                           bool start, float a[12], float r[4]) {
  float f[4], Aj[16];
  cell_step<true>(pv, pg[0], pg[1], pg[2], pg[3], rz, ri, rf, ro, sig, floored, f, Aj);
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = f[k] - sv[k];
#pragma unroll
  for (int q = 0; q < 12; ++q) a[q] = start ? 0.0f : Aj[kSpPlane[q]];
}

template <bool BF16, int TSUB, bool PACKED, bool ALIGNED>
__global__ __launch_bounds__(kFusedBlock, fused_wgs_per_cu<TSUB>()) void newton_iter_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S_in, float* __restrict__ S_out, int T, int d, int n_jt, int n_lg,
    int n_tt, int anchor_stride, int cell_mode, unsigned long long* __restrict__ desc,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch, Control* __restrict__ ctl,
    int k_iter, float tol, const int* __restrict__ cu, int n_seqs,
    const int* __restrict__ seq_tab, const int* __restrict__ tiles, int tile_cap) {
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
  __shared__ unsigned int s_err, s_arrived;  // block residual maximum, waves that added theirs
  const int tid = threadIdx.x;
  if (tid == 0) {
    take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
    s_err = 0u;
    s_arrived = 0u;
  }
  __syncthreads();
  const int tk = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;
  const i64 n_lanes_pad = static_cast<i64>(n_lg) * 64;
  // the tile's position along its look-back chain, its first step, the end of its steps
  int tt = tk, t_tile = tk * 4 * TSUB, t_end = T, aseq = 0;
  unsigned long long* dsc = desc;  // the look-back words of the chain
  if constexpr (ALIGNED) {
    // this ticket's slot of the table, all six values at once (tk < tile_cap)
    const int n_real = __builtin_amdgcn_readfirstlane(tiles[0]);
    const int id = __builtin_amdgcn_readfirstlane(tiles[1 + tk]);
    const int sq = __builtin_amdgcn_readfirstlane(tiles[1 + tile_cap + tk]);
    const int ps = __builtin_amdgcn_readfirstlane(tiles[1 + 2 * tile_cap + tk]);
    const int a0 = __builtin_amdgcn_readfirstlane(tiles[1 + 3 * tile_cap + tk]);
    const int e0 = __builtin_amdgcn_readfirstlane(tiles[1 + 4 * tile_cap + tk]);
    if (tk >= n_real) {  // a ticket past the last tile
      if (blockIdx.x == 0 && tid == 0) ctl->iters = k_iter + 1;
      return;
    }
    aseq = sq;
    tt = ps;
    t_end = e0;
    t_tile = a0 + tt * 4 * TSUB;
    dsc = desc + static_cast<i64>(id - tt) * kLookBackWords * n_lanes_pad;
  }

  // lane layout: the four threads of a quad hold the four consecutive sub-chunks of one feature
  const int l = tid & 63;
  const int sc = l & 3;
  const int lane_in_tile = (tid >> 6) * 16 + (l >> 2);
  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * 64 + lane_in_tile);
  const bool valid = j < ud;
  const int t_start = t_tile + sc * TSUB;
  const i64 my_lane = static_cast<i64>(lg) * 64 + lane_in_tile;
  const bool sig = (cell_mode & kCellSigmoid) != 0;
  const bool floored = (cell_mode & kCellFloored) != 0;
  // scalar bases of this tile's rows; 32-bit lane offsets (elements) within them
  const i64 tile_row = (static_cast<i64>(b) * T + t_tile) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  const rsrc_t rsS = make_rsrc(S_in + tile_row);
  const rsrc_t rsO = make_rsrc(S_out + tile_row);
  const unsigned lane_off = static_cast<unsigned>(sc * TSUB) * 4u * ud + j;

  // this thread's word of the look-back anchor, loaded now so that it arrives meanwhile
  const unsigned long long pf = quad_look_back_prefetch(dsc, n_lanes_pad, my_lane, sc, tt, anchor_stride);

  float pg[TSUB][4], sv[TSUB][4];
  load_sub_chunk<BF16, TSUB>(rsP, rsS, lane_off, ud, t_start, t_end, valid, pg, sv);

  float rz = 0.0f, ri = 0.0f, rf = 0.0f, ro = 0.0f;
  // the state before the sub-chunk: the previous sub-chunk's last step (from the neighbouring
  // thread of the quad), the previous tile's last step, or the initial state
  CellIn pv0 = {quad_perm<0, 0, 1, 2>(sv[TSUB - 1][0]), quad_perm<0, 0, 1, 2>(sv[TSUB - 1][1]),
                quad_perm<0, 0, 1, 2>(sv[TSUB - 1][2]), quad_perm<0, 0, 1, 2>(sv[TSUB - 1][3])};
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
      } else if (t_start < T) {
        const float* sp = S_in + (static_cast<i64>(b) * T + t_start - 1) * 4 * static_cast<i64>(d);
        pv0 = {sp[j], sp[ud + j], sp[2 * ud + j], sp[3 * ud + j]};
      }
    }
  }

  // ---- residual and Jacobian of the sub-chunk, composed on the fly into (M, v) ----
  float keep_a[TSUB][12], keep_r[TSUB][4];
  float M[16], v[4];
  float fmax_local = 0.0f;
  CellIn pv = pv0;
  SeqCursor seq;
  if constexpr (PACKED) seq = seq_cursor(cu, n_seqs, b, t_start, seq_tab);
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    float a[12], r[4];
    // packed: the sequence starting at t (every lane walks the offsets, padding lanes too, so
    // that all lanes of a tile agree on where the maps restart)
    int sq = -1;
    if constexpr (PACKED) {
      if (t < T) sq = seq_begin(seq, t);
    }
    if constexpr (ALIGNED) sq = (tt == 0 && t == t_tile && t < t_end) ? aseq : -1;
    if (valid && t < t_end) {
      const bool start = (PACKED || ALIGNED) ? sq >= 0 : t == 0;
      if ((PACKED || ALIGNED) && start) pv = state0_of(state0, sq, ud, j);
      step_terms(pv, pg[u], sv[u], rz, ri, rf, ro, sig, floored, start, a, r);
#pragma unroll
      for (int k = 0; k < 4; ++k) fmax_local = fmaxf(fmax_local, abs_nan_inf(r[k]));
      pv = {sv[u][0], sv[u][1], sv[u][2], sv[u][3]};
    } else {
      // identity map (zero at a sequence start)
#pragma unroll
      for (int q = 0; q < 12; ++q) a[q] = (kSpPlane[q] % 5 == 0 && sq < 0) ? 1.0f : 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = 0.0f;
    }
    if (u == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = 0.0f;
#pragma unroll
      for (int q = 0; q < 12; ++q) M[kSpPlane[q]] = a[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = r[e];
    } else {
      float vn[4];
      sp_mul_left(a, M);
      sp_vec(a, v, r, vn);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = vn[e];
    }
#pragma unroll
    for (int q = 0; q < 12; ++q) keep_a[u][q] = a[q];
#pragma unroll
    for (int k = 0; k < 4; ++k) keep_r[u][k] = r[k];
  }

  // residual maximum of S_k: waves fold theirs into the block's in LDS; the last to arrive
  // publishes it with one device atomic (no barrier: the waves go on independently)
  const float wm = wave_max(fmax_local);
  if (l == 0) {
    __hip_atomic_fetch_max(&s_err, __float_as_uint(wm), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__hip_atomic_fetch_add(&s_arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) == kFusedBlock / kWave - 1)
      err_publish(&spread_of(ctl)->err[0][k_iter], kErrSlotWords, blockIdx.x,
                  __uint_as_float(__hip_atomic_load(&s_err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)));
  }

  // ---- quad scan of the sub-chunk maps, then the look-back across tiles ----
  quad_inclusive_scan(M, v, sc);
  float carry[4];
  {
    float arow[4], av;
    quad_row_of_last(M, v, sc, arow, av);
    quad_look_back<PACKED>(arow, av, carry, dsc, n_lanes_pad, my_lane, sc, tt, anchor_stride, epoch, pf);
  }

  // ---- re-run each sub-chunk from the value entering it and write the updated iterate ----
  float xs[4];
  {
    float xe[4];
    mat4_vec(M, carry, v, xe);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xs[e] = quad_perm<0, 0, 1, 2>(xe[e]);
      if (sc == 0) xs[e] = carry[e];
    }
  }
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    if (valid && t < t_end) {
      float xn[4];
      sp_vec(keep_a[u], xs, keep_r[u], xn);
      const unsigned o = lane_off + u * 4u * ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xs[e] = xn[e];
        buf_st(sv[u][e] + xs[e], rsO, 4u * o, 4u * e * ud);
      }
    }
  }
  if (blockIdx.x == 0 && tid == 0) ctl->iters = k_iter + 1;
}

static int fused_tsub(int B, int d, bool packed) {
  const i64 n_lg = static_cast<i64>(B) * ((d + 63) / 64);
  return packed || n_lg < kFewLaneGroups ? kFusedLongTSub : kFusedTSub;
}

static void fused_grid(int B, int T, int d, int tsub, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + 63) / 64;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + 4 * tsub - 1) / (4 * tsub);
}

// sized for the shorter tiles (the most tiles), whichever the launch picks
size_t fused_desc_words(int B, int T, int d) {
  i64 n_jt, n_lg, n_tt;
  fused_grid(B, T, d, kFusedTSub, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * kLookBackWords * n_lg * 64);
}

// aligned tiles: the long sub-chunks, as many tiles as the words of the shorter tiles hold
int fused_aligned_steps() { return 4 * kFusedLongTSub; }
int fused_aligned_cap(int T) { return (T + 4 * kFusedTSub - 1) / (4 * kFusedTSub); }
// every aligned tile an anchor: with many sequences in flight a plain chain per sequence
// measured fastest (3.58 ms per iteration on the 292-sequence pack of B = 128, T = 2048,
// d_h = 1024 tokens, against 3.80 and 4.13 for strides 2 and 4)
#ifndef SLSTM_ALIGNED_ANCHOR_STRIDE
#define SLSTM_ALIGNED_ANCHOR_STRIDE 1
#endif

hipError_t launch_newton_iteration(const void* P, bool p_bf16, const float* R, const float* state0,
                                   const float* S_in, float* S_out, int B, int T, int d,
                                   int cell_mode, unsigned long long* desc, unsigned int* tickets,
                                   uint32_t epoch, Control* ctl, int k_iter, float tol,
                                   hipStream_t stream, Seqs seqs) {
  const bool packed = seqs.cu != nullptr;
  const bool aligned = packed && seqs.tiles != nullptr;
  const int tsub = fused_tsub(B, d, packed);
  i64 n_jt, n_lg, n_tt;
  fused_grid(B, T, d, tsub, n_jt, n_lg, n_tt);
  if (aligned) {  // at most one tile more than the row's per sequence; the tickets past the last exit
    n_tt += seqs.n;
    if (B != 1 || tsub != kFusedLongTSub || n_tt > seqs.tile_cap) return hipErrorInvalidValue;
  }
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int stride = look_back_anchor_stride(
      n_lg, tsub == kFusedTSub ? fused_wgs_per_cu<kFusedTSub>() : fused_wgs_per_cu<kFusedLongTSub>());
  // packed rows and other rows of few lane groups along a long T (the long sub-chunks) take
  // the packed anchor stride, measured best there
  const int stride_used =
      aligned ? SLSTM_ALIGNED_ANCHOR_STRIDE : (packed || tsub != kFusedTSub ? kPackedAnchorStride : stride);
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int sig = cell_mode;
#define SLSTM_FUSED_LAUNCH_T(BF, TS, PK, AL)                                                         \
  newton_iter_kernel<BF, TS, PK, AL><<<grid, kFusedBlock, 0, stream>>>(                              \
      P, R, state0, S_in, S_out, T, d, static_cast<int>(n_jt), static_cast<int>(n_lg),                \
      static_cast<int>(n_tt), stride_used, sig, desc, tickets, n_ctr, epoch, ctl, k_iter, tol, seqs.cu, seqs.n, seqs.tab, \
      seqs.tiles, seqs.tile_cap)
#define SLSTM_FUSED_LAUNCH(BF, PK)                                                \
  do {                                                                            \
    if (tsub == kFusedTSub) SLSTM_FUSED_LAUNCH_T(BF, kFusedTSub, PK, false);      \
    else SLSTM_FUSED_LAUNCH_T(BF, kFusedLongTSub, PK, false);                     \
  } while (0)
  if (aligned) {
    if (p_bf16) SLSTM_FUSED_LAUNCH_T(true, kFusedLongTSub, false, true);
    else SLSTM_FUSED_LAUNCH_T(false, kFusedLongTSub, false, true);
  } else if (p_bf16) {
    if (packed) SLSTM_FUSED_LAUNCH(true, true);
    else SLSTM_FUSED_LAUNCH(true, false);
  } else {
    if (packed) SLSTM_FUSED_LAUNCH(false, true);
    else SLSTM_FUSED_LAUNCH(false, false);
  }
#undef SLSTM_FUSED_LAUNCH
#undef SLSTM_FUSED_LAUNCH_T
  return hipGetLastError();
}

}  // namespace slstm
