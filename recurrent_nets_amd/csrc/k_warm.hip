// Initial Newton iterate: the exact trajectory of the sLSTM cell with the recurrent term
// R h_{t-1} removed from the pre-activations. (The pages give no initial guess; with the
// recurrent term dropped every gate is known up front, and this trajectory is the plainest
// starting point that the stabilised equations admit.)
//
// With R dropped, step t is the map (m, c, n) -> (m', c', n'):
//   m' = max(l_t + m, i~_t),  c' = e^{l_t + m - m'} c + e^{i~_t - m'} z_t,
//   n' = e^{l_t + m - m'} n + e^{i~_t - m'}
// (stabiliser and stabilised gates: educational reimplementation page, "Exponential gating +
// the stabilizer (the crux)"; z = tanh, l = f~ or log sigma(f~)). A run of steps composes to
// the same shape, held in log space relative to the run's start as (L, E, cz, nz):
//   L  = sum of the l over the run,
//   E  = max over steps s of e_s, with e_s = i~_s - (l_1 + ... + l_s) the log weight of the
//        input at s seen from the run's start (a (max, +) scan),
//   cz = sum_s e^{e_s - E} z_s,  nz = sum_s e^{e_s - E},
// and it acts on a carried (m, c, n) as
//   x = max(m, E),  c_out = e^{m - x} c + e^{E - x} cz,  n_out likewise,  m_out = L + x.
// Referencing the exponents to the run's start keeps every exponent that carries weight of
// order one: sums of l (which grow by about f~ per step) enter only m_out, never an
// exponent, so a float32 carry is as accurate as the plain step loop.
// Composition (X first, then Y): L = L_X + L_Y, E = max(E_X, E_Y - L_X),
//   cz = e^{E_X - E} cz_X + e^{E_Y - L_X - E} cz_Y, nz likewise. One step: (l, i~ - l, z, 1).
//
// Same decomposition as the 4x4 scan: a tile of 64 features of one batch row x 4*TSUB steps
// per workgroup, per-thread sequential sub-chunks, a DPP quad scan of sub-chunk aggregates,
// tile aggregates and carries staged in LDS, and a decoupled look-back across tiles along T
// with the same fixed, anchored dataflow. The re-run from each carry writes the states
// (c, n, m, h) with h = sigma(p_o) c / n (or the floored read-out, see cell.h).
//
// Packed sequences (PACKED): a run that contains a sequence start forgets whatever enters it;
// it is held in absolute form, E = +inf marking it and (L, cz, nz) holding the (m, c, n) it
// ends with (the start step applied to the sequence's state0, then the steps after it). A run
// composed after an absolute one is applied to its state; an absolute run composed after any
// run replaces it (the head flag of the segmented scan).
#include "cell.h"
#include "kernels.h"

namespace slstm {

constexpr int kWarmBlock = 256;
constexpr int kWarmTSub = 16;
constexpr int kWarmTile = 4 * kWarmTSub;
constexpr int kWarmWords = 8;  // per lane and tile: carry (m, c, n, -), aggregate (L, E, cz, nz)

struct LogAgg {
  float L, E, cz, nz;
};

__device__ __forceinline__ float exp_or_zero(float e, float x) {
  // e^{x} for an exponent built from E; an empty run has E = -inf and weight zero
  return (e == -INFINITY) ? 0.0f : exp_fast(x);
}

__device__ __forceinline__ bool absolute(const LogAgg& X) { return X.E == INFINITY; }

__device__ __forceinline__ void apply_relative(const LogAgg& X, float& m, float& c, float& n);

// X first, then Y
template <bool PACKED = false>
__device__ __forceinline__ LogAgg compose(const LogAgg& X, const LogAgg& Y) {
  if constexpr (PACKED) {
    if (absolute(Y)) return Y;
    if (absolute(X)) {
      float m = X.L, c = X.cz, n = X.nz;
      apply_relative(Y, m, c, n);
      return {m, INFINITY, c, n};
    }
  }
  LogAgg o;
  o.L = X.L + Y.L;
  const float ey = Y.E - X.L;
  o.E = fmaxf(X.E, ey);
  const float wx = exp_or_zero(X.E, X.E - o.E);
  const float wy = exp_or_zero(Y.E, ey - o.E);
  o.cz = fmaf(wx, X.cz, wy * Y.cz);
  o.nz = fmaf(wx, X.nz, wy * Y.nz);
  return o;
}

// apply a run to a carried (m, c, n)
__device__ __forceinline__ void apply_relative(const LogAgg& X, float& m, float& c, float& n) {
  const float x = fmaxf(m, X.E);
  const float wc = exp_fast(m - x);
  const float wz = exp_or_zero(X.E, X.E - x);
  c = fmaf(wc, c, wz * X.cz);
  n = fmaf(wc, n, wz * X.nz);
  m = X.L + x;
}

template <bool PACKED = false>
__device__ __forceinline__ void apply(const LogAgg& X, float& m, float& c, float& n) {
  if (PACKED && absolute(X)) {
    m = X.L;
    c = X.cz;
    n = X.nz;
    return;
  }
  apply_relative(X, m, c, n);
}

__device__ __forceinline__ LogAgg quad_perm_agg_m1(const LogAgg& X) {
  return {quad_perm<0, 0, 1, 2>(X.L), quad_perm<0, 0, 1, 2>(X.E), quad_perm<0, 0, 1, 2>(X.cz),
          quad_perm<0, 0, 1, 2>(X.nz)};
}
__device__ __forceinline__ LogAgg quad_perm_agg_m2(const LogAgg& X) {
  return {quad_perm<0, 1, 0, 1>(X.L), quad_perm<0, 1, 0, 1>(X.E), quad_perm<0, 1, 0, 1>(X.cz),
          quad_perm<0, 1, 0, 1>(X.nz)};
}

template <bool BF16, bool PACKED>
__global__ __launch_bounds__(kWarmBlock) void warm_start_kernel(
    const void* __restrict__ P, const float* __restrict__ state0, float* __restrict__ S, int T,
    int d, int cell_mode, int n_jt, int n_lg, int n_tt, int anchor_stride,
    unsigned long long* __restrict__ desc, unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch,
    const int* __restrict__ cu, int n_seqs,
    const int* __restrict__ seq_tab) {
  __shared__ int s_tile[2];
  __shared__ LogAgg s_agg[64];
  __shared__ float s_carry[64][3];

  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;

  const int wave = tid >> 6;
  const int l = tid & 63;
  const int sc = l & 3;
  const int lane_in_tile = wave * 16 + (l >> 2);
  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * 64 + lane_in_tile);
  const bool valid = j < ud;
  const int t_tile = tt * kWarmTile;
  const int t_start = t_tile + sc * kWarmTSub;
  const i64 n_lanes_pad = static_cast<i64>(n_lg) * 64;
  const bool sig = (cell_mode & kCellSigmoid) != 0;
  const bool floored = (cell_mode & kCellFloored) != 0;
  // scalar bases of this tile's rows, 32-bit lane offsets within them
  const i64 tile_row = (static_cast<i64>(b) * T + t_tile) * 4 * static_cast<i64>(d);
  float* Sb = S + tile_row;
  const unsigned lane_off = static_cast<unsigned>(sc * kWarmTSub) * 4u * ud + j;

  // ---- level 1: gates of the sub-chunk, folded into one aggregate ----
  float lf[kWarmTSub], it[kWarmTSub], zz[kWarmTSub], oo[kWarmTSub];
#pragma unroll
  for (int u = 0; u < kWarmTSub; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
      const unsigned o = lane_off + u * 4u * ud;
      const float pz = load_p<BF16>(P, tile_row + o);
      const float pi = load_p<BF16>(P, tile_row + o + ud);
      const float pf = load_p<BF16>(P, tile_row + o + 2 * ud);
      const float po = load_p<BF16>(P, tile_row + o + 3 * ud);
      zz[u] = tanh_fast(pz);
      oo[u] = sigmoidf(po);
      it[u] = pi;
      lf[u] = sig ? log_sigmoidf(pf) : pf;
    } else {
      zz[u] = 0.0f;
      oo[u] = 0.0f;
      it[u] = -INFINITY;  // padding step: m -> m, c -> c, n -> n
      lf[u] = 0.0f;
    }
  }
  // the sequence starting at each step of the sub-chunk, or -1 (packed only)
  int sq[kWarmTSub];
  if constexpr (PACKED) {
    SeqCursor seq = seq_cursor(cu, n_seqs, b, t_start, seq_tab);
#pragma unroll
    for (int u = 0; u < kWarmTSub; ++u) sq[u] = (t_start + u < T) ? seq_begin(seq, t_start + u) : -1;
  }
  LogAgg agg = {0.0f, -INFINITY, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kWarmTSub; ++u) {
    // one step as a run: L = l, E = i~ - l, cz = z, nz = 1
    LogAgg stp = {lf[u], it[u] - lf[u], zz[u], 1.0f};
    if constexpr (PACKED) {
      if (sq[u] >= 0) {
        // a sequence start: the step from the sequence's state0, in absolute form (a padding
        // lane past d_h takes zeros, so that all lanes of a tile agree on where runs restart)
        const CellIn s0 = valid ? state0_of(state0, sq[u], ud, j) : CellIn{0.0f, 0.0f, 0.0f, 0.0f};
        float m = s0.m, c = s0.c, n = s0.n;
        apply_relative(stp, m, c, n);
        stp = {m, INFINITY, c, n};
      }
    }
    agg = compose<PACKED>(agg, stp);
  }

  // ---- level 2: quad scan (DPP) ----
  {
    const LogAgg p1 = quad_perm_agg_m1(agg);
    if (sc >= 1) agg = compose<PACKED>(p1, agg);
    const LogAgg p2 = quad_perm_agg_m2(agg);
    if (sc >= 2) agg = compose<PACKED>(p2, agg);
  }
  if (sc == 3) s_agg[lane_in_tile] = agg;
  __syncthreads();

  // ---- level 3: decoupled look-back ----
  if (wave == 0) {
    const i64 my_lane = static_cast<i64>(lg) * 64 + l;
    const LogAgg tile = s_agg[l];
    auto word = [&](int tile_idx, int w) {
      return desc + (static_cast<i64>(tile_idx) * kWarmWords + w) * n_lanes_pad + my_lane;
    };
    // state entering the sequence (slots c, n, m of state0; zeros without one)
    float m0 = 0.0f, c0 = 0.0f, n0 = 0.0f;
    const unsigned jl = static_cast<unsigned>(jt * 64 + l);
    if (state0 != nullptr && jl < ud) {
      const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
      c0 = s0[jl];
      n0 = s0[ud + jl];
      m0 = s0[2 * ud + jl];
    }
    float cm = m0, cc = c0, cn = n0;
    // fixed dataflow (results independent of scheduling): anchors publish their carry out,
    // the tiles in between their run aggregate before waiting; a tile folds the aggregates
    // down to the nearest anchor in a fixed order and applies it to the anchor's carry out
    // packed: an absolute run does not depend on what enters it, so the fold stops at the first
    // absolute one (tiles further back cannot change it) and the anchor's carry is not waited
    // for, and an anchor whose own run is absolute publishes its carry out before its look-back:
    // a chain of anchors breaks at every sequence start
    // (wave-uniform tests: the branches on them stay scalar)
    auto wave_abs = [&](const LogAgg& X) {
      return __builtin_amdgcn_ballot_w64(absolute(X)) == __builtin_amdgcn_read_exec();
    };
    const bool anchor = (tt % anchor_stride) == 0;
    const bool own_abs = PACKED && wave_abs(tile);
    if (!anchor) {
      tag_store(word(tt, 4), tile.L, epoch);
      tag_store(word(tt, 5), tile.E, epoch);
      tag_store(word(tt, 6), tile.cz, epoch);
      tag_store(word(tt, 7), tile.nz, epoch);
    } else if (own_abs) {
      tag_store(word(tt, 0), tile.L, epoch);
      tag_store(word(tt, 1), tile.cz, epoch);
      tag_store(word(tt, 2), tile.nz, epoch);
    }
    if (tt > 0) {
      const int a = ((tt - 1) / anchor_stride) * anchor_stride;
      LogAgg acc = {0.0f, -INFINITY, 0.0f, 0.0f};  // runs a+1 .. tt-1, composed
      for (int p = tt - 1; p > a; --p) {
        if (PACKED && wave_abs(acc)) break;
        LogAgg pa;
        while (!(tag_load(word(p, 4), epoch, pa.L) & tag_load(word(p, 5), epoch, pa.E) &
                 tag_load(word(p, 6), epoch, pa.cz) & tag_load(word(p, 7), epoch, pa.nz)))
          poll_pause();
        acc = compose<PACKED>(pa, acc);
      }
      float xm = 0.0f, xc = 0.0f, xn = 0.0f;
      if (!(PACKED && wave_abs(acc))) {
        while (!(tag_load(word(a, 0), epoch, xm) & tag_load(word(a, 1), epoch, xc) &
                 tag_load(word(a, 2), epoch, xn)))
          poll_pause();
      }
      apply<PACKED>(acc, xm, xc, xn);
      cm = xm;
      cc = xc;
      cn = xn;
    }
    s_carry[l][0] = cm;
    s_carry[l][1] = cc;
    s_carry[l][2] = cn;
    if (anchor && !own_abs) {
      float em = cm, ec = cc, en = cn;
      apply<PACKED>(tile, em, ec, en);
      tag_store(word(tt, 0), em, epoch);
      tag_store(word(tt, 1), ec, epoch);
      tag_store(word(tt, 2), en, epoch);
    }
  }
  __syncthreads();

  // ---- re-run each sub-chunk from its carry, writing the states ----
  const float cm = s_carry[lane_in_tile][0];
  const float cc = s_carry[lane_in_tile][1];
  const float cn = s_carry[lane_in_tile][2];
  float em = cm, ec = cc, en = cn;
  apply<PACKED>(agg, em, ec, en);  // inclusive: end of this sub-chunk
  float m = quad_perm<0, 0, 1, 2>(em);
  float c = quad_perm<0, 0, 1, 2>(ec);
  float n = quad_perm<0, 0, 1, 2>(en);
  if (sc == 0) {
    m = cm;
    c = cc;
    n = cn;
  }
#pragma unroll
  for (int u = 0; u < kWarmTSub; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
      if constexpr (PACKED) {
        if (sq[u] >= 0) {
          const CellIn s0 = state0_of(state0, sq[u], ud, j);
          m = s0.m;
          c = s0.c;
          n = s0.n;
        }
      }
      float mn, ig, fg;
      stab_gates(lf[u] + m, it[u], mn, ig, fg);
      c = fmaf(fg, c, ig * zz[u]);
      n = fmaf(fg, n, ig);
      m = mn;
      const unsigned o = lane_off + u * 4u * ud;
      Sb[o] = c;
      Sb[o + ud] = n;
      Sb[o + 2 * ud] = m;
      Sb[o + 3 * ud] = oo[u] * c * readout(n, m, floored).rD;
    }
  }
}

static void warm_grid(int B, int T, int d, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + 63) / 64;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + kWarmTile - 1) / kWarmTile;
}

size_t warm_desc_words(int B, int T, int d) {
  i64 n_jt, n_lg, n_tt;
  warm_grid(B, T, d, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * kWarmWords * n_lg * 64);
}

hipError_t launch_warm_start(const void* P, bool p_bf16, const float* state0, float* S, int B,
                             int T, int d, int cell_mode, unsigned long long* desc,
                             unsigned int* tickets, uint32_t epoch, hipStream_t stream, Seqs seqs) {
  i64 n_jt, n_lg, n_tt;
  warm_grid(B, T, d, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  const int sig = cell_mode;
  const int stride = look_back_anchor_stride(n_lg, 2);
  // packed rows are few lane groups along a long T: anchors every 4 tiles (measured best
  // between 1 and 8 over short and long sequence mixes)
  const int stride_used = seqs.cu != nullptr ? kPackedAnchorStride : stride;
  const int n_ctr = ticket_counters(n_lg);
#define SLSTM_WARM_SCAN_LAUNCH(BF, PK)                                                                    \
  warm_start_kernel<BF, PK><<<grid, kWarmBlock, 0, stream>>>(P, state0, S, T, d, sig, static_cast<int>(n_jt), \
                                                             static_cast<int>(n_lg), static_cast<int>(n_tt), \
                                                             stride_used, desc, tickets, n_ctr, epoch, seqs.cu, seqs.n, seqs.tab)
  const bool packed = seqs.cu != nullptr;
  if (p_bf16) {
    if (packed) SLSTM_WARM_SCAN_LAUNCH(true, true);
    else SLSTM_WARM_SCAN_LAUNCH(true, false);
  } else {
    if (packed) SLSTM_WARM_SCAN_LAUNCH(false, true);
    else SLSTM_WARM_SCAN_LAUNCH(false, false);
  }
#undef SLSTM_WARM_SCAN_LAUNCH
  return hipGetLastError();
}

}  // namespace slstm
