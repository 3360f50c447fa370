// Kernel (b): the block-bidiagonal Newton system solved as an associative scan over 4x4
// affine maps (scan_block4 layout (B, T, 4, 4, d): "Layout" page of the pararnn-torch docs,
// "Naming"; the (J, r) monoid of "sLSTM in this library", "Packed sequences").
//
//   x_1 = rhs_1,   x_t = A_t x_{t-1} + rhs_t        (A at the first step is never used)
//
// Each step is the map x -> A x + r; maps compose as (A2, r2) o (A1, r1) = (A2 A1, A2 r1 + r2).
//
// Work decomposition (one workgroup = 4 waves = one tile of 64 features of one batch row x
// 4*TSUB steps):
//   * lane   = (b, j); a tile covers 64 consecutive features of one batch row, so each load
//              of the tile reads 256 contiguous bytes of one (b, t, plane) row, and b is
//              uniform over the workgroup (scalar row bases, 32-bit lane offsets);
//   * thread = one lane and one sub-chunk of TSUB steps; a wave holds 16 lanes x 4
//              consecutive sub-chunks, the 4 sub-chunks of a lane forming one quad.
// Level 1: every thread composes its sub-chunk sequentially in registers (A and r stay in
//          registers for the whole kernel, so each byte is read from HBM once).
// Level 2: inclusive scan of the 4 sub-chunk aggregates inside each quad with DPP quad
//          permutations; lane 3 of the quad then holds the tile aggregate of its feature.
// Level 3: decoupled look-back across tiles along T, spread over the quad (quad_look_back):
//          each thread publishes, loads and folds one row of the 4x4 maps and receives the
//          other rows by DPP, so every wave runs the look-back of its own 16 features with no
//          LDS staging and no barrier. The fold order is fixed, so results are bitwise
//          reproducible. Tiles take work tickets (take_ticket), so a predecessor always holds a
//          smaller ticket and is running or done.
// Finally every thread re-runs its sub-chunk from its carry and stores x.
// x may alias rhs: each thread reads its rhs values before writing the same addresses.
//
// SPARSE: the sLSTM Jacobian has four structural zeros ((c, n'), (n, c'), (m, c'), (m, n'));
// the Newton solver's scan reads only the other 12 planes and multiplies with them alone
// (48 instead of 64 FMA per 4x4 product). The dense form serves arbitrary 4x4 maps.
#include "affine4.h"
#include "common.h"
#include "kernels.h"

namespace slstm {

constexpr int kScanBlock = 256;
#ifndef SLSTM_SCAN_TSUB
#define SLSTM_SCAN_TSUB 6
#endif
#ifndef SLSTM_SCAN_MIN_WAVES
#define SLSTM_SCAN_MIN_WAVES 3
#endif
constexpr int kScanTSubSparse = SLSTM_SCAN_TSUB;  // sub-chunk length of the Newton solver's sparse scan
constexpr int kScanTSubDense = 4;   // and of the dense scan (16 values per step in registers)
constexpr int kScanWords = kLookBackWords;

template <bool SPARSE, int TSUB>
__global__ __launch_bounds__(kScanBlock, SLSTM_SCAN_MIN_WAVES) void scan_block4_kernel(
    const float* __restrict__ A, const float* rhs, float* x, int T, int d, int n_jt, int n_lg,
    int n_tt, int anchor_stride, unsigned long long* __restrict__ desc,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch, Control* ctl, int k_iter, float tol) {
  constexpr int NA = SPARSE ? 12 : 16;
  if (ctl != nullptr) {
    if (ctl->stopped) return;
    if (tol > 0.0f && err_reduced(ctl, k_iter) < tol) {
      // residual already below the tolerance: stop before solving
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctl->stopped = 1;
        ctl->iters = k_iter;
      }
      return;
    }
  }
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;

  const int wave = tid >> 6;
  const int l = tid & 63;
  (void)wave;
  const int sc = l & 3;
  const int lane_in_tile = wave * 16 + (l >> 2);
  const unsigned j = static_cast<unsigned>(jt * 64 + lane_in_tile);
  const unsigned ud = static_cast<unsigned>(d);
  const bool valid = j < ud;
  const int t_tile = tt * 4 * TSUB;
  const int t_start = t_tile + sc * TSUB;
  const i64 n_lanes_pad = static_cast<i64>(n_lg) * 64;
  // scalar bases of this tile's rows, 32-bit lane offsets within them
  const rsrc_t rsA = make_rsrc(A + (static_cast<i64>(b) * T + t_tile) * 16 * static_cast<i64>(d));
  const rsrc_t rsR = make_rsrc(rhs + (static_cast<i64>(b) * T + t_tile) * 4 * static_cast<i64>(d));
  const rsrc_t rsX = make_rsrc(x + (static_cast<i64>(b) * T + t_tile) * 4 * static_cast<i64>(d));
  const unsigned a_lane = 4u * (static_cast<unsigned>(sc * TSUB) * 16u * ud + j);  // bytes
  const unsigned r_lane = 4u * (static_cast<unsigned>(sc * TSUB) * 4u * ud + j);
  const unsigned row_b = 4u * ud;  // bytes per plane row
  const i64 my_lane = static_cast<i64>(lg) * 64 + lane_in_tile;
  // this thread's word of the look-back anchor, loaded now so that it arrives meanwhile
  const unsigned long long pf = quad_look_back_prefetch(desc, n_lanes_pad, my_lane, sc, tt, anchor_stride);

  // ---- level 1: load the sub-chunk and compose it ----
  float a[TSUB][NA], r[TSUB][4];
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const unsigned plane = SPARSE ? kSpPlane[e] : e;
        a[u][e] = buf_ld(rsA, a_lane, (u * 16u + plane) * row_b);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) r[u][e] = buf_ld(rsR, r_lane, (u * 4u + e) * row_b);
      if (t == 0) {
#pragma unroll
        for (int e = 0; e < NA; ++e) a[u][e] = 0.0f;  // x_0 = 0: the first map is constant
      }
    } else {
      // identity map
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const int plane = SPARSE ? kSpPlane[e] : e;
        a[u][e] = (plane % 5 == 0) ? 1.0f : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) r[u][e] = 0.0f;
    }
  }
  float M[16], v[4];
  if constexpr (SPARSE) {
#pragma unroll
    for (int e = 0; e < 16; ++e) M[e] = 0.0f;
#pragma unroll
    for (int e = 0; e < 12; ++e) M[kSpPlane[e]] = a[0][e];
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) M[e] = a[0][e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = r[0][e];
#pragma unroll
  for (int u = 1; u < TSUB; ++u) {
    // (M, v) <- (a_u, r_u) o (M, v)
    float vn[4];
    if constexpr (SPARSE) {
      sp_mul_left(a[u], M);
      sp_vec(a[u], v, r[u], vn);
    } else {
      mat4_mul_left(a[u], M);
      mat4_vec(a[u], v, r[u], vn);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = vn[e];
  }

  // ---- level 2: inclusive scan of the quad's sub-chunk aggregates (DPP) ----
  quad_inclusive_scan(M, v, sc);

  // ---- level 3: look-back across tiles, spread over the quad ----
  float cin[4];
  {
    float arow[4], av;
    quad_row_of_last(M, v, sc, arow, av);
    quad_look_back(arow, av, cin, desc, n_lanes_pad, my_lane, sc, tt, anchor_stride, epoch, pf);
  }

  // ---- re-run each sub-chunk from its carry ----
  float xe[4], xs[4];
  mat4_vec(M, cin, v, xe);  // value at the end of this sub-chunk
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    xs[e] = quad_perm<0, 0, 1, 2>(xe[e]);
    if (sc == 0) xs[e] = cin[e];
  }
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    float xn[4];
    if constexpr (SPARSE)
      sp_vec(a[u], xs, r[u], xn);
    else
      mat4_vec(a[u], xs, r[u], xn);
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[e] = xn[e];
    if (valid && t < T) {
#pragma unroll
      for (int e = 0; e < 4; ++e) buf_st(xs[e], rsX, r_lane, (u * 4u + e) * row_b);
    }
  }
}

static void scan_grid(int B, int T, int d, int tile, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + 63) / 64;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + tile - 1) / tile;
}

size_t scan_desc_words(int B, int T, int d, bool sparse) {
  i64 n_jt, n_lg, n_tt;
  scan_grid(B, T, d, 4 * (sparse ? kScanTSubSparse : kScanTSubDense), n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * kScanWords * n_lg * 64);
}

hipError_t launch_scan_block4(const float* A, const float* rhs, float* x, int B, int T, int d,
                              bool sparse, unsigned long long* desc, unsigned int* tickets,
                              uint32_t epoch, Control* ctl, int k_iter, float tol,
                              hipStream_t stream) {
  const int tile = 4 * (sparse ? kScanTSubSparse : kScanTSubDense);
  i64 n_jt, n_lg, n_tt;
  scan_grid(B, T, d, tile, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int stride = look_back_anchor_stride(n_lg, SLSTM_SCAN_MIN_WAVES);
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (sparse)
    scan_block4_kernel<true, kScanTSubSparse><<<grid, kScanBlock, 0, stream>>>(
        A, rhs, x, T, d, static_cast<int>(n_jt), static_cast<int>(n_lg), static_cast<int>(n_tt), stride,
        desc, tickets, n_ctr, epoch, ctl, k_iter, tol);
  else
    scan_block4_kernel<false, kScanTSubDense><<<grid, kScanBlock, 0, stream>>>(
        A, rhs, x, T, d, static_cast<int>(n_jt), static_cast<int>(n_lg), static_cast<int>(n_tt), stride,
        desc, tickets, n_ctr, epoch, ctl, k_iter, tol);
  return hipGetLastError();
}

}  // namespace slstm
