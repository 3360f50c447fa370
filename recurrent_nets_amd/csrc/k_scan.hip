// Kernel (b): the block-bidiagonal Newton system solved as an associative scan over 4x4
// affine maps (scan_block4 layout (B, T, 4, 4, d): "Layout" page of the pararnn-torch docs,
// "Naming"; the (J, r) monoid of "sLSTM in this library", "Packed sequences").
//
//   x_1 = rhs_1,   x_t = A_t x_{t-1} + rhs_t        (A at the first step is never used)
//
// Each step is the map x -> A x + r; maps compose as (A2, r2) o (A1, r1) = (A2 A1, A2 r1 + r2).
//
// Work decomposition (one workgroup = 4 data waves + 1 coordinating wave = one tile of 64
// features of one batch row x 4*TS steps):
//   * lane   = (b, j); a tile covers 64 consecutive features of one batch row, so b is uniform
//              over the workgroup (scalar row bases, 32-bit lane offsets);
//   * wave w = sub-chunk w of the tile (TS consecutive steps) for all 64 features, one feature
//              per thread, so every load and store of a wave covers 256 contiguous bytes of one
//              (b, t, plane) row (a whole pair of 128-byte lines; a layout that mixes steps
//              inside a wave touches four 64-byte pieces per instruction and streams about 10%
//              slower on MI355X).
// Level 1: every thread composes its sub-chunk sequentially in registers (A and r stay in
//          registers for the whole kernel, so each byte is read from HBM once) and writes the
//          composed map (M, v) of its lane to LDS.
// Level 2: the fifth wave, which holds no data (so the data waves' registers do not carry the
//          look-back's), finds the value entering the tile by a decoupled look-back across
//          tiles along T (its lanes' words, lane-major), then the value entering each sub-chunk
//          by applying
//          the sub-chunk maps in order (three 4x4 matrix-vector products), and hands them back
//          through LDS. Tiles whose index is a multiple of the anchor stride publish their
//          inclusive value; the others first publish their aggregate (the four sub-chunk maps
//          composed). The fold order is fixed, so results are bitwise reproducible. Tiles take
//          work tickets (take_ticket), so a predecessor always holds a smaller ticket and is
//          running or done.
// Finally every thread re-runs its sub-chunk from its start value and stores x.
// x may alias rhs: each thread reads its rhs values before writing the same addresses.
//
// SPARSE: the sLSTM Jacobian has four structural zeros ((c, n'), (n, c'), (m, c'), (m, n'));
// the Newton solver's scan reads only the other 12 planes and multiplies with them alone
// (48 instead of 64 FMA per 4x4 product), with non-temporal loads (the Jacobian is read once).
// The dense form serves arbitrary 4x4 maps.
#include <algorithm>

#include "affine4.h"
#include "common.h"
#include "kernels.h"

namespace slstm {

constexpr int kScanDataWaves = kRowsDataWaves;
constexpr int kScanBlock = kRowsBlock;  // 320
// sub-chunk lengths of the Newton solver's sparse scan and of the dense scan (16 values per step
// in registers), one feature per thread: 125 and 111 VGPRs, 4 waves per SIMD, so 3 workgroups
// of 5 waves per compute unit. (Two features per thread, 512-byte rows per access, needs
// 3-step sub-chunks to stay at 2 workgroups per compute unit and measured slower: 4.82 against
// 4.65 ms at B = 128, T = 2048, d_h = 1024.)
constexpr int kScanTSubSparse = 6;
constexpr int kScanTSubDense = 3;
// non-temporal loads of the Jacobian (read once): 4.54 against 4.65 ms at B = 128, T = 2048,
// d_h = 1024 on MI355X
#ifndef SLSTM_SCAN_NT
#define SLSTM_SCAN_NT 1
#endif
__host__ __device__ constexpr int scan_wgs_per_cu(int vec) { return vec == 2 ? 2 : 3; }
constexpr int kScanWords = kLookBackWords;

template <bool SPARSE, int TSUB, int VEC>
__global__ __launch_bounds__(kScanBlock, scan_wgs_per_cu(VEC)) void scan_block4_kernel(
    const float* __restrict__ A, const float* rhs, float* x, int T, int d, int n_jt, int n_lg,
    int n_tt, int anchor_stride, unsigned long long* __restrict__ desc,
    unsigned int* __restrict__ tickets, int n_ctr, uint32_t epoch, Control* ctl, int k_iter, float tol) {
  constexpr int NA = SPARSE ? 12 : 16;
  constexpr int TW = VEC * kWave;  // features per tile
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
  __shared__ float s_map[4][20][TW];  // sub-chunk maps: M (16, row-major) and v (4) per feature
  __shared__ float s_x[4][4][TW];     // the value entering each sub-chunk (from the coordinator)

  const int tid = threadIdx.x;
  if (tid == 0) take_ticket(tickets, n_ctr, n_lg, n_tt, s_tile[0], s_tile[1]);
  __syncthreads();
  const int tt = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int lg = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const unsigned j0 = static_cast<unsigned>(jt * TW + VEC * l);  // first feature of the thread
  const unsigned ud = static_cast<unsigned>(d);
  const int t_tile = tt * 4 * TSUB;

  if (wave == kScanDataWaves) {
    scan_coordinate<VEC>(s_map, s_x, desc, static_cast<i64>(n_lg) * TW, static_cast<i64>(lg) * TW + VEC * l, tt,
                         anchor_stride, epoch, l);
    return;
  }

  const int t_start = t_tile + wave * TSUB;
  // scalar bases of this sub-chunk's rows, the feature as a 32-bit lane offset
  const rsrc_t rsA = make_rsrc(A + (static_cast<i64>(b) * T + t_start) * 16 * static_cast<i64>(d));
  const rsrc_t rsR = make_rsrc(rhs + (static_cast<i64>(b) * T + t_start) * 4 * static_cast<i64>(d));
  const rsrc_t rsX = make_rsrc(x + (static_cast<i64>(b) * T + t_start) * 4 * static_cast<i64>(d));
  const unsigned lane_b = 4u * j0;
  const unsigned row_b = 4u * ud;  // bytes per plane row
  const bool valid = j0 < ud;      // d is a multiple of VEC

  // ---- level 1: load the sub-chunk and compose it ----
  float a[TSUB][NA][VEC], r[TSUB][4][VEC];
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const unsigned plane = SPARSE ? kSpPlane[e] : e;
        if (SPARSE && SLSTM_SCAN_NT && VEC == 1)  // aux bit 1: non-temporal
          a[u][e][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsA, lane_b, (u * 16u + plane) * row_b, 2));
        else
          buf_ld_vec<VEC>(rsA, lane_b, (u * 16u + plane) * row_b, a[u][e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) buf_ld_vec<VEC>(rsR, lane_b, (u * 4u + e) * row_b, r[u][e]);
      if (t == 0) {
#pragma unroll
        for (int e = 0; e < NA; ++e)
#pragma unroll
          for (int f = 0; f < VEC; ++f) a[u][e][f] = 0.0f;  // x_0 = 0: the first map is constant
      }
    } else {
      // identity map
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        const int plane = SPARSE ? kSpPlane[e] : e;
#pragma unroll
        for (int f = 0; f < VEC; ++f) a[u][e][f] = (plane % 5 == 0) ? 1.0f : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int f = 0; f < VEC; ++f) r[u][e][f] = 0.0f;
    }
  }
#pragma unroll
  for (int f = 0; f < VEC; ++f) {
    float M[16], v[4], au[NA], ru[4];
    if constexpr (SPARSE) {
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = 0.0f;
#pragma unroll
      for (int e = 0; e < 12; ++e) M[kSpPlane[e]] = a[0][e][f];
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = a[0][e][f];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = r[0][e][f];
#pragma unroll
    for (int u = 1; u < TSUB; ++u) {
      // (M, v) <- (a_u, r_u) o (M, v)
#pragma unroll
      for (int e = 0; e < NA; ++e) au[e] = a[u][e][f];
#pragma unroll
      for (int e = 0; e < 4; ++e) ru[e] = r[u][e][f];
      float vn[4];
      if constexpr (SPARSE) {
        sp_mul_left(au, M);
        sp_vec(au, v, ru, vn);
      } else {
        mat4_mul_left(au, M);
        mat4_vec(au, v, ru, vn);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = vn[e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) s_map[wave][e][VEC * l + f] = M[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) s_map[wave][16 + e][VEC * l + f] = v[e];
  }
  __syncthreads();  // maps in LDS: the coordinating wave reads them
  __syncthreads();  // start values in LDS

  // ---- re-run each sub-chunk from its start value ----
  float xs[VEC][4];
#pragma unroll
  for (int f = 0; f < VEC; ++f)
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[f][e] = s_x[wave][e][VEC * l + f];
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    float xo[4][VEC];
#pragma unroll
    for (int f = 0; f < VEC; ++f) {
      float au[NA], ru[4], xn[4];
#pragma unroll
      for (int e = 0; e < NA; ++e) au[e] = a[u][e][f];
#pragma unroll
      for (int e = 0; e < 4; ++e) ru[e] = r[u][e][f];
      if constexpr (SPARSE)
        sp_vec(au, xs[f], ru, xn);
      else
        mat4_vec(au, xs[f], ru, xn);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xs[f][e] = xn[e];
        xo[e][f] = xn[e];
      }
    }
    if (valid && t < T) {
#pragma unroll
      for (int e = 0; e < 4; ++e) buf_st_vec<VEC>(xo[e], rsX, lane_b, (u * 4u + e) * row_b);
    }
  }
}

static void scan_grid(int B, int T, int d, int tile_t, int tile_f, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + tile_f - 1) / tile_f;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + tile_t - 1) / tile_t;
}

size_t scan_desc_words(int B, int T, int d, bool sparse) {
  i64 n_jt, n_lg, n_tt;
  scan_grid(B, T, d, 4 * (sparse ? kScanTSubSparse : kScanTSubDense), kWave, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * kScanWords * n_lg * kWave);
}

hipError_t launch_scan_block4(const float* A, const float* rhs, float* x, int B, int T, int d,
                              bool sparse, unsigned long long* desc, unsigned int* tickets,
                              uint32_t epoch, Control* ctl, int k_iter, float tol,
                              hipStream_t stream) {
  const int tsub = sparse ? kScanTSubSparse : kScanTSubDense;
  i64 n_jt, n_lg, n_tt;
  scan_grid(B, T, d, 4 * tsub, kWave, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int stride = look_back_anchor_stride(n_lg, scan_wgs_per_cu(1));
  const int n_ctr = ticket_counters(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int a = static_cast<int>(n_jt), c = static_cast<int>(n_lg), e = static_cast<int>(n_tt);
  if (sparse)
    scan_block4_kernel<true, kScanTSubSparse, 1><<<grid, kScanBlock, 0, stream>>>(
        A, rhs, x, T, d, a, c, e, stride, desc, tickets, n_ctr, epoch, ctl, k_iter, tol);
  else
    scan_block4_kernel<false, kScanTSubDense, 1><<<grid, kScanBlock, 0, stream>>>(
        A, rhs, x, T, d, a, c, e, stride, desc, tickets, n_ctr, epoch, ctl, k_iter, tol);
  return hipGetLastError();
}

}  // namespace slstm
