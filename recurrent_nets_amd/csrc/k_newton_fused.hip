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
// Decomposition as in the scan kernel: a tile of 64 features of one batch row x 4*TSUB steps
// per workgroup; each thread holds one feature's sub-chunk of TSUB steps (12 Jacobian entries,
// the right-hand side and the iterate per step, in registers); DPP quad scan of sub-chunk
// maps; tile maps and carries staged in LDS; fixed-dataflow look-back across tiles. The step
// before a sub-chunk (its halo) is read from S_k, which this launch never writes.
//
// The residual maximum of S_k goes to the control block. Early stop is exact although the
// update of iteration k is formed together with F_k: the next launch (or the final residual
// pass) finds max|F_k| < tol and declares S_k final; S_k is still intact in the other buffer.
#include "affine4.h"
#include "cell.h"
#include "kernels.h"

namespace slstm {

// sub-chunk length and the occupancy the register allocation is bounded for (waves per SIMD)
#ifndef SLSTM_FUSED_TSUB
#define SLSTM_FUSED_TSUB 4
#endif
#ifndef SLSTM_FUSED_MIN_WAVES
#define SLSTM_FUSED_MIN_WAVES 2
#endif
constexpr int kFusedBlock = 256;
constexpr int kFusedTSub = SLSTM_FUSED_TSUB;

template <bool BF16, int TSUB>
__global__ __launch_bounds__(kFusedBlock, SLSTM_FUSED_MIN_WAVES) void newton_iter_kernel(
    const void* __restrict__ P, const float* __restrict__ R, const float* __restrict__ state0,
    const float* __restrict__ S_in, float* __restrict__ S_out, int T, int d, int n_jt, int n_lg,
    int n_tt, int anchor_stride, int sig_forget, unsigned long long* __restrict__ desc,
    unsigned int* __restrict__ ticket, uint32_t epoch, Control* __restrict__ ctl, int k_iter,
    float tol) {
  if (ctl->stopped) return;
  if (k_iter > 0 && tol > 0.0f && __uint_as_float(ctl->err_bits[k_iter - 1]) < tol) {
    // the previous iterate already met the tolerance: it is the result
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      ctl->stopped = 1;
      ctl->iters = k_iter - 1;
    }
    return;
  }
  __shared__ unsigned int s_ticket;
  __shared__ float s_agg[64][21];
  __shared__ float s_carry[64][4];
  __shared__ float s_max[kFusedBlock / kWave];

  const int tid = threadIdx.x;
  if (tid == 0) {
    const unsigned int total = static_cast<unsigned int>(n_lg) * n_tt;
    const unsigned int tk = atomicAdd(ticket, 1u);
    if (tk == total - 1) atomicExch(ticket, 0u);
    s_ticket = tk;
  }
  __syncthreads();
  const unsigned int tk = __builtin_amdgcn_readfirstlane(s_ticket);
  const int tt = static_cast<int>(tk / n_lg);
  const int lg = static_cast<int>(tk % n_lg);
  const int b = lg / n_jt;
  const int jt = lg - b * n_jt;

  const int wave = tid >> 6;
  const int l = tid & 63;
  const int sc = l & 3;
  const int lane_in_tile = wave * 16 + (l >> 2);
  const unsigned ud = static_cast<unsigned>(d);
  const unsigned j = static_cast<unsigned>(jt * 64 + lane_in_tile);
  const bool valid = j < ud;
  const int t_tile = tt * 4 * TSUB;
  const int t_start = t_tile + sc * TSUB;
  const i64 n_lanes_pad = static_cast<i64>(n_lg) * 64;
  const bool sig = sig_forget != 0;
  // scalar bases of this tile's rows; 32-bit lane offsets (elements) within them
  const i64 tile_row = (static_cast<i64>(b) * T + t_tile) * 4 * static_cast<i64>(d);
  const rsrc_t rsP = make_rsrc(static_cast<const char*>(P) + tile_row * (BF16 ? 2 : 4));
  const rsrc_t rsS = make_rsrc(S_in + tile_row);
  const rsrc_t rsO = make_rsrc(S_out + tile_row);
  const unsigned lane_off = static_cast<unsigned>(sc * TSUB) * 4u * ud + j;

  // the look-back's anchor words, loaded now so that they arrive during the residual phase
  LookBackPrefetch pf;
  if (wave == 0) pf = look_back_prefetch(desc, n_lanes_pad, static_cast<i64>(lg) * 64 + l, tt, anchor_stride);

  float rz = 0.0f, ri = 0.0f, rf = 0.0f, ro = 0.0f;
  CellIn pv = {0.0f, 0.0f, 0.0f, 0.0f};
  if (valid) {
    rz = R[j];
    ri = R[ud + j];
    rf = R[2 * ud + j];
    ro = R[3 * ud + j];
    if (t_start == 0) {
      if (state0 != nullptr) {
        const float* s0 = state0 + static_cast<i64>(b) * 4 * static_cast<i64>(d);
        pv = {s0[j], s0[ud + j], s0[2 * ud + j], s0[3 * ud + j]};
      }
    } else if (t_start < T) {
      const float* sp = S_in + (static_cast<i64>(b) * T + t_start - 1) * 4 * static_cast<i64>(d);
      pv = {sp[j], sp[ud + j], sp[2 * ud + j], sp[3 * ud + j]};
    }
  }

  // ---- residual, Jacobian and right-hand side of the sub-chunk, in registers ----
  float a[TSUB][12], r[TSUB][4], sv[TSUB][4], pg[TSUB][4];
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
      const unsigned o = lane_off + u * 4u * ud;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pg[u][k] = buf_ld_p<BF16>(rsP, o, k * ud);
        sv[u][k] = buf_ld(rsS, 4u * o, 4u * k * ud);
      }
    }
  }
  float fmax_local = 0.0f;
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
      float f[4], Aj[16];
      cell_step<true>(pv, pg[u][0], pg[u][1], pg[u][2], pg[u][3], rz, ri, rf, ro, sig, f, Aj);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[u][k] = f[k] - sv[u][k];
        fmax_local = fmaxf(fmax_local, abs_nan_inf(r[u][k]));
      }
#pragma unroll
      for (int q = 0; q < 12; ++q) a[u][q] = (t == 0) ? 0.0f : Aj[kSpPlane[q]];  // x_0 = 0
      pv = {sv[u][0], sv[u][1], sv[u][2], sv[u][3]};
    } else {
      // identity map
#pragma unroll
      for (int q = 0; q < 12; ++q) a[u][q] = (kSpPlane[q] % 5 == 0) ? 1.0f : 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[u][k] = 0.0f;
        sv[u][k] = 0.0f;
      }
    }
  }

  // ---- compose the sub-chunk, quad scan, look-back (as in the scan kernel) ----
  float M[16], v[4];
#pragma unroll
  for (int e = 0; e < 16; ++e) M[e] = 0.0f;
#pragma unroll
  for (int q = 0; q < 12; ++q) M[kSpPlane[q]] = a[0][q];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = r[0][e];
#pragma unroll
  for (int u = 1; u < TSUB; ++u) {
    float vn[4];
    sp_mul_left(a[u], M);
    sp_vec(a[u], v, r[u], vn);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = vn[e];
  }
  quad_inclusive_scan(M, v, sc);
  if (sc == 3) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s_agg[lane_in_tile][e] = M[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) s_agg[lane_in_tile][16 + e] = v[e];
  }
  const float wm = wave_max(fmax_local);
  if (l == 0) s_max[wave] = wm;
  __syncthreads();
  if (wave == 0) {
    float carry[4];
    tile_look_back(s_agg[l], carry, desc, n_lanes_pad, static_cast<i64>(lg) * 64 + l, tt,
                   anchor_stride, epoch, &pf);
#pragma unroll
    for (int e = 0; e < 4; ++e) s_carry[l][e] = carry[e];
    if (l == 0) {
      float m = s_max[0];
#pragma unroll
      for (int w = 1; w < kFusedBlock / kWave; ++w) m = fmaxf(m, s_max[w]);
      atomic_max_nonneg(&ctl->err_bits[k_iter], m);
    }
  }
  __syncthreads();

  // ---- re-run each sub-chunk from its carry and write the updated iterate ----
  float cin[4], xe[4], xs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cin[e] = s_carry[lane_in_tile][e];
  mat4_vec(M, cin, v, xe);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    xs[e] = quad_perm<0, 0, 1, 2>(xe[e]);
    if (sc == 0) xs[e] = cin[e];
  }
#pragma unroll
  for (int u = 0; u < TSUB; ++u) {
    const int t = t_start + u;
    float xn[4];
    sp_vec(a[u], xs, r[u], xn);
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[e] = xn[e];
    if (valid && t < T) {
      const unsigned o = lane_off + u * 4u * ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) buf_st(sv[u][e] + xs[e], rsO, 4u * o, 4u * e * ud);
    }
  }
  if (blockIdx.x == 0 && tid == 0) ctl->iters = k_iter + 1;
}

static void fused_grid(int B, int T, int d, i64& n_jt, i64& n_lg, i64& n_tt) {
  n_jt = (d + 63) / 64;
  n_lg = static_cast<i64>(B) * n_jt;
  n_tt = (T + 4 * kFusedTSub - 1) / (4 * kFusedTSub);
}

size_t fused_desc_words(int B, int T, int d) {
  i64 n_jt, n_lg, n_tt;
  fused_grid(B, T, d, n_jt, n_lg, n_tt);
  return static_cast<size_t>(n_tt * kLookBackWords * n_lg * 64);
}

hipError_t launch_newton_iteration(const void* P, bool p_bf16, const float* R, const float* state0,
                                   const float* S_in, float* S_out, int B, int T, int d,
                                   bool sig_forget, unsigned long long* desc, unsigned int* ticket,
                                   uint32_t epoch, Control* ctl, int k_iter, float tol,
                                   hipStream_t stream) {
  i64 n_jt, n_lg, n_tt;
  fused_grid(B, T, d, n_jt, n_lg, n_tt);
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int stride = look_back_anchor_stride(n_lg);
  const dim3 grid(static_cast<unsigned>(blocks));
  const int sig = sig_forget ? 1 : 0;
  if (p_bf16)
    newton_iter_kernel<true, kFusedTSub><<<grid, kFusedBlock, 0, stream>>>(
        P, R, state0, S_in, S_out, T, d, static_cast<int>(n_jt), static_cast<int>(n_lg),
        static_cast<int>(n_tt), stride, sig, desc, ticket, epoch, ctl, k_iter, tol);
  else
    newton_iter_kernel<false, kFusedTSub><<<grid, kFusedBlock, 0, stream>>>(
        P, R, state0, S_in, S_out, T, d, static_cast<int>(n_jt), static_cast<int>(n_lg),
        static_cast<int>(n_tt), stride, sig, desc, ticket, epoch, ctl, k_iter, tol);
  return hipGetLastError();
}

}  // namespace slstm
