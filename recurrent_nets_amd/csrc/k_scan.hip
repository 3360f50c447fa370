// Kernel (b): the block-bidiagonal Newton system solved as an associative scan over 4x4
// affine maps (scan_block4 layout (B, T, 4, 4, d): "Layout" page of the pararnn-torch docs,
// "Naming"; the (J, r) monoid of "sLSTM in this library", "Packed sequences").
//
//   x_1 = rhs_1,   x_t = A_t x_{t-1} + rhs_t        (A at the first step is never used)
//
// Each step is the map x -> A x + r; maps compose as (A2, r2) o (A1, r1) = (A2 A1, A2 r1 + r2).
//
// Work decomposition (one workgroup = 4 waves = one tile of 64 lanes x 4*TSUB steps):
//   * lane   = flattened (b, j); a tile covers 64 consecutive lanes, so each load of the tile
//              reads 256 contiguous bytes of one (b, t, plane) row;
//   * thread = one lane and one sub-chunk of TSUB steps; a wave holds 16 lanes x 4
//              consecutive sub-chunks, the 4 sub-chunks of a lane forming one quad.
// Level 1: every thread composes its sub-chunk sequentially in registers (A and r stay in
//          registers for the whole kernel, so each byte is read from HBM once).
// Level 2: inclusive scan of the 4 sub-chunk aggregates inside each quad with DPP quad
//          permutations; the tile aggregate of each lane is staged in LDS.
// Level 3: decoupled look-back across tiles along T: wave 0 (one thread per lane) publishes
//          the tile aggregate, walks back over predecessor tiles until it meets an inclusive
//          value, and stages the resulting carry in LDS. Tiles take work tickets in launch
//          order, so a predecessor always holds a smaller ticket and is running or done.
// Finally every thread re-runs its sub-chunk from its carry (16 FMA per step) and stores x.
// x may alias rhs: each thread reads its rhs values before writing the same addresses.
#include "common.h"
#include "kernels.h"

namespace slstm {

constexpr int kScanBlock = 256;
constexpr int kScanTSub = 8;
constexpr int kScanTile = 4 * kScanTSub;
constexpr int kScanWords = 24;  // per lane and tile: x_end (4), M (16), v (4)

// C = X Y for row-major 4x4 matrices
__device__ __forceinline__ void mat4_mul(const float X[16], const float Y[16], float C[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      C[4 * i + k] = fmaf(X[4 * i + 0], Y[k],
                          fmaf(X[4 * i + 1], Y[4 + k], fmaf(X[4 * i + 2], Y[8 + k], X[4 * i + 3] * Y[12 + k])));
}

// y = X v + w
__device__ __forceinline__ void mat4_vec(const float X[16], const float v[4], const float w[4],
                                         float y[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    y[i] = fmaf(X[4 * i + 0], v[0], fmaf(X[4 * i + 1], v[1], fmaf(X[4 * i + 2], v[2], fmaf(X[4 * i + 3], v[3], w[i]))));
}

// (M, v) <- (M, v) o (Mp, vp): apply (Mp, vp) first, then (M, v)
__device__ __forceinline__ void compose_after(float M[16], float v[4], const float Mp[16],
                                              const float vp[4]) {
  float Mn[16], vn[4];
  mat4_mul(M, Mp, Mn);
  mat4_vec(M, vp, v, vn);
#pragma unroll
  for (int e = 0; e < 16; ++e) M[e] = Mn[e];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = vn[e];
}

template <int S0, int S1, int S2, int S3>
__device__ __forceinline__ void quad_perm_map(const float M[16], const float v[4], float Mp[16],
                                              float vp[4]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) Mp[e] = quad_perm<S0, S1, S2, S3>(M[e]);
#pragma unroll
  for (int e = 0; e < 4; ++e) vp[e] = quad_perm<S0, S1, S2, S3>(v[e]);
}

__global__ __launch_bounds__(kScanBlock) void scan_block4_kernel(
    const float* __restrict__ A, const float* rhs, float* x, int B, int T, int d, int n_lg,
    int n_tt, unsigned long long* __restrict__ desc, unsigned int* __restrict__ ticket,
    uint32_t epoch, Control* ctl, int k_iter, float tol) {
  if (ctl != nullptr) {
    if (ctl->stopped) return;
    if (tol > 0.0f && __uint_as_float(ctl->err_bits[k_iter]) < tol) {
      // residual already below the tolerance: stop before solving
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctl->stopped = 1;
        ctl->iters = k_iter;
      }
      return;
    }
  }
  __shared__ unsigned int s_ticket;
  __shared__ float s_agg[64][21];
  __shared__ float s_carry[64][4];

  const int tid = threadIdx.x;
  if (tid == 0) {
    const unsigned int total = static_cast<unsigned int>(n_lg) * n_tt;
    const unsigned int tk = atomicAdd(ticket, 1u);
    if (tk == total - 1) atomicExch(ticket, 0u);  // last ticket: reset for the next launch
    s_ticket = tk;
  }
  __syncthreads();
  const unsigned int tk = s_ticket;
  const int tt = static_cast<int>(tk / n_lg);
  const int lg = static_cast<int>(tk % n_lg);

  const int wave = tid >> 6;
  const int l = tid & 63;
  const int sc = l & 3;
  const int lane_in_tile = wave * 16 + (l >> 2);
  const i64 n_lanes = static_cast<i64>(B) * d;
  const i64 n_lanes_pad = static_cast<i64>(n_lg) * 64;
  const i64 lane = static_cast<i64>(lg) * 64 + lane_in_tile;
  const bool valid = lane < n_lanes;
  const int b = valid ? static_cast<int>(lane / d) : 0;
  const int j = valid ? static_cast<int>(lane % d) : 0;
  const int t_start = tt * kScanTile + sc * kScanTSub;
  const i64 dd = d;

  // ---- level 1: load the sub-chunk and compose it ----
  float a[kScanTSub][16], r[kScanTSub][4];
#pragma unroll
  for (int u = 0; u < kScanTSub; ++u) {
    const int t = t_start + u;
    if (valid && t < T) {
      const float* Ap = A + (static_cast<i64>(b) * T + t) * 16 * dd + j;
      const float* rp = rhs + (static_cast<i64>(b) * T + t) * 4 * dd + j;
#pragma unroll
      for (int e = 0; e < 16; ++e) a[u][e] = Ap[e * dd];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[u][e] = rp[e * dd];
      if (t == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) a[u][e] = 0.0f;  // x_0 = 0: the first map is constant
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) a[u][e] = (e % 5 == 0) ? 1.0f : 0.0f;  // identity map
#pragma unroll
      for (int e = 0; e < 4; ++e) r[u][e] = 0.0f;
    }
  }
  float M[16], v[4];
#pragma unroll
  for (int e = 0; e < 16; ++e) M[e] = a[0][e];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = r[0][e];
#pragma unroll
  for (int u = 1; u < kScanTSub; ++u) {
    // (M, v) <- (a_u, r_u) o (M, v)
    float Mn[16], vn[4];
    mat4_mul(a[u], M, Mn);
    mat4_vec(a[u], v, r[u], vn);
#pragma unroll
    for (int e = 0; e < 16; ++e) M[e] = Mn[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = vn[e];
  }

  // ---- level 2: inclusive scan of the quad's sub-chunk aggregates (DPP) ----
  {
    float Mp[16], vp[4];
    quad_perm_map<0, 0, 1, 2>(M, v, Mp, vp);  // from sub-chunk sc - 1
    if (sc >= 1) compose_after(M, v, Mp, vp);
    quad_perm_map<0, 1, 0, 1>(M, v, Mp, vp);  // from sub-chunk sc - 2
    if (sc >= 2) compose_after(M, v, Mp, vp);
  }
  if (sc == 3) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s_agg[lane_in_tile][e] = M[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) s_agg[lane_in_tile][16 + e] = v[e];
  }
  __syncthreads();

  // ---- level 3: decoupled look-back, one thread per lane of the tile ----
  if (wave == 0) {
    const i64 my_lane = static_cast<i64>(lg) * 64 + l;
    float Mt[16], vt[4], carry[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 16; ++e) Mt[e] = s_agg[l][e];
#pragma unroll
    for (int e = 0; e < 4; ++e) vt[e] = s_agg[l][16 + e];
    auto word = [&](int tile, int w) {
      return desc + (static_cast<i64>(tile) * kScanWords + w) * n_lanes_pad + my_lane;
    };
    if (tt > 0) {
      // accumulated map of the tiles between the one being inspected and this one
      float Macc[16], vacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < 16; ++e) Macc[e] = (e % 5 == 0) ? 1.0f : 0.0f;
      bool published = false;
      int p = tt - 1;
      while (true) {
        float xin[4];
        bool inc = true;
#pragma unroll
        for (int e = 0; e < 4; ++e) inc &= tag_load(word(p, e), epoch, xin[e]);
        if (inc) {
          mat4_vec(Macc, xin, vacc, carry);
          break;
        }
        if (!published) {
          // let successors look past this tile while it waits
#pragma unroll
          for (int e = 0; e < 16; ++e) tag_store(word(tt, 4 + e), Mt[e], epoch);
#pragma unroll
          for (int e = 0; e < 4; ++e) tag_store(word(tt, 20 + e), vt[e], epoch);
          published = true;
        }
        float Mp[16], vp[4];
        bool agg = true;
#pragma unroll
        for (int e = 0; e < 16; ++e) agg &= tag_load(word(p, 4 + e), epoch, Mp[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) agg &= tag_load(word(p, 20 + e), epoch, vp[e]);
        if (agg) {
          compose_after(Macc, vacc, Mp, vp);
          if (--p < 0) {  // walked past the first tile: x before it is zero
#pragma unroll
            for (int e = 0; e < 4; ++e) carry[e] = vacc[e];
            break;
          }
          continue;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    float xend[4];
    mat4_vec(Mt, carry, vt, xend);
#pragma unroll
    for (int e = 0; e < 4; ++e) tag_store(word(tt, e), xend[e], epoch);
#pragma unroll
    for (int e = 0; e < 4; ++e) s_carry[l][e] = carry[e];
  }
  __syncthreads();

  // ---- re-run each sub-chunk from its carry ----
  float cin[4], xe[4], xs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cin[e] = s_carry[lane_in_tile][e];
  mat4_vec(M, cin, v, xe);  // value at the end of this sub-chunk
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    xs[e] = quad_perm<0, 0, 1, 2>(xe[e]);
    if (sc == 0) xs[e] = cin[e];
  }
#pragma unroll
  for (int u = 0; u < kScanTSub; ++u) {
    const int t = t_start + u;
    float xn[4];
    mat4_vec(a[u], xs, r[u], xn);
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[e] = xn[e];
    if (valid && t < T) {
      float* xp = x + (static_cast<i64>(b) * T + t) * 4 * dd + j;
#pragma unroll
      for (int e = 0; e < 4; ++e) xp[e * dd] = xs[e];
    }
  }
}

size_t scan_desc_words(int B, int T, int d) {
  const i64 n_lg = (static_cast<i64>(B) * d + 63) / 64;
  const i64 n_tt = (T + kScanTile - 1) / kScanTile;
  return static_cast<size_t>(n_tt * kScanWords * n_lg * 64);
}

hipError_t launch_scan_block4(const float* A, const float* rhs, float* x, int B, int T, int d,
                              unsigned long long* desc, unsigned int* ticket, uint32_t epoch,
                              Control* ctl, int k_iter, float tol, hipStream_t stream) {
  const i64 n_lg = (static_cast<i64>(B) * d + 63) / 64;
  const i64 n_tt = (T + kScanTile - 1) / kScanTile;
  const i64 blocks = n_lg * n_tt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  scan_block4_kernel<<<dim3(static_cast<unsigned>(blocks)), kScanBlock, 0, stream>>>(
      A, rhs, x, B, T, d, static_cast<int>(n_lg), static_cast<int>(n_tt), desc, ticket, epoch, ctl,
      k_iter, tol);
  return hipGetLastError();
}

}  // namespace slstm
