// Input projection P = x W_x^T + bias on the MFMA matrix cores (bfloat16 in, float32 out).
//
//   P[b, t, g, j] = sum_k x[b, t, k] W_x[g, j, k] + bias[g, j]    (gates g = z, i, f, o)
//
// ("sLSTM in this library", "API notes": W_x is applied as a GEMM; the gate pre-activations
// of the sLSTM step pseudocode in the xLSTM summary card, "Key equations".)
// As a matrix product: C (M x N) = X (M x K) * W^T with M = B*T, N = 4*d_h, K = d_in; both
// operands are K-contiguous, and C row-major is exactly P's (B, T, 4, d_h) layout.
//
// Block tile 128 x 128, K step 64, 256 threads = 4 waves in a 2 x 2 arrangement, each wave a
// 64 x 64 sub-tile made of 2 x 2 v_mfma_f32_32x32x16_bf16 accumulators. Tiles are staged
// through LDS with a padded row stride. The bias is added in the epilogue, so P is written
// once. Workgroups are renumbered so that each of the 8 XCDs works through a contiguous
// range of tiles, ordered in groups of 8 row panels so that concurrently running tiles share
// row and column panels in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace slstm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmBK = 64;
constexpr int kGemmLds = kGemmBK + 8;  // padded row stride in bf16 elements
constexpr int kGemmGroupM = 8;
constexpr int kXcds = 8;

__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ W,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ C, int M, int N, int K,
                                                        int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[kGemmBM * kGemmLds];
  __shared__ __attribute__((aligned(16))) uint16_t sW[kGemmBN * kGemmLds];

  // ---- tile selection: XCD-contiguous ranges, grouped row panels ----
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (nb % kXcds == 0) ? (bid % kXcds) * (nb / kXcds) + bid / kXcds : bid;
  const int per_group = kGemmGroupM * tiles_n;
  const int group = logical / per_group;
  const int in_group = logical % per_group;
  const int gm0 = group * kGemmGroupM;
  const int gsize = min(kGemmGroupM, tiles_m - gm0);
  const int tm = gm0 + in_group % gsize;
  const int tn = in_group / gsize;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;

  const i64 row0 = static_cast<i64>(tm) * kGemmBM;
  const i64 col0 = static_cast<i64>(tn) * kGemmBN;
  for (int k0 = 0; k0 < K; k0 += kGemmBK) {
    // global -> LDS: 128 rows x 64 k of each operand, 16-byte chunks, 4 per thread each
#pragma unroll
    for (int c = tid; c < kGemmBM * (kGemmBK / 8); c += 256) {
      const int row = c >> 3;
      const int col = (c & 7) * 8;
      const i64 gm = row0 + row;
      const i64 gn = col0 + row;
      const int gk = k0 + col;
      uint4 vx = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
      if (gm < M && gk < K) vx = *reinterpret_cast<const uint4*>(X + gm * K + gk);
      if (gn < N && gk < K) vw = *reinterpret_cast<const uint4*>(W + gn * K + gk);
      *reinterpret_cast<uint4*>(sX + row * kGemmLds + col) = vx;
      *reinterpret_cast<uint4*>(sW + row * kGemmLds + col) = vw;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 16) {
      bf16x8 a[2], bm[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sX + (wm * 64 + i * 32 + lrow) * kGemmLds + kk + lk);
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        bm[jn] = *reinterpret_cast<const bf16x8*>(sW + (wn * 64 + jn * 32 + lrow) * kGemmLds + kk + lk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bm[jn], acc[i][jn], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: bias, float32 store. Accumulator r of lane l holds row
  //      8*(r/4) + 4*(l/32) + r%4 and column l%32 of its 32 x 32 tile. ----
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) {
    const i64 n = col0 + wn * 64 + jn * 32 + lrow;
    const float bn = (bias != nullptr && n < N) ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const i64 m = row0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M && n < N) C[m * N + n] = acc[i][jn][r] + bn;
      }
    }
  }
}

hipError_t launch_gemm_bf16(const void* X, const void* W, const float* bias, float* C, i64 M,
                            int N, int K, hipStream_t stream) {
  const i64 tiles_m = (M + kGemmBM - 1) / kGemmBM;
  const i64 tiles_n = (N + kGemmBN - 1) / kGemmBN;
  const i64 blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffffLL || M > 0x7fffffffLL) return hipErrorInvalidValue;
  gemm_bf16_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(
      static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), bias, C, static_cast<int>(M),
      N, K, static_cast<int>(tiles_m), static_cast<int>(tiles_n));
  return hipGetLastError();
}

}  // namespace slstm
