// Input projection P = x W_x^T + bias on the MFMA matrix cores (bfloat16 in, float32 out).
//
//   P[b, t, g, j] = sum_k x[b, t, k] W_x[g, j, k] + bias[g, j]    (gates g = z, i, f, o)
//
// ("sLSTM in this library", "API notes": W_x is applied as a GEMM; the gate pre-activations
// of the sLSTM step pseudocode in the xLSTM summary card, "Key equations".)
// As a matrix product: C (M x N) = X (M x K) * W^T with M = B*T, N = 4*d_h, K = d_in; both
// operands are K-contiguous, and C row-major is exactly P's (B, T, 4, d_h) layout.
//
// Block tile 256 x 256, K step 64, 512 threads = 8 waves in a 2 x 4 arrangement, each wave a
// 128 x 64 sub-tile made of 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators (128 accumulator
// registers). Per 16-deep K slice a wave reads 6 KB of LDS for 8 MFMAs. Both operand tiles
// are staged through LDS with a padded row stride, double-buffered: the global loads of K step
// s+1 are in flight (in registers) while step s is multiplied, and one barrier per step
// separates the two buffers. Rows past M or N read zero (buffer loads against the operand's
// extent); a K tail is zeroed explicitly. The bias is added in the epilogue, so P is written
// once. Workgroups are renumbered so that each of the 8 XCDs works through a contiguous range
// of tiles, ordered in groups of row panels so that the tiles an XCD runs together share
// their row and column panels in its L2.
#include "common.h"
#include "kernels.h"

namespace slstm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmLds = kGemmBK + 8;  // padded row stride in bf16 elements
constexpr int kGemmStage = (kGemmBM + kGemmBN) * kGemmLds;  // bf16 elements per LDS stage
constexpr int kGemmThreads = 512;
constexpr int kGemmGroupM = 8;
constexpr int kXcds = 8;
constexpr int kGemmLoads = kGemmBM * kGemmBK / 8 / kGemmThreads;  // 16-byte chunks per thread and operand
// a byte offset beyond every tile extent: buffer loads there return zero, stores are dropped
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc_bytes(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ W,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ C, int M, int N,
                                                                  int K, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kGemmStage];

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
  const int wm = wave >> 2;  // 0..1: 128-row half
  const int wn = wave & 3;   // 0..3: 64-column quarter
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;

  const i64 row0 = static_cast<i64>(tm) * kGemmBM;
  const i64 col0 = static_cast<i64>(tn) * kGemmBN;
  // operand tiles as buffers: rows beyond M (N) fall outside the extent and read as zero
  const uint32_t x_bytes = static_cast<uint32_t>(min<i64>(M - row0, kGemmBM) * K * 2);
  const uint32_t w_bytes = static_cast<uint32_t>(min<i64>(N - col0, kGemmBN) * K * 2);
  const rsrc_t rX = make_rsrc_bytes(X + row0 * K, x_bytes);
  const rsrc_t rW = make_rsrc_bytes(W + col0 * K, w_bytes);

  u32x4 ra[kGemmLoads], rb[kGemmLoads];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kGemmLoads; ++i) {
      const int c = tid + kGemmThreads * i;
      const int row = c >> 3;
      const int gk = k0 + (c & 7) * 8;
      // a K tail chunk is pointed past the extent, where the load returns zero
      const uint32_t off = gk < K ? static_cast<uint32_t>((row * K + gk) * 2) : kOutside;
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0);
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    uint16_t* sA = smem + stage * kGemmStage;
    uint16_t* sB = sA + kGemmBM * kGemmLds;
#pragma unroll
    for (int i = 0; i < kGemmLoads; ++i) {
      const int c = tid + kGemmThreads * i;
      const int row = c >> 3;
      const int col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(sA + row * kGemmLds + col) = ra[i];
      *reinterpret_cast<u32x4*>(sB + row * kGemmLds + col) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;

  const int nk = (K + kGemmBK - 1) / kGemmBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kGemmBK);
    const uint16_t* sA = smem + cur * kGemmStage;
    const uint16_t* sB = sA + kGemmBM * kGemmLds;
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 16) {
      bf16x8 a[4], bm[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * 128 + i * 32 + lrow) * kGemmLds + kk + lk);
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        bm[jn] = *reinterpret_cast<const bf16x8*>(sB + (wn * 64 + jn * 32 + lrow) * kGemmLds + kk + lk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bm[jn], acc[i][jn], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bias, float32 store. Accumulator r of lane l holds row
  //      8*(r/4) + 4*(l/32) + r%4 and column l%32 of its 32 x 32 tile. Stores go through a
  //      buffer over the output tile: rows past M fall outside its extent and are dropped,
  //      columns past N are pointed outside it. ----
  const uint32_t c_bytes = static_cast<uint32_t>(min<i64>(M - row0, kGemmBM) * N * 4);
  const rsrc_t rC = make_rsrc_bytes(C + row0 * N + col0, c_bytes);
  const int n_in = N - static_cast<int>(col0);  // columns of this tile inside C
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) {
    const int nl = wn * 64 + jn * 32 + lrow;
    const bool col_ok = nl < n_in;
    const float bn = (bias != nullptr && col_ok) ? bias[col0 + nl] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const uint32_t off = col_ok ? static_cast<uint32_t>((ml * N + nl) * 4) : kOutside;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][jn][r] + bn), rC, off, 0, 0);
      }
    }
  }
}

hipError_t launch_gemm_bf16(const void* X, const void* W, const float* bias, float* C, i64 M,
                            int N, int K, hipStream_t stream) {
  const i64 tiles_m = (M + kGemmBM - 1) / kGemmBM;
  const i64 tiles_n = (N + kGemmBN - 1) / kGemmBN;
  const i64 blocks = tiles_m * tiles_n;
  // operand and output tiles are addressed with 32-bit byte offsets below kOutside
  if (blocks > 0x7fffffffLL || M > 0x7fffffffLL || static_cast<i64>(kGemmBM) * K * 2 >= kOutside ||
      static_cast<i64>(kGemmBM) * N * 4 >= kOutside)
    return hipErrorInvalidValue;
  gemm_bf16_kernel<<<dim3(static_cast<unsigned>(blocks)), kGemmThreads, 0, stream>>>(
      static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), bias, C, static_cast<int>(M),
      N, K, static_cast<int>(tiles_m), static_cast<int>(tiles_n));
  return hipGetLastError();
}

}  // namespace slstm
