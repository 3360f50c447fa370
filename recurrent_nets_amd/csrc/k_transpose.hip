// Operand preparation for the weight-gradient products of the backward pass.
//
// With P = x W_x^T + bias ("sLSTM in this library", "API notes": W_x is a GEMM), a loss with
// gradient dP gives dW_x = dP^T x and dx = dP W_x (per gate and feature row of W_x). The MFMA
// kernel multiplies K-contiguous bfloat16 operands, so dP^T, x^T and W_x^T are formed here, in
// bfloat16 (float32 dP rounded to nearest even), with the reduction dimension padded by zeros to
// a multiple of 8 (whole 16-byte chunks). The split-K partial products are then summed in a
// fixed order.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace slstm {

constexpr int kTile = 64;

template <bool SRC_F32>
__device__ __forceinline__ float load_elem(const void* src, i64 idx) {
  if constexpr (SRC_F32) {
    return static_cast<const float*>(src)[idx];
  } else {
    return bf16_to_f32(static_cast<const uint16_t*>(src)[idx]);
  }
}

// dst[c, r] = src[r, c] for a rows x cols source; dst rows are ld long, r >= rows is zero.
// Grid: x over 64-row bands of dst's columns (source rows, padding included), y over 64-column
// bands of the source. Reads and writes are each 64 consecutive elements per wave.
template <bool SRC_F32>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const void* __restrict__ src,
                                                             uint16_t* __restrict__ dst, i64 rows,
                                                             int cols, i64 ld) {
  __shared__ float tile[kTile][kTile + 1];
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;  // 0..3
  const i64 r0 = static_cast<i64>(blockIdx.x) * kTile;
  const int c0 = static_cast<int>(blockIdx.y) * kTile;
#pragma unroll
  for (int k = 0; k < kTile / 4; ++k) {
    const int rr = ty + 4 * k;
    const i64 r = r0 + rr;
    const int c = c0 + tx;
    tile[rr][tx] = (r < rows && c < cols) ? load_elem<SRC_F32>(src, r * cols + c) : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kTile / 4; ++k) {
    const int cc = ty + 4 * k;
    const int c = c0 + cc;
    const i64 r = r0 + tx;
    if (c < cols && r < ld) dst[static_cast<i64>(c) * ld + r] = f32_to_bf16_rne(tile[tx][cc]);
  }
}

// dst[r, c] = src[r, c] in bfloat16 for c < cols, zero for cols <= c < ld
template <bool SRC_F32>
__global__ __launch_bounds__(256) void pad_bf16_kernel(const void* __restrict__ src,
                                                       uint16_t* __restrict__ dst, i64 rows,
                                                       int cols, int ld) {
  const i64 n = rows * ld;
  for (i64 i = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<i64>(gridDim.x) * 256) {
    const i64 r = i / ld;
    const int c = static_cast<int>(i - r * ld);
    dst[i] = c < cols ? f32_to_bf16_rne(load_elem<SRC_F32>(src, r * cols + c)) : uint16_t(0);
  }
}

// out[i] = sum over s of part[s * n + i], in order of s
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part,
                                                         float* __restrict__ out, int splits, i64 n) {
  const i64 i = static_cast<i64>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.0f;
  for (int s = 0; s < splits; ++s) acc += part[static_cast<i64>(s) * n + i];
  out[i] = acc;
}

hipError_t launch_transpose_bf16(const void* src, bool src_f32, uint16_t* dst, i64 rows, int cols,
                                 i64 ld, hipStream_t stream) {
  const i64 gx = (ld + kTile - 1) / kTile;
  const i64 gy = (cols + kTile - 1) / kTile;
  if (gx > 0x7fffffffLL || gy > 65535 || ld < rows) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  if (src_f32)
    transpose_bf16_kernel<true><<<grid, 256, 0, stream>>>(src, dst, rows, cols, ld);
  else
    transpose_bf16_kernel<false><<<grid, 256, 0, stream>>>(src, dst, rows, cols, ld);
  return hipGetLastError();
}

hipError_t launch_pad_bf16(const void* src, bool src_f32, uint16_t* dst, i64 rows, int cols, int ld,
                           hipStream_t stream) {
  const i64 n = rows * ld;
  const i64 blocks = std::min<i64>((n + 255) / 256, 65536);
  if (src_f32)
    pad_bf16_kernel<true><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(src, dst, rows, cols, ld);
  else
    pad_bf16_kernel<false><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(src, dst, rows, cols, ld);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, float* out, int splits, i64 n, hipStream_t stream) {
  const i64 blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  sum_splits_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(part, out, splits, n);
  return hipGetLastError();
}

}  // namespace slstm
