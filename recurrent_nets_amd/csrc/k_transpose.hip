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

// dst[c, r] = src[r, c] for a rows x cols source; dst rows are ld long (ld a multiple of 8),
// r >= rows is zero. Grid: x over 64-row bands of the source (dst's columns, padding included),
// y over 64-column bands. A 64 x 64 tile goes through LDS as bfloat16: loads of 16 bytes along
// the source rows (scalar loads where the rows are not whole 16-byte chunks), then each thread
// gathers two adjacent columns of 8 consecutive rows (8 LDS words) and writes two 16-byte chunks
// of dst rows.
template <bool SRC_F32>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const void* __restrict__ src,
                                                             uint16_t* __restrict__ dst, i64 rows,
                                                             int cols, i64 ld) {
  constexpr int kLdsRow = kTile + 8;  // 144-byte rows: 16-byte aligned, spread over banks
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile][kLdsRow];
  const int tid = threadIdx.x;
  const i64 r0 = static_cast<i64>(blockIdx.x) * kTile;
  const int c0 = static_cast<int>(blockIdx.y) * kTile;
  if constexpr (SRC_F32) {
    const float* s = static_cast<const float*>(src);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = tid + 256 * k;  // 1024 chunks of 4
      const int rr = q >> 4, cc = (q & 15) * 4;
      const i64 r = r0 + rr;
      const int c = c0 + cc;
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (r < rows) {
        if (c + 4 <= cols && (cols & 3) == 0) {
          const float4 f = *reinterpret_cast<const float4*>(s + r * cols + c);
          v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < cols) v[e] = s[r * cols + c + e];
        }
      }
      uint2 packed;
      packed.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
      packed.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
      *reinterpret_cast<uint2*>(&tile[rr][cc]) = packed;
    }
  } else {
    const uint16_t* s = static_cast<const uint16_t*>(src);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = tid + 256 * k;  // 512 chunks of 8
      const int rr = q >> 3, cc = (q & 7) * 8;
      const i64 r = r0 + rr;
      const int c = c0 + cc;
      uint4 v = {0u, 0u, 0u, 0u};
      if (r < rows) {
        if (c + 8 <= cols && (cols & 7) == 0) {
          v = *reinterpret_cast<const uint4*>(s + r * cols + c);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < cols) w[e >> 1] |= static_cast<uint32_t>(s[r * cols + c + e]) << (16 * (e & 1));
          v = {w[0], w[1], w[2], w[3]};
        }
      }
      *reinterpret_cast<uint4*>(&tile[rr][cc]) = v;
    }
  }
  __syncthreads();
  // thread: columns cc, cc + 1 of the tile (two dst rows), source rows rq .. rq + 7
  const int cc = 2 * (tid >> 3);
  const int rq = (tid & 7) * 8;
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = *reinterpret_cast<const uint32_t*>(&tile[rq + 2 * i][cc]);
    const uint32_t b = *reinterpret_cast<const uint32_t*>(&tile[rq + 2 * i + 1][cc]);
    lo[i] = (a & 0xffffu) | (b << 16);            // column cc, rows rq + 2i, rq + 2i + 1
    hi[i] = (a >> 16) | (b & 0xffff0000u);        // column cc + 1
  }
  const i64 r = r0 + rq;
  if (r < ld) {
    const int c = c0 + cc;
    if (c < cols) *reinterpret_cast<uint4*>(dst + static_cast<i64>(c) * ld + r) = {lo[0], lo[1], lo[2], lo[3]};
    if (c + 1 < cols) *reinterpret_cast<uint4*>(dst + static_cast<i64>(c + 1) * ld + r) = {hi[0], hi[1], hi[2], hi[3]};
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
  if (gx > 0x7fffffffLL || gy > 65535 || ld < rows || ld % 8 != 0) return hipErrorInvalidValue;
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
