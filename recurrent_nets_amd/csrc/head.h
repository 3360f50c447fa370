// Helpers of the head-mixing kernels (block-diagonal recurrent matrices): a workgroup per
// (batch row, head), one thread per (unit i, gate g) at lane 4 i + g, so the four lanes of a
// unit form a quad and exchange values by DPP.
#pragma once

#include "affine4.h"
#include "common.h"

namespace slstm {

constexpr int kHeadPrefetch = 8;

// barrier for the step-to-step LDS exchange: this thread's LDS accesses have completed
// (lgkmcnt 0, the other counters left at their maxima); global loads stay in flight
__device__ __forceinline__ void head_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// the four values of a unit (one per lane of its quad), in every lane of the quad
__device__ __forceinline__ void quad_gather(float v, float out[4]) {
  out[0] = quad_bcast<0>(v);
  out[1] = quad_bcast<1>(v);
  out[2] = quad_bcast<2>(v);
  out[3] = quad_bcast<3>(v);
}

// row i of gate g's block of head a, d_head floats (R is (4, n_heads, d_head, d_head))
template <int DH>
__device__ __forceinline__ void load_block_row(const float* __restrict__ R, int nh, int a, int i, int g,
                                               float row[DH]) {
  const float4* src = reinterpret_cast<const float4*>(R + ((static_cast<i64>(g) * nh + a) * DH + i) * DH);
#pragma unroll
  for (int k = 0; k < DH / 4; ++k) {
    const float4 v = src[k];
    row[4 * k] = v.x;
    row[4 * k + 1] = v.y;
    row[4 * k + 2] = v.z;
    row[4 * k + 3] = v.w;
  }
}

// v[g] for the lane's gate g = 2 g1 + g0 (the bits held as loop-invariant lane masks): three
// selects, where indexing a register array by g would select among every element
struct GateSel {
  bool g0, g1;
  __device__ __forceinline__ explicit GateSel(int g) : g0((g & 1) != 0), g1((g & 2) != 0) {}
  __device__ __forceinline__ float operator()(float v0, float v1, float v2, float v3) const {
    const float lo = g0 ? v1 : v0;
    const float hi = g0 ? v3 : v2;
    return g1 ? hi : lo;
  }
  __device__ __forceinline__ float operator()(const float v[4]) const { return (*this)(v[0], v[1], v[2], v[3]); }
};

template <int DH>
__device__ __forceinline__ float block_dot(const float row[DH], const float* __restrict__ v) {
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int k = 0; k < DH / 4; ++k) {
    const float4 x = v4[k];
    acc0 = fmaf(row[4 * k], x.x, acc0);
    acc1 = fmaf(row[4 * k + 1], x.y, acc1);
    acc0 = fmaf(row[4 * k + 2], x.z, acc0);
    acc1 = fmaf(row[4 * k + 3], x.w, acc1);
  }
  return acc0 + acc1;
}


// Dynamic LDS reserved by a head-kernel launch (unused by the kernel) so that its n_wg
// workgroups spread evenly over the chip's 256 CUs (160 KiB of LDS each): a workgroup walks all
// of T, so a CU that received more of them than its share would set the kernel's duration. At
// most 64 KiB, the per-workgroup default limit.
inline unsigned int head_spread_lds(long long n_wg, unsigned int static_lds) {
  constexpr long long kCUs = 256, kLdsPerCU = 160 * 1024, kMax = 64 * 1024;
  const long long per_cu = (n_wg + kCUs - 1) / kCUs;
  long long bytes = kLdsPerCU / (per_cu < 1 ? 1 : per_cu) - static_cast<long long>(static_lds) - 1024;
  if (bytes > kMax) bytes = kMax;
  return bytes > 0 ? static_cast<unsigned int>(bytes) : 0u;
}

// DH = d_head as a compile-time constant for the widths the kernels are built for
#define SLSTM_HEAD_DH_DISPATCH(DHV, BODY) \
  switch (DHV) {                          \
    case 8: { constexpr int DH = 8; BODY; break; }    \
    case 16: { constexpr int DH = 16; BODY; break; }  \
    case 32: { constexpr int DH = 32; BODY; break; }  \
    case 64: { constexpr int DH = 64; BODY; break; }  \
    default: return hipErrorInvalidValue;             \
  }

}  // namespace slstm
