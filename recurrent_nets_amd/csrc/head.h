// Helpers of the head-mixing kernels (block-diagonal recurrent matrices): a workgroup per
// (batch row, head), one thread per (unit i, gate g) at lane 4 i + g, so the four lanes of a
// unit form a quad and exchange values by DPP.
#pragma once

#include "affine4.h"
#include "cell.h"
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
  // all of v's LDS reads first, then the FMAs: the scheduling fence keeps the reads in flight
  // together (otherwise the scheduler may trade them for registers and wait on each in turn)
  // (in chunks of at most 8 reads, which bounds the registers they hold; heads of 64 units keep
  // the compiler's own schedule)
  constexpr int kChunk = DH / 4 < 8 ? DH / 4 : 8;
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int k0 = 0; k0 < DH / 4; k0 += kChunk) {
    float4 x[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) x[k] = v4[k0 + k];
    if constexpr (DH <= 32) __builtin_amdgcn_sched_barrier(0);  // at 64 the held reads spill
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float* r = row + 4 * (k0 + k);
      acc0 = fmaf(r[0], x[k].x, acc0);
      acc1 = fmaf(r[1], x[k].y, acc1);
      acc0 = fmaf(r[2], x[k].z, acc0);
      acc1 = fmaf(r[3], x[k].w, acc1);
    }
  }
  return acc0 + acc1;
}

// One cell step under head mixing in linearised form: the next state s (c, n, m, h) from the
// previous state pv (its h enters only through the pre-activations x, which already hold R h')
// and the coefficients of the step's Jacobian in the structure the cell gives it (the nonzero
// entries of its own-state and gate Jacobians):
//   own-state columns: dc/dc' = dn/dn' = f', dc/dm' = c_m, dn/dm' = n_m, dm/dm' = mm;
//   gate columns: dc/dz~ = g_z, dc/di~ = -c_m, dc/df~ = c_m l', dn/di~ = -n_m, dn/df~ = n_m l',
//   dm/di~ = g_mi, dm/df~ = g_mf; the h row is the quotient rule q1 dc - qn dn - qm dm plus
//   dh/do~ = g_o.
struct CellLin {
  float fg, c_m, n_m, gz, mm, gm_i, gm_f, dlf, q1, qn, qm, go;
};

__device__ __forceinline__ void cell_step_lin(const CellIn& pv, const float x[4], bool sig_forget, bool floored,
                                              float s[4], CellLin& L) {
  const float z = tanh_fast(x[0]);
  const float it = x[1];
  const float o = sigmoidf(x[3]);
  float lf, dlf;
  if (sig_forget) {
    lf = log_sigmoidf(x[2]);
    dlf = sigmoidf(-x[2]);
  } else {
    lf = x[2];
    dlf = 1.0f;
  }
  const float a = lf + pv.m;
  const bool beta = a >= it;
  const float m = beta ? a : it;
  const float e = exp_fast(-fabsf(a - it));
  const float ig = beta ? e : 1.0f;
  const float fg = beta ? 1.0f : e;
  const float c = fmaf(fg, pv.c, ig * z);
  const float n = fmaf(fg, pv.n, ig);
  const Readout rdn = readout(n, m, floored);
  const float rn = rdn.rD;
  const float q1 = o * rn;  // h = (o / D) c, as the channelwise cell forms it
  const float h = q1 * c;
  s[0] = c;
  s[1] = n;
  s[2] = m;
  s[3] = h;
  L.fg = fg;
  L.c_m = e * (beta ? -z : pv.c);
  L.n_m = e * (beta ? -1.0f : pv.n);
  L.gz = ig * fmaf(-z, z, 1.0f);
  L.mm = beta ? 1.0f : 0.0f;
  L.gm_i = beta ? 0.0f : 1.0f;
  L.gm_f = beta ? dlf : 0.0f;
  L.dlf = dlf;
  L.q1 = q1;
  const float q2 = h * rn;
  L.qn = floored ? q2 * rdn.dn : q2;
  L.qm = floored ? q2 * rdn.dm : 0.0f;
  L.go = (c * rn) * fmaf(-o, o, o);
}

// Jacobian-vector product of the step: d = A_own (ds_c, ds_n, ds_m) + G y for every slot, with
// ds the change of the previous state and y the change of the pre-activations (z, i, f, o)
__device__ __forceinline__ void cell_jvp(const CellLin& L, const float ds[4], const float y[4], float d[4]) {
  const float u = fmaf(L.dlf, y[2], ds[2] - y[1]);
  d[0] = fmaf(L.fg, ds[0], fmaf(L.c_m, u, L.gz * y[0]));
  d[1] = fmaf(L.fg, ds[1], L.n_m * u);
  d[2] = fmaf(L.mm, ds[2], fmaf(L.gm_i, y[1], L.gm_f * y[2]));
  d[3] = fmaf(L.q1, d[0], fmaf(-L.qn, d[1], fmaf(-L.qm, d[2], L.go * y[3])));
}

// Vector-Jacobian product of the step, the transpose of cell_jvp: for the adjoint lam of the
// next state, dx = G^T lam (the gradient of the pre-activations z, i, f, o) and the own-state
// part of A^T lam (the previous state's c, n, m)
__device__ __forceinline__ void cell_vjp_lin(const CellLin& L, const float lam[4], float dx[4], float dprev[3]) {
  const float lc = fmaf(L.q1, lam[3], lam[0]);
  const float ln = fmaf(-L.qn, lam[3], lam[1]);
  const float lm = fmaf(-L.qm, lam[3], lam[2]);
  const float w = fmaf(L.c_m, lc, L.n_m * ln);  // c_m lc + n_m ln
  dx[0] = L.gz * lc;
  dx[1] = fmaf(L.gm_i, lm, -w);
  dx[2] = fmaf(L.dlf, w, L.gm_f * lm);
  dx[3] = L.go * lam[3];
  dprev[0] = L.fg * lc;
  dprev[1] = L.fg * ln;
  dprev[2] = fmaf(L.mm, lm, w);
}

// Dynamic LDS reserved by a head-kernel launch (unused by the kernel) so that its n_wg
// workgroups spread evenly over the chip's 256 CUs (160 KiB of LDS each): a workgroup walks all
// of T, so a CU that received more of them than its share would set the kernel's duration. At
// most 64 KiB, the per-workgroup default limit.
// compute units of the current device (256 on MI355X when the query fails)
inline int head_device_cus() {
  static int cus = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return cus;
}

inline unsigned int head_spread_lds(long long n_wg, unsigned int static_lds) {
  constexpr long long kLdsPerCU = 160 * 1024, kMax = 64 * 1024;
  const long long cus = head_device_cus();
  const long long per_cu = (n_wg + cus - 1) / cus;
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
    case 128: { constexpr int DH = 128; BODY; break; } \
    default: return hipErrorInvalidValue;             \
  }
// the widths of the one-sweep Newton kernel (a 128-unit head's K + 2 stages exceed the register
// file; such heads iterate kernel by kernel)
#define SLSTM_HEAD_SWEEP_DH_DISPATCH(DHV, BODY) \
  switch (DHV) {                          \
    case 8: { constexpr int DH = 8; BODY; break; }    \
    case 16: { constexpr int DH = 16; BODY; break; }  \
    case 32: { constexpr int DH = 32; BODY; break; }  \
    case 64: { constexpr int DH = 64; BODY; break; }  \
    default: return hipErrorInvalidValue;             \
  }

}  // namespace slstm
