// The stabilised sLSTM cell for one feature (channelwise mixing, mix='diag'), float32.
//
// Equations: "xLSTM: Extended Long Short-Term Memory" (summary card), sLSTM step pseudocode
// under "Key equations" (paper section 2.2, appendix A.2), with the stabiliser of the
// educational reimplementation page, section "Exponential gating + the stabilizer (the crux)":
//   x~ = p_x + r_x h'  (x = z, i, f, o; channelwise R, "sLSTM in this library", "Cell")
//   z = tanh z~, o = sigma(o~), l = f~ (exponential forget gate) or log sigma(f~) (sigmoid)
//   a = l + m', m = max(a, i~) (ties take a), i' = exp(i~ - m), f' = exp(a - m)
//   c = f' c' + i' z, n = f' n' + i', h = o c / n
// The 4x4 Jacobian A = d(c, n, m, h) / d(c', n', m', h') is the analytic derivative of these
// equations, on the branch the max takes; (c, n', m) rows have structural zeros.
#pragma once
#include "common.h"

namespace slstm {

struct CellIn {
  float c, n, m, h;  // previous state
};

// Transcendentals on the hardware units, from their defining identities. Each is within a
// few units in the last place of float32 where its value carries weight (absolute error
// around 1e-7 where it is small), which is well inside the state's float32 rounding floor.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// e^x = 2^(x log2 e) (v_exp_f32)
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// 1 / x (v_rcp_f32)
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
// sigma(x) = 1 / (1 + e^-x)
__device__ __forceinline__ float sigmoidf(float x) { return rcp_fast(1.0f + exp_fast(-x)); }
// tanh x = 1 - 2 / (1 + e^{2x})
__device__ __forceinline__ float tanh_fast(float x) { return 1.0f - 2.0f * rcp_fast(1.0f + exp_fast(2.0f * x)); }
// log sigma(x) = -softplus(-x) = -(max(-x, 0) + ln(1 + e^{-|x|})), finite for any finite x
__device__ __forceinline__ float log_sigmoidf(float x) {
  return -(fmaxf(-x, 0.0f) + kLn2 * __builtin_amdgcn_logf(1.0f + exp_fast(-fabsf(x))));
}

// One step. Writes the next state s[4] = (c, n, m, h); with JAC also A[16] row-major
// (A[4*row + col] = d s[row] / d prev[col]).
template <bool JAC>
__device__ __forceinline__ void cell_step(const CellIn& pv, float pz, float pi, float pf, float po,
                                          float rz, float ri, float rf, float ro, bool sig_forget,
                                          float s[4], float A[16]) {
  const float zt = fmaf(rz, pv.h, pz);
  const float it = fmaf(ri, pv.h, pi);
  const float ft = fmaf(rf, pv.h, pf);
  const float ot = fmaf(ro, pv.h, po);
  const float z = tanh_fast(zt);
  const float o = sigmoidf(ot);
  float lf, dlf;
  if (sig_forget) {
    lf = log_sigmoidf(ft);
    dlf = sigmoidf(-ft);
  } else {
    lf = ft;
    dlf = 1.0f;
  }
  const float a = lf + pv.m;
  const bool beta = a >= it;
  const float m = beta ? a : it;
  const float ig = exp_fast(it - m);
  const float fg = exp_fast(a - m);
  const float c = fmaf(fg, pv.c, ig * z);
  const float n = fmaf(fg, pv.n, ig);
  const float rn = rcp_fast(n);
  const float h = o * c * rn;
  s[0] = c;
  s[1] = n;
  s[2] = m;
  s[3] = h;
  if constexpr (JAC) {
    const float b = beta ? 1.0f : 0.0f;
    const float dm_dh = beta ? dlf * rf : ri;
    const float dig_dm = -b * ig;
    const float dig_dh = ig * (ri - dm_dh);
    const float dfg_dm = (1.0f - b) * fg;
    const float dfg_dh = fg * (dlf * rf - dm_dh);
    const float dz_dh = (1.0f - z * z) * rz;
    const float do_dh = o * (1.0f - o) * ro;
    // rows c and n
    const float c_m = pv.c * dfg_dm + z * dig_dm;
    const float c_h = pv.c * dfg_dh + z * dig_dh + ig * dz_dh;
    const float n_m = pv.n * dfg_dm + dig_dm;
    const float n_h = pv.n * dfg_dh + dig_dh;
    // row h = o c / n: (o/n) dc - (o c / n^2) dn, plus (c/n) do on h'
    const float q1 = o * rn;
    const float q2 = h * rn;
    A[0] = fg;     A[1] = 0.0f;   A[2] = c_m;   A[3] = c_h;
    A[4] = 0.0f;   A[5] = fg;     A[6] = n_m;   A[7] = n_h;
    A[8] = 0.0f;   A[9] = 0.0f;   A[10] = b;    A[11] = dm_dh;
    A[12] = q1 * fg;
    A[13] = -q2 * fg;
    A[14] = q1 * c_m - q2 * n_m;
    A[15] = q1 * c_h - q2 * n_h + (c * rn) * do_dh;
  }
}

}  // namespace slstm
