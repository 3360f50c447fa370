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
//
// m = max(a, i~) makes one of the two gates exactly e^0 = 1: with beta = (a >= i~) and
// e = e^{-|a - i~|}, (i', f') = (e, 1) when beta and (1, e) otherwise. Both are bitwise the
// values e^{i~ - m} and e^{a - m}, from one exponential. On the branch the max takes, the
// derivatives of the c and n rows reduce to (with l' = dl/df~ and D = l' r_f - r_i)
//   dc/dm' = e (beta ? -z : c'),   dn/dm' = e (beta ? -1 : n'),
//   dc/dh' = D dc/dm' + i' dz/dh',  dn/dh' = D dn/dm',
// and dm/dm' = beta, dm/dh' = beta ? l' r_f : r_i.
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
  const float e = exp_fast(-fabsf(a - it));
  const float ig = beta ? e : 1.0f;
  const float fg = beta ? 1.0f : e;
  const float c = fmaf(fg, pv.c, ig * z);
  const float n = fmaf(fg, pv.n, ig);
  const float rn = rcp_fast(n);
  const float h = o * c * rn;
  s[0] = c;
  s[1] = n;
  s[2] = m;
  s[3] = h;
  if constexpr (JAC) {
    const float lrf = dlf * rf;
    const float D = lrf - ri;
    const float c_m = e * (beta ? -z : pv.c);
    const float n_m = e * (beta ? -1.0f : pv.n);
    const float dz_dh = fmaf(-z, z, 1.0f) * rz;
    const float do_dh = fmaf(-o, o, o) * ro;
    const float c_h = fmaf(c_m, D, ig * dz_dh);
    const float n_h = n_m * D;
    // row h = o c / n: (o/n) dc - (o c / n^2) dn, plus (c/n) do on h'
    const float q1 = o * rn;
    const float q2 = h * rn;
    A[0] = fg;     A[1] = 0.0f;   A[2] = c_m;   A[3] = c_h;
    A[4] = 0.0f;   A[5] = fg;     A[6] = n_m;   A[7] = n_h;
    A[8] = 0.0f;   A[9] = 0.0f;   A[10] = beta ? 1.0f : 0.0f;   A[11] = beta ? lrf : ri;
    A[12] = q1 * fg;
    A[13] = -q2 * fg;
    A[14] = fmaf(q1, c_m, -q2 * n_m);
    A[15] = fmaf(q1, c_h, fmaf(-q2, n_h, (c * rn) * do_dh));
  }
}

// Vector-Jacobian product of one step at the state before it (pv) and its pre-activations:
// given lam = dL/ds for the state the step produces, returns dx = dL/dx~ for the gate
// pre-activations (z, i, f, o) (= dL/dP of the step) and lam_prev = dL/ds' = A^T lam. The
// backward of "sLSTM in this library", section "Backward", one step of it:
//   h = o c / n folds into the c and n adjoints: lc = lam_c + (o/n) lam_h, ln = lam_n - (h/n) lam_h,
//   c = f' c' + i' z, n = f' n' + i':  dL/df' = lc c' + ln n',  dL/di' = lc z + ln,  dL/dz = lc i'
//   one of (i', f') is 1 and the other e = e^{-|a - i~|} (see cell_step); with
//   w = beta ? e dL/di' : -e dL/df', the stabiliser m = max(a, i~) gives
//   dL/di~ = w + (1 - beta) lam_m,  dL/da = -w + beta lam_m  (a = l(f~) + m')
//   dL/dz~ = dL/dz (1 - z^2),  dL/do~ = (c/n) lam_h o (1 - o),  dL/df~ = dL/da l'(f~)
//   lam_prev = (lc f', ln f', dL/da, sum_x r_x dL/dx~)   (h' enters only through x~ = p + r h')
__device__ __forceinline__ void cell_vjp(const CellIn& pv, float pz, float pi, float pf, float po,
                                         float rz, float ri, float rf, float ro, bool sig_forget,
                                         const float lam[4], float dx[4], float lam_prev[4]) {
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
  const float e = exp_fast(-fabsf(a - it));
  const float ig = beta ? e : 1.0f;
  const float fg = beta ? 1.0f : e;
  const float c = fmaf(fg, pv.c, ig * z);
  const float n = fmaf(fg, pv.n, ig);
  const float rn = rcp_fast(n);
  const float cn = c * rn;
  const float lc = fmaf(o * rn, lam[3], lam[0]);
  const float ln = fmaf(-o * cn * rn, lam[3], lam[1]);
  const float lfg = fmaf(lc, pv.c, ln * pv.n);
  const float lig = fmaf(lc, z, ln);
  const float w = beta ? e * lig : -e * lfg;
  const float da = beta ? lam[2] - w : -w;
  dx[0] = lc * ig * fmaf(-z, z, 1.0f);
  dx[1] = beta ? w : w + lam[2];
  dx[2] = da * dlf;
  dx[3] = cn * lam[3] * fmaf(-o, o, o);
  lam_prev[0] = lc * fg;
  lam_prev[1] = ln * fg;
  lam_prev[2] = da;
  lam_prev[3] = fmaf(rz, dx[0], fmaf(ri, dx[1], fmaf(rf, dx[2], ro * dx[3])));
}

}  // namespace slstm
