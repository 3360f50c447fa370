// The stabilised sLSTM cell for one feature (channelwise mixing, mix='diag'), float32.
//
// Equations: "xLSTM: Extended Long Short-Term Memory" (summary card), sLSTM step pseudocode
// under "Key equations" (paper section 2.2, appendix A.2), with the stabiliser of the
// educational reimplementation page, section "Exponential gating + the stabilizer (the crux)":
//   x~ = p_x + r_x h'  (x = z, i, f, o; channelwise R, "sLSTM in this library", "Cell")
//   z = tanh z~, o = sigma(o~), l = f~ (exponential forget gate) or log sigma(f~) (sigmoid)
//   a = l + m', m = max(a, i~) (ties take a), i' = exp(i~ - m), f' = exp(a - m)
//   c = f' c' + i' z, n = f' n' + i', h = o c / n
// or, with the floored read-out of the educational page (same section, and its deviations
// item 1), h = o c / max(|n|, e^{-m}, 1e-6).
// The 4x4 Jacobian A = d(c, n, m, h) / d(c', n', m', h') is the analytic derivative of these
// equations, on the branch each max takes; (c, n', m) rows have structural zeros.
//
// The cell mode of a kernel is an int: bit 0 the sigmoid forget gate (else exponential), bit 1
// the floored read-out.
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
// tanh x = 1 - 2 / (1 + e^{2x}), e^{2x} = 2^(x (2 log2 e)): the doubled constant is exact, so this
// is bitwise exp_fast(2 x) with one multiply fewer
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.0f - 2.0f * rcp_fast(1.0f + __builtin_amdgcn_exp2f(x * (2.0f * kLog2e)));
}
// The same two from their exponent arguments already scaled: tanh_scaled(x * kTanhScale) and
// sigmoid_scaled(x * kSigScale) are bitwise tanh_fast(x) and sigmoidf(x). A kernel that keeps a
// step's pre-activations in registers through several evaluations scales them once.
constexpr float kTanhScale = 2.0f * kLog2e;
constexpr float kSigScale = -kLog2e;
__device__ __forceinline__ float tanh_scaled(float xs) {
  return 1.0f - 2.0f * rcp_fast(1.0f + __builtin_amdgcn_exp2f(xs));
}
__device__ __forceinline__ float sigmoid_scaled(float xs) { return rcp_fast(1.0f + __builtin_amdgcn_exp2f(xs)); }
// log sigma(x) = -softplus(-x) = -(max(-x, 0) + ln(1 + e^{-|x|})), finite for any finite x
__device__ __forceinline__ float log_sigmoidf(float x) {
  return -(fmaxf(-x, 0.0f) + kLn2 * __builtin_amdgcn_logf(1.0f + exp_fast(-fabsf(x))));
}

// Expands LAUNCH(CM) with the compile-time cell mode CM equal to the runtime value cell_mode.
#define SLSTM_CELL_MODE_DISPATCH(cell_mode, LAUNCH) \
  switch (cell_mode) {                              \
    case 0: LAUNCH(0); break;                       \
    case 1: LAUNCH(1); break;                       \
    case 2: LAUNCH(2); break;                       \
    default: LAUNCH(3); break;                      \
  }
constexpr float kReadoutFloor = 1e-6f;

// Denominator D of the read-out h = o c / D: returns 1 / D and the derivatives dD/dn, dD/dm.
// D = n, or (floored) max(|n|, e^{-m}, 1e-6) on the branch the max takes (ties go to |n|, then
// to e^{-m}).
struct Readout {
  float rD, dn, dm;
};
__device__ __forceinline__ Readout readout(float n, float m, bool floored) {
  if (!floored) return {rcp_fast(n), 1.0f, 0.0f};
  const float an = fabsf(n);
  const float em = exp_fast(-m);
  const bool on_n = an >= em && an >= kReadoutFloor;
  const bool on_m = !on_n && em >= kReadoutFloor;
  const float D = on_n ? an : (on_m ? em : kReadoutFloor);
  return {rcp_fast(D), on_n ? copysignf(1.0f, n) : 0.0f, on_m ? -em : 0.0f};
}

// The state before the first step of sequence s (state0 (n_seqs, 4, d), zeros without one)
__device__ __forceinline__ CellIn state0_of(const float* state0, int s, unsigned ud, unsigned j) {
  if (state0 == nullptr) return {0.0f, 0.0f, 0.0f, 0.0f};
  const float* s0 = state0 + static_cast<i64>(s) * 4 * static_cast<i64>(ud);
  return {s0[j], s0[ud + j], s0[2 * ud + j], s0[3 * ud + j]};
}

// The stabilised gates of a step from a = l + m' and i~: m = max(a, i~) (a tie takes a) and
// (i', f') = (e^{i~ - m}, e^{a - m}), one of which is e^0 = 1 and the other e^{-|a - i~|}, so one
// exponential gives both, bitwise.
__device__ __forceinline__ void stab_gates(float a, float it, float& m, float& ig, float& fg) {
  const bool beta = a >= it;
  const float e = exp_fast(-fabsf(a - it));
  m = beta ? a : it;
  ig = beta ? e : 1.0f;
  fg = beta ? 1.0f : e;
}

// The values of one step that the state, its Jacobian and its linearisation share.
//
// m = max(a, i~) makes one of the two gates exactly e^0 = 1: with beta = (a >= i~) and
// e = e^{-|a - i~|}, (i', f') = (e, 1) when beta and (1, e) otherwise. Both are bitwise the
// values e^{i~ - m} and e^{a - m}, from one exponential.
//
// The z and o pre-activations enter their exponentials scaled: z~ kTanhScale = r_z kTanhScale h'
// + p_z kTanhScale as one FMA (likewise o with kSigScale). With PRE the caller passes p_z and p_o
// already scaled (the same float32 products, so the same bits); r_z and r_o are always raw.
// h = (o / D) c, the product the Jacobian's h row reuses.
struct CellCore {
  float z, o, dlf, e, ig, fg, c, n, m, h, rn, q1;
  bool beta;
  Readout rdn;
};
template <bool PRE = false>
__device__ __forceinline__ CellCore cell_core(const CellIn& pv, float pz, float pi, float pf, float po, float rz,
                                              float ri, float rf, float ro, bool sig_forget, bool floored) {
  CellCore k;
  const float zs = fmaf(rz * kTanhScale, pv.h, PRE ? pz : pz * kTanhScale);
  const float it = fmaf(ri, pv.h, pi);
  const float ft = fmaf(rf, pv.h, pf);
  const float os = fmaf(ro * kSigScale, pv.h, PRE ? po : po * kSigScale);
  k.z = tanh_scaled(zs);
  k.o = sigmoid_scaled(os);
  float lf;
  if (sig_forget) {
    lf = log_sigmoidf(ft);
    k.dlf = sigmoidf(-ft);
  } else {
    lf = ft;
    k.dlf = 1.0f;
  }
  const float a = lf + pv.m;
  k.beta = a >= it;
  k.m = k.beta ? a : it;
  k.e = exp_fast(-fabsf(a - it));
  k.ig = k.beta ? k.e : 1.0f;
  k.fg = k.beta ? 1.0f : k.e;
  k.c = fmaf(k.fg, pv.c, k.ig * k.z);
  k.n = fmaf(k.fg, pv.n, k.ig);
  k.rdn = readout(k.n, k.m, floored);
  k.rn = k.rdn.rD;
  k.q1 = k.o * k.rn;
  k.h = k.q1 * k.c;
  return k;
}

// One step. Writes the next state s[4] = (c, n, m, h); with JAC also A[16] row-major
// (A[4*row + col] = d s[row] / d prev[col]).
//
// On the branch the max takes, the derivatives of the c and n rows reduce to (with
// l' = dl/df~ and D = l' r_f - r_i)
//   dc/dm' = e (beta ? -z : c'),   dn/dm' = e (beta ? -1 : n'),
//   dc/dh' = D dc/dm' + i' dz/dh',  dn/dh' = D dn/dm',
// and dm/dm' = beta, dm/dh' = beta ? l' r_f : r_i. The h row is the quotient rule through c
// and through the read-out's denominator D(n, m).
template <bool JAC, bool PRE = false>
__device__ __forceinline__ void cell_step(const CellIn& pv, float pz, float pi, float pf, float po,
                                          float rz, float ri, float rf, float ro, bool sig_forget,
                                          bool floored, float s[4], float A[16]) {
  const CellCore k = cell_core<PRE>(pv, pz, pi, pf, po, rz, ri, rf, ro, sig_forget, floored);
  s[0] = k.c;
  s[1] = k.n;
  s[2] = k.m;
  s[3] = k.h;
  if constexpr (JAC) {
    const float z = k.z, o = k.o, e = k.e, ig = k.ig, fg = k.fg, c = k.c, h = k.h, rn = k.rn;
    const bool beta = k.beta;
    const float lrf = k.dlf * rf;
    const float D = lrf - ri;
    const float c_m = e * (beta ? -z : pv.c);
    const float n_m = e * (beta ? -1.0f : pv.n);
    const float dz_dh = fmaf(-z, z, 1.0f) * rz;
    const float do_dh = fmaf(-o, o, o) * ro;
    const float c_h = fmaf(c_m, D, ig * dz_dh);
    const float n_h = n_m * D;
    // row h = o c / D: (o/D) dc - (o c / D^2) (D_n dn + D_m dm), plus (c/D) do on h'
    const float q1 = k.q1;
    const float q2 = h * rn;
    A[0] = fg;     A[1] = 0.0f;   A[2] = c_m;   A[3] = c_h;
    A[4] = 0.0f;   A[5] = fg;     A[6] = n_m;   A[7] = n_h;
    A[8] = 0.0f;   A[9] = 0.0f;   A[10] = beta ? 1.0f : 0.0f;   A[11] = beta ? lrf : ri;
    A[12] = q1 * fg;
    if (!floored) {
      A[13] = -q2 * fg;
      A[14] = fmaf(q1, c_m, -q2 * n_m);
      A[15] = fmaf(q1, c_h, fmaf(-q2, n_h, (c * rn) * do_dh));
    } else {
      const float qn = q2 * k.rdn.dn, qm = q2 * k.rdn.dm;
      A[13] = -qn * fg;
      A[14] = fmaf(q1, c_m, fmaf(-qn, n_m, -qm * A[10]));
      A[15] = fmaf(q1, c_h, fmaf(-qn, n_h, fmaf(-qm, A[11], (c * rn) * do_dh)));
    }
  }
}

// The Jacobian of one step in factored form, for recurrences that apply it to one vector per
// step (Delta_t = A_t Delta_{t-1} + rhs_t) rather than compose it: with Delta' = (c', n', m', h')
// and y = m' + D h' (the direction the gates see through a = l + m' and i~), the rows of A
// above give
//   A_c Delta' = f' c' + c_m y + g h'        (g = i' dz/dh')
//   A_n Delta' = f' n' + n_m y
//   A_m Delta' = r_i h' + (beta ? y : 0)
//   A_h Delta' = q1 A_c Delta' - qn A_n Delta' - qm A_m Delta' + dov h'
// (q1 = o / D, qn = (h / D) D_n, qm = (h / D) D_m, dov = (c / D) do/dh' = (h - h o) r_o), which
// reuses the c, n and m rows instead of forming the h row's four entries. PRE as in cell_core.
struct DiagLin {
  float fg, c_m, n_m, g, D, ri, q1, qn, qm, dov;
  bool beta;
};
template <bool PRE = false>
__device__ __forceinline__ void cell_step_diag(const CellIn& pv, float pz, float pi, float pf, float po, float rz,
                                               float ri, float rf, float ro, bool sig_forget, bool floored,
                                               float s[4], DiagLin& L) {
  const CellCore k = cell_core<PRE>(pv, pz, pi, pf, po, rz, ri, rf, ro, sig_forget, floored);
  s[0] = k.c;
  s[1] = k.n;
  s[2] = k.m;
  s[3] = k.h;
  L.beta = k.beta;
  L.fg = k.fg;
  L.c_m = k.e * (k.beta ? -k.z : pv.c);
  L.n_m = k.e * (k.beta ? -1.0f : pv.n);
  L.g = k.ig * (fmaf(-k.z, k.z, 1.0f) * rz);
  L.D = fmaf(k.dlf, rf, -ri);
  L.ri = ri;
  L.q1 = k.q1;
  const float q2 = k.h * k.rn;
  L.qn = floored ? q2 * k.rdn.dn : q2;
  L.qm = floored ? q2 * k.rdn.dm : 0.0f;
  L.dov = fmaf(-k.h, k.o, k.h) * ro;
}

// x <- A x + rhs for the step L linearises (x holds Delta_{t-1} on entry, Delta_t on return)
__device__ __forceinline__ void diag_jvp(const DiagLin& L, bool floored, const float rhs[4], float x[4]) {
  const float y = fmaf(L.D, x[3], x[2]);
  const float u0 = fmaf(L.fg, x[0], fmaf(L.c_m, y, L.g * x[3]));
  const float u1 = fmaf(L.fg, x[1], L.n_m * y);
  const float u2 = fmaf(L.ri, x[3], L.beta ? y : 0.0f);
  const float tail = fmaf(L.dov, x[3], rhs[3]);
  const float x3 = floored ? fmaf(L.q1, u0, fmaf(-L.qn, u1, fmaf(-L.qm, u2, tail)))
                           : fmaf(L.q1, u0, fmaf(-L.qn, u1, tail));
  x[0] = u0 + rhs[0];
  x[1] = u1 + rhs[1];
  x[2] = u2 + rhs[2];
  x[3] = x3;
}

// Vector-Jacobian product of one step at the state before it (pv) and its pre-activations:
// given lam = dL/ds for the state the step produces, returns dx = dL/dx~ for the gate
// pre-activations (z, i, f, o) (= dL/dP of the step) and lam_prev = dL/ds' = A^T lam. The
// backward of "sLSTM in this library", section "Backward", one step of it:
//   h = o c / D folds into the c, n and m adjoints: lc = lam_c + (o/D) lam_h,
//   ln = lam_n - (h/D) D_n lam_h, lam_m += -(h/D) D_m lam_h (D = n: D_n = 1, D_m = 0),
//   c = f' c' + i' z, n = f' n' + i':  dL/df' = lc c' + ln n',  dL/di' = lc z + ln,  dL/dz = lc i'
//   one of (i', f') is 1 and the other e = e^{-|a - i~|} (see cell_step); with
//   w = beta ? e dL/di' : -e dL/df', the stabiliser m = max(a, i~) gives
//   dL/di~ = w + (1 - beta) lam_m,  dL/da = -w + beta lam_m  (a = l(f~) + m')
//   dL/dz~ = dL/dz (1 - z^2),  dL/do~ = (c/n) lam_h o (1 - o),  dL/df~ = dL/da l'(f~)
//   lam_prev = (lc f', ln f', dL/da, sum_x r_x dL/dx~)   (h' enters only through x~ = p + r h')
__device__ __forceinline__ void cell_vjp(const CellIn& pv, float pz, float pi, float pf, float po,
                                         float rz, float ri, float rf, float ro, bool sig_forget,
                                         bool floored, const float lam[4], float dx[4], float lam_prev[4]) {
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
  const Readout rdn = readout(n, beta ? a : it, floored);
  const float rn = rdn.rD;
  const float cn = c * rn;
  const float lc = fmaf(o * rn, lam[3], lam[0]);
  const float hq = -o * cn * rn;  // -(h / D)
  const float ln = floored ? fmaf(hq * rdn.dn, lam[3], lam[1]) : fmaf(hq, lam[3], lam[1]);
  const float lm = floored ? fmaf(hq * rdn.dm, lam[3], lam[2]) : lam[2];
  const float lfg = fmaf(lc, pv.c, ln * pv.n);
  const float lig = fmaf(lc, z, ln);
  const float w = beta ? e * lig : -e * lfg;
  const float da = beta ? lm - w : -w;
  dx[0] = lc * ig * fmaf(-z, z, 1.0f);
  dx[1] = beta ? w : w + lm;
  dx[2] = da * dlf;
  dx[3] = cn * lam[3] * fmaf(-o, o, o);
  lam_prev[0] = lc * fg;
  lam_prev[1] = ln * fg;
  lam_prev[2] = da;
  lam_prev[3] = fmaf(rz, dx[0], fmaf(ri, dx[1], fmaf(rf, dx[2], ro * dx[3])));
}

}  // namespace slstm
