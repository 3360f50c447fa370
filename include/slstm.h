/*
 * slstm.h -- C ABI of the MI355X (gfx950) sLSTM forward library: channelwise recurrence
 * (mix='diag'), state (c, n, m, h) per feature, solved in parallel over time by Newton's
 * method with a 4x4 affine scan, or step by step.
 *
 * Sources (the pages the method is described on):
 *  [SL]  pararnn-torch docs, "sLSTM in this library": sections "Cell" (state layout
 *        (B, T, 4, d_h) = (c, n, m, h), hidden slot 3; mix='diag' = channelwise R of shape
 *        (4, d_h), a 4x4 Jacobian per feature), "API notes" (Newton / sequential solver
 *        modes, T = 1 decode step, W_x applied as a GEMM), "Outputs".
 *  [LY]  pararnn-torch docs, "Layout": "Current surface (0.17)" (fused kernels prepend h0;
 *        NewtonStats; residual early stop; divergence error when max|F| > 1 after K),
 *        "Naming" (scan_block4 for the (B, T, 4, 4, d) layout).
 *  [XL]  "xLSTM: Extended Long Short-Term Memory" summary card, "Key equations": the sLSTM
 *        step pseudocode (paper section 2.2, appendix A.2), gate order (z, i, f, o).
 *  [ED]  "xLSTM -- a from-scratch, educational reimplementation", section "Exponential gating
 *        + the stabilizer (the crux)": stabiliser m_t and the stabilised gates.
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, row-major, in device memory owned by the caller. The library never
 *    allocates, frees or keeps a pointer after a call returns (workspaces are caller memory).
 *  - Layouts (feature index innermost):
 *      P        (B, T, 4, d_h)      gate pre-activations, gates (z, i, f, o); float32 or bf16
 *      R        (4, d_h)  float32   channelwise recurrent weights, same gate order
 *      state0   (B, 4, d_h) float32 initial state, slots (c, n, m, h); NULL means all zeros
 *      states   (B, T, 4, d_h) float32, slots (c, n, m, h); states[:, T-1] is the final state
 *      h_out    (B, T, d_h) float32, the hidden slot; optional (NULL skips it)
 *      final_state (B, 4, d_h) float32, the last step's state (c, n, m, h) as a contiguous
 *               tensor, ready to be the next call's state0 ([SL] "Outputs": return_hidden adds
 *               the final state); optional (NULL skips it)
 *      A        (B, T, 4, 4, d_h) float32, A[b,t,row,col,j] = d s_t[row] / d s_{t-1}[col]
 *  - Every call enqueues work on `stream` (a hipStream_t; NULL is the default stream) and
 *    returns without waiting, unless stated otherwise.
 *  - Status: negative values mean invalid input or a HIP failure and that no output is valid;
 *    slstm_last_error() then describes the problem (per thread). Positive values report a
 *    solver outcome with outputs written.
 *  - Alignment: states, h_out, A, rhs/x and workspaces 16-byte aligned; P 4-byte (float32) or
 *    2-byte (bf16); x and W_x of the input projection 16-byte aligned.
 */
#ifndef SLSTM_H
#define SLSTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLSTM_OK = 0,
  SLSTM_DIVERGED = 1,   /* Newton: finite max|F| > 1 after the last iterate ([LY]) */
  SLSTM_NONFINITE = 2,  /* Newton: residual of the last iterate is NaN or infinite */
  SLSTM_EINVAL = -1,    /* invalid argument */
  SLSTM_EWORKSPACE = -2,/* workspace smaller than required */
  SLSTM_EHIP = -3       /* a HIP runtime call or kernel launch failed */
} slstm_status;

typedef enum { SLSTM_F32 = 0, SLSTM_BF16 = 1 } slstm_dtype;

/* forget gate: log f = f~ (exponential) or log sigma(f~) (sigmoid) ([XL] "Method"; [ED]).
 * SLSTM_READOUT_FLOORED may be OR-ed into every argument of this type: the read-out becomes
 * h = o c / max(|n|, e^{-m}, 1e-6), the stabilised read-out of [ED] ("Exponential gating + the
 * stabilizer (the crux)", with the 1e-6 floor of its "Implementation notes / deviations" item 1,
 * read as a lower bound), instead of the paper's h = o c / n. Any other bit is rejected. */
typedef enum {
  SLSTM_FORGET_EXP = 0,
  SLSTM_FORGET_SIGMOID = 1,
  SLSTM_READOUT_FLOORED = 0x100
} slstm_forget;

/* initial Newton iterate: the trajectory with the recurrent term R h_{t-1} dropped, or zeros */
typedef enum { SLSTM_INIT_WARM = 0, SLSTM_INIT_ZERO = 1 } slstm_init;

/* How a Newton iteration is laid out in kernels (same iterates up to float32 rounding):
 *  SLSTM_SCHEDULE_FUSED_SCAN   one kernel per iteration: residual, Jacobian, the 4x4 affine
 *                              scan of the block-bidiagonal system and the update, all in
 *                              registers; reads P and the iterate, writes the next iterate
 *                              (double-buffered in the workspace);
 *  SLSTM_SCHEDULE_FUSED_CHAIN  one kernel per iteration as above, but each tile of 8 steps
 *                              solves its part of the system as a plain recurrence from the
 *                              Newton step entering it, published by the tile before; no 4x4
 *                              maps are composed. The last iteration also forms the final
 *                              residual and h, so no separate pass over the states follows.
 *                              A fixed-count solve (tol = 0, max_iters <= 4) runs as ONE
 *                              kernel: each tile keeps P and its iterate in registers through
 *                              the warm start and all iterations (a wavefront along T), so P
 *                              is read once and only the final states are written.
 *                              Fast when there are many independent lanes, serial along T;
 *  SLSTM_SCHEDULE_FUSED        FUSED_CHAIN when B * ceil(d_h / 256) is at least the GPU's
 *                              compute-unit count, or at least 32 for a fixed-count solve
 *                              (tol = 0, max_iters <= 4, unpacked: the one-kernel form, which
 *                              reads P once; under FUSED max_iters <= 8) or an early-stop
 *                              solve (tol > 0, max_iters <= 8, unpacked); FUSED_SCAN
 *                              otherwise. Under FUSED a fixed count up to 8 on the chain form
 *                              runs as the one-kernel solve, and an early stop on
 *                              the chain form runs the one-kernel form twice: max_iters
 *                              iterations with every iterate's residual, then, if an iterate k
 *                              met tol first, k iterations again, so that the outputs are the
 *                              iterate the stop returns;
 *  SLSTM_SCHEDULE_LAYERED      three kernels per iteration: (a) residual + Jacobian to HBM in
 *                              the scan_block4 layout, (b) the 4x4 affine scan, (c) the update.
 * Each schedule's results are bitwise reproducible on a given device. */
typedef enum {
  SLSTM_SCHEDULE_FUSED = 0,
  SLSTM_SCHEDULE_LAYERED = 1,
  SLSTM_SCHEDULE_FUSED_SCAN = 2,
  SLSTM_SCHEDULE_FUSED_CHAIN = 3
} slstm_schedule;

#define SLSTM_MAX_ITERS 64

/* Newton bookkeeping ([LY] NewtonStats). max_abs_F[k] = max |F| over all (b, t, slot, j) at
 * the iterate after k updates, k = 0 .. iters; entries past `iters` are 0. A non-finite
 * residual is recorded as +inf. */
typedef struct {
  int32_t iters;      /* updates applied */
  int32_t converged;  /* tol > 0 and max_abs_F[iters] < tol */
  int32_t diverged;   /* max_abs_F[iters] > 1 or not finite */
  int32_t nonfinite;  /* max_abs_F[iters] not finite */
  float max_abs_F[SLSTM_MAX_ITERS + 1];
} slstm_newton_stats;

const char* slstm_status_string(slstm_status s);
/* Detail of the last negative status returned on the calling thread ("" if none). */
const char* slstm_last_error(void);

/* Bytes of device workspace slstm_newton_forward needs for these sizes and schedule (0 if
 * invalid). */
size_t slstm_newton_workspace_bytes(int B, int T, int d_h, slstm_schedule schedule);

/*
 * Newton-parallel forward ([SL] "API notes": solver='newton'; [LY] "Current surface"): the
 * whole sequence s_1..s_T of the recurrence s_t = f(s_{t-1}, P_t) with s_0 = state0, where f
 * is the stabilised sLSTM step of [XL]/[ED] with channelwise R:
 *   x~ = p_x + r_x h'; z = tanh z~; o = sigma(o~); l = f~ or log sigma(f~);
 *   a = l + m'; m = max(a, i~) (a tie takes a); i' = e^{i~ - m}; f' = e^{a - m};
 *   c = f' c' + i' z; n = f' n' + i'; h = o c / n.
 * Each iteration k evaluates F_t = s_t - f(s_{t-1}) and A_t = df/ds' at every step; if
 * tol > 0 and max|F| < tol it stops before solving; otherwise it solves
 *   Delta_1 = -F_1, Delta_t = A_t Delta_{t-1} - F_t     (block-bidiagonal system)
 * by a 4x4 affine scan (or, FUSED_CHAIN, tile-serial recurrences) and sets s <- s + Delta. After max_iters updates (or the stop) the
 * residual of the final iterate gives the flags.
 *
 *  P, P_dtype   gate pre-activations (B, T, 4, d_h), float32 or bf16
 *  R            (4, d_h); state0 (B, 4, d_h) or NULL
 *  states       output (B, T, 4, d_h); also the Newton iterate while solving. May be NULL
 *               when the call resolves to the one-kernel solve (unpacked; tol = 0 and
 *               max_iters <= 4 with FUSED_CHAIN; max_iters <= 8 with FUSED where it picks
 *               FUSED_CHAIN, with or without a tolerance): that form keeps its
 *               iterate on chip, and h_out and final_state are then the outputs, as in the
 *               layer's default output, the hidden slot ([SL] "Outputs"). NULL for any other
 *               form is SLSTM_EINVAL.
 *  h_out        optional output (B, T, d_h); final_state optional output (B, 4, d_h)
 *  fmode        forget-gate form; max_iters in 1..64; tol >= 0 (0: fixed iteration count)
 *  init         SLSTM_INIT_WARM (default reading) or SLSTM_INIT_ZERO
 *  schedule     one of the slstm_schedule values (see above)
 *  workspace    >= slstm_newton_workspace_bytes(B, T, d_h, schedule) bytes of device memory;
 *               holds the solver control block (later readable with slstm_newton_read_stats)
 *               and look-back words, plus the second iterate buffer (fused) or the Jacobians
 *               and right-hand sides / Newton steps (layered)
 *  stats        NULL: fully asynchronous, returns SLSTM_OK once everything is enqueued.
 *               non-NULL: waits for the stream, fills *stats and returns SLSTM_DIVERGED or
 *               SLSTM_NONFINITE when the flags say so (outputs are still written).
 */
slstm_status slstm_newton_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                  const float* state0, float* states, float* h_out,
                                  float* final_state, int B, int T, int d_h, slstm_forget fmode,
                                  int max_iters, float tol, slstm_init init,
                                  slstm_schedule schedule, void* workspace,
                                  size_t workspace_bytes, void* stream, slstm_newton_stats* stats);

/* Waits for `stream` and copies the stats of the last slstm_newton_forward that used this
 * workspace into *stats; returns the status that call would have returned with stats. */
slstm_status slstm_newton_read_stats(const void* workspace, size_t workspace_bytes, void* stream,
                                     slstm_newton_stats* stats);

/* Size of the library's fixed device scratch used by slstm_newton_forward_noalloc (64 MiB). */
#define SLSTM_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): slstm_newton_forward without a workspace argument.
 * Same arguments, semantics, layouts and results as slstm_newton_forward (the same kernels);
 * the solver's workspace is a fixed array of SLSTM_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, allocated when the library's code is loaded onto that GPU and held until the
 * process ends. The call allocates nothing (no hipMalloc, hipFree or allocating library call)
 * and records no profiling events.
 *  - Problems whose workspace, slstm_newton_workspace_bytes(B, T, d_h, schedule), exceeds
 *    SLSTM_NOALLOC_SCRATCH_BYTES are rejected with SLSTM_EWORKSPACE before any work is enqueued.
 *  - The scratch lives on the device of `stream` (the current device for NULL); the solver's
 *    control block is cleared by a kernel at the start of each call.
 *  - Every call on one GPU shares that GPU's scratch: calls that overlap in time on one GPU
 *    (on different streams, or from different threads) race and give undefined results;
 *    serialise them. Solver statistics are only returned through `stats` (which waits for the
 *    stream); slstm_newton_read_stats cannot address the scratch.
 */
slstm_status slstm_newton_forward_noalloc(const void* P, slstm_dtype P_dtype, const float* R,
                                          const float* state0, float* states, float* h_out,
                                          float* final_state, int B, int T, int d_h,
                                          slstm_forget fmode, int max_iters, float tol,
                                          slstm_init init, slstm_schedule schedule, void* stream,
                                          slstm_newton_stats* stats);

/*
 * Sequential forward ([SL] "API notes": solver='sequential'; at T = 1 the decode step):
 * s_t = f(s_{t-1}, P_t) for t = 1..T, one thread per lane (b, j). Same arguments and layouts
 * as slstm_newton_forward; needs no workspace. states may be NULL (unpacked calls): h_out and
 * final_state are then the outputs, the layer's default output ([SL] "Outputs").
 */
slstm_status slstm_sequential_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                      const float* state0, float* states, float* h_out,
                                      float* final_state, int B, int T, int d_h,
                                      slstm_forget fmode, void* stream);

/*
 * Input projection on the MFMA matrix cores ([SL] "API notes": W_x is a GEMM; [XL]
 * pre-activations W x + b):  P[b,t,g,j] = sum_k x[b,t,k] W_x[g,j,k] + bias[g,j].
 *  x (B, T, d_in) and W_x (4, d_h, d_in) in bf16 (xw_dtype must be SLSTM_BF16), bias (4, d_h)
 *  float32 (NULL: no bias), P (B, T, 4, d_h) float32 output. d_in must be a multiple of 8.
 *  Accumulates in float32.
 */
slstm_status slstm_input_projection(const void* x, const void* W_x, const float* bias, float* P,
                                    int B, int T, int d_in, int d_h, slstm_dtype xw_dtype,
                                    void* stream);

/*
 * One residual + Jacobian evaluation (the first half of a Newton iteration, [LY]):
 *   rhs_t = f(s_{t-1}, P_t) - s_t = -F_t and A_t = df/ds' at s_{t-1}, for t = 1..T, s_0 = state0.
 *  states (B, T, 4, d_h) is the iterate; A (B, T, 4, 4, d_h) and rhs (B, T, 4, d_h) are outputs.
 *  max_abs_F: device pointer to one float, overwritten with max |F| (NaN counted as +inf).
 */
slstm_status slstm_residual_jacobian(const void* P, slstm_dtype P_dtype, const float* R,
                                     const float* state0, const float* states, float* A,
                                     float* rhs, float* max_abs_F, int B, int T, int d_h,
                                     slstm_forget fmode, void* stream);

/* Workspace bytes of slstm_scan_block4 (0 if invalid). */
size_t slstm_scan_block4_workspace_bytes(int B, int T, int d_h);

/*
 * Associative scan over 4x4 affine maps in the scan_block4 layout ([LY] "Naming"; the (J, r)
 * monoid of [SL] "Packed sequences"): x_1 = rhs_1, x_t = A_t x_{t-1} + rhs_t, per lane (b, j).
 * A at the first step is not read as a multiplier (x_0 = 0). A (B, T, 4, 4, d_h), rhs and x
 * (B, T, 4, d_h); x may be the same buffer as rhs.
 */
slstm_status slstm_scan_block4(const float* A, const float* rhs, float* x, int B, int T, int d_h,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of slstm_warm_start (0 if invalid). */
size_t slstm_warm_start_workspace_bytes(int B, int T, int d_h, slstm_schedule schedule);

/*
 * The initial Newton iterate: the exact trajectory of the cell with R h_{t-1} dropped from the
 * pre-activations, from state0's (c, n, m) (a reading: the pages give no initial guess).
 * Writes states (B, T, 4, d_h) with h = sigma(p_o) c / n. schedule picks the kernel form the
 * Newton solver would use for it: SLSTM_SCHEDULE_FUSED_CHAIN runs tile-serial recurrences,
 * SLSTM_SCHEDULE_FUSED_SCAN and SLSTM_SCHEDULE_LAYERED a log-space scan with look-back, and
 * SLSTM_SCHEDULE_FUSED chooses as slstm_newton_forward does.
 */
slstm_status slstm_warm_start(const void* P, slstm_dtype P_dtype, const float* state0,
                              float* states, int B, int T, int d_h, slstm_forget fmode,
                              slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Workspace bytes of slstm_backward (0 if invalid). */
size_t slstm_backward_workspace_bytes(int B, int T, int d_h, slstm_schedule schedule);

/*
 * Gradients through the recurrence ("sLSTM in this library", section "Backward"): the adjoint
 * lam_t = dL/ds_t, from lam_{T-1} = g_{T-1} and lam_t = g_t + A_{t+1}^T lam_{t+1} (A_t the 4x4
 * Jacobian of step t with respect to the state before it), then per step the vector-Jacobian
 * product of the cell with respect to its pre-activations.
 *   P (B, T, 4, d_h) f32 or bf16, R (4, d_h), state0 (B, 4, d_h) or NULL (zeros): as given to
 *     the forward call.
 *   states (B, T, 4, d_h) f32: the forward solution s_1..s_T (slots c, n, m, h), as the Newton
 *     or the sequential forward wrote it. 16-byte aligned.
 *   g_states (B, T, 4, d_h) or NULL: dL/d states.  g_h (B, T, d_h) or NULL: dL/d h, added to
 *     slot 3.  g_final (B, 4, d_h) or NULL: dL/d of the final state, added at step T-1. A NULL
 *     gradient counts as zeros.
 *   dP (B, T, 4, d_h), written: dL/dP per gate (z, i, f, o), float32 (dP_dtype SLSTM_F32) or
 *     rounded to bfloat16, nearest even (SLSTM_BF16, the operand of
 *     slstm_input_projection_backward). P = W_x x + bias, so the gradients of W_x and x are
 *     products of dP with x and W_x.
 *   dR (4, d_h) f32, written: dL/dR = sum over b, t of dP[b, t, g, j] * h_{t-1}[b, j], with
 *     h_0 taken from state0.
 *   dbias (4, d_h) f32 or NULL, written: dL/dbias = sum over b, t of dP[b, t, g, j] (from the
 *     float32 values).
 *   dstate0 (B, 4, d_h) f32 or NULL, written: dL/d state0 (at the zero state if state0 is NULL).
 * schedule: SLSTM_SCHEDULE_FUSED and SLSTM_SCHEDULE_FUSED_SCAN run one kernel that scans the
 * maps y -> A_t^T (g_t + y) along T with a look-back across tiles (parallel along T at any
 * batch size); SLSTM_SCHEDULE_FUSED_CHAIN runs tile-serial reverse chains instead;
 * SLSTM_SCHEDULE_LAYERED is rejected. Two small kernels then sum dR in a fixed order. The workspace (slstm_backward_workspace_bytes, 256-byte aligned) is the caller's;
 * results are bitwise reproducible. Negative status: nothing valid was written. Outputs must
 * not alias inputs.
 */
slstm_status slstm_backward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                            const float* states, const float* g_states, const float* g_h,
                            const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR,
                            float* dbias, float* dstate0, int B, int T, int d_h, slstm_forget fmode,
                            slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes of slstm_input_projection_backward (0 if invalid). */
size_t slstm_input_projection_backward_workspace_bytes(int B, int T, int d_in, int d_h);

/*
 * Gradients of the input projection P = x W_x^T + bias ("sLSTM in this library", "API notes":
 * W_x is a GEMM; "Backward": the gradient of W_x follows from the cell's VJP by a GEMM):
 *   dW_x[g, j, k] = sum over b, t of dP[b, t, g, j] x[b, t, k]   (dW_x = dP^T x)
 *   dx[b, t, k]   = sum over g, j of dP[b, t, g, j] W_x[g, j, k]  (dx = dP W_x)
 * (the bias gradient is slstm_backward's dbias).
 *   x (B, T, d_in) bf16, W_x (4, d_h, d_in) bf16: as given to slstm_input_projection.
 *   dP (B, T, 4, d_h), f32 (rounded to bfloat16, nearest even, for the products) or bf16
 *     (dP_dtype), as slstm_backward writes it.
 *   dx (B, T, d_in) f32 or NULL; dW_x (4, d_h, d_in) f32 or NULL: written when non-NULL.
 * Both products run on the bf16 MFMA units with float32 accumulation; dW_x, whose reduction
 * runs over all B*T rows, splits that range over workgroups and adds the partial products in a
 * fixed order (bitwise reproducible). d_in must be a positive multiple of 8; 16-byte aligned
 * x, W_x and dP. The workspace (slstm_input_projection_backward_workspace_bytes, 256-byte
 * aligned) holds the bfloat16 transposes of dP, x and W_x and the partial products.
 */
slstm_status slstm_input_projection_backward(const void* x, const void* W_x, const void* dP,
                                             slstm_dtype dP_dtype, float* dx, float* dW_x, int B,
                                             int T, int d_in, int d_h, void* workspace,
                                             size_t workspace_bytes, void* stream);

/*
 * Packed sequences ([SL] "Packed sequences"; "Scan backend" item 4): S ragged sequences laid
 * end to end along time in one row, B = 1. Sequence s covers steps cu_seqlens[s] ..
 * cu_seqlens[s+1] - 1 of P, states, h_out and the gradients (cu_seqlens: exclusive prefix sums
 * of the lengths, S + 1 entries, cu_seqlens[0] = 0, non-decreasing, cu_seqlens[S] = T; empty
 * sequences allowed). Each sequence starts from its own initial state: state0 is (S, 4, d_h)
 * or NULL (zeros), and the step at each sequence's start does not depend on the step before
 * it (the head flag of the segmented (J, r) scan: that step's Jacobian is zero).
 *   cu_seqlens   device pointer to S + 1 int32 values, 4-byte aligned; its contents are read
 *                by the kernels and not checked (a malformed array gives unspecified results,
 *                every access staying in bounds). n_seqs = S, 1 .. 2^24.
 *   final_state  (S, 4, d_h): each sequence's last state (its state0 for an empty one).
 *   g_final      (S, 4, d_h): added at each sequence's last step (an empty sequence passes it
 *                to its dstate0).  dstate0 (S, 4, d_h).
 * Everything else is as in the entry point without the suffix, at B = 1. Packed Newton solves
 * under SLSTM_SCHEDULE_FUSED (max_iters <= 8; an early stop in two passes) run the one-kernel
 * solve on tiles aligned to the sequence starts, each sequence's chain beside the others, when
 * the tile table holds the pack (about T / 48 sequences or fewer) and ceil(d_h / 256) times S
 * is at least 32; otherwise, and for the other packed calls, SLSTM_SCHEDULE_FUSED means
 * SLSTM_SCHEDULE_FUSED_SCAN. Size the Newton workspace with SLSTM_SCHEDULE_FUSED, which covers
 * both (B = 1). SLSTM_SCHEDULE_LAYERED is accepted by the Newton solve and the warm start, and
 * SLSTM_SCHEDULE_FUSED_CHAIN is rejected. states may be NULL for a packed solve that runs the
 * one-kernel form.
 */
slstm_status slstm_newton_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                         const float* state0, const int* cu_seqlens, int n_seqs,
                                         float* states, float* h_out, float* final_state, int T,
                                         int d_h, slstm_forget fmode, int max_iters, float tol,
                                         slstm_init init, slstm_schedule schedule, void* workspace,
                                         size_t workspace_bytes, void* stream,
                                         slstm_newton_stats* stats);
slstm_status slstm_sequential_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                             const float* state0, const int* cu_seqlens, int n_seqs,
                                             float* states, float* h_out, float* final_state, int T,
                                             int d_h, slstm_forget fmode, void* stream);
slstm_status slstm_warm_start_varlen(const void* P, slstm_dtype P_dtype, const float* state0,
                                     const int* cu_seqlens, int n_seqs, float* states, int T, int d_h,
                                     slstm_forget fmode, slstm_schedule schedule, void* workspace,
                                     size_t workspace_bytes, void* stream);
slstm_status slstm_backward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                   const float* state0, const int* cu_seqlens, int n_seqs,
                                   const float* states, const float* g_states, const float* g_h,
                                   const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR,
                                   float* dbias, float* dstate0, int T, int d_h, slstm_forget fmode,
                                   slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Head mixing ([SL] "Cell", the mix table's 'head' row; [XL] "Method" item 2 and the one-head
 * step pseudocode: recurrent matrices from h' to every gate, block-diagonal with one block per
 * head, no mixing across heads). R is (4, n_heads, d_head, d_head) float32, 16-byte aligned,
 * n_heads * d_head = d_h, d_head one of 8, 16, 32, 64, 128; unit i of head a (feature
 * j = a d_head + i) has the pre-activations x~_g = P[.., g, j] + sum_k R[g, a, i, k] h'[a d_head + k].
 * Every other argument is as for the channelwise calls (P, states, h_out, final_state, state0
 * layouts, forget modes with the floored read-out flag, statuses, stream semantics).
 *
 * slstm_head_newton_forward: Newton as slstm_newton_forward (warm start with R h' dropped, the
 * same stop rule, flags and stats). One workgroup per (batch row, head) walks T, forms the
 * residual at the iterate and solves the block-bidiagonal system with the Jacobian applied in
 * factored form (the unit's own-state columns plus the gate Jacobian times R_g Delta h'), so no
 * (4 d_head)^2 block is formed; the solve is a recurrence along T and parallelism comes from
 * B * n_heads. With tol = 0, max_iters <= 4 and d_head <= 64 the warm start and all iterations
 * run as one kernel, pipelined along T; otherwise (and always for heads of 128 units, whose
 * pipeline stages would not fit the register file) the warm start, then one kernel per iteration.
 * Workspace: slstm_head_newton_workspace_bytes (0 if the sizes are invalid).
 * slstm_head_sequential_forward: the step loop, one workgroup per (batch row, head); no
 * workspace.
 * slstm_head_backward: gradients through the head-mixing recurrence at the forward solution
 * `states`, as slstm_backward ([SL] "Backward"): g_states (B, T, 4, d_h), g_h (B, T, d_h) and
 * g_final (B, 4, d_h) are the loss's direct gradients (each may be NULL: zero); outputs dP
 * (B, T, 4, d_h) in dP_dtype (F32 or BF16, rounded to nearest even), dR (4, n_heads, d_head,
 * d_head), dbias (4, d_h; may be NULL), dstate0 (B, 4, d_h; may be NULL); d_head 8, 16, 32, 64
 * or 128 (heads of 128 units read their blocks of R from memory at every step: a lane's block
 * row and dR row would not fit in registers, nor the head's blocks in LDS). One workgroup per
 * (batch row, head) walks T backwards; dR and dbias are added over the batch in a fixed order
 * from per-row partial sums in the workspace (slstm_head_backward_workspace_bytes; 0 if the
 * sizes are invalid; for heads of 128 units it also holds the transposed blocks of R), so
 * results are reproducible bit for bit.
 * The _varlen forms take packed sequences as the channelwise _varlen calls do (one row of T steps,
 * cu_seqlens (n_seqs + 1 device ints), state0, final_state, g_final and dstate0 per sequence):
 * a sequence start takes state0[s] as the state before it, its Jacobian is zero for the Newton
 * solve and the adjoint does not cross it. Packed Newton with tol = 0, max_iters <= 4 and d_head <= 64
 * runs the one-sweep kernel in its single-group form (one workgroup per head along the row),
 * otherwise the warm start and one kernel per iteration; the workspace sizes are those of the
 * unpacked calls with B = 1.
 */
size_t slstm_head_newton_workspace_bytes(int B, int T, int d_h, int n_heads);
slstm_status slstm_head_newton_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                       const float* state0, float* states, float* h_out,
                                       float* final_state, int B, int T, int d_h, int n_heads,
                                       slstm_forget fmode, int max_iters, float tol, slstm_init init,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       slstm_newton_stats* stats);
slstm_status slstm_head_sequential_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                           const float* state0, float* states, float* h_out,
                                           float* final_state, int B, int T, int d_h, int n_heads,
                                           slstm_forget fmode, void* stream);
slstm_status slstm_head_newton_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                              const float* state0, const int* cu_seqlens, int n_seqs,
                                              float* states, float* h_out, float* final_state, int T,
                                              int d_h, int n_heads, slstm_forget fmode, int max_iters,
                                              float tol, slstm_init init, void* workspace,
                                              size_t workspace_bytes, void* stream,
                                              slstm_newton_stats* stats);
slstm_status slstm_head_sequential_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                                  const float* state0, const int* cu_seqlens, int n_seqs,
                                                  float* states, float* h_out, float* final_state, int T,
                                                  int d_h, int n_heads, slstm_forget fmode, void* stream);
size_t slstm_head_backward_workspace_bytes(int B, int T, int d_h, int n_heads);
slstm_status slstm_head_backward(const void* P, slstm_dtype P_dtype, const float* R,
                                 const float* state0, const float* states, const float* g_states,
                                 const float* g_h, const float* g_final, void* dP,
                                 slstm_dtype dP_dtype, float* dR, float* dbias, float* dstate0, int B,
                                 int T, int d_h, int n_heads, slstm_forget fmode, void* workspace,
                                 size_t workspace_bytes, void* stream);
slstm_status slstm_head_backward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                        const float* state0, const int* cu_seqlens, int n_seqs,
                                        const float* states, const float* g_states, const float* g_h,
                                        const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR,
                                        float* dbias, float* dstate0, int T, int d_h, int n_heads,
                                        slstm_forget fmode, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Kernel timing with HIP events recorded on the launching stream around every kernel the
 * library launches, for measurement. Off by default; process-wide; not thread-safe.
 * slstm_profile_read waits for the recorded events and returns the summed duration (ms) and
 * the launch count of one kernel kind since the last reset.
 */
typedef enum {
  SLSTM_KERNEL_WARM_START = 0,
  SLSTM_KERNEL_RESIDUAL_JACOBIAN = 1,
  SLSTM_KERNEL_SCAN_BLOCK4 = 2,
  SLSTM_KERNEL_UPDATE = 3,
  SLSTM_KERNEL_FINAL_RESIDUAL = 4,
  SLSTM_KERNEL_INPUT_PROJECTION = 5,
  SLSTM_KERNEL_SEQUENTIAL = 6,
  SLSTM_KERNEL_NEWTON_ITERATION = 7,
  SLSTM_KERNEL_NEWTON_SOLVE = 8, /* the one-kernel fixed-count solve of the chain form */
  SLSTM_KERNEL_BACKWARD = 9,     /* the adjoint and cell VJP pass of slstm_backward */
  SLSTM_KERNEL_WEIGHT_GRADIENT = 10, /* slstm_input_projection_backward's dW_x product */
  SLSTM_KERNEL_INPUT_GRADIENT = 11,  /* slstm_input_projection_backward's dx product */
  SLSTM_KERNEL_HEAD_ITERATION = 12,  /* one Newton iteration under head mixing */
  SLSTM_KERNEL_HEAD_SEQUENTIAL = 13, /* the sequential forward under head mixing */
  SLSTM_KERNEL_HEAD_SOLVE = 14,      /* the whole Newton solve under head mixing, one sweep */
  SLSTM_KERNEL_HEAD_BACKWARD = 15,   /* the backward under head mixing (recurrence and sums) */
  SLSTM_KERNEL_KINDS = 16
} slstm_kernel_kind;

slstm_status slstm_profile_enable(int on);
slstm_status slstm_profile_reset(void);
slstm_status slstm_profile_read(slstm_kernel_kind kind, double* total_ms, int* launches);
/* The individual durations (ms, in launch order) of one kernel kind since the last reset:
 * writes min(count, capacity) values to out_ms and the full count to *launches. */
slstm_status slstm_profile_durations(slstm_kernel_kind kind, double* out_ms, int capacity,
                                     int* launches);

#ifdef __cplusplus
}
#endif

#endif /* SLSTM_H */
