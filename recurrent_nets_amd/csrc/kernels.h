// Host-side launchers of the kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace slstm {

// `tickets` arguments: the kSpreadSlots work counters of one kind (Spread::ticket[kind]), zero
// before the launch and zero again after it.

// Jacobian planes the residual kernel writes: all 16, the 12 non-structural ones, or none
enum class ResidualMode { kDense, kSparse, kNone };

// With a control block and stop_check_iter >= 0, the launch first declares the iterate
// stop_check_iter final (and does nothing else) when its residual maximum met tol. h_out
// (kNone only, optional) receives the hidden slot of S. The residual maximum goes to
// err_base[slot * err_stride] (see err_publish; stride 0 for a single word).
hipError_t launch_residual(const void* P, bool p_bf16, const float* R, const float* state0,
                           const float* S, float* A, float* rhs, int B, int T, int d,
                           int cell_mode, Control* ctl, unsigned int* err_base, int err_stride,
                           ResidualMode mode, int stop_check_iter, float tol, hipStream_t stream,
                           float* h_out = nullptr, Seqs seqs = {});

size_t fused_desc_words(int B, int T, int d);
hipError_t launch_newton_iteration(const void* P, bool p_bf16, const float* R, const float* state0,
                                   const float* S_in, float* S_out, int B, int T, int d,
                                   int cell_mode, unsigned long long* desc, unsigned int* tickets,
                                   uint32_t epoch, Control* ctl, int k_iter, float tol,
                                   hipStream_t stream, Seqs seqs = {});
// chain form of the fused iteration (256 features x 8 steps per tile); `last` also writes the
// residual of the new iterate (slot k_iter + 1) and, if h_out is not NULL, its hidden slot
long long chain_lane_groups(int B, int d);
size_t chain_desc_words(int B, int T, int d);
hipError_t launch_newton_chain(const void* P, bool p_bf16, const float* R, const float* state0,
                               const float* S_in, float* S_out, float* h_out, int B, int T, int d,
                               int cell_mode, unsigned long long* carry, unsigned int* tickets,
                               uint32_t epoch, Control* ctl, int k_iter, float tol, bool last,
                               hipStream_t stream);
// a whole fixed-count solve of the chain form in one pipelined pass (warm or zero initial
// iterate, 1 <= K <= kPipeMaxIters iterations, final residual and h); writes S_K to S_out
constexpr int kPipeMaxIters = 4;
// an early-stop solve (tol > 0) of at most this many iterations runs as two one-kernel passes:
// K iterations with every iterate's residual maximum, the stop test, then the count it chose
constexpr int kPipeMaxItersStop = 8;
size_t pipe_desc_words(int B, int T, int d, int K);
hipError_t launch_newton_pipe(const void* P, bool p_bf16, const float* R, const float* state0,
                              float* S_out, float* h_out, float* fs_out, int B, int T, int d, int cell_mode,
                              bool warm, int K, bool k_from_ctl, int tile_steps, unsigned long long* carry,
                              unsigned int* tickets, uint32_t epoch, Control* ctl, const int* tiles,
                              int tile_cap, hipStream_t stream);
// final states of the empty sequences of a pack: state0, or zeros without one
hipError_t launch_empty_seq_final(const int* cu, int n_seqs, int T, const float* state0, float* final_state, int d,
                                  hipStream_t stream);
hipError_t launch_pipe_stop(Control* ctl, int K, float tol, hipStream_t stream);
// steps per tile of the one-kernel solve for a shape on a GPU of n_cus compute units
int pipe_tile_steps(int B, int d, int n_cus);
// after the last chain iteration: declares iterate k final when its residual met tol
hipError_t launch_settle(Control* ctl, int k, float tol, hipStream_t stream);
// copies the final iterate into `states` when it ended in the other buffer (iterate k lives in
// buf0 for even k, buf1 for odd k)
hipError_t launch_select_iterate(const Control* ctl, const float* buf0, const float* buf1,
                                 float* states, i64 n_floats, hipStream_t stream);

size_t scan_desc_words(int B, int T, int d, bool sparse);
hipError_t launch_scan_block4(const float* A, const float* rhs, float* x, int B, int T, int d,
                              bool sparse, unsigned long long* desc, unsigned int* tickets,
                              uint32_t epoch, Control* ctl, int k_iter, float tol,
                              hipStream_t stream);

size_t warm_desc_words(int B, int T, int d);
hipError_t launch_warm_start(const void* P, bool p_bf16, const float* state0, float* S, int B,
                             int T, int d, int cell_mode, unsigned long long* desc,
                             unsigned int* tickets, uint32_t epoch, hipStream_t stream,
                             Seqs seqs = {});

size_t warm_chain_desc_words(int B, int T, int d);
hipError_t launch_warm_chain(const void* P, bool p_bf16, const float* state0, float* S, int B,
                             int T, int d, int cell_mode, unsigned long long* carry,
                             unsigned int* tickets, uint32_t epoch, hipStream_t stream);

// backward (adjoint + cell VJP) as chains or as a scan along T, then the fixed-order sums of
// dR and dbias over the tiles' rows; rows holds backward_row_floats floats
size_t backward_desc_words(int B, int T, int d, bool scan);
size_t backward_row_floats(int B, int T, int d, bool scan);
// packed rows on aligned tiles (Seqs::tiles, positions counted from each sequence's last tile):
// a table of backward_aligned_cap(T) slots of backward_aligned_steps() steps, which the words
// and rows of the scan form hold
int backward_aligned_steps();
int backward_aligned_cap(int T);
hipError_t launch_backward(const void* P, bool p_bf16, const float* R, const float* state0,
                           const float* S, const float* g, const float* g_h, const float* g_final,
                           void* dP, bool dp_bf16, float* dR, float* dbias, float* dstate0,
                           float* rows, int B, int T, int d, int cell_mode, bool scan,
                           unsigned long long* desc, unsigned int* tickets, uint32_t epoch,
                           hipStream_t stream, Seqs seqs = {});

hipError_t launch_update(float* S, const float* D, i64 n_floats, Control* ctl, int k_iter,
                         hipStream_t stream);
hipError_t launch_init_control(Control* ctl, hipStream_t stream);
hipError_t launch_finalize(Control* ctl, float tol, hipStream_t stream);
// hidden slot (unless the final residual pass already wrote it: then only after an early stop,
// signalled by ctl) and final state; with packed sequences the final state of each sequence
// (its state0 for an empty one)
hipError_t launch_outputs(const float* S, float* h, float* final_state, int B, int T, int d,
                          const Control* ctl, hipStream_t stream, const float* state0 = nullptr,
                          Seqs seqs = {});
hipError_t launch_zero(float* p, i64 n_floats, hipStream_t stream);
// the sequence table of packed offsets (seq_table_ints(T) ints; see kSeqTabShift)
size_t seq_table_ints(int T);
hipError_t launch_seq_table(const int* cu, int n_seqs, int T, int* tab, hipStream_t stream);
// tiles aligned to packed sequences for the scan-form iteration (see Seqs::tiles):
// aligned_tile_ints(cap) ints; fused_aligned_cap(T) tiles fit the iteration's look-back words,
// and a pack of n_seqs sequences over T steps needs at most ceil(T / fused_aligned_steps()) +
// n_seqs of them
size_t aligned_tile_ints(int cap);
hipError_t launch_aligned_tiles(const int* cu, int n_seqs, int T, int tile_steps, int cap, int* tiles,
                                hipStream_t stream);
int fused_aligned_cap(int T);
int fused_aligned_steps();

hipError_t launch_sequential(const void* P, bool p_bf16, const float* R, const float* state0,
                             float* S, float* h_out, float* final_state, int B, int T, int d,
                             int cell_mode, hipStream_t stream, Seqs seqs = {});

// head mixing (R of shape (4, n_heads, d_head, d_head), d_head in {8, 16, 32, 64}): the
// sequential forward, and one Newton iteration (residual of S_in, the factored block solve,
// S_out; `last` also the residual of S_out, slot k_iter + 1, and h into h_out if not NULL)
bool head_width_supported(int d_head);
hipError_t launch_head_sequential(const void* P, bool p_bf16, const float* R, const float* state0, float* S,
                                  float* h_out, float* final_state, int B, int T, int d, int n_heads,
                                  int cell_mode, hipStream_t stream, Seqs seqs = {});
hipError_t launch_head_iteration(const void* P, bool p_bf16, const float* R, const float* state0, const float* S_in,
                                 float* S_out, float* h_out, int B, int T, int d, int n_heads, int cell_mode,
                                 Control* ctl, int k_iter, float tol, bool last, hipStream_t stream,
                                 Seqs seqs = {});
// The whole head-mixing Newton solve in one sweep over T: K (1..kHeadSolveMaxIters) iterations
// pipelined stage by stage, the warm start (or zero_init's zero iterate) formed in the sweep;
// writes S (iterate K), h_out (may be NULL), the residual maxima of iterates 0..K into ctl's
// error slots and ctl->iters = K. Packed rows (seqs, B = 1) run the single-group form.
constexpr int kHeadSolveMaxIters = 4;
constexpr int kHeadSolveMaxWidth = 64;  // widest head the one-sweep kernel takes
hipError_t launch_head_solve(const void* P, bool p_bf16, const float* R, const float* state0, float* S,
                             float* h_out, int B, int T, int d, int n_heads, int cell_mode, int K, bool zero_init,
                             Control* ctl, hipStream_t stream, Seqs seqs = {});

// Backward under head mixing at the stored states S: dP (float32 or bf16), dR (4, n_heads,
// d_head, d_head), dbias (4, d; may be NULL), dstate0 (B, 4, d; may be NULL); g_states, g_h and
// g_final may be NULL. `part` holds head_backward_part_floats(B, d, n_heads) floats: per-row
// partial sums, added over the batch in a fixed order, and for heads of 128 units the
// transposed blocks of R.
size_t head_backward_part_floats(int B, int d, int n_heads);
bool head_backward_width_supported(int d_head);  // 8, 16, 32, 64, 128
hipError_t launch_head_backward(const void* P, bool p_bf16, const float* R, const float* state0, const float* S,
                                const float* g_states, const float* g_h, const float* g_final, void* dP,
                                bool dp_bf16, float* dR, float* dbias, float* dstate0, int B, int T, int d,
                                int n_heads, int cell_mode, float* part, hipStream_t stream, Seqs seqs = {});

// C = X W^T (+ bias) in bf16 MFMA with float32 accumulation; X (M x K), W (N x K), both
// K-contiguous. With splits > 1 the K range is split and split s writes its partial product to
// C + s * M * N (bias must then be null); gemm_splits_for gives an accepted split count.
hipError_t launch_gemm_bf16(const void* X, const void* W, const float* bias, float* C, i64 M,
                            int N, int K, hipStream_t stream, int splits = 1);
int gemm_tiles(i64 M, int N);
int gemm_splits_for(i64 M, int N, int K, int want);

// operand preparation for the weight-gradient products (bfloat16, rounded to nearest even)
hipError_t launch_transpose_bf16(const void* src, bool src_f32, uint16_t* dst, i64 rows, int cols,
                                 i64 ld, hipStream_t stream);
hipError_t launch_pad_bf16(const void* src, bool src_f32, uint16_t* dst, i64 rows, int cols, int ld,
                           hipStream_t stream);
hipError_t launch_sum_splits(const float* part, float* out, int splits, i64 n, hipStream_t stream);

}  // namespace slstm
