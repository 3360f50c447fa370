// C ABI of the library: argument checks, workspace layout, the host-side Newton loop and timing.
// The solver loop follows "Layout" (pararnn-torch docs), "Current surface (0.17)":
// initial state prepended, residual early stop, flags after the last iterate.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>
#include <vector>

#include "../../include/slstm.h"
#include "common.h"
#include "kernels.h"

using slstm::Control;
using slstm::i64;

namespace {

thread_local char g_err[512] = "";

slstm_status fail(slstm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(SLSTM_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));             \
  } while (0)

// Launch epochs tag the look-back words of every scan launch. The sequence starts at a random
// point so that words left in recycled device memory by another process do not match.
std::atomic<uint32_t> g_epoch{[] {
  std::random_device rd;
  return static_cast<uint32_t>(rd());
}()};

uint32_t next_epoch() {
  uint32_t e;
  do {
    e = g_epoch.fetch_add(1u) + 1u;
  } while (e == 0u);
  return e;
}

// ---- kernel timing ------------------------------------------------------------------------
struct ProfRec {
  hipEvent_t a, b;
  int kind;
};
struct Profiler {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<ProfRec> pool;
  hipError_t acquire(ProfRec& r) {
    if (!pool.empty()) {
      r = pool.back();
      pool.pop_back();
      return hipSuccess;
    }
    hipError_t e = hipEventCreate(&r.a);
    if (e != hipSuccess) return e;
    return hipEventCreate(&r.b);
  }
};
Profiler g_prof;

// set for the duration of a call that must not create HIP objects (the no-allocation entry)
thread_local bool g_no_timing = false;

template <class F>
hipError_t timed(slstm_kernel_kind kind, hipStream_t s, F&& launch) {
  if (!g_prof.on || g_no_timing) return launch();
  ProfRec r;
  hipError_t e = g_prof.acquire(r);
  if (e != hipSuccess) return e;
  r.kind = kind;
  e = hipEventRecord(r.a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.b, s);
  if (e == hipSuccess) g_prof.recs.push_back(r);
  return e;
}

// ---- argument checks and workspace layout ----------------------------------------------------
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

slstm_status check_dims(int B, int T, int d) {
  if (B < 1 || T < 1 || d < 1) return fail(SLSTM_EINVAL, "B, T, d_h must be >= 1 (got %d, %d, %d)", B, T, d);
  // grid limits of the kernels' launch shapes (batch and time on grid dimensions of <= 65535
  // blocks) and 32-bit byte offsets inside one tile's rows (a scan tile spans 2 KiB * d_h)
  if (B > 65535 || T > (1 << 22) || d > (1 << 20))
    return fail(SLSTM_EINVAL, "B <= 65535, T <= 4194304 and d_h <= 1048576 required (got %d, %d, %d)", B, T, d);
  // the largest tensor, A, has B*T*16*d floats; keep every element offset well inside int64
  const double elems = 16.0 * B * T * d;
  if (elems > 4.0e15) return fail(SLSTM_EINVAL, "sizes too large");
  return SLSTM_OK;
}

int device_cus() {
  static int cus = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return cus;
}

// the kernel layout a schedule resolves to for a shape
enum class Form { kScan, kChain, kLayered };

bool known_schedule(slstm_schedule s) {
  return s == SLSTM_SCHEDULE_FUSED || s == SLSTM_SCHEDULE_LAYERED || s == SLSTM_SCHEDULE_FUSED_SCAN ||
         s == SLSTM_SCHEDULE_FUSED_CHAIN;
}

// Lane groups from which FUSED runs a fixed-count solve (tol = 0, max_iters <= 4) as the
// one-kernel form even when they do not cover every compute unit: its wavefront along T then
// waits on each tile's predecessor (a few microseconds a tile), yet reads P once where the scan
// form makes K + 2 passes over HBM. Measured on MI355X (K = 3 and 4): 32 lane groups at
// T = 16384 (B = 4, d_h = 2048) 4.2 ms against 9.3 ms; 64 at T = 2048 (B = 16, d_h = 1024)
// 0.73 ms against 1.95 ms.
constexpr long long kOneKernelMinLaneGroups = 32;

// one_kernel_ok: the call is an unpacked solve that the one-kernel form can run (a fixed count
// up to kPipeMaxIters; under FUSED up to kPipeMaxItersStop, an early stop in two passes)
Form newton_form(int B, int d, slstm_schedule s, bool one_kernel_ok = false) {
  switch (s) {
    case SLSTM_SCHEDULE_LAYERED: return Form::kLayered;
    case SLSTM_SCHEDULE_FUSED_SCAN: return Form::kScan;
    case SLSTM_SCHEDULE_FUSED_CHAIN: return Form::kChain;
    default: {
      // chains along T cost no waiting once the lane groups cover every compute unit
      const long long lg = slstm::chain_lane_groups(B, d);
      if (lg >= device_cus()) return Form::kChain;
      return one_kernel_ok && lg >= kOneKernelMinLaneGroups ? Form::kChain : Form::kScan;
    }
  }
}

struct NewtonLayout {
  size_t ctl, desc, A, rhs, S2, tab, tiles, total;
};

// control block, look-back words, then either the second iterate buffer (fused) or the
// Jacobians and right-hand sides (layered)
NewtonLayout newton_layout(int B, int T, int d, Form form) {
  NewtonLayout L;
  const size_t n_state = static_cast<size_t>(B) * T * 4 * d;
  L.ctl = 0;
  L.desc = align_up(slstm::kControlBytes);
  if (form != Form::kLayered) {
    const bool chain = form == Form::kChain;
    const size_t iter_words = chain ? slstm::chain_desc_words(B, T, d) : slstm::fused_desc_words(B, T, d);
    const size_t desc_words = std::max(iter_words, chain ? slstm::warm_chain_desc_words(B, T, d)
                                                         : slstm::warm_desc_words(B, T, d));
    L.S2 = align_up(L.desc + desc_words * 8);
    L.A = L.rhs = 0;
    L.total = align_up(L.S2 + n_state * sizeof(float));
    if (chain)  // the one-kernel solve keeps its words from L.desc on, in place of S2
      L.total = std::max(L.total, align_up(L.desc + slstm::pipe_desc_words(B, T, d, slstm::kPipeMaxItersStop) * 8));
  } else {
    const size_t desc_words = std::max(slstm::scan_desc_words(B, T, d, true), slstm::warm_desc_words(B, T, d));
    L.A = align_up(L.desc + desc_words * 8);
    L.rhs = align_up(L.A + 4 * n_state * sizeof(float));
    L.S2 = 0;
    L.total = align_up(L.rhs + n_state * sizeof(float));
  }
  // the sequence table of packed calls and their aligned tiles (unused otherwise)
  L.tab = L.total;
  L.tiles = align_up(L.tab + slstm::seq_table_ints(T) * sizeof(int));
  L.total = align_up(L.tiles + slstm::aligned_tile_ints(slstm::fused_aligned_cap(T)) * sizeof(int));
  return L;
}

// whether a pack of n_seqs sequences over T steps fits the aligned tiles of the scan-form
// iteration (at most one tile per sequence beyond the row's own count)
// whether the one-kernel solve's tiles of `steps` steps, aligned to the sequences, fit the table
bool pipe_aligned_fit(int T, int n_seqs, int steps) {
  return (T + steps - 1) / steps + static_cast<long long>(n_seqs) <= slstm::fused_aligned_cap(T);
}

bool aligned_tiles_fit(int T, int n_seqs) {
  const long long steps = slstm::fused_aligned_steps();
  return (T + steps - 1) / steps + static_cast<long long>(n_seqs) <= slstm::fused_aligned_cap(T);
}

// the warm start's kernel for a schedule: chains where the solver would use them
bool warm_chain_form(int B, int d, slstm_schedule schedule) {
  return newton_form(B, d, schedule) == Form::kChain;
}

size_t warm_desc_words_for(int B, int T, int d, bool chain) {
  return chain ? slstm::warm_chain_desc_words(B, T, d) : slstm::warm_desc_words(B, T, d);
}

hipError_t launch_warm(const void* P, bool bf16, const float* state0, float* S, int B, int T, int d,
                       int cm, bool chain, unsigned long long* desc, Control* ctl, hipStream_t st,
                       slstm::Seqs seqs) {
  const uint32_t ep = next_epoch();
  unsigned int* tickets = slstm::spread_of(ctl)->ticket[slstm::kTicketWarm][0];
  return timed(SLSTM_KERNEL_WARM_START, st, [&] {
    return chain ? slstm::launch_warm_chain(P, bf16, state0, S, B, T, d, cm, desc, tickets, ep, st)
                 : slstm::launch_warm_start(P, bf16, state0, S, B, T, d, cm, desc, tickets, ep, st, seqs);
  });
}

struct ScanLayout {
  size_t ctl, desc, tab, total;
};

// control block, look-back words, then (table_T > 0) a sequence table for table_T steps
ScanLayout scan_layout(size_t desc_words, int table_T = 0) {
  ScanLayout L;
  L.ctl = 0;
  L.desc = align_up(slstm::kControlBytes);
  L.tab = align_up(L.desc + desc_words * 8);
  L.total = table_T > 0 ? align_up(L.tab + slstm::seq_table_ints(table_T) * sizeof(int)) : L.tab;
  return L;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// the kernels' cell mode: bit 0 sigmoid forget gate, bit 1 floored read-out
bool known_cell_mode(slstm_forget f) {
  const int v = static_cast<int>(f);
  const int base = v & ~static_cast<int>(SLSTM_READOUT_FLOORED);
  return base == SLSTM_FORGET_EXP || base == SLSTM_FORGET_SIGMOID;
}

int cell_mode_of(slstm_forget f) {
  const int v = static_cast<int>(f);
  return ((v & ~static_cast<int>(SLSTM_READOUT_FLOORED)) == SLSTM_FORGET_SIGMOID ? slstm::kCellSigmoid : 0) |
         ((v & SLSTM_READOUT_FLOORED) ? slstm::kCellFloored : 0);
}

slstm_status check_common(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                          const float* states, const float* h_out, const float* final_state, int B,
                          int T, int d, slstm_forget fmode, bool states_required = true) {
  slstm_status s = check_dims(B, T, d);
  if (s != SLSTM_OK) return s;
  if (P == nullptr || R == nullptr || (states_required && states == nullptr))
    return fail(SLSTM_EINVAL, "P, R and states must not be NULL");
  if (P_dtype != SLSTM_F32 && P_dtype != SLSTM_BF16) return fail(SLSTM_EINVAL, "unknown P dtype %d", (int)P_dtype);
  if (!known_cell_mode(fmode)) return fail(SLSTM_EINVAL, "unknown forget mode %d", (int)fmode);
  if (!aligned(P, P_dtype == SLSTM_F32 ? 4 : 2) || !aligned(R, 4) || !aligned(state0, 4))
    return fail(SLSTM_EINVAL, "P, R or state0 misaligned");
  if (!aligned(states, 16) || !aligned(h_out, 16) || !aligned(final_state, 16))
    return fail(SLSTM_EINVAL, "states, h_out and final_state must be 16-byte aligned");
  return SLSTM_OK;
}

slstm_status stats_from_control(const Control& c, slstm_newton_stats* st) {
  std::memset(st, 0, sizeof(*st));
  st->iters = c.iters;
  st->converged = c.converged;
  st->diverged = c.diverged;
  st->nonfinite = c.nonfinite;
  for (int k = 0; k <= c.iters && k <= SLSTM_MAX_ITERS; ++k) {
    float v;
    std::memcpy(&v, &c.err_bits[k], 4);
    st->max_abs_F[k] = v;
  }
  if (c.nonfinite) return SLSTM_NONFINITE;
  if (c.diverged) return SLSTM_DIVERGED;
  return SLSTM_OK;
}

__global__ void store_u32_kernel(unsigned int* p, unsigned int v) { *p = v; }

#define HIP_RET(expr)            \
  do {                           \
    hipError_t e_ = (expr);      \
    if (e_ != hipSuccess) return e_; \
  } while (0)

// the solver as one launch per iteration (every schedule; the only way with an early stop)
hipError_t iterate(const void* P, bool bf16, const float* R, const float* state0, float* states,
                   float* h_out, int B, int T, int d_h, int cm, int max_iters, float tol,
                   slstm_init init, Form form, const NewtonLayout& L, void* workspace, Control* ctl,
                   unsigned int* tickets, hipStream_t st, slstm::Seqs seqs) {
  auto* desc = at<unsigned long long>(workspace, L.desc);
  const i64 n_state = static_cast<i64>(B) * T * 4 * d_h;
  // iterate buffers: the layered schedule updates `states` in place; the fused one alternates
  // between `states` and a workspace buffer, arranged so that iterate max_iters lands in
  // `states` (iterate k lives in buf[k % 2])
  float* buf[2] = {states, states};
  if (form != Form::kLayered) {
    float* other = at<float>(workspace, L.S2);
    buf[0] = (max_iters % 2 == 0) ? states : other;
    buf[1] = (max_iters % 2 == 0) ? other : states;
  }
  if (init == SLSTM_INIT_WARM) {
    HIP_RET(launch_warm(P, bf16, state0, buf[0], B, T, d_h, cm, form == Form::kChain, desc, ctl, st, seqs));
  } else {
    HIP_RET(slstm::launch_zero(buf[0], n_state, st));
  }
  if (form == Form::kChain) {
    for (int k = 0; k < max_iters; ++k) {
      const uint32_t ep = next_epoch();
      const bool last = k + 1 == max_iters;
      HIP_RET(timed(SLSTM_KERNEL_NEWTON_ITERATION, st, [&] {
        return slstm::launch_newton_chain(P, bf16, R, state0, buf[k % 2], buf[(k + 1) % 2], last ? h_out : nullptr,
                                          B, T, d_h, cm, desc, tickets, ep, ctl, k, tol, last, st);
      }));
    }
    // the last launch formed the final residual and h; what remains of the stop rule is the
    // check of the iterate before it
    HIP_RET(slstm::launch_settle(ctl, max_iters - 1, tol, st));
  } else if (form == Form::kScan) {
    for (int k = 0; k < max_iters; ++k) {
      const uint32_t ep = next_epoch();
      HIP_RET(timed(SLSTM_KERNEL_NEWTON_ITERATION, st, [&] {
        return slstm::launch_newton_iteration(P, bf16, R, state0, buf[k % 2], buf[(k + 1) % 2], B, T, d_h,
                                              cm, desc, tickets, ep, ctl, k, tol, st, seqs);
      }));
    }
  } else {
    float* A = at<float>(workspace, L.A);
    float* rhs = at<float>(workspace, L.rhs);
    for (int k = 0; k < max_iters; ++k) {
      HIP_RET(timed(SLSTM_KERNEL_RESIDUAL_JACOBIAN, st, [&] {
        return slstm::launch_residual(P, bf16, R, state0, states, A, rhs, B, T, d_h, cm, ctl,
                                      &slstm::spread_of(ctl)->err[0][k], slstm::kErrSlotWords,
                                      slstm::ResidualMode::kSparse, -1, tol, st, nullptr, seqs);
      }));
      const uint32_t ep = next_epoch();
      HIP_RET(timed(SLSTM_KERNEL_SCAN_BLOCK4, st, [&] {
        return slstm::launch_scan_block4(A, rhs, rhs, B, T, d_h, true, desc, tickets, ep, ctl, k, tol, st);
      }));
      HIP_RET(timed(SLSTM_KERNEL_UPDATE, st, [&] { return slstm::launch_update(states, rhs, n_state, ctl, k, st); }));
    }
  }
  if (form != Form::kChain) {
    // residual of the last iterate (the scan form first checks whether the iterate before it
    // already met the tolerance)
    const int chk = (form == Form::kScan) ? max_iters - 1 : -1;
    HIP_RET(timed(SLSTM_KERNEL_FINAL_RESIDUAL, st, [&] {
      return slstm::launch_residual(P, bf16, R, state0, buf[max_iters % 2], nullptr, nullptr, B, T, d_h, cm,
                                    ctl, &slstm::spread_of(ctl)->err[0][max_iters], slstm::kErrSlotWords,
                                    slstm::ResidualMode::kNone, chk, tol, st, h_out, seqs);
    }));
  }
  if (form != Form::kLayered)
    HIP_RET(slstm::launch_select_iterate(ctl, buf[0], buf[1], states, n_state, st));
  return hipSuccess;
}


// control block, the look-back words, then the dR rows and their chunk sums
struct BackwardLayout {
  size_t ctl, desc, rows, tab, tiles, total;
};

bool backward_schedule(slstm_schedule s) {
  return s == SLSTM_SCHEDULE_FUSED || s == SLSTM_SCHEDULE_FUSED_SCAN || s == SLSTM_SCHEDULE_FUSED_CHAIN;
}

// The backward's scan form measured at least as fast as its chains at every shape tried on
// MI355X (B = 128 with 512 lane groups included): one VJP pass per step costs about as much as
// the chain's, and the look-back words shrink to the anchors' values when the lane groups
// cover the GPU. Chains on request only.
bool backward_scan_form(int /*B*/, int /*d*/, slstm_schedule s) {
  return s != SLSTM_SCHEDULE_FUSED_CHAIN;
}

BackwardLayout backward_layout(int B, int T, int d, bool scan) {
  BackwardLayout L;
  L.ctl = 0;
  L.desc = align_up(slstm::kControlBytes);
  L.rows = align_up(L.desc + slstm::backward_desc_words(B, T, d, scan) * 8);
  L.tab = align_up(L.rows + slstm::backward_row_floats(B, T, d, scan) * sizeof(float));
  // packed calls only: the sequence table, then the aligned tiles
  L.tiles = align_up(L.tab + slstm::seq_table_ints(T) * sizeof(int));
  L.total = align_up(L.tiles + slstm::aligned_tile_ints(slstm::backward_aligned_cap(T)) * sizeof(int));
  return L;
}

// workspace of the input projection's backward: bfloat16 operands with the reduction dimension
// padded to whole 16-byte chunks, then the split-K partial products of dW_x
struct ProjBackLayout {
  i64 k_bt, k_4d;  // padded reduction lengths of dW_x (B*T) and dx (4*d_h)
  int splits;
  size_t dPb, WT, dPT, xT, part, total;
};

i64 pad8(i64 v) { return (v + 7) / 8 * 8; }

ProjBackLayout proj_back_layout(int B, int T, int d_in, int d_h) {
  ProjBackLayout L;
  const i64 bt = static_cast<i64>(B) * T;
  const i64 n4 = 4 * static_cast<i64>(d_h);
  L.k_bt = pad8(bt);
  L.k_4d = pad8(n4);
  // enough workgroups for SLSTM_DW_WAVES rounds of two per compute unit, each split at least
  // 32 K steps long
#ifndef SLSTM_DW_WAVES
#define SLSTM_DW_WAVES 1
#endif
  const int tiles = slstm::gemm_tiles(n4, d_in);
  int want = (SLSTM_DW_WAVES * 2 * device_cus() + tiles - 1) / tiles;
  want = std::min<i64>(want, std::max<i64>(1, L.k_bt / 1024));
  L.splits = slstm::gemm_splits_for(n4, d_in, static_cast<int>(L.k_bt), std::min(want, 64));
  L.dPb = 0;
  L.WT = align_up(L.dPb + static_cast<size_t>(bt * L.k_4d) * 2);
  L.dPT = align_up(L.WT + static_cast<size_t>(d_in * L.k_4d) * 2);
  L.xT = align_up(L.dPT + static_cast<size_t>(n4 * L.k_bt) * 2);
  L.part = align_up(L.xT + static_cast<size_t>(d_in * L.k_bt) * 2);
  L.total = align_up(L.part + (L.splits > 1 ? static_cast<size_t>(L.splits) * n4 * d_in * 4 : 0));
  return L;
}

}  // namespace

namespace slstm {

int look_back_anchor_stride(long long n_lane_groups, int wgs_per_cu) {
  const long long resident = static_cast<long long>(wgs_per_cu) * device_cus();
  long long s = (resident + n_lane_groups - 1) / n_lane_groups;
  return static_cast<int>(s < 1 ? 1 : (s > 8 ? 8 : s));
}

}  // namespace slstm

namespace {

// packed sequences: the offsets array's contents stay on the device and are not checked here;
// the kernels keep every access in bounds whatever they hold
slstm_status check_seqs(const int* cu_seqlens, int n_seqs, slstm::Seqs& seqs) {
  if (cu_seqlens == nullptr || !aligned(cu_seqlens, 4))
    return fail(SLSTM_EINVAL, "cu_seqlens must be a non-NULL, 4-byte aligned device pointer");
  if (n_seqs < 1 || n_seqs > (1 << 24)) return fail(SLSTM_EINVAL, "n_seqs must be in 1..16777216 (got %d)", n_seqs);
  seqs.cu = cu_seqlens;
  seqs.n = n_seqs;
  return SLSTM_OK;
}

// ---- scratch of the no-allocation Newton entry point --------------------------------------------
// One statically sized array per device, loaded with the code object and kept until the process
// ends. Host code must never pass the array's name to a kernel (on the host it is only a stand-in
// for the symbol): the device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(SLSTM_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// the scratch address on device `dev` (nullptr and the HIP error on failure)
void* scratch_on_device(int dev, hipError_t& err) {
  err = hipSuccess;
  if (dev < 0 || dev >= kMaxScratchDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] != nullptr) return g_scratch_ptr[dev];
  int cur = 0;
  err = hipGetDevice(&cur);
  if (err != hipSuccess) return nullptr;
  if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return nullptr;
  void* p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
  if (err != hipSuccess) return nullptr;
  if (back != hipSuccess) {
    err = back;
    return nullptr;
  }
  g_scratch_ptr[dev] = p;
  return p;
}

slstm_status newton_forward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                            float* states, float* h_out, float* final_state, int B, int T, int d_h,
                            slstm_forget fmode, int max_iters, float tol, slstm_init init,
                            slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                            void* stream, slstm_newton_stats* stats, slstm::Seqs seqs) {
  slstm_status s = check_common(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode, false);
  if (s != SLSTM_OK) return s;
  if (max_iters < 1 || max_iters > SLSTM_MAX_ITERS)
    return fail(SLSTM_EINVAL, "max_iters must be in 1..%d (got %d)", SLSTM_MAX_ITERS, max_iters);
  if (!(tol >= 0.0f) || std::isinf(tol)) return fail(SLSTM_EINVAL, "tol must be finite and >= 0");
  if (init != SLSTM_INIT_WARM && init != SLSTM_INIT_ZERO) return fail(SLSTM_EINVAL, "unknown init %d", (int)init);
  if (!known_schedule(schedule)) return fail(SLSTM_EINVAL, "unknown schedule %d", (int)schedule);
  if (workspace == nullptr || !aligned(workspace, kAlign))
    return fail(SLSTM_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (seqs.cu != nullptr && schedule == SLSTM_SCHEDULE_FUSED_CHAIN)
    return fail(SLSTM_EINVAL, "packed sequences run the scan and layered forms only (not FUSED_CHAIN)");
  // The one-kernel (pipelined) solve of the chain form: a fixed count up to kPipeMaxIters, and
  // under FUSED any count up to kPipeMaxItersStop, an early stop as two passes of it
  const bool fused = schedule == SLSTM_SCHEDULE_FUSED;
  const bool count_ok = tol == 0.0f ? max_iters <= (fused ? slstm::kPipeMaxItersStop : slstm::kPipeMaxIters)
                                    : fused && max_iters <= slstm::kPipeMaxItersStop;
  const bool one_kernel_ok = seqs.cu == nullptr && count_ok;
  // A packed row under FUSED runs it on tiles aligned to the sequence starts when the tile table
  // holds them and the sequences give enough chains (each lane group of each sequence is one)
  const int pipe_tile = slstm::pipe_tile_steps(B, d_h, device_cus());
  const bool packed_pipe = seqs.cu != nullptr && fused && count_ok && B == 1 && pipe_aligned_fit(T, seqs.n, pipe_tile) &&
                           slstm::chain_lane_groups(B, d_h) * seqs.n >= kOneKernelMinLaneGroups;
  const Form form = packed_pipe ? Form::kChain
                                : (seqs.cu != nullptr && fused ? Form::kScan : newton_form(B, d_h, schedule, one_kernel_ok));
  const bool one_kernel = (one_kernel_ok && form == Form::kChain) || packed_pipe;
  const bool stop_passes = one_kernel && tol > 0.0f;
  // only the one-kernel solve keeps its iterate on chip; every other form keeps it in `states`
  if (states == nullptr && !one_kernel)
    return fail(SLSTM_EINVAL, "states may be NULL only for a solve that resolves to the one-kernel form "
                "(tol = 0 and max_iters <= %d with FUSED_CHAIN, unpacked; max_iters <= %d with FUSED on "
                "enough lanes or sequences)", slstm::kPipeMaxIters, slstm::kPipeMaxItersStop);
  const NewtonLayout L = newton_layout(B, T, d_h, form);
  if (workspace_bytes < L.total)
    return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = P_dtype == SLSTM_BF16;
  const int cm = cell_mode_of(fmode);
  Control* ctl = at<Control>(workspace, L.ctl);
  auto* desc = at<unsigned long long>(workspace, L.desc);
  const i64 n_state = static_cast<i64>(B) * T * 4 * d_h;

  HIP_TRY(slstm::launch_init_control(ctl, st));
  if (seqs.cu != nullptr) {  // the sequence table the packed kernels start their cursors from
    int* tab = at<int>(workspace, L.tab);
    HIP_TRY(slstm::launch_seq_table(seqs.cu, seqs.n, T, tab, st));
    seqs.tab = tab;
    if (packed_pipe) {
      // the one-kernel solve's tiles aligned to the sequences, of its own length
      int* tiles = at<int>(workspace, L.tiles);
      seqs.tile_cap = slstm::fused_aligned_cap(T);
      HIP_TRY(slstm::launch_aligned_tiles(seqs.cu, seqs.n, T, pipe_tile, seqs.tile_cap, tiles, st));
      seqs.tiles = tiles;
    } else if (form == Form::kScan && aligned_tiles_fit(T, seqs.n)) {
      // the scan-form iterations on tiles aligned to the sequences
      int* tiles = at<int>(workspace, L.tiles);
      seqs.tile_cap = slstm::fused_aligned_cap(T);
      HIP_TRY(slstm::launch_aligned_tiles(seqs.cu, seqs.n, T, slstm::fused_aligned_steps(), seqs.tile_cap, tiles, st));
      seqs.tiles = tiles;
    }
  }
  unsigned int* tickets = slstm::spread_of(ctl)->ticket[slstm::kTicketTiles][0];
  if (one_kernel) {
    // the whole fixed-count solve in one pass; it writes the states (if asked for), h, the
    // final state and every residual. An early stop runs it for max_iters iterations, finds
    // the first iterate below tol, and runs it again for that count (skipped on the device when
    // none is), so the outputs are the iterate the stop returns
    auto pass = [&](bool k_from_ctl) {
      const uint32_t ep = next_epoch();
      return timed(SLSTM_KERNEL_NEWTON_SOLVE, st, [&] {
        return slstm::launch_newton_pipe(P, bf16, R, state0, states, h_out, final_state, B, T, d_h, cm,
                                         init == SLSTM_INIT_WARM, max_iters, k_from_ctl, pipe_tile, desc,
                                         tickets, ep, ctl, packed_pipe ? seqs.tiles : nullptr,
                                         packed_pipe ? seqs.tile_cap : 0, st);
      });
    };
    HIP_TRY(pass(false));
    if (stop_passes) {
      HIP_TRY(slstm::launch_pipe_stop(ctl, max_iters, tol, st));
      HIP_TRY(pass(true));
    }
    HIP_TRY(slstm::launch_finalize(ctl, tol, st));
    if (packed_pipe && final_state != nullptr)  // sequences without steps keep their state0
      HIP_TRY(slstm::launch_empty_seq_final(seqs.cu, seqs.n, T, state0, final_state, d_h, st));
  } else {
    HIP_TRY(iterate(P, bf16, R, state0, states, h_out, B, T, d_h, cm, max_iters, tol, init, form, L,
                    workspace, ctl, tickets, st, seqs));
    HIP_TRY(slstm::launch_finalize(ctl, tol, st));
    if (h_out != nullptr || final_state != nullptr)
      HIP_TRY(slstm::launch_outputs(states, h_out, final_state, B, T, d_h, ctl, st, state0, seqs));
  }
  if (stats == nullptr) return SLSTM_OK;
  Control host;
  HIP_TRY(hipMemcpyAsync(&host, ctl, sizeof(Control), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  return stats_from_control(host, stats);
}


slstm_status sequential_forward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                                float* states, float* h_out, float* final_state, int B, int T, int d_h,
                                slstm_forget fmode, void* stream, slstm::Seqs seqs) {
  slstm_status s = check_common(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode, false);
  if (s != SLSTM_OK) return s;
  // packed final states are gathered from the state tensor afterwards
  if (states == nullptr && seqs.cu != nullptr)
    return fail(SLSTM_EINVAL, "states may be NULL only for unpacked sequences");
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(timed(SLSTM_KERNEL_SEQUENTIAL, st, [&] {
    return slstm::launch_sequential(P, P_dtype == SLSTM_BF16, R, state0, states, h_out, final_state,
                                    B, T, d_h, cell_mode_of(fmode), st, seqs);
  }));
  // packed: each sequence's final state is gathered from its last step
  if (seqs.cu != nullptr && final_state != nullptr)
    HIP_TRY(slstm::launch_outputs(states, nullptr, final_state, B, T, d_h, nullptr, st, state0, seqs));
  return SLSTM_OK;
}

slstm_status warm_start(const void* P, slstm_dtype P_dtype, const float* state0, float* states, int B,
                        int T, int d_h, slstm_forget fmode, slstm_schedule schedule, void* workspace,
                        size_t workspace_bytes, void* stream, slstm::Seqs seqs) {
  static const float kDummyR = 0.0f;  // R is not used by the warm start; the shared check wants one
  slstm_status s = check_common(P, P_dtype, &kDummyR, state0, states, nullptr, nullptr, B, T, d_h, fmode);
  if (s != SLSTM_OK) return s;
  if (!known_schedule(schedule)) return fail(SLSTM_EINVAL, "unknown schedule %d", (int)schedule);
  if (workspace == nullptr || !aligned(workspace, kAlign)) return fail(SLSTM_EINVAL, "workspace must be 256-byte aligned");
  if (seqs.cu != nullptr && schedule == SLSTM_SCHEDULE_FUSED_CHAIN)
    return fail(SLSTM_EINVAL, "packed sequences run the scan form only (not FUSED_CHAIN)");
  const bool chain = seqs.cu == nullptr && warm_chain_form(B, d_h, schedule);
  const ScanLayout L = scan_layout(warm_desc_words_for(B, T, d_h, chain), T);
  if (workspace_bytes < L.total) return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Control* ctl = at<Control>(workspace, L.ctl);
  HIP_TRY(slstm::launch_init_control(ctl, st));
  if (seqs.cu != nullptr) {  // the sequence table the packed kernels start their cursors from
    int* tab = at<int>(workspace, L.tab);
    HIP_TRY(slstm::launch_seq_table(seqs.cu, seqs.n, T, tab, st));
    seqs.tab = tab;
  }
  HIP_TRY(launch_warm(P, P_dtype == SLSTM_BF16, state0, states, B, T, d_h, cell_mode_of(fmode),
                      chain, at<unsigned long long>(workspace, L.desc), ctl, st, seqs));
  return SLSTM_OK;
}

slstm_status backward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                      const float* states, const float* g_states, const float* g_h, const float* g_final,
                      void* dP, slstm_dtype dP_dtype, float* dR, float* dbias, float* dstate0, int B, int T,
                      int d_h, slstm_forget fmode, slstm_schedule schedule, void* workspace,
                      size_t workspace_bytes, void* stream, slstm::Seqs seqs) {
  slstm_status s = check_common(P, P_dtype, R, state0, states, nullptr, nullptr, B, T, d_h, fmode);
  if (s != SLSTM_OK) return s;
  if (dP == nullptr || dR == nullptr) return fail(SLSTM_EINVAL, "dP and dR must not be NULL");
  if (dP_dtype != SLSTM_F32 && dP_dtype != SLSTM_BF16) return fail(SLSTM_EINVAL, "unknown dP dtype %d", (int)dP_dtype);
  if (!aligned(dP, 16) || !aligned(dR, 4) || !aligned(dbias, 4) || !aligned(dstate0, 4) ||
      !aligned(g_states, 4) || !aligned(g_h, 4) || !aligned(g_final, 4))
    return fail(SLSTM_EINVAL, "dP must be 16-byte aligned; gradients and dR, dbias, dstate0 4-byte aligned");
  if (!known_schedule(schedule)) return fail(SLSTM_EINVAL, "unknown schedule %d", (int)schedule);
  if (!backward_schedule(schedule))
    return fail(SLSTM_EINVAL, "the backward pass has fused forms only: schedule FUSED, FUSED_SCAN or FUSED_CHAIN");
  if (workspace == nullptr || !aligned(workspace, kAlign))
    return fail(SLSTM_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (seqs.cu != nullptr && schedule == SLSTM_SCHEDULE_FUSED_CHAIN)
    return fail(SLSTM_EINVAL, "packed sequences run the scan form only (not FUSED_CHAIN)");
  const bool scan = backward_scan_form(B, d_h, schedule);
  const BackwardLayout L = backward_layout(B, T, d_h, scan);
  if (workspace_bytes < L.total)
    return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Control* ctl = at<Control>(workspace, L.ctl);
  HIP_TRY(slstm::launch_init_control(ctl, st));
  if (seqs.cu != nullptr) {  // the sequence table the packed kernels start their cursors from
    int* tab = at<int>(workspace, L.tab);
    HIP_TRY(slstm::launch_seq_table(seqs.cu, seqs.n, T, tab, st));
    seqs.tab = tab;
    const long long steps = slstm::backward_aligned_steps();
    if (scan && (T + steps - 1) / steps + static_cast<long long>(seqs.n) <= slstm::backward_aligned_cap(T)) {
      // the reverse scan on tiles aligned to the sequences (each chain runs from a sequence's
      // last tile to its first)
      int* tiles = at<int>(workspace, L.tiles);
      seqs.tile_cap = slstm::backward_aligned_cap(T);
      HIP_TRY(slstm::launch_aligned_tiles(seqs.cu, seqs.n, T, static_cast<int>(steps), seqs.tile_cap, tiles, st));
      seqs.tiles = tiles;
    }
  }
  const uint32_t ep = next_epoch();
  HIP_TRY(timed(SLSTM_KERNEL_BACKWARD, st, [&] {
    return slstm::launch_backward(P, P_dtype == SLSTM_BF16, R, state0, states, g_states, g_h, g_final, dP,
                                  dP_dtype == SLSTM_BF16, dR, dbias, dstate0, at<float>(workspace, L.rows), B, T, d_h,
                                  cell_mode_of(fmode), scan, at<unsigned long long>(workspace, L.desc),
                                  slstm::spread_of(ctl)->ticket[slstm::kTicketTiles][0], ep, st, seqs);
  }));
  return SLSTM_OK;
}

// head mixing with one launch per iteration (an early stop, or more iterations than the
// one-sweep kernel holds): the warm start or zero iterate, then K iteration kernels; iterate k
// lives in buf[k % 2], arranged so that iterate max_iters lands in `states`, and the early stop
// leaves its iterate there through select_iterate
hipError_t head_newton_iterations(const void* P, bool bf16, const float* R, const float* state0, float* states,
                                  float* h_out, int B, int T, int d_h, int n_heads, int cm, int max_iters, float tol,
                                  slstm_init init, Control* ctl, unsigned long long* desc, float* other,
                                  hipStream_t st, slstm::Seqs seqs) {
  const i64 n_state = static_cast<i64>(B) * T * 4 * d_h;
  float* buf[2] = {(max_iters % 2 == 0) ? states : other, (max_iters % 2 == 0) ? other : states};
  if (init == SLSTM_INIT_WARM) {
    HIP_RET(launch_warm(P, bf16, state0, buf[0], B, T, d_h, cm, false, desc, ctl, st, seqs));
  } else {
    HIP_RET(slstm::launch_zero(buf[0], n_state, st));
  }
  for (int k = 0; k < max_iters; ++k) {
    const bool last = k + 1 == max_iters;
    HIP_RET(timed(SLSTM_KERNEL_HEAD_ITERATION, st, [&] {
      return slstm::launch_head_iteration(P, bf16, R, state0, buf[k % 2], buf[(k + 1) % 2], last ? h_out : nullptr,
                                          B, T, d_h, n_heads, cm, ctl, k, tol, last, st, seqs);
    }));
  }
  // the last launch formed the final residual and h; what remains of the stop rule is the check
  // of the iterate before it
  HIP_RET(slstm::launch_settle(ctl, max_iters - 1, tol, st));
  return slstm::launch_select_iterate(ctl, buf[0], buf[1], states, n_state, st);
}

// head mixing: control block, the warm start's look-back words, the second iterate buffer
struct HeadLayout {
  size_t ctl, desc, S2, tab, total;
};

HeadLayout head_layout(int B, int T, int d) {
  HeadLayout L;
  L.ctl = 0;
  L.desc = align_up(slstm::kControlBytes);
  L.S2 = align_up(L.desc + slstm::warm_desc_words(B, T, d) * 8);
  L.tab = align_up(L.S2 + static_cast<size_t>(B) * T * 4 * d * sizeof(float));  // packed: sequence table
  L.total = align_up(L.tab + slstm::seq_table_ints(T) * sizeof(int));
  return L;
}

bool head_shape_ok(int d, int n_heads) {
  return n_heads >= 1 && d % n_heads == 0 && slstm::head_width_supported(d / n_heads);
}

slstm_status check_heads(int d, int n_heads, const float* R) {
  if (!head_shape_ok(d, n_heads))
    return fail(SLSTM_EINVAL, "n_heads (%d) must divide d_h (%d) into heads of 8, 16, 32, 64 or 128 units", n_heads, d);
  if (!aligned(R, 16)) return fail(SLSTM_EINVAL, "R must be 16-byte aligned");
  return SLSTM_OK;
}

}  // namespace

extern "C" {

const char* slstm_status_string(slstm_status s) {
  switch (s) {
    case SLSTM_OK: return "ok";
    case SLSTM_DIVERGED: return "diverged: max|F| > 1 after the last Newton iterate";
    case SLSTM_NONFINITE: return "non-finite residual after the last Newton iterate";
    case SLSTM_EINVAL: return "invalid argument";
    case SLSTM_EWORKSPACE: return "workspace too small";
    case SLSTM_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* slstm_last_error(void) { return g_err; }

size_t slstm_newton_workspace_bytes(int B, int T, int d_h, slstm_schedule schedule) {
  if (check_dims(B, T, d_h) != SLSTM_OK) return 0;
  if (!known_schedule(schedule)) return 0;
  // FUSED may resolve differently by iteration count and tolerance, and a packed row (B = 1) may
  // take the chain form's one-kernel solve whatever its lanes: room for each form it can pick
  size_t need = std::max(newton_layout(B, T, d_h, newton_form(B, d_h, schedule, false)).total,
                         newton_layout(B, T, d_h, newton_form(B, d_h, schedule, true)).total);
  if (schedule == SLSTM_SCHEDULE_FUSED && B == 1) need = std::max(need, newton_layout(B, T, d_h, Form::kChain).total);
  return need;
}

slstm_status slstm_newton_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                  const float* state0, float* states, float* h_out,
                                  float* final_state, int B, int T, int d_h, slstm_forget fmode,
                                  int max_iters, float tol, slstm_init init,
                                  slstm_schedule schedule, void* workspace,
                                  size_t workspace_bytes, void* stream, slstm_newton_stats* stats) {
  g_err[0] = '\0';
  return newton_forward(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode, max_iters, tol,
                        init, schedule, workspace, workspace_bytes, stream, stats, {});
}

slstm_status slstm_newton_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                         const float* state0, const int* cu_seqlens, int n_seqs,
                                         float* states, float* h_out, float* final_state, int T,
                                         int d_h, slstm_forget fmode, int max_iters, float tol,
                                         slstm_init init, slstm_schedule schedule, void* workspace,
                                         size_t workspace_bytes, void* stream,
                                         slstm_newton_stats* stats) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return newton_forward(P, P_dtype, R, state0, states, h_out, final_state, 1, T, d_h, fmode, max_iters, tol,
                        init, schedule, workspace, workspace_bytes, stream, stats, seqs);
}

slstm_status slstm_newton_read_stats(const void* workspace, size_t workspace_bytes, void* stream,
                                     slstm_newton_stats* stats) {
  g_err[0] = '\0';
  if (workspace == nullptr || stats == nullptr || workspace_bytes < sizeof(Control))
    return fail(SLSTM_EINVAL, "workspace and stats must be valid");
  hipStream_t st = static_cast<hipStream_t>(stream);
  Control host;
  HIP_TRY(hipMemcpyAsync(&host, workspace, sizeof(Control), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  return stats_from_control(host, stats);
}

slstm_status slstm_newton_forward_noalloc(const void* P, slstm_dtype P_dtype, const float* R,
                                          const float* state0, float* states, float* h_out,
                                          float* final_state, int B, int T, int d_h, slstm_forget fmode,
                                          int max_iters, float tol, slstm_init init,
                                          slstm_schedule schedule, void* stream,
                                          slstm_newton_stats* stats) {
  if (!known_schedule(schedule)) return fail(SLSTM_EINVAL, "unknown schedule %d", (int)schedule);
  const size_t need = slstm_newton_workspace_bytes(B, T, d_h, schedule);
  if (need == 0) {
    const slstm_status s = check_dims(B, T, d_h);
    return s != SLSTM_OK ? s : fail(SLSTM_EINVAL, "invalid sizes");
  }
  if (need > kNoAllocScratchBytes)
    return fail(SLSTM_EWORKSPACE,
                "slstm_newton_forward_noalloc: this problem needs %zu bytes of scratch, more than the "
                "library's fixed %zu; call slstm_newton_forward with a workspace instead",
                need, kNoAllocScratchBytes);
  int dev = 0;
  if (stream != nullptr) {
    HIP_TRY(hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev));
  } else {
    HIP_TRY(hipGetDevice(&dev));
  }
  hipError_t err;
  void* ws = scratch_on_device(dev, err);
  if (ws == nullptr) return fail(SLSTM_EHIP, "scratch address on device %d: %s", dev, hipGetErrorString(err));
  g_no_timing = true;
  const slstm_status s = newton_forward(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode,
                                        max_iters, tol, init, schedule, ws, kNoAllocScratchBytes, stream,
                                        stats, {});
  g_no_timing = false;
  return s;
}

slstm_status slstm_sequential_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                      const float* state0, float* states, float* h_out,
                                      float* final_state, int B, int T, int d_h,
                                      slstm_forget fmode, void* stream) {
  g_err[0] = '\0';
  return sequential_forward(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode, stream, {});
}

slstm_status slstm_sequential_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                             const float* state0, const int* cu_seqlens, int n_seqs,
                                             float* states, float* h_out, float* final_state, int T,
                                             int d_h, slstm_forget fmode, void* stream) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return sequential_forward(P, P_dtype, R, state0, states, h_out, final_state, 1, T, d_h, fmode, stream, seqs);
}

slstm_status slstm_input_projection(const void* x, const void* W_x, const float* bias, float* P,
                                    int B, int T, int d_in, int d_h, slstm_dtype xw_dtype,
                                    void* stream) {
  g_err[0] = '\0';
  slstm_status s = check_dims(B, T, d_h);
  if (s != SLSTM_OK) return s;
  if (d_in < 8 || d_in % 8 != 0) return fail(SLSTM_EINVAL, "d_in must be a positive multiple of 8 (got %d)", d_in);
  if (xw_dtype != SLSTM_BF16) return fail(SLSTM_EINVAL, "the input projection takes bf16 x and W_x");
  if (x == nullptr || W_x == nullptr || P == nullptr) return fail(SLSTM_EINVAL, "x, W_x and P must not be NULL");
  if (!aligned(x, 16) || !aligned(W_x, 16) || !aligned(P, 4) || !aligned(bias, 4))
    return fail(SLSTM_EINVAL, "x and W_x must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const i64 M = static_cast<i64>(B) * T;
  HIP_TRY(timed(SLSTM_KERNEL_INPUT_PROJECTION, st, [&] {
    return slstm::launch_gemm_bf16(x, W_x, bias, P, M, 4 * d_h, d_in, st);
  }));
  return SLSTM_OK;
}

slstm_status slstm_residual_jacobian(const void* P, slstm_dtype P_dtype, const float* R,
                                     const float* state0, const float* states, float* A,
                                     float* rhs, float* max_abs_F, int B, int T, int d_h,
                                     slstm_forget fmode, void* stream) {
  g_err[0] = '\0';
  slstm_status s = check_common(P, P_dtype, R, state0, states, nullptr, nullptr, B, T, d_h, fmode);
  if (s != SLSTM_OK) return s;
  if (A == nullptr || rhs == nullptr || max_abs_F == nullptr)
    return fail(SLSTM_EINVAL, "A, rhs and max_abs_F must not be NULL");
  if (!aligned(A, 16) || !aligned(rhs, 16) || !aligned(max_abs_F, 4)) return fail(SLSTM_EINVAL, "A or rhs misaligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned int* err = reinterpret_cast<unsigned int*>(max_abs_F);
  store_u32_kernel<<<1, 1, 0, st>>>(err, 0u);
  HIP_TRY(hipGetLastError());
  HIP_TRY(timed(SLSTM_KERNEL_RESIDUAL_JACOBIAN, st, [&] {
    return slstm::launch_residual(P, P_dtype == SLSTM_BF16, R, state0, states, A, rhs, B, T, d_h,
                                  cell_mode_of(fmode), nullptr, err, 0, slstm::ResidualMode::kDense, -1,
                                  0.0f, st);
  }));
  return SLSTM_OK;
}

size_t slstm_scan_block4_workspace_bytes(int B, int T, int d_h) {
  if (check_dims(B, T, d_h) != SLSTM_OK) return 0;
  return scan_layout(slstm::scan_desc_words(B, T, d_h, false)).total;
}

slstm_status slstm_scan_block4(const float* A, const float* rhs, float* x, int B, int T, int d_h,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  slstm_status s = check_dims(B, T, d_h);
  if (s != SLSTM_OK) return s;
  if (A == nullptr || rhs == nullptr || x == nullptr) return fail(SLSTM_EINVAL, "A, rhs and x must not be NULL");
  if (!aligned(A, 4) || !aligned(rhs, 4) || !aligned(x, 4)) return fail(SLSTM_EINVAL, "A, rhs or x misaligned");
  if (workspace == nullptr || !aligned(workspace, kAlign)) return fail(SLSTM_EINVAL, "workspace must be 256-byte aligned");
  const ScanLayout L = scan_layout(slstm::scan_desc_words(B, T, d_h, false));
  if (workspace_bytes < L.total) return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Control* ctl = at<Control>(workspace, L.ctl);
  HIP_TRY(slstm::launch_init_control(ctl, st));
  const uint32_t ep = next_epoch();
  HIP_TRY(timed(SLSTM_KERNEL_SCAN_BLOCK4, st, [&] {
    return slstm::launch_scan_block4(A, rhs, x, B, T, d_h, false, at<unsigned long long>(workspace, L.desc),
                                     slstm::spread_of(ctl)->ticket[slstm::kTicketTiles][0], ep, nullptr, 0, 0.0f, st);
  }));
  return SLSTM_OK;
}

size_t slstm_warm_start_workspace_bytes(int B, int T, int d_h, slstm_schedule schedule) {
  if (check_dims(B, T, d_h) != SLSTM_OK || !known_schedule(schedule)) return 0;
  return scan_layout(warm_desc_words_for(B, T, d_h, warm_chain_form(B, d_h, schedule)), T).total;
}

slstm_status slstm_warm_start(const void* P, slstm_dtype P_dtype, const float* state0,
                              float* states, int B, int T, int d_h, slstm_forget fmode,
                              slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                              void* stream) {
  g_err[0] = '\0';
  return warm_start(P, P_dtype, state0, states, B, T, d_h, fmode, schedule, workspace, workspace_bytes, stream, {});
}

slstm_status slstm_warm_start_varlen(const void* P, slstm_dtype P_dtype, const float* state0,
                                     const int* cu_seqlens, int n_seqs, float* states, int T, int d_h,
                                     slstm_forget fmode, slstm_schedule schedule, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return warm_start(P, P_dtype, state0, states, 1, T, d_h, fmode, schedule, workspace, workspace_bytes, stream,
                    seqs);
}

size_t slstm_backward_workspace_bytes(int B, int T, int d_h, slstm_schedule schedule) {
  if (check_dims(B, T, d_h) != SLSTM_OK || !backward_schedule(schedule)) return 0;
  return backward_layout(B, T, d_h, backward_scan_form(B, d_h, schedule)).total;
}

slstm_status slstm_backward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                            const float* states, const float* g_states, const float* g_h,
                            const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR,
                            float* dbias, float* dstate0, int B, int T, int d_h, slstm_forget fmode,
                            slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err[0] = '\0';
  return backward(P, P_dtype, R, state0, states, g_states, g_h, g_final, dP, dP_dtype, dR, dbias, dstate0, B, T,
                  d_h, fmode, schedule, workspace, workspace_bytes, stream, {});
}

slstm_status slstm_backward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                   const float* state0, const int* cu_seqlens, int n_seqs,
                                   const float* states, const float* g_states, const float* g_h,
                                   const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR,
                                   float* dbias, float* dstate0, int T, int d_h, slstm_forget fmode,
                                   slstm_schedule schedule, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return backward(P, P_dtype, R, state0, states, g_states, g_h, g_final, dP, dP_dtype, dR, dbias, dstate0, 1, T,
                  d_h, fmode, schedule, workspace, workspace_bytes, stream, seqs);
}

size_t slstm_input_projection_backward_workspace_bytes(int B, int T, int d_in, int d_h) {
  if (check_dims(B, T, d_h) != SLSTM_OK || d_in < 8 || d_in % 8 != 0) return 0;
  return proj_back_layout(B, T, d_in, d_h).total;
}

slstm_status slstm_input_projection_backward(const void* x, const void* W_x, const void* dP,
                                             slstm_dtype dP_dtype, float* dx, float* dW_x, int B,
                                             int T, int d_in, int d_h, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  slstm_status s = check_dims(B, T, d_h);
  if (s != SLSTM_OK) return s;
  if (d_in < 8 || d_in % 8 != 0) return fail(SLSTM_EINVAL, "d_in must be a positive multiple of 8 (got %d)", d_in);
  if (dP_dtype != SLSTM_F32 && dP_dtype != SLSTM_BF16) return fail(SLSTM_EINVAL, "unknown dP dtype %d", (int)dP_dtype);
  if (dP == nullptr || (dW_x != nullptr && x == nullptr) || (dx != nullptr && W_x == nullptr))
    return fail(SLSTM_EINVAL, "dP, and x for dW_x and W_x for dx, must not be NULL");
  if (!aligned(x, 16) || !aligned(W_x, 16) || !aligned(dP, 16) || !aligned(dx, 4) || !aligned(dW_x, 4))
    return fail(SLSTM_EINVAL, "x, W_x and dP must be 16-byte aligned");
  if (workspace == nullptr || !aligned(workspace, kAlign))
    return fail(SLSTM_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  const ProjBackLayout L = proj_back_layout(B, T, d_in, d_h);
  if (workspace_bytes < L.total)
    return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f32 = dP_dtype == SLSTM_F32;
  const i64 bt = static_cast<i64>(B) * T;
  const int n4 = 4 * d_h;
  if (dW_x != nullptr) {
    uint16_t* dPT = at<uint16_t>(workspace, L.dPT);
    uint16_t* xT = at<uint16_t>(workspace, L.xT);
    float* part = at<float>(workspace, L.part);
    HIP_TRY(timed(SLSTM_KERNEL_WEIGHT_GRADIENT, st, [&]() -> hipError_t {
      hipError_t e = slstm::launch_transpose_bf16(dP, f32, dPT, bt, n4, L.k_bt, st);
      if (e != hipSuccess) return e;
      e = slstm::launch_transpose_bf16(x, false, xT, bt, d_in, L.k_bt, st);
      if (e != hipSuccess) return e;
      if (L.splits == 1) return slstm::launch_gemm_bf16(dPT, xT, nullptr, dW_x, n4, d_in, static_cast<int>(L.k_bt), st, 1);
      e = slstm::launch_gemm_bf16(dPT, xT, nullptr, part, n4, d_in, static_cast<int>(L.k_bt), st, L.splits);
      if (e != hipSuccess) return e;
      return slstm::launch_sum_splits(part, dW_x, L.splits, static_cast<i64>(n4) * d_in, st);
    }));
  }
  if (dx != nullptr) {
    uint16_t* WT = at<uint16_t>(workspace, L.WT);
    HIP_TRY(timed(SLSTM_KERNEL_INPUT_GRADIENT, st, [&]() -> hipError_t {
      hipError_t e = slstm::launch_transpose_bf16(W_x, false, WT, n4, d_in, L.k_4d, st);
      if (e != hipSuccess) return e;
      const void* A = dP;
      if (f32 || L.k_4d != n4) {
        uint16_t* dPb = at<uint16_t>(workspace, L.dPb);
        e = slstm::launch_pad_bf16(dP, f32, dPb, bt, n4, static_cast<int>(L.k_4d), st);
        if (e != hipSuccess) return e;
        A = dPb;
      }
      return slstm::launch_gemm_bf16(A, WT, nullptr, dx, bt, d_in, static_cast<int>(L.k_4d), st, 1);
    }));
  }
  return SLSTM_OK;
}

size_t slstm_head_newton_workspace_bytes(int B, int T, int d_h, int n_heads) {
  if (check_dims(B, T, d_h) != SLSTM_OK || !head_shape_ok(d_h, n_heads)) return 0;
  return head_layout(B, T, d_h).total;
}

}  // extern "C"

namespace {

slstm_status head_newton_forward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                                 float* states, float* h_out, float* final_state, int B, int T, int d_h,
                                 int n_heads, slstm_forget fmode, int max_iters, float tol, slstm_init init,
                                 void* workspace, size_t workspace_bytes, void* stream, slstm_newton_stats* stats,
                                 slstm::Seqs seqs) {
  slstm_status s = check_common(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode);
  if (s != SLSTM_OK) return s;
  s = check_heads(d_h, n_heads, R);
  if (s != SLSTM_OK) return s;
  if (max_iters < 1 || max_iters > SLSTM_MAX_ITERS)
    return fail(SLSTM_EINVAL, "max_iters must be in 1..%d (got %d)", SLSTM_MAX_ITERS, max_iters);
  if (!(tol >= 0.0f) || std::isinf(tol)) return fail(SLSTM_EINVAL, "tol must be finite and >= 0");
  if (init != SLSTM_INIT_WARM && init != SLSTM_INIT_ZERO) return fail(SLSTM_EINVAL, "unknown init %d", (int)init);
  if (workspace == nullptr || !aligned(workspace, kAlign))
    return fail(SLSTM_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  const HeadLayout L = head_layout(B, T, d_h);
  if (workspace_bytes < L.total)
    return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = P_dtype == SLSTM_BF16;
  const int cm = cell_mode_of(fmode);
  Control* ctl = at<Control>(workspace, L.ctl);
  auto* desc = at<unsigned long long>(workspace, L.desc);
  HIP_TRY(slstm::launch_init_control(ctl, st));
  if (seqs.cu != nullptr) {
    int* tab = at<int>(workspace, L.tab);
    HIP_TRY(slstm::launch_seq_table(seqs.cu, seqs.n, T, tab, st));
    seqs.tab = tab;
  }
  // the one-sweep kernel serves fixed counts on heads up to 64 units (packed rows in its
  // single-group form); 128-unit heads and solves with a tolerance iterate kernel by kernel
  if (tol == 0.0f && max_iters <= slstm::kHeadSolveMaxIters && d_h / n_heads <= slstm::kHeadSolveMaxWidth) {
    // a fixed count of iterations: the whole solve in one sweep over T
    HIP_TRY(timed(SLSTM_KERNEL_HEAD_SOLVE, st, [&] {
      return slstm::launch_head_solve(P, bf16, R, state0, states, h_out, B, T, d_h, n_heads, cm, max_iters,
                                      init == SLSTM_INIT_ZERO, ctl, st, seqs);
    }));
  } else {
    HIP_TRY(head_newton_iterations(P, bf16, R, state0, states, h_out, B, T, d_h, n_heads, cm, max_iters, tol, init,
                                   ctl, desc, at<float>(workspace, L.S2), st, seqs));
  }
  HIP_TRY(slstm::launch_finalize(ctl, tol, st));
  if (h_out != nullptr || final_state != nullptr)
    HIP_TRY(slstm::launch_outputs(states, h_out, final_state, B, T, d_h, ctl, st, state0, seqs));
  if (stats == nullptr) return SLSTM_OK;
  Control host;
  HIP_TRY(hipMemcpyAsync(&host, ctl, sizeof(Control), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  return stats_from_control(host, stats);
}
slstm_status head_sequential_forward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                                     float* states, float* h_out, float* final_state, int B, int T, int d_h,
                                     int n_heads, slstm_forget fmode, void* stream, slstm::Seqs seqs) {
  slstm_status s = check_common(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, fmode);
  if (s != SLSTM_OK) return s;
  s = check_heads(d_h, n_heads, R);
  if (s != SLSTM_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(timed(SLSTM_KERNEL_HEAD_SEQUENTIAL, st, [&] {
    return slstm::launch_head_sequential(P, P_dtype == SLSTM_BF16, R, state0, states, h_out,
                                         seqs.cu != nullptr ? nullptr : final_state, B, T, d_h, n_heads,
                                         cell_mode_of(fmode), st, seqs);
  }));
  if (seqs.cu != nullptr && final_state != nullptr)  // each sequence's last state, or its state0 if empty
    HIP_TRY(slstm::launch_outputs(states, nullptr, final_state, B, T, d_h, nullptr, st, state0, seqs));
  return SLSTM_OK;
}


slstm_status head_backward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                           const float* states, const float* g_states, const float* g_h, const float* g_final,
                           void* dP, slstm_dtype dP_dtype, float* dR, float* dbias, float* dstate0, int B, int T,
                           int d_h, int n_heads, slstm_forget fmode, void* workspace, size_t workspace_bytes,
                           void* stream, slstm::Seqs seqs) {
  slstm_status s = check_common(P, P_dtype, R, state0, states, nullptr, nullptr, B, T, d_h, fmode);
  if (s != SLSTM_OK) return s;
  s = check_heads(d_h, n_heads, R);
  if (s != SLSTM_OK) return s;
  if (!slstm::head_backward_width_supported(d_h / n_heads))
    return fail(SLSTM_EINVAL, "the head-mixing backward takes heads of 8, 16, 32, 64 or 128 units (got %d)", d_h / n_heads);
  if (dP == nullptr || dR == nullptr) return fail(SLSTM_EINVAL, "dP and dR must not be NULL");
  if (dP_dtype != SLSTM_F32 && dP_dtype != SLSTM_BF16) return fail(SLSTM_EINVAL, "unknown dP dtype %d", (int)dP_dtype);
  if (!aligned(dP, 4) || !aligned(dR, 4) || !aligned(dbias, 4) || !aligned(dstate0, 4) || !aligned(g_states, 4) ||
      !aligned(g_h, 4) || !aligned(g_final, 4))
    return fail(SLSTM_EINVAL, "dP, the gradients and dR, dbias, dstate0 must be 4-byte aligned");
  if (workspace == nullptr || !aligned(workspace, kAlign))
    return fail(SLSTM_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  const size_t need = slstm_head_backward_workspace_bytes(B, T, d_h, n_heads);
  if (workspace_bytes < need) return fail(SLSTM_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(timed(SLSTM_KERNEL_HEAD_BACKWARD, st, [&] {
    return slstm::launch_head_backward(P, P_dtype == SLSTM_BF16, R, state0, states, g_states, g_h, g_final, dP,
                                       dP_dtype == SLSTM_BF16, dR, dbias, dstate0, B, T, d_h, n_heads,
                                       cell_mode_of(fmode), static_cast<float*>(workspace), st, seqs);
  }));
  return SLSTM_OK;
}

}  // namespace

extern "C" {

size_t slstm_head_backward_workspace_bytes(int B, int T, int d_h, int n_heads) {
  if (check_dims(B, T, d_h) != SLSTM_OK || !head_shape_ok(d_h, n_heads) ||
      !slstm::head_backward_width_supported(d_h / n_heads))
    return 0;
  return align_up(slstm::head_backward_part_floats(B, d_h, n_heads) * sizeof(float));
}

slstm_status slstm_head_newton_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                       const float* state0, float* states, float* h_out,
                                       float* final_state, int B, int T, int d_h, int n_heads,
                                       slstm_forget fmode, int max_iters, float tol, slstm_init init,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       slstm_newton_stats* stats) {
  g_err[0] = '\0';
  return head_newton_forward(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, n_heads, fmode, max_iters,
                             tol, init, workspace, workspace_bytes, stream, stats, {});
}

slstm_status slstm_head_newton_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                              const float* state0, const int* cu_seqlens, int n_seqs,
                                              float* states, float* h_out, float* final_state, int T,
                                              int d_h, int n_heads, slstm_forget fmode, int max_iters,
                                              float tol, slstm_init init, void* workspace,
                                              size_t workspace_bytes, void* stream,
                                              slstm_newton_stats* stats) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return head_newton_forward(P, P_dtype, R, state0, states, h_out, final_state, 1, T, d_h, n_heads, fmode, max_iters,
                             tol, init, workspace, workspace_bytes, stream, stats, seqs);
}

slstm_status slstm_head_sequential_forward(const void* P, slstm_dtype P_dtype, const float* R,
                                           const float* state0, float* states, float* h_out,
                                           float* final_state, int B, int T, int d_h, int n_heads,
                                           slstm_forget fmode, void* stream) {
  g_err[0] = '\0';
  return head_sequential_forward(P, P_dtype, R, state0, states, h_out, final_state, B, T, d_h, n_heads, fmode, stream,
                                 {});
}

slstm_status slstm_head_sequential_forward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                                  const float* state0, const int* cu_seqlens, int n_seqs,
                                                  float* states, float* h_out, float* final_state, int T,
                                                  int d_h, int n_heads, slstm_forget fmode, void* stream) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return head_sequential_forward(P, P_dtype, R, state0, states, h_out, final_state, 1, T, d_h, n_heads, fmode, stream,
                                 seqs);
}

slstm_status slstm_head_backward(const void* P, slstm_dtype P_dtype, const float* R, const float* state0,
                                 const float* states, const float* g_states, const float* g_h,
                                 const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR, float* dbias,
                                 float* dstate0, int B, int T, int d_h, int n_heads, slstm_forget fmode,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  return head_backward(P, P_dtype, R, state0, states, g_states, g_h, g_final, dP, dP_dtype, dR, dbias, dstate0, B, T,
                       d_h, n_heads, fmode, workspace, workspace_bytes, stream, {});
}

slstm_status slstm_head_backward_varlen(const void* P, slstm_dtype P_dtype, const float* R,
                                        const float* state0, const int* cu_seqlens, int n_seqs,
                                        const float* states, const float* g_states, const float* g_h,
                                        const float* g_final, void* dP, slstm_dtype dP_dtype, float* dR,
                                        float* dbias, float* dstate0, int T, int d_h, int n_heads,
                                        slstm_forget fmode, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  g_err[0] = '\0';
  slstm::Seqs seqs;
  slstm_status s = check_seqs(cu_seqlens, n_seqs, seqs);
  if (s != SLSTM_OK) return s;
  return head_backward(P, P_dtype, R, state0, states, g_states, g_h, g_final, dP, dP_dtype, dR, dbias, dstate0, 1, T,
                       d_h, n_heads, fmode, workspace, workspace_bytes, stream, seqs);
}

slstm_status slstm_profile_enable(int on) {
  g_prof.on = on != 0;
  return SLSTM_OK;
}

slstm_status slstm_profile_reset(void) {
  for (auto& r : g_prof.recs) g_prof.pool.push_back(r);
  g_prof.recs.clear();
  return SLSTM_OK;
}

slstm_status slstm_profile_read(slstm_kernel_kind kind, double* total_ms, int* launches) {
  g_err[0] = '\0';
  if (total_ms == nullptr || launches == nullptr) return fail(SLSTM_EINVAL, "NULL output");
  double sum = 0.0;
  int n = 0;
  for (auto& r : g_prof.recs) {
    if (r.kind != static_cast<int>(kind)) continue;
    HIP_TRY(hipEventSynchronize(r.b));
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return SLSTM_OK;
}

slstm_status slstm_profile_durations(slstm_kernel_kind kind, double* out_ms, int capacity,
                                     int* launches) {
  g_err[0] = '\0';
  if (launches == nullptr || (capacity > 0 && out_ms == nullptr)) return fail(SLSTM_EINVAL, "NULL output");
  int n = 0;
  for (auto& r : g_prof.recs) {
    if (r.kind != static_cast<int>(kind)) continue;
    if (n < capacity) {
      HIP_TRY(hipEventSynchronize(r.b));
      float ms = 0.0f;
      HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
      out_ms[n] = ms;
    }
    ++n;
  }
  *launches = n;
  return SLSTM_OK;
}

}  // extern "C"
