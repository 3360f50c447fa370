// Kernel (c) and the solver's control kernels.
//
// update:    s <- s + Delta over all (b, t, slot, j) (the Newton step, Delta from the scan);
//            records the number of applied updates. Skipped once the solver has stopped.
// init:      clears the control block (residual maxima, counters, flags) at the start of a
//            solve; a plain fill kernel, so the whole solve can be replayed from a graph.
// finalize:  flags from the residual of the last iterate: divergence when max|F| > 1 or it is
//            not finite, convergence when a tolerance is set and met ("Layout" page of the
//            pararnn-torch docs, "Current surface (0.17)": NewtonStats, residual early stop,
//            divergence error when max|F| > 1 after K).
// select:    copies the final iterate into the caller's states when an early stop left it in
//            the fused schedule's other iterate buffer.
// outputs:   copies the hidden slot (slot 3) of the states into a (B, T, d) output and the
//            last step's state into a contiguous (B, 4, d) output.
#include "common.h"
#include "kernels.h"

namespace slstm {

constexpr int kUpdBlock = 256;
// residual maxima reduced at the end of a solve: iterations 0 .. 64 (the largest iteration cap)
constexpr int kFinalizeIters = 65;
static_assert(kFinalizeIters <= kErrSlotWords && kFinalizeIters <= 72, "slot words per iteration");

__global__ __launch_bounds__(kUpdBlock) void update_kernel(float4* __restrict__ S,
                                                           const float4* __restrict__ D, i64 n4,
                                                           Control* __restrict__ ctl, int k_iter) {
  if (ctl->stopped) return;
  const i64 stride = static_cast<i64>(gridDim.x) * kUpdBlock;
  for (i64 i = static_cast<i64>(blockIdx.x) * kUpdBlock + threadIdx.x; i < n4; i += stride) {
    float4 s = S[i];
    const float4 dl = D[i];
    s.x += dl.x;
    s.y += dl.y;
    s.z += dl.z;
    s.w += dl.w;
    S[i] = s;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) ctl->iters = k_iter + 1;
}

__global__ __launch_bounds__(kUpdBlock) void init_control_kernel(Control* __restrict__ ctl) {
  // the control block and its spread counters
  unsigned int* w = reinterpret_cast<unsigned int*>(ctl);
  constexpr int n = static_cast<int>(kControlBytes / 4);
  for (int i = blockIdx.x * kUpdBlock + threadIdx.x; i < n; i += gridDim.x * kUpdBlock) w[i] = 0u;
}

// one wave per iteration k: the residual maximum reduced over the slots into err_bits[k];
// the wave of the final iterate also sets the flags
__global__ __launch_bounds__(kWave) void finalize_kernel(Control* __restrict__ ctl, float tol) {
  const int k = blockIdx.x;
  const float e = err_reduced(ctl, k);
  if (threadIdx.x != 0) return;
  ctl->err_bits[k] = __float_as_uint(e);
  if (k != ctl->iters) return;
  const bool finite = e == e && e != INFINITY;
  ctl->nonfinite = finite ? 0 : 1;
  ctl->diverged = (!finite || e > 1.0f) ? 1 : 0;
  ctl->converged = (tol > 0.0f && finite && e < tol) ? 1 : 0;
}

// one wave: the stop decision the next iteration's launch would have taken for iterate k
__global__ __launch_bounds__(kWave) void settle_kernel(Control* __restrict__ ctl, int k, float tol) {
  const float e = err_reduced(ctl, k);
  if (threadIdx.x == 0 && !ctl->stopped && tol > 0.0f && e < tol) {
    ctl->stopped = 1;
    ctl->iters = k;
  }
}

__global__ __launch_bounds__(kUpdBlock) void hidden_kernel(const float* __restrict__ S,
                                                           float* __restrict__ h, i64 rows, int d,
                                                           const Control* __restrict__ ctl) {
  // the final residual pass writes h unless an early stop skipped it
  if (ctl != nullptr && !ctl->stopped) return;
  // rows = B*T; element i of h is feature i % d of row i / d
  const i64 n = rows * d;
  const i64 stride = static_cast<i64>(gridDim.x) * kUpdBlock;
  for (i64 i = static_cast<i64>(blockIdx.x) * kUpdBlock + threadIdx.x; i < n; i += stride) {
    const i64 row = i / d;
    const i64 j = i - row * d;
    h[i] = S[(row * 4 + 3) * d + j];
  }
}

__global__ __launch_bounds__(kUpdBlock) void final_state_kernel(const float* __restrict__ S,
                                                                float* __restrict__ out, int B,
                                                                int T, int d) {
  const i64 n = static_cast<i64>(B) * 4 * d;  // (b, slot, j) of the last step
  for (i64 i = static_cast<i64>(blockIdx.x) * kUpdBlock + threadIdx.x; i < n;
       i += static_cast<i64>(gridDim.x) * kUpdBlock) {
    const i64 b = i / (4 * static_cast<i64>(d));
    const i64 rest = i - b * 4 * d;
    out[i] = S[(b * T + (T - 1)) * 4 * d + rest];
  }
}

// packed sequences: out[s] = the last state of sequence s (steps cu[s] .. cu[s+1]-1 of the one
// batch row), or state0[s] (zeros without one) for an empty sequence; cu is read only within
// its n_seqs + 1 entries and the step is clamped into [0, T)
__global__ __launch_bounds__(kUpdBlock) void packed_final_state_kernel(const float* __restrict__ S,
                                                                       const float* __restrict__ state0,
                                                                       const int* __restrict__ cu,
                                                                       float* __restrict__ out,
                                                                       int n_seqs, int T, int d) {
  const i64 n = static_cast<i64>(n_seqs) * 4 * d;  // (s, slot, j)
  for (i64 i = static_cast<i64>(blockIdx.x) * kUpdBlock + threadIdx.x; i < n;
       i += static_cast<i64>(gridDim.x) * kUpdBlock) {
    const int s = static_cast<int>(i / (4 * static_cast<i64>(d)));
    const i64 rest = i - static_cast<i64>(s) * 4 * d;
    const int a = cu[s], e = cu[s + 1];
    if (e > a) {
      const int t = e - 1 < 0 ? 0 : (e - 1 >= T ? T - 1 : e - 1);
      out[i] = S[static_cast<i64>(t) * 4 * d + rest];
    } else {
      out[i] = state0 != nullptr ? state0[i] : 0.0f;
    }
  }
}

__global__ __launch_bounds__(kUpdBlock) void zero_kernel(float4* __restrict__ p, i64 n4) {
  const i64 stride = static_cast<i64>(gridDim.x) * kUpdBlock;
  for (i64 i = static_cast<i64>(blockIdx.x) * kUpdBlock + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

__global__ __launch_bounds__(kUpdBlock) void select_iterate_kernel(const Control* __restrict__ ctl,
                                                                   const float4* buf0,
                                                                   const float4* buf1, float4* states,
                                                                   i64 n4) {
  const float4* src = (ctl->iters % 2 == 0) ? buf0 : buf1;
  if (src == states) return;  // the final iterate is already in place
  const i64 stride = static_cast<i64>(gridDim.x) * kUpdBlock;
  for (i64 i = static_cast<i64>(blockIdx.x) * kUpdBlock + threadIdx.x; i < n4; i += stride) states[i] = src[i];
}

static unsigned int stream_grid(i64 n) {
  // enough blocks to fill 256 CUs several times over; the kernels stride the rest
  const i64 want = (n + kUpdBlock - 1) / kUpdBlock;
  return static_cast<unsigned int>(want < 8192 ? (want > 0 ? want : 1) : 8192);
}

hipError_t launch_update(float* S, const float* D, i64 n_floats, Control* ctl, int k_iter,
                         hipStream_t stream) {
  const i64 n4 = n_floats / 4;
  // four workgroups per compute unit striding the whole tensor: streams S and Delta faster
  // on MI355X than more, shorter-lived workgroups (5.2 against 4.9 TB/s measured)
  const i64 want = (n4 + kUpdBlock - 1) / kUpdBlock;
  const unsigned grid = static_cast<unsigned>(want < 1024 ? (want > 0 ? want : 1) : 1024);
  update_kernel<<<grid, kUpdBlock, 0, stream>>>(
      reinterpret_cast<float4*>(S), reinterpret_cast<const float4*>(D), n4, ctl, k_iter);
  return hipGetLastError();
}

hipError_t launch_init_control(Control* ctl, hipStream_t stream) {
  init_control_kernel<<<16, kUpdBlock, 0, stream>>>(ctl);
  return hipGetLastError();
}

hipError_t launch_finalize(Control* ctl, float tol, hipStream_t stream) {
  finalize_kernel<<<kFinalizeIters, kWave, 0, stream>>>(ctl, tol);
  return hipGetLastError();
}

hipError_t launch_settle(Control* ctl, int k, float tol, hipStream_t stream) {
  settle_kernel<<<1, kWave, 0, stream>>>(ctl, k, tol);
  return hipGetLastError();
}

hipError_t launch_outputs(const float* S, float* h, float* final_state, int B, int T, int d,
                          const Control* ctl, hipStream_t stream, const float* state0, Seqs seqs) {
  if (h != nullptr) {
    const i64 rows = static_cast<i64>(B) * T;
    hidden_kernel<<<stream_grid(rows * d), kUpdBlock, 0, stream>>>(S, h, rows, d, ctl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (final_state != nullptr && seqs.cu != nullptr) {
    if (seqs.n > 0)
      packed_final_state_kernel<<<stream_grid(static_cast<i64>(seqs.n) * 4 * d), kUpdBlock, 0, stream>>>(
          S, state0, seqs.cu, final_state, seqs.n, T, d);
  } else if (final_state != nullptr) {
    final_state_kernel<<<stream_grid(static_cast<i64>(B) * 4 * d), kUpdBlock, 0, stream>>>(
        S, final_state, B, T, d);
  }
  return hipGetLastError();
}

hipError_t launch_select_iterate(const Control* ctl, const float* buf0, const float* buf1,
                                 float* states, i64 n_floats, hipStream_t stream) {
  const i64 n4 = n_floats / 4;
  select_iterate_kernel<<<stream_grid(n4), kUpdBlock, 0, stream>>>(
      ctl, reinterpret_cast<const float4*>(buf0), reinterpret_cast<const float4*>(buf1),
      reinterpret_cast<float4*>(states), n4);
  return hipGetLastError();
}

// entry k of the sequence table: the sequence holding step 4k (a binary search per entry, all
// entries in parallel)
__global__ __launch_bounds__(kUpdBlock) void seq_table_kernel(const int* __restrict__ cu, int n_seqs,
                                                             int* __restrict__ tab, int n_tab) {
  const int k = blockIdx.x * kUpdBlock + threadIdx.x;
  if (k >= n_tab) return;
  tab[k] = seq_cursor(cu, n_seqs, 0, k << kSeqTabShift).s;
}

size_t seq_table_ints(int T) { return (static_cast<size_t>(T) + (1u << kSeqTabShift) - 1) >> kSeqTabShift; }

hipError_t launch_seq_table(const int* cu, int n_seqs, int T, int* tab, hipStream_t stream) {
  const int n_tab = static_cast<int>(seq_table_ints(T));
  seq_table_kernel<<<(n_tab + kUpdBlock - 1) / kUpdBlock, kUpdBlock, 0, stream>>>(cu, n_seqs, tab, n_tab);
  return hipGetLastError();
}

// Tiles aligned to packed sequences: sequence s gets ceil(len_s / tile_steps) tiles, numbered
// consecutively (tile id = the sequence's first tile + its position p), none straddling a start.
// The order they are handed out in is by position (any order among the tiles of one position):
// every tile comes after the tiles before it in its sequence (the only ones it waits on), while
// the tiles in flight at once belong to many sequences. One workgroup builds it, once per solve:
// block scans give each sequence its first id; a histogram of the tile counts, summed from the
// top, gives the tiles at each position and its exclusive prefix the first slot of each
// position; each tile then takes the next slot of its position. At most cap tiles are made,
// whatever the offsets hold (offsets are clamped into [0, T]).
// Layout of tiles: [0] count, then per slot of the hand-out order (cap each): the tile id, its
// sequence, its position, the sequence's first step and its end (a tile reads its five values
// in one round of independent loads); then cap each of scratch: sequence and position by id,
// counters.
constexpr int kTileBlock = 1024;

// inclusive sum over the workgroup's threads in thread order; *total receives the sum of all
template <class V>
__device__ V block_inclusive_sum(V v, V* s_wave, V* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave[w] = v;
  __syncthreads();
  if (w == 0) {
    V t = lane < kTileBlock / 64 ? s_wave[lane] : V(0);
#pragma unroll
    for (int o = 1; o < kTileBlock / 64; o <<= 1) {
      const V u = __shfl_up(t, o, 64);
      if (lane >= o) t += u;
    }
    if (lane < kTileBlock / 64) s_wave[lane] = t;
  }
  __syncthreads();
  if (w > 0) v += s_wave[w - 1];
  *total = s_wave[kTileBlock / 64 - 1];
  __syncthreads();  // s_wave is free again
  return v;
}

__global__ __launch_bounds__(kTileBlock) void aligned_tiles_kernel(const int* __restrict__ cu, int n_seqs, int T,
                                                                  int tile_steps, int cap, int* __restrict__ tiles) {
  __shared__ long long s_wave[kTileBlock / 64];  // 64-bit: tile counts of clamped offsets may be large
  __shared__ int s_max;
  int* order = tiles + 1;
  int* slot_seq = tiles + 1 + cap;
  int* slot_pos = tiles + 1 + 2 * cap;
  int* slot_start = tiles + 1 + 3 * cap;
  int* slot_end = tiles + 1 + 4 * cap;
  int* seq = tiles + 1 + 5 * cap;
  int* pos = tiles + 1 + 6 * cap;
  int* cnt = tiles + 1 + 7 * cap;  // histogram, then tiles per position, then next slot per position
  const int tid = threadIdx.x;
  for (int i = tid; i < cap; i += kTileBlock) cnt[i] = 0;
  if (tid == 0) s_max = 0;
  __syncthreads();
  // each sequence's tiles: ids first .. first + nt - 1 (cut at cap), positions 0 .. nt - 1
  int made = 0;  // ids handed out so far (uniform)
  for (int base = 0; base < n_seqs; base += kTileBlock) {
    const int s = base + tid;
    long long nt = 0;
    if (s < n_seqs) {
      const int a = min(max(cu[s], 0), T);
      const int e = min(max(cu[s + 1], a), T);
      nt = (e - a + tile_steps - 1) / tile_steps;
    }
    long long chunk = 0;
    const long long first = made + block_inclusive_sum(nt, s_wave, &chunk) - nt;
    const int kept = static_cast<int>(max(0LL, min(nt, cap - first)));
    for (int p = 0; p < kept; ++p) {
      seq[first + p] = s;
      pos[first + p] = p;
    }
    if (kept > 0) {
      atomicAdd(&cnt[kept - 1], 1);  // sequences with exactly `kept` tiles
      atomicMax(&s_max, kept);
    }
    made = static_cast<int>(min(made + chunk, static_cast<long long>(cap)));
  }
  __syncthreads();
  const int n = made;
  const int max_nt = s_max;
  // tiles at position p = sequences with more than p tiles: the histogram summed from the top
  long long carry = 0;
  for (int top = max_nt; top > 0; top -= kTileBlock) {
    const int i = top - 1 - tid;
    const long long v = i >= 0 ? cnt[i] : 0;
    long long chunk = 0;
    const long long incl = block_inclusive_sum(v, s_wave, &chunk);
    if (i >= 0) cnt[i] = static_cast<int>(carry + incl);
    carry += chunk;
  }
  __syncthreads();
  // the first slot of each position: exclusive prefix of the tiles per position
  carry = 0;
  for (int base = 0; base < max_nt; base += kTileBlock) {
    const int i = base + tid;
    const long long v = i < max_nt ? cnt[i] : 0;
    long long chunk = 0;
    const long long incl = block_inclusive_sum(v, s_wave, &chunk);
    if (i < max_nt) cnt[i] = static_cast<int>(carry + incl - v);
    carry += chunk;
  }
  __syncthreads();
  for (int id = tid; id < n; id += kTileBlock) {
    const int s = seq[id], p = pos[id];
    const int slot = atomicAdd(&cnt[p], 1);
    const int a = min(max(cu[s], 0), T);
    order[slot] = id;
    slot_seq[slot] = s;
    slot_pos[slot] = p;
    slot_start[slot] = a;
    slot_end[slot] = min(max(cu[s + 1], a), T);
  }
  if (tid == 0) tiles[0] = n;
}

size_t aligned_tile_ints(int cap) { return 1 + 8 * static_cast<size_t>(cap); }

hipError_t launch_aligned_tiles(const int* cu, int n_seqs, int T, int tile_steps, int cap, int* tiles,
                                hipStream_t stream) {
  aligned_tiles_kernel<<<1, kTileBlock, 0, stream>>>(cu, n_seqs, T, tile_steps, cap, tiles);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, i64 n_floats, hipStream_t stream) {
  const i64 n4 = n_floats / 4;
  zero_kernel<<<stream_grid(n4), kUpdBlock, 0, stream>>>(reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

}  // namespace slstm
