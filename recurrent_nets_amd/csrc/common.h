// Shared device helpers for the sLSTM Newton kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slstm {

constexpr int kWave = 64;

// 64-bit element offsets: the Jacobian tensor of a large layer exceeds 2^32 floats.
typedef long long i64;

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (add half an ulp of the kept part, less
// one unless the kept part is odd, then truncate); NaN stays a quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Load one gate pre-activation, stored as float32 or bfloat16.
template <bool BF16>
__device__ __forceinline__ float load_p(const void* __restrict__ P, i64 idx) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(P)[idx]);
  } else {
    return static_cast<const float*>(P)[idx];
  }
}

// Cell mode of the kernels: bit 0 the sigmoid forget gate (else exponential), bit 1 the floored
// read-out h = o c / max(|n|, e^{-m}, 1e-6) (else h = o c / n).
constexpr int kCellSigmoid = 1;
constexpr int kCellFloored = 2;

// ---- packed sequences -------------------------------------------------------------------------
// With packed sequences ("sLSTM in this library", "Packed sequences") the single batch row holds
// n_seqs sequences one after the other along T, sequence s on steps cu[s] .. cu[s+1]-1 (cu: the
// n_seqs + 1 exclusive prefix offsets), each started from its own state0[s]. Without them
// (cu == nullptr) batch row b is sequence b and starts at t = 0. A cursor walks the steps of a
// run in increasing order and names the sequence, if any, that starts at each. Every read of cu
// stays within its n_seqs + 1 entries whatever they hold.
// packed-sequence offsets as the launchers take them (cu == nullptr: one sequence per row)
struct Seqs {
  const int* cu = nullptr;
  int n = 0;
  const int* tab = nullptr;  // optional: seq_table entries (see build_seq_table)
  // optional: tiles aligned to the sequences (see launch_aligned_tiles), for the scan-form
  // iteration: tiles[0] the number of tiles, then the order they are handed out in, each
  // tile's sequence and each tile's position in it (tile_cap entries each)
  const int* tiles = nullptr;
  int tile_cap = 0;
};

// seq_table: entry k holds the sequence containing step k << kSeqTabShift, i.e. the s with
// cu[s] <= 4k < cu[s+1] (the largest s with cu[s] <= 4k); ceil(T / 4) entries
constexpr int kSeqTabShift = 2;
// look-back anchor stride of the packed scan kernels
#ifndef SLSTM_PACKED_ANCHOR_STRIDE
#define SLSTM_PACKED_ANCHOR_STRIDE 2
#endif
constexpr int kPackedAnchorStride = SLSTM_PACKED_ANCHOR_STRIDE;

struct SeqCursor {
  const int* cu;
  int n_seqs;
  int s;      // the sequence holding the current step
  int start;  // its first step
  int end;    // one past its last step
};

// cursor at step t (t >= 0): the last sequence whose first step is <= t. With a sequence table
// one load finds the sequence at the table step at or before t, then the cursor walks forward;
// without one, a binary search over the offsets. Table entries are clamped into [0, n_seqs), so
// every access stays in bounds whatever the offsets hold.
__device__ __forceinline__ SeqCursor seq_cursor(const int* cu, int n_seqs, int b, int t,
                                                const int* tab = nullptr) {
  if (cu == nullptr) return {nullptr, 0, b, 0, 0x7fffffff};
  int lo;
  if (tab != nullptr) {
    lo = min(max(tab[t >> kSeqTabShift], 0), n_seqs - 1);
    while (lo + 1 < n_seqs && cu[lo + 1] <= t) ++lo;
  } else {
    lo = 0;
    int hi = n_seqs - 1;  // largest s in [0, n_seqs) with cu[s] <= t (0 if none)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
  }
  return {cu, n_seqs, lo, cu[lo], cu[lo + 1]};
}

// The sequence that starts at step t, or -1. Steps must be visited one by one in increasing
// order (t = the cursor's step, then +1, ...).
__device__ __forceinline__ int seq_begin(SeqCursor& c, int t) {
  if (c.cu == nullptr) return t == 0 ? c.s : -1;
  while (t >= c.end && c.s + 1 < c.n_seqs) {
    ++c.s;
    c.start = c.cu[c.s];
    c.end = c.cu[c.s + 1];
  }
  return (t == c.start && t < c.end) ? c.s : -1;
}

// ---- buffer resources -------------------------------------------------------------------------
// A buffer resource holds a wave-uniform base address in scalar registers; each access adds a
// 32-bit per-lane byte offset (one VGPR) and a wave-uniform byte offset (an SGPR). Kernels that
// issue many loads from rows at uniform strides keep one VGPR per stream instead of a 64-bit
// address per load. The third descriptor word is the raw-buffer setting of the gfx9 family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), -1,
                                           0x00020000);
}
__device__ __forceinline__ float buf_ld(rsrc_t r, unsigned voff_bytes, unsigned soff_bytes) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff_bytes, soff_bytes, 0));
}
__device__ __forceinline__ void buf_st(float v, rsrc_t r, unsigned voff_bytes, unsigned soff_bytes) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff_bytes, soff_bytes, 0);
}
// gate pre-activation at element offsets (lane part, uniform part) of a float32 or bf16 tensor
template <bool BF16>
__device__ __forceinline__ float buf_ld_p(rsrc_t r, unsigned voff_elems, unsigned soff_elems) {
  if constexpr (BF16) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, 2u * voff_elems, 2u * soff_elems, 0));
  } else {
    return buf_ld(r, 4u * voff_elems, 4u * soff_elems);
  }
}

// |x| for the residual maximum; NaN counts as +inf so that a max reduction cannot drop it.
__device__ __forceinline__ float abs_nan_inf(float x) {
  float a = fabsf(x);
  return (a == a) ? a : __int_as_float(0x7f800000);
}

// Running maximum of |x| over float32 values with NaN counted as +inf, kept on the bit
// patterns of |x| as unsigned integers: they order like the magnitudes, and every NaN pattern
// (exponent all ones, mantissa non-zero) lies above +inf, so a single integer max per value
// keeps the NaN; res_max_value maps the result to a float once.
__device__ __forceinline__ unsigned int res_max(unsigned int acc, float x) {
  return max(acc, __float_as_uint(x) & 0x7fffffffu);
}
// The same maximum for a kernel that folds many values in: a float running maximum of |x| with
// the NaN-propagating maximum (IEEE 754-2019 maximum, one v_maximum3_f32 per two values, the
// absolute values as operand modifiers). Its bit pattern is then that of the largest |x|, or of
// a quiet NaN, which lies above +inf like the patterns res_max keeps.
struct ResMax2 {
  float v = 0.0f;
};
__device__ __forceinline__ void res_max2(ResMax2& acc, float a, float b) {
  acc.v = __builtin_elementwise_maximum(__builtin_elementwise_maximum(acc.v, fabsf(a)), fabsf(b));
}
__device__ __forceinline__ unsigned int res_max2_bits(const ResMax2& acc) { return __float_as_uint(acc.v); }
__device__ __forceinline__ float res_max_value(unsigned int acc) {
  return acc > 0x7f800000u ? __int_as_float(0x7f800000) : __uint_as_float(acc);
}
__device__ __forceinline__ unsigned int wave_max_u32(unsigned int v) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<unsigned int>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}

// Device-wide running maximum of non-negative floats (bit patterns order like the values).
__device__ __forceinline__ void atomic_max_nonneg(unsigned int* dst, float v) {
  atomicMax(dst, __float_as_uint(v));
}

// ---- DPP quad permutations (lanes grouped in fours) ---------------------------------------
// quad_perm selector: lane k of each quad reads lane sel[k] of the same quad.
template <int S0, int S1, int S2, int S3>
__device__ __forceinline__ float quad_perm(float v) {
  constexpr int ctrl = S0 | (S1 << 2) | (S2 << 4) | (S3 << 6);
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), ctrl,
                                                    0xf, 0xf, false));
}

// ---- wave / block maximum --------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ---- epoch-tagged words for the decoupled look-back -------------------------------------------
// Each published float travels in a 64-bit word whose high half is the launch's epoch. A reader
// accepts a word only when its tag matches, so every word validates itself: no flag-after-data
// ordering is needed, and stale words from earlier launches are never mistaken for new ones.
__device__ __forceinline__ void tag_store(unsigned long long* p, float v, uint32_t epoch) {
  unsigned long long w = (static_cast<unsigned long long>(epoch) << 32) | __float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool tag_load(const unsigned long long* p, uint32_t epoch, float& v) {
  unsigned long long w = __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
  v = __uint_as_float(static_cast<uint32_t>(w));
  return static_cast<uint32_t>(w >> 32) == epoch;
}

// Pause between two polls of a look-back word (s_sleep units of 64 cycles)
#ifndef SLSTM_POLL_SLEEP
#define SLSTM_POLL_SLEEP 2
#endif
__device__ __forceinline__ void poll_pause() { __builtin_amdgcn_s_sleep(SLSTM_POLL_SLEEP); }

// Anchor stride of the look-back along T: tiles of one lane group are n_lg work tickets
// apart, so when the lane groups outnumber the workgroups resident on the GPU a predecessor
// has finished before its successor starts and a plain chain (stride 1) never waits. With few
// lane groups several tiles of a chain run at once, and every stride-th tile anchors the
// chain, so a tile waits on at most one anchor and on aggregates published before any wait.
// A function of the shape, the kernel's residency (workgroups per compute unit) and the device
// alone, so results stay reproducible.
int look_back_anchor_stride(long long n_lane_groups, int wgs_per_cu);

// ---- spread counters ----------------------------------------------------------------------------
// Device-scope atomics on one address serialise (about 10 ns apiece on MI355X), so a launch of
// 2^18 workgroups that all touch one word spends milliseconds there. Work tickets and residual
// maxima are therefore spread over kSpreadSlots words in separate cache lines.
constexpr int kSpreadSlots = 64;   // one per lane of a wave: a reduction is a single wave load
constexpr int kErrSlotWords = 128; // per slot one word per Newton iteration (slots 512 B apart)
constexpr int kTicketWords = 64;   // ticket counters 256 B apart
enum { kTicketWarm = 0, kTicketTiles = 1 };

// Solver control block kept at the start of the workspace, followed by its Spread block.
struct Control {
  unsigned int err_bits[72];  // max|F| after k updates (float bits; NaN stored as +inf),
                              // reduced from the slots when the solve is finalised
  int iters;                  // Newton updates applied
  int stopped;                // early stop taken
  int converged;
  int diverged;
  int nonfinite;
  int pad[51];
};
static_assert(sizeof(Control) == 512, "control block layout");

struct Spread {
  unsigned int err[kSpreadSlots][kErrSlotWords];             // residual maxima per slot
  unsigned int ticket[2][kSpreadSlots][kTicketWords];        // work counters (self-resetting)
};
constexpr size_t kControlBytes = sizeof(Control) + sizeof(Spread);

__host__ __device__ inline Spread* spread_of(Control* c) {
  return reinterpret_cast<Spread*>(reinterpret_cast<char*>(c) + sizeof(Control));
}
__host__ __device__ inline const Spread* spread_of(const Control* c) {
  return reinterpret_cast<const Spread*>(reinterpret_cast<const char*>(c) + sizeof(Control));
}

// Residual maximum of iteration k over all slots. Every lane of the wave must take part; the
// result is wave-uniform.
__device__ __forceinline__ float err_reduced(const Control* c, int k) {
  const unsigned int w = spread_of(c)->err[threadIdx.x & (kSpreadSlots - 1)][k];
  return wave_max(__uint_as_float(w));
}

// Publish a (non-negative) residual maximum: into word err_base[slot * stride], slot chosen
// by the caller. stride 0 folds every slot into the one word err_base.
__device__ __forceinline__ void err_publish(unsigned int* err_base, int stride, unsigned int slot,
                                            float v) {
  atomic_max_nonneg(err_base + static_cast<i64>(slot % kSpreadSlots) * stride, v);
}

// Work tickets (thread 0 of a workgroup). Tiles are numbered (tt, lg): lane group lg of tile
// row tt. Lane group lg draws from counter lg % n_ctr, which hands its tiles out in order of
// tt; workgroup b draws from counter b % n_ctr. n_ctr divides n_lg, so each counter serves as
// many workgroups as it has tiles, and a tile's predecessors along T (same lane group, smaller
// tt) hold smaller tickets of the same counter: they have been taken by running workgroups, so
// the look-back's waits always end, whatever order the hardware dispatches workgroups in.
// The last ticket of a counter resets it for the next launch.
__device__ __forceinline__ void take_ticket(unsigned int* counters, int n_ctr, int n_lg, int n_tt,
                                            int& tt, int& lg) {
  const int c = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_ctr));
  const int per = n_lg / n_ctr;  // lane groups per counter
  unsigned int* ctr = counters + c * kTicketWords;
  const unsigned int tk = atomicAdd(ctr, 1u);
  if (tk == static_cast<unsigned int>(per) * n_tt - 1) atomicExch(ctr, 0u);
  tt = static_cast<int>(tk / per);
  lg = c + n_ctr * static_cast<int>(tk % per);
}

// number of ticket counters for n_lg lane groups: the largest power of two <= kSpreadSlots
// that divides n_lg
inline int ticket_counters(long long n_lg) {
  int c = kSpreadSlots;
  while (c > 1 && n_lg % c != 0) c >>= 1;
  return c;
}

}  // namespace slstm
