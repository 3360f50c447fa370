// Input projection P = x W_x^T + bias on the MFMA matrix cores (bfloat16 in, float32 out).
//
//   P[b, t, g, j] = sum_k x[b, t, k] W_x[g, j, k] + bias[g, j]    (gates g = z, i, f, o)
//
// ("sLSTM in this library", "API notes": W_x is applied as a GEMM; the gate pre-activations
// of the sLSTM step pseudocode in the xLSTM summary card, "Key equations".)
// As a matrix product: C (M x N) = X (M x K) * W^T with M = B*T, N = 4*d_h, K = d_in; both
// operands are K-contiguous, and C row-major is exactly P's (B, T, 4, d_h) layout.
//
// Workgroup tile 256 x 256 (rows of x by rows of W_x), 8 waves in a 2 x 4 arrangement, each wave
// a 128 x 64 sub-tile made of 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators (128 registers); one
// workgroup per compute unit. K advances 64 at a time, so every operand row of a step is one
// whole 128-byte line, through two 64 KiB LDS stages filled by direct global-to-LDS buffer
// loads (no staging registers, no LDS stores in the instruction stream): the loads of step q+1
// are in flight while step q is multiplied. The barrier between steps orders LDS only (each
// wave first waits for its own loads into the stage and for its own LDS reads), so nothing
// else is drained there. Inside a step the fragment reads of the next 16-deep slice are
// interleaved one by one with the MFMAs of the current slice. LDS rows are 128 bytes (eight
// 16-byte chunks of 8 bf16); chunk c of row r sits in slot c ^ ((r >> 1) & 7), which keeps
// the 16 lanes the LDS serves together on distinct banks (rows r and r+1 fall in different
// halves of the 64 banks). Rows past M or N read zero (buffer loads against the tile's extent);
// a K tail is pointed outside the extent, which also reads zero. The bias is added in the
// epilogue, so P is written once. The same kernel serves the weight-gradient products of the
// backward pass, whose reduction length (B*T) is long and whose output is small: there the K
// range is split and each split writes its partial product to its own slice of C. Splits are
// numbered with the tiles, split-major, so each XCD's contiguous range of work covers one K
// range: the workgroups an XCD runs together read the same K slices of their row and column
// panels from its L2. Workgroups are renumbered so that each of the 8 XCDs works through a
// contiguous range of tiles, ordered in groups of row panels so that the tiles an XCD runs
// together share row and column panels in its L2.
#include "common.h"
#include "kernels.h"

namespace slstm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmWavesM = 2;
constexpr int kGemmWavesN = 4;
constexpr int kGemmThreads = kGemmWavesM * kGemmWavesN * kWave;          // 512
constexpr int kGemmTM = kGemmBM / kGemmWavesM;                           // 128 rows per wave
constexpr int kGemmTN = kGemmBN / kGemmWavesN;                           // 64 columns per wave
constexpr int kGemmFM = kGemmTM / 32;                                    // 4 MFMA tiles
constexpr int kGemmFN = kGemmTN / 32;                                    // 2 MFMA tiles
constexpr int kGemmSlices = kGemmBK / 16;                                // 16-deep K slices
constexpr int kGemmRowBytes = kGemmBK * 2;                               // 128
constexpr int kGemmChunks = kGemmRowBytes / 16;                          // 8
constexpr int kGemmRowsPerBlock = 1024 / kGemmRowBytes;                  // 8
constexpr int kGemmStageBytes = (kGemmBM + kGemmBN) * kGemmRowBytes;     // 64 KiB
constexpr int kGemmBlocksA = kGemmBM * kGemmRowBytes / 1024;             // 1 KiB loads: 32 for x
constexpr int kGemmBlocks = kGemmStageBytes / 1024;                      // 64 per stage
constexpr int kGemmBlocksPerWave = kGemmBlocks / (kGemmThreads / kWave);  // 8
constexpr int kGemmGroupM = 4;
constexpr int kXcds = 8;
static_assert(kGemmBlocksA % kGemmBlocksPerWave == 0, "every wave loads blocks of one operand");
// a byte offset beyond every tile extent: buffer loads there return zero, stores are dropped
constexpr uint32_t kOutside = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ rsrc_t make_rsrc_bytes(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// slot of chunk c of row r in the swizzled LDS layout
__device__ __forceinline__ uint32_t gemm_slot(uint32_t r, uint32_t c) { return c ^ ((r >> 1) & 7u); }

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier for the LDS ring: this wave's LDS reads have completed (lgkmcnt 0, the
// other counters left at their maxima), and the compiler keeps every memory access on its side
// of the barrier. Unlike __syncthreads it does not wait for outstanding global loads.
__device__ __forceinline__ void gemm_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ W,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ C, int M, int N,
                                                                  int K, int tiles_m, int tiles_n,
                                                                  int k_split, i64 c_split) {
  // two separate objects, so that the compiler sees which stage a fragment read touches
  __shared__ __attribute__((aligned(1024))) unsigned char st0[kGemmStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[kGemmStageBytes];

  // ---- tile selection: XCD-contiguous ranges, grouped row panels ----
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical_all = (nb % kXcds == 0) ? (bid % kXcds) * (nb / kXcds) + bid / kXcds : bid;
  const int n_tiles = tiles_m * tiles_n;
  const int split = logical_all / n_tiles;
  const int logical = logical_all - split * n_tiles;
  const int per_group = kGemmGroupM * tiles_n;
  const int group = logical / per_group;
  const int in_group = logical % per_group;
  const int gm0 = group * kGemmGroupM;
  const int gsize = min(kGemmGroupM, tiles_m - gm0);
  const int tm = gm0 + in_group % gsize;
  const int tn = in_group / gsize;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / kGemmWavesN;  // 0..1: 128-row half of the tile
  const int wn = wave % kGemmWavesN;  // 0..3: 64-column quarter

  const i64 row0 = static_cast<i64>(tm) * kGemmBM;
  const i64 col0 = static_cast<i64>(tn) * kGemmBN;
  // this split's range of K: [kb, kb + kl)
  const int kb = split * k_split;
  const int kl = min(k_split, K - kb);
  // extents of the operand tiles (uniform; integer selects keep them in scalar registers)
  const int x_rows = (M - row0 < kGemmBM) ? static_cast<int>(M - row0) : kGemmBM;
  const int w_rows = (N - col0 < kGemmBN) ? static_cast<int>(N - col0) : kGemmBN;
  const uint32_t x_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x_rows) * static_cast<uint32_t>(K) * 2u - static_cast<uint32_t>(kb) * 2u);
  const uint32_t w_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(w_rows) * static_cast<uint32_t>(K) * 2u - static_cast<uint32_t>(kb) * 2u);
  const rsrc_t rX = make_rsrc_bytes(X + row0 * K + kb, x_bytes);
  const rsrc_t rW = make_rsrc_bytes(W + col0 * K + kb, w_bytes);

  // ---- global -> LDS: each wave fills 8 of the 64 blocks of a stage (a block: 8 rows x 128 B,
  //      one 1 KiB direct load); waves 0-3 the x rows, waves 4-7 the W_x rows. Lane l fills slot
  //      l & 7 of row l >> 3 of its block, i.e. fetches that row's chunk gemm_slot(row, slot)
  //      (the swizzle is an involution). ----
  const bool wave_x = wave * kGemmBlocksPerWave < kGemmBlocksA;
  const rsrc_t rOp = wave_x ? rX : rW;
  const int blk0 = wave_x ? wave * kGemmBlocksPerWave : wave * kGemmBlocksPerWave - kGemmBlocksA;
  const uint32_t lrow = static_cast<uint32_t>(lane) >> 3;
  const uint32_t lslot = static_cast<uint32_t>(lane) & 7u;
  auto issue = [&](unsigned char* stg, int k0) {
    unsigned char* dst0 = stg + (wave_x ? 0 : kGemmBM * kGemmRowBytes);
#pragma unroll
    for (int i = 0; i < kGemmBlocksPerWave; ++i) {
      const int blk = blk0 + i;
      const uint32_t r = static_cast<uint32_t>(blk * kGemmRowsPerBlock) + lrow;
      const uint32_t c = gemm_slot(r, lslot);
      const int gk = k0 + static_cast<int>(c) * 8;
      const uint32_t off = gk < kl ? (r * static_cast<uint32_t>(K) + static_cast<uint32_t>(gk)) * 2u : kOutside;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rOp, (lds_ptr_t)(dst0 + blk * 1024), 16, off, 0, 0, 0);
    }
  };

  f32x16 acc[kGemmFM][kGemmFN];
#pragma unroll
  for (int i = 0; i < kGemmFM; ++i)
#pragma unroll
    for (int jn = 0; jn < kGemmFN; ++jn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;

  // fragment addresses within a stage: lane l reads row (l & 31) of a 32-row strip, chunk
  // 2 * slice + (l >> 5)
  const uint32_t frow = static_cast<uint32_t>(lane) & 31u;
  const uint32_t fhalf = static_cast<uint32_t>(lane) >> 5;
  auto load_frag = [&](const unsigned char* stg, int sl, bf16x8 (&a)[kGemmFM], bf16x8 (&bm)[kGemmFN]) {
    const uint32_t c = static_cast<uint32_t>(2 * sl) + fhalf;
#pragma unroll
    for (int i = 0; i < kGemmFM; ++i) {
      const uint32_t r = static_cast<uint32_t>(wm * kGemmTM + i * 32) + frow;
      a[i] = *reinterpret_cast<const bf16x8*>(stg + r * kGemmRowBytes + (gemm_slot(r, c) << 4));
    }
#pragma unroll
    for (int jn = 0; jn < kGemmFN; ++jn) {
      const uint32_t r = static_cast<uint32_t>(wn * kGemmTN + jn * 32) + frow;
      bm[jn] = *reinterpret_cast<const bf16x8*>(stg + kGemmBM * kGemmRowBytes + r * kGemmRowBytes +
                                                (gemm_slot(r, c) << 4));
    }
  };
  auto multiply = [&](const unsigned char* stg) {
    bf16x8 fa[kGemmSlices][kGemmFM], fb[kGemmSlices][kGemmFN];
    load_frag(stg, 0, fa[0], fb[0]);
#pragma unroll
    for (int sl = 0; sl < kGemmSlices; ++sl) {
      if (sl + 1 < kGemmSlices) load_frag(stg, sl + 1, fa[sl + 1], fb[sl + 1]);
#pragma unroll
      for (int i = 0; i < kGemmFM; ++i)
#pragma unroll
        for (int jn = 0; jn < kGemmFN; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][i], fb[sl][jn], acc[i][jn], 0, 0, 0);
    }
    // schedule: the first slice's reads, then per slice its MFMAs with the next slice's reads
    // placed one after each MFMA (mask 0x100: LDS reads, 0x008: MFMA)
    constexpr int kReads = kGemmFM + kGemmFN;
    constexpr int kMfmas = kGemmFM * kGemmFN;
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
    for (int sl = 0; sl < kGemmSlices; ++sl) {
      if (sl + 1 < kGemmSlices) {
#pragma unroll
        for (int e = 0; e < kReads; ++e) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kReads, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas, 0);
      }
    }
  };
  // step q: wait for this wave's loads into stage q, barrier (every wave's have landed; every
  // wave is done reading the other stage), refill the other stage with step q+1, multiply
  // stage q
  const int nk = (kl + kGemmBK - 1) / kGemmBK;
  auto step = [&](int q, unsigned char* cur, unsigned char* refill) {
    wait_vmcnt<0>();
    gemm_lds_barrier();
    if (q + 1 < nk) issue(refill, (q + 1) * kGemmBK);
    multiply(cur);
  };
  issue(st0, 0);
  int q = 0;
  for (; q + 2 <= nk; q += 2) {
    step(q, st0, st1);
    step(q + 1, st1, st0);
  }
  if (q < nk) step(q, st0, st1);

  // ---- epilogue: bias, float32 store. Accumulator r of lane l holds row
  //      8*(r/4) + 4*(l/32) + r%4 and column l%32 of its 32 x 32 tile. Stores go through a
  //      buffer over the output tile: rows past M fall outside its extent and are dropped,
  //      columns past N are pointed outside it. ----
  const uint32_t c_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x_rows) * static_cast<uint32_t>(N) * 4u);
  const rsrc_t rC = make_rsrc_bytes(C + static_cast<i64>(split) * c_split + row0 * N + col0, c_bytes);
  const int n_in = N - static_cast<int>(col0);  // columns of this tile inside C
#pragma unroll
  for (int jn = 0; jn < kGemmFN; ++jn) {
    const int nl = wn * kGemmTN + jn * 32 + static_cast<int>(frow);
    const bool col_ok = nl < n_in;
    const float bn = (bias != nullptr && col_ok) ? bias[col0 + nl] : 0.0f;
#pragma unroll
    for (int i = 0; i < kGemmFM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = wm * kGemmTM + i * 32 + (r >> 2) * 8 + static_cast<int>(fhalf) * 4 + (r & 3);
        const uint32_t off = col_ok ? static_cast<uint32_t>((ml * N + nl) * 4) : kOutside;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][jn][r] + bn), rC, off, 0, 0);
      }
    }
  }
}

int gemm_tiles(i64 M, int N) {
  return static_cast<int>(((M + kGemmBM - 1) / kGemmBM) * ((N + kGemmBN - 1) / kGemmBN));
}

hipError_t launch_gemm_bf16(const void* X, const void* W, const float* bias, float* C, i64 M,
                            int N, int K, hipStream_t stream, int splits) {
  const i64 tiles_m = (M + kGemmBM - 1) / kGemmBM;
  const i64 tiles_n = (N + kGemmBN - 1) / kGemmBN;
  const i64 blocks = tiles_m * tiles_n * splits;
  // operand and output tiles are addressed with 32-bit byte offsets below kOutside
  if (splits < 1 || blocks > 0x7fffffffLL || M > 0x7fffffffLL || static_cast<i64>(kGemmBM) * K * 2 >= kOutside ||
      static_cast<i64>(kGemmBM) * N * 4 >= kOutside)
    return hipErrorInvalidValue;
  // K range per split: a whole number of K steps; every split gets at least one
  const int k_split = ((K + splits - 1) / splits + kGemmBK - 1) / kGemmBK * kGemmBK;
  const int used = (K + k_split - 1) / k_split;
  if (used != splits) return hipErrorInvalidValue;
  gemm_bf16_kernel<<<dim3(static_cast<unsigned>(blocks)), kGemmThreads, 0, stream>>>(
      static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), bias, C, static_cast<int>(M),
      N, K, static_cast<int>(tiles_m), static_cast<int>(tiles_n), k_split, M * static_cast<i64>(N));
  return hipGetLastError();
}

int gemm_splits_for(i64 M, int N, int K, int want) {
  // the number of splits launch_gemm_bf16 accepts closest to want (each split a whole number of
  // K steps, none empty)
  int s = want < 1 ? 1 : want;
  while (s > 1) {
    const int k_split = ((K + s - 1) / s + kGemmBK - 1) / kGemmBK * kGemmBK;
    if ((K + k_split - 1) / k_split == s) break;
    --s;
  }
  (void)M;
  (void)N;
  return s;
}

}  // namespace slstm
