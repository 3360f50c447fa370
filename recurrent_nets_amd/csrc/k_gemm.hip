// Input projection P = x W_x^T + bias on the MFMA matrix cores (bfloat16 in, float32 out).
//
//   P[b, t, g, j] = sum_k x[b, t, k] W_x[g, j, k] + bias[g, j]    (gates g = z, i, f, o)
//
// ("sLSTM in this library", "API notes": W_x is applied as a GEMM; the gate pre-activations
// of the sLSTM step pseudocode in the xLSTM summary card, "Key equations".)
// As a matrix product: C (M x N) = X (M x K) * W^T with M = B*T, N = 4*d_h, K = d_in; both
// operands are K-contiguous, and C row-major is exactly P's (B, T, 4, d_h) layout.
//
// Workgroup tile 256 x 128 (rows of x by rows of W_x), 4 waves in a 2 x 2 arrangement, each wave
// a 128 x 64 sub-tile made of 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators (128 registers), so
// two workgroups share a compute unit and one's epilogue (the float32 P write, as large as the
// arithmetic) overlaps the other's main loop. K advances 32 at a time through a three-stage
// LDS ring (72 KiB) filled by direct global-to-LDS buffer loads: no staging registers and no LDS
// stores in the instruction stream, two stages in flight while one is multiplied, one barrier
// per step. LDS rows are 64 bytes (four 16-byte chunks of 8 bf16); chunk c of row r sits in
// slot c ^ ((r >> 1) & 3), which keeps every 8-lane group of a fragment read on distinct banks.
// Rows past M or N read zero (buffer loads against the tile's extent); a K tail is pointed
// outside the extent, which also reads zero. The bias is added in the epilogue, so P is written
// once. The same kernel serves the weight-gradient products of the backward pass, whose
// reduction length (B*T) is long and whose output is small: there the K range is split and each
// split writes its partial product to its own slice of C. Splits are numbered with the tiles,
// split-major, so each XCD's contiguous range of work covers one K range: the workgroups an XCD
// runs together read the same K slices of their row and column panels from its L2. Workgroups are renumbered so that each of the 8 XCDs works through a contiguous range of
// tiles, ordered in groups of row panels so that the tiles an XCD runs together share row and
// column panels in its L2.
#include "common.h"
#include "kernels.h"

namespace slstm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmBM = 256;
constexpr int kGemmBN = 128;
constexpr int kGemmBK = 32;
constexpr int kGemmStages = 3;
constexpr int kGemmThreads = 256;
constexpr int kGemmRowBytes = kGemmBK * 2;                               // 64
constexpr int kGemmStageBytes = (kGemmBM + kGemmBN) * kGemmRowBytes;     // 24 KiB
constexpr int kGemmBlocksA = kGemmBM * kGemmRowBytes / 1024;             // 1 KiB loads: 16 for x
constexpr int kGemmBlocks = kGemmStageBytes / 1024;                      // 24 per stage
constexpr int kGemmBlocksPerWave = kGemmBlocks / (kGemmThreads / kWave);  // 6
constexpr int kGemmGroupM = 4;
constexpr int kXcds = 8;
// a byte offset beyond every tile extent: buffer loads there return zero, stores are dropped
constexpr uint32_t kOutside = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ rsrc_t make_rsrc_bytes(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// slot of chunk c of row r in the swizzled LDS layout
__device__ __forceinline__ uint32_t gemm_slot(uint32_t r, uint32_t c) { return c ^ ((r >> 1) & 3u); }

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// one stage of the LDS ring: the x rows of the tile, then the W_x rows
struct GemmStage {
  unsigned char a[kGemmBM * kGemmRowBytes];
  unsigned char b[kGemmBN * kGemmRowBytes];
};

__global__ __launch_bounds__(kGemmThreads, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ W,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ C, int M, int N,
                                                                  int K, int tiles_m, int tiles_n,
                                                                  int k_split, i64 c_split) {
  // three separate objects, so that the compiler sees which stage a fragment read touches and
  // waits only for the loads into that stage
  __shared__ __attribute__((aligned(1024))) GemmStage st0;
  __shared__ __attribute__((aligned(1024))) GemmStage st1;
  __shared__ __attribute__((aligned(1024))) GemmStage st2;

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
  const int wm = wave >> 1;  // 0..1: 128-row half of the tile
  const int wn = wave & 1;   // 0..1: 64-column half

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

  // ---- global -> LDS: each wave fills 4 of the 16 x blocks and 2 of the 8 W_x blocks of a
  //      stage (a block: 16 rows x 64 B, one 1 KiB direct load). Lane l fills slot l & 3 of row
  //      l >> 2 of its block, i.e. fetches that row's chunk gemm_slot(row, slot) (the swizzle
  //      is an involution). ----
  const uint32_t lrow = static_cast<uint32_t>(lane) >> 2;
  const uint32_t lslot = static_cast<uint32_t>(lane) & 3u;
  auto load_block = [&](rsrc_t rs, unsigned char* dst_rows, int blk, int k0) {
    const uint32_t r = static_cast<uint32_t>(blk * 16) + lrow;
    const uint32_t c = gemm_slot(r, lslot);
    const int gk = k0 + static_cast<int>(c) * 8;
    const uint32_t off = gk < kl ? (r * static_cast<uint32_t>(K) + static_cast<uint32_t>(gk)) * 2u : kOutside;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst_rows + blk * 1024), 16, off, 0, 0, 0);
  };
  auto issue = [&](GemmStage& stg, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) load_block(rX, stg.a, wave * 4 + i, k0);
#pragma unroll
    for (int i = 0; i < 2; ++i) load_block(rW, stg.b, wave * 2 + i, k0);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.0f;

  // fragment addresses within a stage: lane l reads row (l & 31) of a 32-row strip, chunk
  // (kk / 8) + (l >> 5)
  const uint32_t frow = static_cast<uint32_t>(lane) & 31u;
  const uint32_t fhalf = static_cast<uint32_t>(lane) >> 5;
  auto multiply = [&](const GemmStage& stg) {
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 16) {
      const uint32_t c = static_cast<uint32_t>(kk / 8) + fhalf;
      bf16x8 a[4], bm[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t r = static_cast<uint32_t>(wm * 128 + i * 32) + frow;
        a[i] = *reinterpret_cast<const bf16x8*>(stg.a + r * kGemmRowBytes + (gemm_slot(r, c) << 4));
      }
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const uint32_t r = static_cast<uint32_t>(wn * 64 + jn * 32) + frow;
        bm[jn] = *reinterpret_cast<const bf16x8*>(stg.b + r * kGemmRowBytes + (gemm_slot(r, c) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bm[jn], acc[i][jn], 0, 0, 0);
    }
  };
  // step q: wait for this wave's loads into stage q (those of stage q+1 may still be in flight),
  // barrier (every wave's have landed; every wave is done with the stage of step q-1), refill
  // that stage with step q+2, multiply stage q
  const int nk = (kl + kGemmBK - 1) / kGemmBK;
  auto step = [&](int q, GemmStage& cur, GemmStage& refill) {
    if (q + 1 < nk)
      wait_vmcnt<kGemmBlocksPerWave>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (q + 2 < nk) issue(refill, (q + 2) * kGemmBK);
    multiply(cur);
  };
  issue(st0, 0);
  if (nk > 1) issue(st1, kGemmBK);
  int q = 0;
  for (; q + 3 <= nk; q += 3) {
    step(q, st0, st2);
    step(q + 1, st1, st0);
    step(q + 2, st2, st1);
  }
  if (q < nk) step(q, st0, st2);
  if (q + 1 < nk) step(q + 1, st1, st0);

  // ---- epilogue: bias, float32 store. Accumulator r of lane l holds row
  //      8*(r/4) + 4*(l/32) + r%4 and column l%32 of its 32 x 32 tile. Stores go through a
  //      buffer over the output tile: rows past M fall outside its extent and are dropped,
  //      columns past N are pointed outside it. ----
  const uint32_t c_bytes = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x_rows) * static_cast<uint32_t>(N) * 4u);
  const rsrc_t rC = make_rsrc_bytes(C + static_cast<i64>(split) * c_split + row0 * N + col0, c_bytes);
  const int n_in = N - static_cast<int>(col0);  // columns of this tile inside C
#pragma unroll
  for (int jn = 0; jn < 2; ++jn) {
    const int nl = wn * 64 + jn * 32 + static_cast<int>(frow);
    const bool col_ok = nl < n_in;
    const float bn = (bias != nullptr && col_ok) ? bias[col0 + nl] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = wm * 128 + i * 32 + (r >> 2) * 8 + static_cast<int>(fhalf) * 4 + (r & 3);
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
