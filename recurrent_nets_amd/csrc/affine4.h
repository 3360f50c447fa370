// 4x4 affine maps x -> A x + v and the tile look-back shared by the scan kernels.
//
// Maps compose as (A2, v2) o (A1, v1) = (A2 A1, A2 v1 + v2) (the (J, r) monoid of the
// associative scan, "sLSTM in this library", "Packed sequences"; scan_block4 layout of the
// "Layout" page, "Naming"). Matrices are row-major float[16].
#pragma once
#include "common.h"

namespace slstm {

// the 12 entries of the sLSTM Jacobian that are not structural zeros, as row-major positions
__device__ constexpr int kSpPlane[12] = {0, 2, 3, 5, 6, 7, 10, 11, 12, 13, 14, 15};

// y = X v + w
__device__ __forceinline__ void mat4_vec(const float X[16], const float v[4], const float w[4],
                                         float y[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    y[i] = fmaf(X[4 * i + 0], v[0], fmaf(X[4 * i + 1], v[1], fmaf(X[4 * i + 2], v[2], fmaf(X[4 * i + 3], v[3], w[i]))));
}

// Y <- A Y with A given by its 12 non-structural entries (order of kSpPlane); in place,
// column by column (column k of A Y needs only column k of Y)
__device__ __forceinline__ void sp_mul_left(const float a[12], float Y[16]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float y0 = Y[k], y1 = Y[4 + k], y2 = Y[8 + k], y3 = Y[12 + k];
    Y[k] = fmaf(a[0], y0, fmaf(a[1], y2, a[2] * y3));
    Y[4 + k] = fmaf(a[3], y1, fmaf(a[4], y2, a[5] * y3));
    Y[8 + k] = fmaf(a[6], y2, a[7] * y3);
    Y[12 + k] = fmaf(a[8], y0, fmaf(a[9], y1, fmaf(a[10], y2, a[11] * y3)));
  }
}

// Y <- X Y for a dense X; in place, column by column
__device__ __forceinline__ void mat4_mul_left(const float X[16], float Y[16]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float y0 = Y[k], y1 = Y[4 + k], y2 = Y[8 + k], y3 = Y[12 + k];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Y[4 * i + k] = fmaf(X[4 * i], y0, fmaf(X[4 * i + 1], y1, fmaf(X[4 * i + 2], y2, X[4 * i + 3] * y3)));
  }
}

// y = A v + w, A sparse
__device__ __forceinline__ void sp_vec(const float a[12], const float v[4], const float w[4],
                                       float y[4]) {
  y[0] = fmaf(a[0], v[0], fmaf(a[1], v[2], fmaf(a[2], v[3], w[0])));
  y[1] = fmaf(a[3], v[1], fmaf(a[4], v[2], fmaf(a[5], v[3], w[1])));
  y[2] = fmaf(a[6], v[2], fmaf(a[7], v[3], w[2]));
  y[3] = fmaf(a[8], v[0], fmaf(a[9], v[1], fmaf(a[10], v[2], fmaf(a[11], v[3], w[3]))));
}

// (M, v) <- (M, v) o (Mp, vp): apply (Mp, vp) first, then (M, v). In place, row by row: the
// new v needs the old M, and row i of the new M needs only row i of the old M.
__device__ __forceinline__ void compose_after(float M[16], float v[4], const float Mp[16],
                                              const float vp[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = fmaf(M[4 * i], vp[0], fmaf(M[4 * i + 1], vp[1], fmaf(M[4 * i + 2], vp[2], fmaf(M[4 * i + 3], vp[3], v[i]))));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float row[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      row[k] = fmaf(M[4 * i], Mp[k], fmaf(M[4 * i + 1], Mp[4 + k], fmaf(M[4 * i + 2], Mp[8 + k], M[4 * i + 3] * Mp[12 + k])));
#pragma unroll
    for (int k = 0; k < 4; ++k) M[4 * i + k] = row[k];
  }
}

template <int S0, int S1, int S2, int S3>
__device__ __forceinline__ void quad_perm_map(const float M[16], const float v[4], float Mp[16],
                                              float vp[4]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) Mp[e] = quad_perm<S0, S1, S2, S3>(M[e]);
#pragma unroll
  for (int e = 0; e < 4; ++e) vp[e] = quad_perm<S0, S1, S2, S3>(v[e]);
}

// Inclusive scan of the four sub-chunk maps held by the lanes of each quad (DPP): afterwards
// lane sc of a quad holds sub-chunks 0..sc composed. Every lane of the wave must take part.
__device__ __forceinline__ void quad_inclusive_scan(float M[16], float v[4], int sc) {
  float Mp[16], vp[4];
  quad_perm_map<0, 0, 1, 2>(M, v, Mp, vp);  // from sub-chunk sc - 1
  if (sc >= 1) compose_after(M, v, Mp, vp);
  quad_perm_map<0, 1, 0, 1>(M, v, Mp, vp);  // from sub-chunk sc - 2
  if (sc >= 2) compose_after(M, v, Mp, vp);
}

constexpr int kLookBackWords = 24;  // per lane and tile: x_end (4), M (16), v (4)

// Broadcast lane K of each quad to the whole quad.
template <int K>
__device__ __forceinline__ float quad_bcast(float x) {
  return quad_perm<K, K, K, K>(x);
}

// Row q (the lane's position in its quad) of the map held by lane 3 of the quad; every lane of
// the wave must take part.
__device__ __forceinline__ void quad_row_of_last(const float M[16], const float v[4], int q,
                                                 float row[4], float& vq) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = quad_bcast<3>(M[k]), x1 = quad_bcast<3>(M[4 + k]);
    const float x2 = quad_bcast<3>(M[8 + k]), x3 = quad_bcast<3>(M[12 + k]);
    row[k] = q == 0 ? x0 : (q == 1 ? x1 : (q == 2 ? x2 : x3));
  }
  const float y0 = quad_bcast<3>(v[0]), y1 = quad_bcast<3>(v[1]);
  const float y2 = quad_bcast<3>(v[2]), y3 = quad_bcast<3>(v[3]);
  vq = q == 0 ? y0 : (q == 1 ? y1 : (q == 2 ? y2 : y3));
}

// Look-back along T for one lane of a tile, spread over the four threads of a quad: thread q
// holds row q of the tile's composed map (arow = M[q][0..3], av = v[q]) and publishes, loads and
// folds only the words of row q; the rows it needs from the other threads of its quad arrive by
// DPP. Returns in carry, in every thread of the quad, the value entering the tile (x before the
// tile's first step; zero before the first tile). Every lane of the wave must take part (the
// quad broadcasts run after the waits).
//
// Fixed dataflow, so results do not depend on scheduling: tiles whose index is a multiple of
// the anchor stride publish their inclusive value x_end = M carry + v; the others publish their
// aggregate (M, v) before waiting. A tile folds its predecessors' aggregates down to the nearest
// anchor, always in the same order, and applies the anchor's inclusive value. Words are
// epoch-tagged (see tag_store); the word w of tile t for lane L sits at
// desc[(t * kLookBackWords + w) * n_lanes_pad + L]: w = 0..3 the inclusive value, 4 + 4 i + k
// the entry (i, k) of M, 20 + i the entry i of v.
// With CUT (packed sequences only: the test costs the unpacked kernels' schedule), maps that
// are exactly zero in every lane of the wave (a packed sequence starts inside them)
// make everything before them irrelevant: the fold stops there and the anchor's value is not
// waited for, and an anchor whose own maps are zero publishes its inclusive value (its v)
// before its look-back, so a chain of anchors breaks at every sequence start. For finite values
// the result is the one the full fold gives (0 * x = 0); a non-finite value is not carried
// across such a map.
//   pf_word: this thread's word of the anchor's inclusive value, loaded ahead of time
//            (quad_look_back_prefetch); it costs no wait when it already carries the epoch.
__device__ __forceinline__ unsigned long long quad_look_back_prefetch(
    const unsigned long long* __restrict__ desc, i64 n_lanes_pad, i64 my_lane, int q, int tt,
    int anchor_stride) {
  if (tt == 0) return 0ull;
  const int a = ((tt - 1) / anchor_stride) * anchor_stride;
  return __hip_atomic_load(const_cast<unsigned long long*>(desc) + (static_cast<i64>(a) * kLookBackWords + q) * n_lanes_pad + my_lane,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool CUT = false>
__device__ __forceinline__ void quad_look_back(const float arow[4], float av, float carry[4],
                                               unsigned long long* __restrict__ desc,
                                               i64 n_lanes_pad, i64 my_lane, int q, int tt,
                                               int anchor_stride, uint32_t epoch,
                                               unsigned long long pf_word) {
  auto word = [&](int tile, int w) {
    return desc + (static_cast<i64>(tile) * kLookBackWords + w) * n_lanes_pad + my_lane;
  };
  // whether the maps of every lane of the wave are exactly zero (each thread holds one row of
  // its lane's map): a wave-uniform answer, so the branches on it stay scalar
  auto wave_zero = [&](const float r[4]) {
    const bool z = r[0] == 0.0f && r[1] == 0.0f && r[2] == 0.0f && r[3] == 0.0f;
    return __builtin_amdgcn_ballot_w64(z) == __builtin_amdgcn_read_exec();
  };
  const bool anchor = (tt % anchor_stride) == 0;
  const bool own_zero = CUT && wave_zero(arow);
  if (!anchor) {
#pragma unroll
    for (int k = 0; k < 4; ++k) tag_store(word(tt, 4 + 4 * q + k), arow[k], epoch);
    tag_store(word(tt, 20 + q), av, epoch);
  } else if (own_zero) {
    tag_store(word(tt, q), av, epoch);  // the inclusive value does not depend on the carry
  }
  float cq = 0.0f;  // carry[q]
  if (tt > 0) {
    const int a = ((tt - 1) / anchor_stride) * anchor_stride;  // nearest anchor below
    // row q of the accumulated map of the tiles a+1 .. tt-1
    float mrow[4], vacc = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) mrow[k] = (k == q) ? 1.0f : 0.0f;
    bool cut = false;  // the accumulated map is zero: tiles further back cannot change the carry
    for (int p = tt - 1; p > a; --p) {
      if (CUT && wave_zero(mrow)) {
        cut = true;
        break;
      }
      float prow[4], pv;
      while (true) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < 4; ++k) ok &= tag_load(word(p, 4 + 4 * q + k), epoch, prow[k]);
        ok &= tag_load(word(p, 20 + q), epoch, pv);
        if (ok) break;
        poll_pause();
      }
      // (Macc, vacc) <- (Macc, vacc) o (Mp, vp), row q: sum_k Macc[q][k] (Mp[k][.], vp[k])
      float nrow[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      float nv = vacc;
      auto fold = [&](float mk, float r0, float r1, float r2, float r3, float vk) {
        nrow[0] = fmaf(mk, r0, nrow[0]);
        nrow[1] = fmaf(mk, r1, nrow[1]);
        nrow[2] = fmaf(mk, r2, nrow[2]);
        nrow[3] = fmaf(mk, r3, nrow[3]);
        nv = fmaf(mk, vk, nv);
      };
      fold(mrow[0], quad_bcast<0>(prow[0]), quad_bcast<0>(prow[1]), quad_bcast<0>(prow[2]), quad_bcast<0>(prow[3]), quad_bcast<0>(pv));
      fold(mrow[1], quad_bcast<1>(prow[0]), quad_bcast<1>(prow[1]), quad_bcast<1>(prow[2]), quad_bcast<1>(prow[3]), quad_bcast<1>(pv));
      fold(mrow[2], quad_bcast<2>(prow[0]), quad_bcast<2>(prow[1]), quad_bcast<2>(prow[2]), quad_bcast<2>(prow[3]), quad_bcast<2>(pv));
      fold(mrow[3], quad_bcast<3>(prow[0]), quad_bcast<3>(prow[1]), quad_bcast<3>(prow[2]), quad_bcast<3>(prow[3]), quad_bcast<3>(pv));
#pragma unroll
      for (int k = 0; k < 4; ++k) mrow[k] = nrow[k];
      vacc = nv;
    }
    cut = cut || (CUT && wave_zero(mrow));
    if (cut) {
      cq = vacc;
    } else {
      // the anchor's inclusive value, element q
      float xq = __uint_as_float(static_cast<uint32_t>(pf_word));
      bool ok = static_cast<uint32_t>(pf_word >> 32) == epoch;
      while (!ok) {
        ok = tag_load(word(a, q), epoch, xq);
        if (ok) break;
        poll_pause();
      }
      cq = fmaf(mrow[0], quad_bcast<0>(xq), fmaf(mrow[1], quad_bcast<1>(xq), fmaf(mrow[2], quad_bcast<2>(xq), fmaf(mrow[3], quad_bcast<3>(xq), vacc))));
    }
  }
  carry[0] = quad_bcast<0>(cq);
  carry[1] = quad_bcast<1>(cq);
  carry[2] = quad_bcast<2>(cq);
  carry[3] = quad_bcast<3>(cq);
  if (anchor && !own_zero) {
    const float xe = fmaf(arow[0], carry[0], fmaf(arow[1], carry[1], fmaf(arow[2], carry[2], fmaf(arow[3], carry[3], av))));
    tag_store(word(tt, q), xe, epoch);
  }
}

// ---- tiles of 4 data waves and a coordinating wave ------------------------------------------
// Wave-major scan tiles: wave w (w = 0..3) of a workgroup holds sub-chunk w (consecutive steps)
// of the tile's features, one or two per thread, so every access of a wave covers whole
// 256- or 512-byte rows; a fifth wave, which holds no data, does the look-back across tiles.
constexpr int kRowsDataWaves = 4;
constexpr int kRowsBlock = (kRowsDataWaves + 1) * kWave;  // 320

// VEC consecutive floats at a byte offset (one 4- or 8-byte buffer access)
template <int VEC>
__device__ __forceinline__ void buf_ld_vec(rsrc_t r, unsigned voff, unsigned soff, float (&out)[VEC]) {
  if constexpr (VEC == 1) {
    out[0] = buf_ld(r, voff, soff);
  } else {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    out[0] = __uint_as_float(static_cast<uint32_t>(w[0]));
    out[1] = __uint_as_float(static_cast<uint32_t>(w[1]));
  }
}
template <int VEC>
__device__ __forceinline__ void buf_st_vec(const float (&v)[VEC], rsrc_t r, unsigned voff, unsigned soff) {
  if constexpr (VEC == 1) {
    buf_st(v[0], r, voff, soff);
  } else {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 w;
    w[0] = __float_as_uint(v[0]);
    w[1] = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, 0);
  }
}

// The coordinating wave of a scan tile, lane l = features VEC l .. VEC l + VEC - 1 of the
// tile: between the two workgroup barriers of the data waves it publishes the tile's aggregate
// (non-anchor tiles), looks back across tiles for the value entering the tile and writes the
// value entering each sub-chunk to s_x. Look-back words: word w of tile t for feature lane L at
// desc[(t * kLookBackWords + w) * n_lanes_pad + L]; w = 0..3 the tile's inclusive value
// (anchors), 4 + 4 i + k the entry (i, k) of its aggregate map, 20 + i the entry i of its offset.
template <int VEC>
__device__ __forceinline__ void scan_coordinate(float (&s_map)[4][20][VEC * kWave], float (&s_x)[4][4][VEC * kWave],
                                                unsigned long long* __restrict__ desc, i64 n_lanes_pad,
                                                i64 lane0, int tt, int anchor_stride, uint32_t epoch,
                                                int l) {
  auto word = [&](int tile, int w, int f) {
    return desc + (static_cast<i64>(tile) * kLookBackWords + w) * n_lanes_pad + lane0 + f;
  };
  const int anchor_a = tt > 0 ? ((tt - 1) / anchor_stride) * anchor_stride : 0;
  const bool anchor = (tt % anchor_stride) == 0;
  // the anchor's inclusive value, loaded now so that it arrives while the data waves load
  unsigned long long pf[VEC][4];
#pragma unroll
  for (int f = 0; f < VEC; ++f)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pf[f][e] = tt > 0 ? __hip_atomic_load(word(anchor_a, e, f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
  __syncthreads();  // the data waves' maps are in LDS
#pragma unroll
  for (int f = 0; f < VEC; ++f) {
    const int lf = VEC * l + f;  // the feature's column in LDS
    auto load_map = [&](int w, float (&Mw)[16], float (&vw)[4]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) Mw[e] = s_map[w][e][lf];
#pragma unroll
      for (int e = 0; e < 4; ++e) vw[e] = s_map[w][16 + e][lf];
    };
    if (!anchor) {
      // the tile's aggregate: sub-chunk maps 3 o 2 o 1 o 0, published before any wait
      float G[16], gv[4];
      load_map(0, G, gv);
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        float Mw[16], vw[4];
        load_map(w, Mw, vw);
        compose_after(Mw, vw, G, gv);  // (Mw, vw) <- (Mw, vw) o (G, gv)
#pragma unroll
        for (int e = 0; e < 16; ++e) G[e] = Mw[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[e] = vw[e];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) tag_store(word(tt, 4 + e, f), G[e], epoch);
#pragma unroll
      for (int e = 0; e < 4; ++e) tag_store(word(tt, 20 + e, f), gv[e], epoch);
    }
  }
#pragma unroll
  for (int f = 0; f < VEC; ++f) {
    const int lf = VEC * l + f;
    float xs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (tt > 0) {
      // accumulated map of the tiles anchor_a+1 .. tt-1, folded from the nearest one back
      float Macc[16], vacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < 16; ++e) Macc[e] = (e % 5 == 0) ? 1.0f : 0.0f;
      for (int p = tt - 1; p > anchor_a; --p) {
        float Mp[16], vp[4];
        while (true) {
          bool ok = true;
#pragma unroll
          for (int e = 0; e < 16; ++e) ok &= tag_load(word(p, 4 + e, f), epoch, Mp[e]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ok &= tag_load(word(p, 20 + e, f), epoch, vp[e]);
          if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
          poll_pause();
        }
        compose_after(Macc, vacc, Mp, vp);  // (Macc, vacc) <- (Macc, vacc) o (Mp, vp)
      }
      float xa[4];
      bool ok = true;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = __uint_as_float(static_cast<uint32_t>(pf[f][e]));
        ok &= static_cast<uint32_t>(pf[f][e] >> 32) == epoch;
      }
      while (__builtin_amdgcn_ballot_w64(!ok) != 0) {
        poll_pause();
        ok = true;
#pragma unroll
        for (int e = 0; e < 4; ++e) ok &= tag_load(word(anchor_a, e, f), epoch, xa[e]);
      }
      mat4_vec(Macc, xa, vacc, xs);
    }
    // start values of the sub-chunks, then the tile's inclusive value
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_x[w][e][lf] = xs[e];
      float Mw[16], vw[4], xn[4];
#pragma unroll
      for (int e = 0; e < 16; ++e) Mw[e] = s_map[w][e][lf];
#pragma unroll
      for (int e = 0; e < 4; ++e) vw[e] = s_map[w][16 + e][lf];
      mat4_vec(Mw, xs, vw, xn);
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[e] = xn[e];
    }
    if (anchor) {
#pragma unroll
      for (int e = 0; e < 4; ++e) tag_store(word(tt, e, f), xs[e], epoch);
    }
  }
  __syncthreads();  // start values in LDS
}

}  // namespace slstm
