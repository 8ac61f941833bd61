// Per-row moments of a residual stream, handed from the kernel that writes
// the stream to the kernels that normalise it.
//
// The writer stores partial moments per column tile: part[t * M + m] =
// (mean, M2) of row m over columns [t*tw, min(N, (t+1)*tw)). A reader
// merges the T partials of a row (Chan et al. pairwise update, fixed order
// in a fixed butterfly), so no kernel needs a grid-wide reduction and the
// result is the same on every run.
#pragma once
#include "common.h"

namespace vla {

struct RowStats {
  const float2* part;   // [T][M]
  int T;                // number of column tiles (1..256)
  int tw;               // columns per tile (the last tile may be shorter)
  int N;                // row length
  int M;                // rows (leading dimension of part)
};

// Merged (mean, biased variance) of RPW rows handled by one wave (rows[j] <
// 0 means "no row"). Lanes form groups of G = 64 / P lanes, one group per
// row, each lane covering ceil(T / G) <= 4 tiles; P rows are merged per pass.
// Every partial of the wave is loaded before any merge.
// a[j] for a runtime j without dynamic register indexing (-1 when out of range)
template <int N>
__device__ __forceinline__ int pick_row(const int (&a)[N], int j) {
  int v = -1;
#pragma unroll
  for (int i = 0; i < N; i++) v = (i == j) ? a[i] : v;
  return v;
}

template <int RPW>
__device__ __forceinline__ void rows_moments_wave(const RowStats& rs, const int (&rows)[RPW], float2 (&out)[RPW]) {
  const int lane = threadIdx.x & 63;
  int G = 1;
  while (G < 64 && 4 * G < rs.T) G <<= 1;      // lanes per row (power of two)
  const int P = 64 / G;                        // rows per pass
  const int gl = lane & (G - 1), grp = lane / G;
  constexpr int MAXP = RPW;                    // passes needed when P == 1
  float2 v[MAXP][4];
#pragma unroll
  for (int q = 0; q < MAXP; q++) {
    int j = q * P + grp;                       // row slot handled by this lane group in pass q
    int m = pick_row(rows, j);
#pragma unroll
    for (int u = 0; u < 4; u++) {
      int t = gl + u * G;
      v[q][u] = (m >= 0 && t < rs.T) ? rs.part[(size_t)t * rs.M + m] : make_float2(0.f, 0.f);
    }
  }
#pragma unroll
  for (int q = 0; q < MAXP; q++) {
    if (q * P >= RPW) break;
    int j = q * P + grp;
    int m = pick_row(rows, j);
    float n = 0.f, mean = 0.f, m2 = 0.f;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      int t = gl + u * G;
      if (m >= 0 && t < rs.T) moments_merge(n, mean, m2, (float)min(rs.tw, rs.N - t * rs.tw), v[q][u].x, v[q][u].y);
    }
    for (int o = G >> 1; o >= 1; o >>= 1) {
      float n2 = __shfl_xor(n, o, WAVE), mean2 = __shfl_xor(mean, o, WAVE), m22 = __shfl_xor(m2, o, WAVE);
      moments_merge(n, mean, m2, n2, mean2, m22);
    }
    // the group's first lane holds the row result; hand it to every lane
#pragma unroll
    for (int jj = 0; jj < RPW; jj++) {
      if (jj / P != q) continue;               // wave-uniform
      int src = (jj % P) * G;
      float nn = __shfl(n, src, WAVE), mm = __shfl(mean, src, WAVE), qq = __shfl(m2, src, WAVE);
      out[jj] = make_float2(mm, nn > 0.f ? qq / nn : 0.f);
    }
  }
}

}  // namespace vla
