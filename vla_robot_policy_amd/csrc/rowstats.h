// Per-row moments of a residual stream, handed from the kernel that writes
// the stream to the kernels that normalise it.
//
// The writer stores partial moments per column tile: part[t * M + m] =
// (mean, M2) of row m over columns [t*tw, min(N, (t+1)*tw)). A reader merges
// the T partials of a row itself, so no kernel needs a grid-wide reduction:
// each of the G threads serving a row accumulates a strided subset of the
// tiles as shifted sums (shift = the mean of its first tile; no divisions),
// then the G results are merged pairwise (Chan et al.) in a fixed butterfly.
// The order is fixed, so the result is the same on every run.
#pragma once
#include "common.h"

namespace vla {

struct RowStats {
  const float2* part;   // [T][M]
  int T;                // number of column tiles (>= 1)
  int tw;               // columns per tile (the last tile may be shorter)
  int N;                // row length
  int M;                // rows (leading dimension of part)
};

// Shifted sums of a thread's tiles: with c the first tile's mean,
// s1 = sum n_t (mean_t - c), s2 = sum (M2_t + n_t (mean_t - c)^2).
struct ShiftSum {
  float c = 0.f, n = 0.f, s1 = 0.f, s2 = 0.f;
  __device__ __forceinline__ void add(float nt, float2 v) {
    c = n > 0.f ? c : v.x;
    float d = v.x - c;
    n += nt;
    s1 = fmaf(nt, d, s1);
    s2 += fmaf(nt * d, d, v.y);
  }
  // (count, mean, M2) of the accumulated tiles
  __device__ __forceinline__ void moments(float& cnt, float& mean, float& m2) const {
    cnt = n;
    float q = n > 0.f ? s1 / n : 0.f;
    mean = c + q;
    m2 = s2 - s1 * q;
  }
};

__device__ __forceinline__ float tile_count(const RowStats& rs, int t) { return (float)min(rs.tw, rs.N - t * rs.tw); }

// Merge (count, mean, M2) across the G lanes of an aligned lane group (G a
// power of two <= 64): both partners of each butterfly step merge the same
// ordered pair (lower lane first), so every lane ends with the same result.
__device__ __forceinline__ void group_merge(float& n, float& mean, float& m2, int G) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < G; o <<= 1) {
    float n2 = __shfl_xor(n, o, WAVE), mean2 = __shfl_xor(mean, o, WAVE), m22 = __shfl_xor(m2, o, WAVE);
    if (lane & o) {
      float tn = n, tmean = mean, tm2 = m2;
      n = n2; mean = mean2; m2 = m22;
      n2 = tn; mean2 = tmean; m22 = tm2;
    }
    if (n <= 0.f) { n = n2; mean = mean2; m2 = m22; }
    else moments_merge(n, mean, m2, n2, mean2, m22);
  }
}

// (mean, biased variance) of row m by one whole wave: lane l takes tiles
// l, l + 64, ... Every lane returns the result.
__device__ __forceinline__ float2 row_moments_wave(const RowStats& rs, int m) {
  const int lane = threadIdx.x & 63;
  ShiftSum a;
  for (int t = lane; t < rs.T; t += 64) a.add(tile_count(rs, t), rs.part[(size_t)t * rs.M + m]);
  float n, mean, m2;
  a.moments(n, mean, m2);
  group_merge(n, mean, m2, 64);
  return make_float2(mean, n > 0.f ? m2 / n : 0.f);
}

// (value to subtract, reciprocal standard deviation) of a row from its
// (mean, variance): LayerNorm centres on the mean, RMSNorm uses the mean
// square var + mean^2.
__device__ __forceinline__ float2 norm_coeffs(float2 mv, int rms, float eps) {
  float ms = rms ? mv.y + mv.x * mv.x : mv.y;
  return make_float2(rms ? 0.f : mv.x, rsqrtf(ms + eps));
}

}  // namespace vla
