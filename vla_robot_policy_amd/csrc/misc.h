// Small kernels around the GEMMs: input staging with row statistics, the
// standalone final norm, the fused Euler tail of the flow sampler, and a fill.
#pragma once
#include "common.h"
#include "rowstats.h"
#include "tail.h"

namespace vla {

// Fill n uint32 words with a value (used instead of a memset node so the
// clearing of counters can sit inside a captured graph).
__global__ void k_fill_u32(unsigned* p, unsigned v, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// x[r] = src[r - r0] for r in [r0, r1) (bf16 or fp32 source), then the
// moments of every row r < M as a single column tile (stats[r] = (mean,
// sum of squared deviations)). One wave per row.
__global__ __launch_bounds__(256) void k_stage_rows(float* x, int ldx, int M, int N, const void* src, int src_f32,
                                                  int ld_src, int r0, int r1, float2* stats) {
  int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (r >= M) return;
  float* xr = x + (size_t)r * ldx;
  if (src && r >= r0 && r < r1) {
    for (int c = lane; c < N; c += 64) {
      size_t o = (size_t)(r - r0) * ld_src + c;
      xr[c] = src_f32 ? ((const float*)src)[o] : bf2f(((const uint16_t*)src)[o]);
    }
  }
  float s = 0.f;
  for (int c = lane; c < N; c += 64) s += xr[c];
  float mean = wave_sum(s) / (float)N;
  float q = 0.f;
  for (int c = lane; c < N; c += 64) { float d = xr[c] - mean; q += d * d; }
  float m2 = wave_sum(q);
  if (lane == 0) stats[r] = make_float2(mean, m2);
}

// out[r] = RMSNorm(x[r]) * gain, from the row moments left by x's writer.
__global__ __launch_bounds__(256) void k_rmsnorm_out(const float* x, int ldx, int M, int N, RowStats st_in,
                                                   const float* gain, float eps, void* out, int ldo, int out_f32) {
  int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (r >= M) return;
  float rs = norm_coeffs(row_moments_wave(st_in, r), 1, eps).y;
  for (int c = lane; c < N; c += 64) {
    float v = x[(size_t)r * ldx + c] * rs * gain[c];
    if (out_f32) ((float*)out)[(size_t)r * ldo + c] = v;
    else ((uint16_t*)out)[(size_t)r * ldo + c] = f2bf(v);
  }
}

// One normalised row per workgroup, in bf16, for the GEMMs that read it:
// RMSNorm (x * rstd * g) or LayerNorm ((x - mean) * rstd * g + b, g given as
// 1 + g when g_plus_one), the row moments merged from the writer's tiles.
// With out_lo, also the remainder lo = bf16(v - hi) of each value.
__global__ __launch_bounds__(256) void k_norm_rows(NormArgs p) {
  __shared__ float2 snc;
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* xr = p.x + (size_t)r * p.ldx;
  // the row's first 4096 values (and their gain / shift) are requested
  // before the row moments, so both share one memory latency
  constexpr int PRE = 4;
  float4 v[PRE], g[PRE], b[PRE];
#pragma unroll
  for (int i = 0; i < PRE; i++) {
    const int k = tid * 4 + i * 1024;
    const bool ok = k < p.K;
    v[i] = ok ? *reinterpret_cast<const float4*>(xr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    g[i] = ok && p.g ? *reinterpret_cast<const float4*>(p.g + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    b[i] = ok && p.bsh ? *reinterpret_cast<const float4*>(p.bsh + k) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid < 64) {
    float2 nc = norm_coeffs(row_moments_wave(p.rs, r), p.rms, p.eps);
    if (tid == 0) snc = nc;
  }
  __syncthreads();
  const float2 nc = snc;
  auto put = [&](int k, float4 x, float4 gg, float4 bb) {
    if (!p.g) gg = make_float4(1.f, 1.f, 1.f, 1.f);
    else if (p.g_plus_one) { gg.x += 1.f; gg.y += 1.f; gg.z += 1.f; gg.w += 1.f; }
    const float u0 = (x.x - nc.x) * nc.y * gg.x + bb.x, u1 = (x.y - nc.x) * nc.y * gg.y + bb.y;
    const float u2 = (x.z - nc.x) * nc.y * gg.z + bb.z, u3 = (x.w - nc.x) * nc.y * gg.w + bb.w;
    uint2 h;
    h.x = pack_bf2(u0, u1);
    h.y = pack_bf2(u2, u3);
    *reinterpret_cast<uint2*>(p.out + (size_t)r * p.ldo + k) = h;
    if (p.out_lo) {
      uint2 l;
      l.x = pack_bf2(u0 - bf2f(f2bf(u0)), u1 - bf2f(f2bf(u1)));
      l.y = pack_bf2(u2 - bf2f(f2bf(u2)), u3 - bf2f(f2bf(u3)));
      *reinterpret_cast<uint2*>(p.out_lo + (size_t)r * p.ldo + k) = l;
    }
  };
#pragma unroll
  for (int i = 0; i < PRE; i++) {
    const int k = tid * 4 + i * 1024;
    if (k < p.K) put(k, v[i], g[i], b[i]);
  }
  for (int k = tid * 4 + PRE * 1024; k < p.K; k += 1024) {
    const float4 x = *reinterpret_cast<const float4*>(xr + k);
    const float4 gg = p.g ? *reinterpret_cast<const float4*>(p.g + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 bb = p.bsh ? *reinterpret_cast<const float4*>(p.bsh + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    put(k, x, gg, bb);
  }
}

template <typename WT> __device__ __forceinline__ float wget(const void* w, size_t i);
template <> __device__ __forceinline__ float wget<uint16_t>(const void* w, size_t i) { return bf2f(((const uint16_t*)w)[i]); }
template <> __device__ __forceinline__ float wget<float>(const void* w, size_t i) { return ((const float*)w)[i]; }
template <> __device__ __forceinline__ float wget<uint8_t>(const void* w, size_t i) { return fp8_to_f32(((const uint8_t*)w)[i]); }



// One workgroup per action row m:
//   v = (LN(x_m)(1 + scale) + shift) W_out^T + b_out;  a_m <- a_m + v / K
//   x_m <- a_m W_in^T + b_in, with its (mean, var) for the next LayerNorm.
template <typename WT>
__global__ __launch_bounds__(256) void k_euler_tail(TailArgs p) {
  extern __shared__ __align__(16) float sh[];
  float* su = sh;                 // [D]
  float* sa = sh + p.D;           // [A]
  __shared__ float red[8];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* arow = p.a_in + (size_t)m * p.A;
  if (p.w_out) {
    // LayerNorm of x_m: two-pass mean / variance over the row (this
    // workgroup reads the whole row anyway)
    const float* xr = p.x + (size_t)m * p.D;
    float s1 = 0.f;
    for (int d = tid; d < p.D; d += 256) s1 += xr[d];
    s1 = wave_sum(s1);
    if (lane == 0) red[wave] = s1;
    __syncthreads();
    const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)p.D;
    float s2 = 0.f;
    for (int d = tid; d < p.D; d += 256) { float dd = xr[d] - mean; s2 += dd * dd; }
    s2 = wave_sum(s2);
    if (lane == 0) red[4 + wave] = s2;
    __syncthreads();
    const float rstd = rsqrtf((red[4] + red[5] + red[6] + red[7]) / (float)p.D + p.eps);
    __syncthreads();   // red is reused below
    for (int d = tid; d < p.D; d += 256)
      su[d] = (xr[d] - mean) * rstd * (1.f + p.scale[d]) + p.shift[d];
    __syncthreads();
    for (int a = wave; a < p.A; a += 4) {
      float acc = 0.f;
      for (int d = lane; d < p.D; d += 64) acc += su[d] * wget<WT>(p.w_out, (size_t)a * p.D + d);
      acc = wave_sum(acc);
      if (lane == 0) {
        float v = acc * (p.s_out ? p.s_out[a] : 1.f) + p.b_out[a];
        if (p.v_out) p.v_out[(size_t)m * p.A + a] = v;
        float an = arow[a] + v / (float)p.K;
        sa[a] = an;
      }
    }
    __syncthreads();
    for (int a = tid; a < p.A; a += 256) p.a_out[(size_t)m * p.A + a] = sa[a];
  } else {
    for (int a = tid; a < p.A; a += 256) {
      sa[a] = arow[a];
      if (p.a_out != p.a_in) p.a_out[(size_t)m * p.A + a] = arow[a];
    }
  }
  __syncthreads();
  if (!p.w_in) return;
  float s = 0.f;
  for (int d = tid; d < p.D; d += 256) {
    float acc = p.b_in[d];
    float sc = p.s_in ? p.s_in[d] : 1.f;
    float dot = 0.f;
    for (int a = 0; a < p.A; a++) dot += sa[a] * wget<WT>(p.w_in, (size_t)d * p.A + a);
    acc += dot * sc;
    p.x_out[(size_t)m * p.D + d] = acc;
    su[d] = acc;
    s += acc;
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  float mean = (red[0] + red[1] + red[2] + red[3]) / (float)p.D;
  __syncthreads();
  float q = 0.f;
  for (int d = tid; d < p.D; d += 256) { float dd = su[d] - mean; q += dd * dd; }
  q = wave_sum(q);
  if (lane == 0) red[4 + wave] = q;
  __syncthreads();
  if (tid == 0) p.rs_out[m] = make_float2(mean, red[4] + red[5] + red[6] + red[7]);
}

}  // namespace vla
