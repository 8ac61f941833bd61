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
// Largest value over a 256-thread workgroup (every thread gets it).
__device__ __forceinline__ float block_max256(float v) {
  __shared__ float wm[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

// Four E4M3FN codes (bytes in order x, y, z, w) of u * inv, clamped to the
// largest finite magnitude and rounded to nearest even by the converter.
__device__ __forceinline__ uint32_t e4m3x4(float4 u, float inv) {
  auto c = [&](float t) { return fminf(fmaxf(t * inv, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(u.x), c(u.y), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c(u.z), c(u.w), w, true);
  return (uint32_t)w;
}
// Four int8 codes of u * inv: nearest integer (halves to even), clipped to 127.
__device__ __forceinline__ uint32_t i8x4(float4 u, float inv) {
  auto c = [&](float t) { return (uint32_t)(int)fminf(fmaxf(rintf(t * inv), -127.f), 127.f) & 0xFFu; };
  return c(u.x) | (c(u.y) << 8) | (c(u.z) << 16) | (c(u.w) << 24);
}
// 8-bit codes of four values: E4M3FN (qmax 448) or int8 (qmax 127)
__device__ __forceinline__ uint32_t codes4(float4 u, float inv, int int8) { return int8 ? i8x4(u, inv) : e4m3x4(u, inv); }

// W8A8: E4M3FN (int8 = 0) or int8 (int8 = 1) codes of bf16 or fp32 rows
// [M, ldx] (K values each, K a multiple of 8 and at most 16384), one float32
// scale max|x| / qmax per row (qmax 448 or 127); one workgroup per row, the
// row held in registers.
__global__ __launch_bounds__(256) void k_quant_rows(const void* x, int x_f32, int ldx, int K, uint8_t* out, int ldo,
                                                    float* scale, int int8) {
  const float qmax = int8 ? 127.f : 448.f;
  constexpr int G = 8;                           // 8-value groups per thread
  const int r = blockIdx.x, tid = threadIdx.x;
  float4 v[G][2];
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < G; i++) {
    const int k = (tid + i * 256) * 8;
    v[i][0] = v[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < K) {
      if (x_f32) {
        const float* xr = (const float*)x + (size_t)r * ldx + k;
        v[i][0] = *reinterpret_cast<const float4*>(xr);
        v[i][1] = *reinterpret_cast<const float4*>(xr + 4);
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>((const uint16_t*)x + (size_t)r * ldx + k);
        auto f4 = [](uint32_t a, uint32_t b) {
          return make_float4(bf2f((uint16_t)(a & 0xFFFFu)), bf2f((uint16_t)(a >> 16)), bf2f((uint16_t)(b & 0xFFFFu)),
                             bf2f((uint16_t)(b >> 16)));
        };
        v[i][0] = f4(w.x, w.y);
        v[i][1] = f4(w.z, w.w);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
      am = fmaxf(am, fmaxf(fmaxf(fabsf(v[i][h].x), fabsf(v[i][h].y)), fmaxf(fabsf(v[i][h].z), fabsf(v[i][h].w))));
  }
  am = block_max256(am);
  const float inv = am > 0.f ? __fdiv_rn(qmax, am) : 0.f;
#pragma unroll
  for (int i = 0; i < G; i++) {
    const int k = (tid + i * 256) * 8;
    if (k >= K) continue;
    uint2 c;
    c.x = codes4(v[i][0], inv, int8);
    c.y = codes4(v[i][1], inv, int8);
    *reinterpret_cast<uint2*>(out + (size_t)r * ldo + k) = c;
  }
  if (tid == 0) scale[r] = __fdiv_rn(am, qmax);
}

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
  auto norm4 = [&](float4 x, float4 gg, float4 bb) -> float4 {
    if (!p.g) gg = make_float4(1.f, 1.f, 1.f, 1.f);
    else if (p.g_plus_one) { gg.x += 1.f; gg.y += 1.f; gg.z += 1.f; gg.w += 1.f; }
    return make_float4((x.x - nc.x) * nc.y * gg.x + bb.x, (x.y - nc.x) * nc.y * gg.y + bb.y,
                       (x.z - nc.x) * nc.y * gg.z + bb.z, (x.w - nc.x) * nc.y * gg.w + bb.w);
  };
  if (p.out8) {
    // W8A8: the normalised row as 8-bit codes with the scale max|u| / qmax
    // (the whole row is in this thread's registers: K <= 4 * 1024)
    float4 u[PRE];
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < PRE; i++) {
      const int k = tid * 4 + i * 1024;
      u[i] = k < p.K ? norm4(v[i], g[i], b[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
      am = fmaxf(am, fmaxf(fmaxf(fabsf(u[i].x), fabsf(u[i].y)), fmaxf(fabsf(u[i].z), fabsf(u[i].w))));
    }
    am = block_max256(am);
    const float qmax = p.out8_int8 ? 127.f : 448.f;
    const float inv = am > 0.f ? __fdiv_rn(qmax, am) : 0.f;
#pragma unroll
    for (int i = 0; i < PRE; i++) {
      const int k = tid * 4 + i * 1024;
      if (k < p.K) *reinterpret_cast<uint32_t*>(p.out8 + (size_t)r * p.ldo + k) = codes4(u[i], inv, p.out8_int8);
    }
    if (tid == 0) p.oscale[r] = __fdiv_rn(am, qmax);
    return;
  }
  auto put = [&](int k, float4 x, float4 gg, float4 bb) {
    const float4 uu = norm4(x, gg, bb);
    const float u0 = uu.x, u1 = uu.y, u2 = uu.z, u3 = uu.w;
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
template <> __device__ __forceinline__ float wget<int8_t>(const void* w, size_t i) { return (float)((const int8_t*)w)[i]; }



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
