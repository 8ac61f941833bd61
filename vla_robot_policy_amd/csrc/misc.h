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

// Rows are read as float4 (bf16: four values per 8-byte load); a lane holds
// RW_V of them per pass, every load of a pass requested before the first is
// used, so a row costs one memory latency per 4096 columns.
constexpr int RW_V = 16;

__device__ __forceinline__ float4 bf16x4_to_f4(uint2 b) {
  return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u), __uint_as_float(b.y << 16),
                     __uint_as_float(b.y & 0xFFFF0000u));
}

// x[r] = src[r - r0] for r in [r0, r1) (bf16 or fp32 source), then the
// moments of every row r < M as a single column tile (stats[r] = (mean,
// sum of squared deviations)). One wave per row; N, ldx and ld_src are
// multiples of 4 (checked by the launcher). Each pass of 4096 columns gives
// exact two-pass moments from registers; passes merge by Chan et al.
__global__ __launch_bounds__(256) void k_stage_rows(float* x, int ldx, int M, int N, const void* src, int src_f32,
                                                  int ld_src, int r0, int r1, float2* stats) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= M) return;
  float* xr = x + (size_t)r * ldx;
  const bool copy = src && r >= r0 && r < r1;
  const brsrc xs = make_brsrc(xr);
  const brsrc ss = make_brsrc(!copy ? (const void*)xr
                                    : src_f32 ? (const void*)((const float*)src + (size_t)(r - r0) * ld_src)
                                              : (const void*)((const uint16_t*)src + (size_t)(r - r0) * ld_src));
  float n = 0.f, mean = 0.f, m2 = 0.f;
  for (int c0 = 0; c0 < N; c0 += 64 * 4 * RW_V) {
    float4 v[RW_V];
#pragma unroll
    for (int i = 0; i < RW_V; i++) {
      const int c = c0 + (lane + 64 * i) * 4;
      const bool ok = c < N;
      if (copy && !src_f32) v[i] = bf16x4_to_f4(bload8(ss, ok ? (uint32_t)c * 2u : BUF_OOB));
      else v[i] = as_f4(bload16(copy ? ss : xs, ok ? (uint32_t)c * 4u : BUF_OOB));
    }
    if (copy) {
#pragma unroll
      for (int i = 0; i < RW_V; i++) {
        const int c = c0 + (lane + 64 * i) * 4;
        if (c < N) *reinterpret_cast<float4*>(xr + c) = v[i];
      }
    }
    const int cn = min(N - c0, 64 * 4 * RW_V);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RW_V; i++) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);   // zeros beyond N
    const float cm = wave_sum(s) / (float)cn;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < RW_V; i++) {
      if (c0 + (lane + 64 * i) * 4 < N) {
        const float d0 = v[i].x - cm, d1 = v[i].y - cm, d2 = v[i].z - cm, d3 = v[i].w - cm;
        q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
      }
    }
    moments_merge(n, mean, m2, (float)cn, cm, wave_sum(q));
  }
  if (lane == 0) stats[r] = make_float2(mean, m2);
}

// out[r] = RMSNorm(x[r]) * gain, from the row moments left by x's writer.
// One wave per row; the row and the gains are requested before the row
// moments are merged, so both share one memory latency.
__global__ __launch_bounds__(256) void k_rmsnorm_out(const float* x, int ldx, int M, int N, RowStats st_in,
                                                   const float* gain, float eps, void* out, int ldo, int out_f32) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= M) return;
  const brsrc xs = make_brsrc(x + (size_t)r * ldx), gs = make_brsrc(gain);
  float rs = 0.f;
  for (int c0 = 0; c0 < N; c0 += 64 * 4 * RW_V) {
    float4 v[RW_V], g[RW_V];
#pragma unroll
    for (int i = 0; i < RW_V; i++) {
      const int c = c0 + (lane + 64 * i) * 4;
      v[i] = as_f4(bload16(xs, c < N ? (uint32_t)c * 4u : BUF_OOB));
      g[i] = as_f4(bload16(gs, c < N ? (uint32_t)c * 4u : BUF_OOB));
    }
    if (c0 == 0) rs = norm_coeffs(row_moments_wave(st_in, r), 1, eps).y;
#pragma unroll
    for (int i = 0; i < RW_V; i++) {
      const int c = c0 + (lane + 64 * i) * 4;
      if (c >= N) continue;
      const float4 y = make_float4(v[i].x * rs * g[i].x, v[i].y * rs * g[i].y, v[i].z * rs * g[i].z, v[i].w * rs * g[i].w);
      if (out_f32) {
        *reinterpret_cast<float4*>((float*)out + (size_t)r * ldo + c) = y;
      } else {
        uint2 u;
        u.x = pack_bf2(y.x, y.y);
        u.y = pack_bf2(y.z, y.w);
        *reinterpret_cast<uint2*>((uint16_t*)out + (size_t)r * ldo + c) = u;
      }
    }
  }
}

// Packed weight layout (vla_pack_weights): a row-major W [N, K] of esz-byte
// elements (2: bf16, 1: E4M3FN or int8 codes) becomes blocks of 16 rows x 32
// columns, ordered [row block][column block]; inside a block, lane l of a
// wave holds the 8 elements of row l % 16 at columns 8 (l / 16) .. + 7, the
// B operand fragment of one 16x16x32 MFMA step, so a wave-wide load of one
// block is contiguous (1 KB for bf16). Rows and columns beyond N and K are
// zero. One thread per 8-element lane chunk.
__global__ __launch_bounds__(256) void k_pack_weights(const uint8_t* w, int N, int K, int ldw, int esz, uint8_t* out) {
  const int KB = (K + 31) / 32, NB = (N + 15) / 16;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (size_t)NB * KB * 64) return;
  const int lane = (int)(e % 64);
  const size_t blk = e / 64;
  const int kb = (int)(blk % KB), nb = (int)(blk / KB);
  const int row = nb * 16 + lane % 16, k0 = kb * 32 + (lane / 16) * 8;
  uint8_t v[16];
#pragma unroll
  for (int j = 0; j < 8; j++)
#pragma unroll
    for (int b = 0; b < 2; b++) {
      if (b >= esz) continue;
      const int k = k0 + j;
      v[j * esz + b] = (row < N && k < K) ? w[((size_t)row * ldw + k) * esz + b] : (uint8_t)0;
    }
  uint8_t* o = out + e * 8 * esz;
  for (int i = 0; i < 8 * esz; i++) o[i] = v[i];
}

// Context values of every layer transposed for the action expert's
// cross-attention: vt[l][d][c] = V_l[c][d], where V_l is columns l 2D + D ..
// l 2D + 2D - 1 of the cross K / V rows kv[c] (C rows, pitch L 2D), and zero
// for c >= C (Cp keys per row, a multiple of 8). A thread writes 8 keys of
// one (l, d); consecutive threads take consecutive d, so each of its 8 reads
// is coalesced across the wave.
__global__ __launch_bounds__(256) void k_ctx_vt(const uint16_t* kv, int C, int L, int D, int Cp, uint16_t* vt) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int n8 = Cp / 8;
  if (e >= (size_t)L * n8 * D) return;
  const int d = (int)(e % D);
  const size_t r = e / D;
  const int c0 = (int)(r % n8) * 8, l = (int)(r / n8);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int c = c0 + 2 * j;
    const size_t base = (size_t)l * 2 * D + D + d, ld = (size_t)L * 2 * D;
    const uint32_t lo = c < C ? kv[(size_t)c * ld + base] : 0u;
    const uint32_t hi = c + 1 < C ? kv[(size_t)(c + 1) * ld + base] : 0u;
    w[j] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(vt + ((size_t)l * D + d) * Cp + c0) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Patch rows of a batch of images (bf16 [n_img][chans][img][img]): row m =
// patch (pr, pc) of image m / n_patches with features in (channel, row,
// column) order, zero from k = chans * patch^2 up to the row pitch; one
// thread per 8 features (one 16-byte store).
__global__ __launch_bounds__(256) void k_patch_rows(const uint16_t* img, int n_img, int chans, int size, int patch,
                                                    int grid, int pitch, uint16_t* out) {
  const int n8 = pitch / 8;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int np = grid * grid;
  if (e >= (size_t)n_img * np * n8) return;
  const int m = (int)(e / n8), k0 = (int)(e % n8) * 8;
  const int im = m / np, pi = m % np, pr = pi / grid, pc = pi % grid;
  const int P2 = patch * patch, K = chans * P2;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    uint32_t h[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int k = k0 + 2 * j + q;
      h[q] = 0u;
      if (k < K) {
        const int c = k / P2, r = k % P2, ky = r / patch, kx = r % patch;
        h[q] = img[(((size_t)im * chans + c) * size + pr * patch + ky) * size + pc * patch + kx];
      }
    }
    w[j] = h[0] | (h[1] << 16);
  }
  *reinterpret_cast<uint4*>(out + (size_t)m * pitch + k0) = make_uint4(w[0], w[1], w[2], w[3]);
}

// RoPE tables of a pass: cs[pos][i] = cos(pos theta_i), sn[pos][i] =
// sin(pos theta_i), theta_i = base^(-2i / D), i < D / 2, pos < S (half-split
// rotation of the pairs (i, i + D/2)). The frequency and the angle are formed
// in double and reduced to [-pi, pi] before the float sine and cosine: a
// float frequency times a position of several hundred is off by up to 1e-4
// radians.
__global__ __launch_bounds__(256) void k_rope_table(float* cs, float* sn, int S, int D, float base) {
  const int hd = D / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= S * hd) return;
  const int pos = e / hd, i = e % hd;
  const double theta = pow((double)base, -2.0 * (double)i / (double)D);
  double a = (double)pos * theta;
  a -= rint(a * (0.5 / M_PI)) * (2.0 * M_PI);
  float s, c;
  sincosf((float)a, &s, &c);
  cs[e] = c;
  sn[e] = s;
}

// Sinusoidal features of the sampler's time grid t_k = k / K (k < K): row k
// is [cos(s t_k w_i) | sin(s t_k w_i)], w_i = base^(-i / half), i < half, in
// bf16 [K][2 half]. The frequency and the argument are formed in double and
// reduced to [-pi, pi] before the float sine and cosine (the arguments reach
// s radians).
__global__ __launch_bounds__(256) void k_time_embed(uint16_t* phi, int K, int half, float time_scale, float freq_base) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= K * half) return;
  const int k = e / half, i = e % half;
  const double w = pow((double)freq_base, -(double)i / (double)half);
  double a = (double)time_scale * ((double)k / (double)K) * w;
  a -= rint(a * (0.5 / M_PI)) * (2.0 * M_PI);
  float sn, cs;
  sincosf((float)a, &sn, &cs);
  phi[(size_t)k * 2 * half + i] = f2bf(cs);
  phi[(size_t)k * 2 * half + half + i] = f2bf(sn);
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
// With out_lo, also the remainder lo = bf16(v - hi) of each value. With a
// merge geometry, each row (a patch) lands in its segment of a merged row.
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
  // destination of the row: its own row, or its segment of a merged row
  size_t obase = (size_t)r * p.ldo;
  if (p.merge) {
    const int im = r / p.n_patches, pi = r % p.n_patches, pr = pi / p.vgrid, pc = pi % p.vgrid;
    const int gq = p.vgrid / p.merge;
    const int mrow = im * (p.n_patches / (p.merge * p.merge)) + (pr / p.merge) * gq + pc / p.merge;
    const int seg = (pr % p.merge) * p.merge + pc % p.merge;
    obase = (size_t)mrow * p.ldo + (size_t)seg * p.K;
  }
  auto put = [&](int k, float4 x, float4 gg, float4 bb) {
    const float4 uu = norm4(x, gg, bb);
    const float u0 = uu.x, u1 = uu.y, u2 = uu.z, u3 = uu.w;
    uint2 h;
    h.x = pack_bf2(u0, u1);
    h.y = pack_bf2(u2, u3);
    *reinterpret_cast<uint2*>(p.out + obase + k) = h;
    if (p.out_lo) {
      uint2 l;
      l.x = pack_bf2(u0 - bf2f(f2bf(u0)), u1 - bf2f(f2bf(u1)));
      l.y = pack_bf2(u2 - bf2f(f2bf(u2)), u3 - bf2f(f2bf(u3)));
      *reinterpret_cast<uint2*>(p.out_lo + obase + k) = l;
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



// Eight consecutive weights from element i (a multiple of 8) as floats,
// in one vector load (the matrices are 16-byte aligned, rows a multiple of 8).
template <typename WT> __device__ __forceinline__ void wload8(const void* w, size_t i, float (&f)[8]);
template <> __device__ __forceinline__ void wload8<uint16_t>(const void* w, size_t i, float (&f)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>((const uint16_t*)w + i);
  const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; k++) { f[2 * k] = __uint_as_float(h[k] << 16); f[2 * k + 1] = __uint_as_float(h[k] & 0xFFFF0000u); }
}
template <> __device__ __forceinline__ void wload8<float>(const void* w, size_t i, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>((const float*)w + i), b = *reinterpret_cast<const float4*>((const float*)w + i + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <> __device__ __forceinline__ void wload8<uint8_t>(const void* w, size_t i, float (&f)[8]) {
  const uint2 u = *reinterpret_cast<const uint2*>((const uint8_t*)w + i);
  const uint32_t h[2] = {u.x, u.y};
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)h[k], false), hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)h[k], true);
    f[4 * k] = lo[0]; f[4 * k + 1] = lo[1]; f[4 * k + 2] = hi[0]; f[4 * k + 3] = hi[1];
  }
}
template <> __device__ __forceinline__ void wload8<int8_t>(const void* w, size_t i, float (&f)[8]) {
  const uint2 u = *reinterpret_cast<const uint2*>((const int8_t*)w + i);
#pragma unroll
  for (int k = 0; k < 8; k++) f[k] = (float)(int8_t)((k < 4 ? u.x : u.y) >> (8 * (k & 3)));
}

// One workgroup per action row m:
//   v = (LN(x_m)(1 + scale) + shift) W_out^T + b_out;  a_m <- a_m + v / K
//   x_m <- a_m W_in^T + b_in, with its (mean, var) for the next LayerNorm.
// The row is read once into LDS. In the velocity head wave w takes actions
// w, w + 4, ... of each group of 32 and every lane accumulates all of them
// over its 8-wide column groups, so the weight loads of all the wave's
// actions are in flight together (D is a multiple of 8).
template <typename WT>
__global__ __launch_bounds__(256) void k_euler_tail(TailArgs p) {
  extern __shared__ __align__(16) float sh[];
  float* su = sh;                 // [D]
  float* sa = sh + p.D;           // [A]
  __shared__ float red[8];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = p.D, A = p.A;
  const float* arow = p.a_in + (size_t)m * A;
  if (p.w_out) {
    // LayerNorm of x_m: the row into LDS with its sum, then the variance
    // from LDS (two-pass)
    const float4* xr4 = reinterpret_cast<const float4*>(p.x + (size_t)m * D);
    float s1 = 0.f;
    for (int d4 = tid; d4 < D / 4; d4 += 256) {
      const float4 v = xr4[d4];
      reinterpret_cast<float4*>(su)[d4] = v;
      s1 += (v.x + v.y) + (v.z + v.w);
    }
    s1 = wave_sum(s1);
    if (lane == 0) red[wave] = s1;
    __syncthreads();
    const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)D;
    float s2 = 0.f;
    for (int d = tid; d < D; d += 256) { const float dd = su[d] - mean; s2 += dd * dd; }
    s2 = wave_sum(s2);
    if (lane == 0) red[4 + wave] = s2;
    __syncthreads();
    const float rstd = rsqrtf((red[4] + red[5] + red[6] + red[7]) / (float)D + p.eps);
    for (int d = tid; d < D; d += 256) su[d] = (su[d] - mean) * rstd * (1.f + p.scale[d]) + p.shift[d];
    __syncthreads();
    for (int a0 = 0; a0 < A; a0 += 32) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = 0.f;
#pragma unroll 2
      for (int g = lane; g < D / 8; g += 64) {
        const float4 u0 = reinterpret_cast<const float4*>(su)[2 * g], u1 = reinterpret_cast<const float4*>(su)[2 * g + 1];
        const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int a = a0 + wave + 4 * i;
          if (a < A) {
            float wv[8];
            wload8<WT>(p.w_out, (size_t)a * D + 8 * g, wv);
#pragma unroll
            for (int e = 0; e < 8; e++) acc[i] = fmaf(u[e], wv[e], acc[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int a = a0 + wave + 4 * i;
        const float dot = wave_sum(acc[i]);
        if (lane == 0 && a < A) {
          const float v = dot * (p.s_out ? p.s_out[a] : 1.f) + p.b_out[a];
          if (p.v_out) p.v_out[(size_t)m * A + a] = v;
          sa[a] = arow[a] + v / (float)p.K;
        }
      }
    }
    __syncthreads();
    for (int a = tid; a < A; a += 256) p.a_out[(size_t)m * A + a] = sa[a];
  } else {
    for (int a = tid; a < A; a += 256) {
      sa[a] = arow[a];
      if (p.a_out != p.a_in) p.a_out[(size_t)m * A + a] = arow[a];
    }
  }
  __syncthreads();
  if (!p.w_in) return;
  // input projection: rows of W_in are A long; 8-wide loads when A allows
  const bool vec = A % 8 == 0;
  float s = 0.f;
  for (int d = tid; d < D; d += 256) {
    float dot = 0.f;
    if (vec) {
      for (int a8 = 0; a8 < A; a8 += 8) {
        float wv[8];
        wload8<WT>(p.w_in, (size_t)d * A + a8, wv);
#pragma unroll
        for (int e = 0; e < 8; e++) dot = fmaf(sa[a8 + e], wv[e], dot);
      }
    } else {
      for (int a = 0; a < A; a++) dot = fmaf(sa[a], wget<WT>(p.w_in, (size_t)d * A + a), dot);
    }
    const float acc = p.b_in[d] + dot * (p.s_in ? p.s_in[d] : 1.f);
    p.x_out[(size_t)m * D + d] = acc;
    su[d] = acc;
    s += acc;
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  float mean = (red[0] + red[1] + red[2] + red[3]) / (float)D;
  __syncthreads();
  float q = 0.f;
  for (int d = tid; d < D; d += 256) { float dd = su[d] - mean; q += dd * dd; }
  q = wave_sum(q);
  if (lane == 0) red[4 + wave] = q;
  __syncthreads();
  if (tid == 0) p.rs_out[m] = make_float2(mean, red[4] + red[5] + red[6] + red[7]);
}

}  // namespace vla
