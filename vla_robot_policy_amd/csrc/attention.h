// Flash attention (online softmax) for GQA / MHA, causal or full, on MFMA.
//
// Each wave owns 16 query rows of one query head and walks the keys in
// blocks of 32 staged in LDS (K row-major, V transposed). The scores are
// computed transposed, S^T = K Q^T, so a lane holds 8 keys of a single query:
// the running max / sum of that query live in the lane (plus a 4-way
// exchange across lane groups), and the exponentiated scores are already in
// the B-operand layout of O^T = V^T P^T. No LDS round trip for P.
// With grouped KV heads one workgroup serves up to 4 query heads that share
// one KV head, so each K/V block is fetched once for all of them.
#pragma once
#include "common.h"

namespace vla {

struct AttnArgs {
  const void* q; int ldq;    // [Sq, ldq]; head h starts at column h*D
  const void* k; int ldk;    // [Sk, ldk]; kv head g starts at column g*D
  const void* v; int ldv;
  void* o; int ldo;          // [Sq, ldo]; head h starts at column h*D
  int Sq, Sk, Hq, Hkv, D;
  int causal;                // key j visible to query i iff j <= i
  float scale_log2;          // log2(e) / sqrt(D)
};

template <typename CT> struct ATraits;
template <> struct ATraits<__bf16> {
  using F = FragBF16;
  static constexpr int ESZ = 2;
  __device__ static F gload(const void* base, size_t off) {
    F f; f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>((const uint16_t*)base + off)); return f;
  }
  __device__ static void lstore8(char* dst, const void* base, size_t off) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>((const uint16_t*)base + off);
  }
  __device__ static void lzero8(char* dst) { *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0); }
  __device__ static float get(const void* base, size_t off) { return bf2f(((const uint16_t*)base)[off]); }
  __device__ static void lput(char* dst, float v) { *reinterpret_cast<uint16_t*>(dst) = f2bf(v); }
  __device__ static void lput_raw(char* dst, const void* base, size_t off) {
    *reinterpret_cast<uint16_t*>(dst) = ((const uint16_t*)base)[off];
  }
  __device__ static void lzero1(char* dst) { *reinterpret_cast<uint16_t*>(dst) = 0; }
  __device__ static F lfrag(const char* p) { F f; f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p)); return f; }
  // V^T fragment: keys {4g..4g+3} at p0 and {16+4g..} at p1 (4 elements each)
  __device__ static F lfrag2(const char* p0, const char* p1) {
    uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
    F f; f.v = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y)); return f;
  }
  __device__ static void store(void* base, size_t off, float v) { ((uint16_t*)base)[off] = f2bf(v); }
};
template <> struct ATraits<float> {
  using F = FragF32;
  static constexpr int ESZ = 4;
  __device__ static F gload(const void* base, size_t off) {
    const float4* p = reinterpret_cast<const float4*>((const float*)base + off);
    float4 a = p[0], b = p[1];
    F f; f.lo = (f32x4){a.x, a.y, a.z, a.w}; f.hi = (f32x4){b.x, b.y, b.z, b.w}; return f;
  }
  __device__ static void lstore8(char* dst, const void* base, size_t off) {
    const float4* p = reinterpret_cast<const float4*>((const float*)base + off);
    reinterpret_cast<float4*>(dst)[0] = p[0];
    reinterpret_cast<float4*>(dst)[1] = p[1];
  }
  __device__ static void lzero8(char* dst) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(0, 0, 0, 0);
    reinterpret_cast<float4*>(dst)[1] = make_float4(0, 0, 0, 0);
  }
  __device__ static float get(const void* base, size_t off) { return ((const float*)base)[off]; }
  __device__ static void lput(char* dst, float v) { *reinterpret_cast<float*>(dst) = v; }
  __device__ static void lput_raw(char* dst, const void* base, size_t off) {
    *reinterpret_cast<float*>(dst) = ((const float*)base)[off];
  }
  __device__ static void lzero1(char* dst) { *reinterpret_cast<float*>(dst) = 0.f; }
  __device__ static F lfrag(const char* p) {
    float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    F f; f.lo = (f32x4){a.x, a.y, a.z, a.w}; f.hi = (f32x4){b.x, b.y, b.z, b.w}; return f;
  }
  __device__ static F lfrag2(const char* p0, const char* p1) {
    float4 a = *reinterpret_cast<const float4*>(p0), b = *reinterpret_cast<const float4*>(p1);
    F f; f.lo = (f32x4){a.x, a.y, a.z, a.w}; f.hi = (f32x4){b.x, b.y, b.z, b.w}; return f;
  }
  __device__ static void store(void* base, size_t off, float v) { ((float*)base)[off] = v; }
};

// DP: head dim padded to a multiple of 32 (64, 96, 128). HPW: query heads per
// workgroup (1, 2 or 4); the 4 waves cover HPW heads x (4 / HPW) row blocks.
template <typename CT, int DP, int HPW>
__global__ __launch_bounds__(256) void k_attention(AttnArgs p) {
  using TR = ATraits<CT>;
  using F = typename TR::F;
  constexpr int ESZ = TR::ESZ;
  constexpr int RB = 4 / HPW;                // 16-row blocks per workgroup
  constexpr int KB = 32;                     // keys per block
  constexpr int KPITCH = DP * ESZ + 16;      // K tile row pitch (bytes)
  constexpr int VPITCH = KB * ESZ + 16;      // V^T tile row pitch (bytes)
  __shared__ __align__(16) char sK[KB * KPITCH];
  __shared__ __align__(16) char sV[DP * VPITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = p.Hq / p.Hkv;
  const int hsets = group / HPW;             // head subsets per kv head
  const int nrb = (p.Sq + 16 * RB - 1) / (16 * RB);
  int bid = blockIdx.x;
  const int rb = bid % nrb;  bid /= nrb;
  const int hs = bid % hsets; bid /= hsets;
  const int g = bid;                          // kv head
  const int head = g * group + hs * HPW + (wave % HPW);
  const int row0 = (rb * RB + wave / HPW) * 16;     // this wave's first query row
  const int wg_row_end = min(p.Sq, (rb + 1) * RB * 16);
  const int qn = lane & 15, grp = lane >> 4;
  const int qrow = row0 + qn;

  // Q^T fragments (B operand): query qn, dims ds*32 + grp*8 .. +8
  F qf[DP / 32];
#pragma unroll
  for (int ds = 0; ds < DP / 32; ds++) {
    int d = ds * 32 + grp * 8;
    if (qrow < p.Sq && d < p.D) qf[ds] = TR::gload(p.q, (size_t)qrow * p.ldq + (size_t)head * p.D + d);
    else qf[ds] = zero_frag(F{});
  }

  f32x4 oacc[DP / 16];
#pragma unroll
  for (int i = 0; i < DP / 16; i++) oacc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  const int kend = p.causal ? min(p.Sk, wg_row_end) : p.Sk;
  for (int kb = 0; kb < kend; kb += KB) {
    __syncthreads();
    // stage K [32][DP] and V^T [DP][32] of kv head g
    for (int e = tid; e < KB * (DP / 8); e += 256) {
      int key = e / (DP / 8), d8 = (e % (DP / 8)) * 8;
      int j = kb + key;
      char* kd = sK + key * KPITCH + d8 * ESZ;
      if (j < p.Sk && d8 < p.D) {
        TR::lstore8(kd, p.k, (size_t)j * p.ldk + (size_t)g * p.D + d8);
        size_t vo = (size_t)j * p.ldv + (size_t)g * p.D + d8;
#pragma unroll
        for (int t = 0; t < 8; t++) TR::lput_raw(sV + (d8 + t) * VPITCH + key * ESZ, p.v, vo + t);
      } else {
        TR::lzero8(kd);
#pragma unroll
        for (int t = 0; t < 8; t++) TR::lzero1(sV + (d8 + t) * VPITCH + key * ESZ);
      }
    }
    __syncthreads();
    // S^T for keys kb + hb*16 + 4*grp + i, query qn
    f32x4 s[2];
#pragma unroll
    for (int hb = 0; hb < 2; hb++) {
      s[hb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DP / 32; ds++) {
        F kf = TR::lfrag(sK + (hb * 16 + qn) * KPITCH + (ds * 32 + grp * 8) * ESZ);
        mma32(s[hb], kf, qf[ds]);
      }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < 2; hb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int j = kb + hb * 16 + grp * 4 + i;
        bool ok = j < p.Sk && (!p.causal || j <= qrow);
        float v = ok ? s[hb][i] * p.scale_log2 : -INFINITY;
        s[hb][i] = v;
        bmax = fmaxf(bmax, v);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, WAVE));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, WAVE));
    float mnew = fmaxf(mrun, bmax);
    float corr = (mnew == -INFINITY) ? 1.f : exp2f(mrun - mnew);
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      pv[i] = (mnew == -INFINITY) ? 0.f : exp2f(s[0][i] - mnew);
      pv[4 + i] = (mnew == -INFINITY) ? 0.f : exp2f(s[1][i] - mnew);
      psum += pv[i] + pv[4 + i];
    }
    lrun = lrun * corr + psum;
    mrun = mnew;
    F pf;
    frag_from_floats(pf, pv);
#pragma unroll
    for (int db = 0; db < DP / 16; db++) {
      oacc[db] = oacc[db] * corr;
      const char* vr = sV + (db * 16 + qn) * VPITCH;
      F vf = TR::lfrag2(vr + (grp * 4) * ESZ, vr + (16 + grp * 4) * ESZ);
      mma32(oacc[db], vf, pf);
    }
  }
  float lsum = lrun;
  lsum += __shfl_xor(lsum, 16, WAVE);
  lsum += __shfl_xor(lsum, 32, WAVE);
  float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (qrow < p.Sq) {
#pragma unroll
    for (int db = 0; db < DP / 16; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int d = db * 16 + grp * 4 + i;
        if (d < p.D) TR::store(p.o, (size_t)qrow * p.ldo + (size_t)head * p.D + d, oacc[db][i] * inv);
      }
  }
}

}  // namespace vla
