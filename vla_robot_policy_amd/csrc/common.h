// Device-side building blocks shared by the kernels of libvla (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr int WAVE = 64;

// ---------------------------------------------------------------- scalar conversion
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- 8-wide fragments
// A fragment is the 8 contraction-dimension values one lane contributes to a
// 16x16x32 MFMA step. For bf16 it is one bf16x8 register quad; for fp32 it is
// 8 floats fed to 8 consecutive 16x16x4 fp32 MFMAs. Lane group g = lane/16
// owns contraction indices 8g..8g+7 of each 32-wide step in both cases (for
// fp32, MFMA j pairs index 8g+j of A with 8g+j of B), so any operand loaded
// with that convention on both sides contracts correctly.
struct FragBF16 {
  bf16x8 v;
};
struct FragF32 {
  f32x4 lo, hi;
};

template <typename T> struct Frag;
template <> struct Frag<__bf16> { using type = FragBF16; };
template <> struct Frag<float> { using type = FragF32; };

__device__ __forceinline__ void mma32(f32x4& acc, const FragBF16& a, const FragBF16& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma32(f32x4& acc, const FragF32& a, const FragF32& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

__device__ __forceinline__ FragBF16 zero_frag(FragBF16) {
  FragBF16 f;
  f.v = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
  return f;
}
__device__ __forceinline__ FragF32 zero_frag(FragF32) {
  FragF32 f;
  f.lo = (f32x4){0, 0, 0, 0};
  f.hi = (f32x4){0, 0, 0, 0};
  return f;
}

// Build a fragment from 8 floats (rounding to bf16 when needed).
__device__ __forceinline__ void frag_from_floats(FragBF16& f, const float* x) {
  uint4 u;
  u.x = pack_bf2(x[0], x[1]);
  u.y = pack_bf2(x[2], x[3]);
  u.z = pack_bf2(x[4], x[5]);
  u.w = pack_bf2(x[6], x[7]);
  f.v = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void frag_from_floats(FragF32& f, const float* x) {
  f.lo = (f32x4){x[0], x[1], x[2], x[3]};
  f.hi = (f32x4){x[4], x[5], x[6], x[7]};
}

// ---------------------------------------------------------------- fp8 (OCP E4M3FN, gfx950 native)
// 8 codes (two dwords) -> bf16 fragment. Every E4M3FN value is exact in bf16.
__device__ __forceinline__ FragBF16 fp8x8_to_frag(uint2 codes) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, 1.0f, true);
  FragBF16 f;
  f.v = (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return f;
}

// Eight int8 codes widened to bf16: |code| <= 127 needs 7 significant bits,
// so the float32 value's upper half is the exact bf16
__device__ __forceinline__ FragBF16 int8x8_to_frag(uint2 codes) {
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t w = j < 2 ? codes.x : codes.y;
    const int sh = (j & 1) * 16;
    const float lo = (float)(int8_t)(w >> sh), hi = (float)(int8_t)(w >> (sh + 8));
    h[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  FragBF16 f;
  f.v = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  return f;
}

__device__ __forceinline__ float fp8_to_f32(uint8_t c) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
  return v[0];
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads return zeros for an offset at or beyond the resource's
// size, so edge tiles select an out-of-range offset instead of branching:
// every load of a loop is then unconditional and the compiler can wait for
// exactly the loads a step needs (vmcnt) instead of draining the queue.
typedef __amdgpu_buffer_rsrc_t brsrc;
constexpr uint32_t BUF_LIMIT = 0x7FFFFFF0u;   // resource size; larger offsets read 0
constexpr uint32_t BUF_OOB = BUF_LIMIT;       // the offset used for "no element"
constexpr int CP_NONE = 0, CP_NT = 2, CP_SC1 = 16;   // cache policy bits of a buffer access

__device__ __forceinline__ brsrc make_brsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)BUF_LIMIT, 0x00020000);
}
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
template <int CP = CP_NONE>
__device__ __forceinline__ uint4 bload16(brsrc r, uint32_t off) {
  i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int CP = CP_NONE>
__device__ __forceinline__ uint2 bload8(brsrc r, uint32_t off) {
  i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ float4 as_f4(uint4 u) {
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
template <int CP = CP_NONE>
__device__ __forceinline__ float bloadf(brsrc r, uint32_t off) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP));
}
template <int CP = CP_NONE>
__device__ __forceinline__ uint16_t bload2(brsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP);
}

// ---------------------------------------------------------------- wave reductions
// DPP lane moves within rows of 16 lanes (quad permutes and row rotations)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each row of 16 lanes, in every lane of the row: swap neighbours,
// swap pairs, then add the quads 4 and 8 lanes around the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);   // row_ror:4
  v += dpp_f<0x128>(v);   // row_ror:8
  return v;
}
// Sum over the whole wave (wave-uniform result): row sums, then the four
// rows' sums read from lanes 0, 16, 32, 48 in that order.
__device__ __forceinline__ float wave_sum_rows(float v) {
  v = row16_sum(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Exact GELU z * Phi(z) and SiLU z / (1 + e^-z), with the device math library.
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Chan et al. pairwise merge of (count, mean, M2) partial moments.
__device__ __forceinline__ void moments_merge(float& n, float& mean, float& m2, float nb, float meanb, float m2b) {
  if (nb <= 0.f) return;
  float nn = n + nb;
  float d = meanb - mean;
  mean += d * (nb / nn);
  m2 += m2b + d * d * (n * nb / nn);
  n = nn;
}

}  // namespace vla
