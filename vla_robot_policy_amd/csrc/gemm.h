// Weight-streaming GEMM for small M (16..600 rows), y = prologue(A) . W^T,
// with fused prologues (row norms, patch gather, merge gather, sinusoidal
// timestep features) and fused epilogues (bias, GELU/SiLU, RoPE, SwiGLU,
// residual / gated residual with per-tile row moments for the next norm).
//
// Layout: A is [M, K] row-major (token-major activations); W is [N, K]
// row-major (PyTorch Linear); each lane's 16-byte W load is exactly the
// MFMA B-operand fragment, so weights go HBM -> registers without LDS. A is
// staged through LDS and shared by the workgroup's waves.
// Pipeline: weights stream through a 4-deep register ring (three chunks in
// flight while a fourth is consumed), activations through a 2-deep register
// ring into a double-buffered LDS tile, one barrier per chunk. Every load is
// a raw buffer load; rows or k beyond the edge get an out-of-range offset
// (the hardware returns zeros), so the loop has no conditional loads and the
// waits are exact.
// Compensated activations (AC = 1): the bf16 A operand is carried as a pair
// hi + lo (hi = bf16(a), lo = bf16(a - hi)) and both halves meet the same
// weight fragment, so the product keeps ~16 significant bits of a at twice
// the MFMA work and LDS traffic; the weights are read once either way. The
// pair is formed from a float source, or read as two bf16 planes (a, a_lo).
// Split-K partial tiles are reduced in a fixed order by the last workgroup
// of each output tile (no float atomics), so results are bitwise
// reproducible run to run.
#pragma once
#include "common.h"
#include "rowstats.h"

namespace vla {

enum AMode { A_BF16 = 0, A_F32 = 1, A_NORM = 2, A_PATCH = 3, A_MERGE = 4, A_TIME = 5 };
enum EMode { E_STORE = 0, E_ROPE = 1, E_SWIGLU = 2, E_RESID = 3 };
enum ActKind { ACT_NONE = 0, ACT_GELU = 1, ACT_SILU = 2 };

struct GemmArgs {
  int M, N, K;
  // ---- A source
  const void* a;         // BF16/F32/NORM/MERGE: matrix [rows, lda]; PATCH: bf16 images
  const void* a_lo;      // BF16 with compensation: remainder plane, same layout as a
  int lda;
  RowStats rs;           // NORM/MERGE: per-tile row moments of the source rows
  int norm_rms;          // 1: RMSNorm (no mean subtraction), 0: LayerNorm
  float eps;
  const float* g;        // per-k gain (NULL = 1)
  int g_plus_one;        // gain is 1 + g[k] (adaLN scale)
  const float* bsh;      // per-k shift (NULL = 0)
  int img, patch, chans, vgrid, n_patches;   // PATCH / MERGE geometry
  int merge, n_merged;                       // MERGE
  int tsteps; float time_scale, freq_base; int half;   // TIME
  // ---- W
  const void* w;
  int ldw;
  const float* wscale;   // fp8: per-row scale
  int n_half;            // SWIGLU: row offset of the up projection
  // ---- epilogue
  const float* bias;
  int act;
  void* c;
  void* c_lo;            // STORE / SWIGLU in bf16: also the remainder plane bf16(v - hi) (NULL = none)
  int ldc;
  int c_f32;
  int q_cols, k_cols, head_dim, pos0; float rope_base;   // ROPE
  float* x; int ldx;                                      // RESID
  int x_init;                                             // RESID: x = y (+ table) instead of x += y
  const float* addrow; int addrow_rows;                   // RESID: + table[m % rows][n]
  const float* gate;                                      // RESID: per-n gate (NULL = 1)
  float2* rs_out;                                         // RESID: [n_tiles_n][M] tile moments of the new stream
  // ---- tiling / split-K (filled by the launcher)
  int split, ksplit;
  float* part;
  unsigned* cnt_tile;
  int n_tiles_n, n_tiles_m;
};

// ---------------------------------------------------------------- weight fragments
// Weights are streamed once per use: loads are non-temporal (CP_NT).
template <typename WT> struct WLoad;
template <> struct WLoad<uint16_t> {
  using raw = uint4;
  using frag = FragBF16;
  static constexpr int ESZ = 2;
  __device__ static raw load(brsrc r, uint32_t off) { return bload16<CP_NT>(r, off); }
  __device__ static frag cvt(raw r) { FragBF16 f; f.v = __builtin_bit_cast(bf16x8, r); return f; }
};
template <> struct WLoad<uint8_t> {
  using raw = uint2;
  using frag = FragBF16;
  static constexpr int ESZ = 1;
  __device__ static raw load(brsrc r, uint32_t off) { return bload8<CP_NT>(r, off); }
  __device__ static frag cvt(raw r) { return fp8x8_to_frag(r); }
};
struct F32x8 { uint4 a, b; };
template <> struct WLoad<float> {
  using raw = F32x8;
  using frag = FragF32;
  static constexpr int ESZ = 4;
  __device__ static raw load(brsrc r, uint32_t off) {
    F32x8 v; v.a = bload16<CP_NT>(r, off); v.b = bload16<CP_NT>(r, off == BUF_OOB ? BUF_OOB : off + 16); return v;
  }
  __device__ static frag cvt(raw r) {
    FragF32 f;
    f.lo = (f32x4){__uint_as_float(r.a.x), __uint_as_float(r.a.y), __uint_as_float(r.a.z), __uint_as_float(r.a.w)};
    f.hi = (f32x4){__uint_as_float(r.b.x), __uint_as_float(r.b.y), __uint_as_float(r.b.z), __uint_as_float(r.b.w)};
    return f;
  }
};

// ---------------------------------------------------------------- LDS A fragments
__device__ __forceinline__ void lds_frag(FragBF16& f, const char* p) {
  f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void lds_frag(FragF32& f, const char* p) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  f.lo = (f32x4){a.x, a.y, a.z, a.w};
  f.hi = (f32x4){b.x, b.y, b.z, b.w};
}
__device__ __forceinline__ void lds_store4(__bf16*, char* p, float4 v) {
  uint2 u; u.x = pack_bf2(v.x, v.y); u.y = pack_bf2(v.z, v.w);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void lds_store4(float*, char* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
// hi = bf16(v) into p, lo = bf16(v - hi) into p + plane
__device__ __forceinline__ void lds_store4_pair(char* p, int plane, float4 v) {
  float hx = bf2f(f2bf(v.x)), hy = bf2f(f2bf(v.y)), hz = bf2f(f2bf(v.z)), hw = bf2f(f2bf(v.w));
  uint2 h; h.x = pack_bf2(hx, hy); h.y = pack_bf2(hz, hw);
  uint2 l; l.x = pack_bf2(v.x - hx, v.y - hy); l.y = pack_bf2(v.z - hz, v.w - hw);
  *reinterpret_cast<uint2*>(p) = h;
  *reinterpret_cast<uint2*>(p + plane) = l;
}

// ---------------------------------------------------------------- cross-workgroup hand-off
// Device-scope relaxed atomic accesses compile to sc1 loads / stores, which
// are coherent across the XCDs' private L2s without the L2 write-back and
// invalidate that a device-scope fence costs.
__device__ __forceinline__ void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_dev(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Called by every thread after its st_dev() stores: waits for them to
// complete, counts this workgroup in *cnt, and returns true for every
// workgroup except the one that arrives last.
__device__ __forceinline__ bool tile_arrive(unsigned* cnt, int expected, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = (old == (unsigned)(expected - 1));
  }
  __syncthreads();
  return !flag[0];
}

constexpr int SPLIT_MAX = 16;

// ---------------------------------------------------------------- tile geometry
template <typename WT, typename CT, int MB, int WN, int WK, int NBW, int AM, int EM, int UU = 4, int AC = 0>
struct GemmTile {
  static constexpr int THREADS = 64 * WN * WK;
  static constexpr int NW = WN * WK;             // waves
  static constexpr int BM = 16 * MB;
  static constexpr int BN = 16 * NBW * WN;
  static constexpr int U = UU;                   // 32-wide k-steps per wave per chunk
  static constexpr int BK = 32 * WK * U;         // chunk width
  static constexpr int ESZ = sizeof(CT);
#ifndef VLA_LDS_PAD
#define VLA_LDS_PAD 16
#endif
  static constexpr int LROW = BK * ESZ + VLA_LDS_PAD;   // LDS row pitch (bytes), padded
  static constexpr int PLANES = AC ? 2 : 1;      // compensated A: hi and lo planes
  static constexpr int APLANE = BM * LROW;
  static constexpr int ABUF = PLANES * APLANE;
  static constexpr int AG = (AM == A_BF16) ? 8 : 4;  // A elements per loader group
  static constexpr int AGROUPS = BM * BK / AG;   // A groups per chunk
  static constexpr int GPT = (AGROUPS + THREADS - 1) / THREADS;  // A groups per thread per chunk
  static constexpr int TPITCH = BN + 4;          // fp32 tile pitch (elements)
  static constexpr int SMEM_A = 2 * ABUF;
  static constexpr int SMEM_T = WK * BM * TPITCH * 4;   // one fp32 tile slice per k-wave
  static constexpr int NROWST = (AM == A_MERGE) ? 4 * BM : BM;   // normaliser entries
  static constexpr int SMEM = (SMEM_A > SMEM_T ? SMEM_A : SMEM_T) + NROWST * 8 + 64;
  // threads serving one normalised row: a power of two, at most 64
  static constexpr int TPR0 = THREADS / NROWST;
  static constexpr int TPR = TPR0 >= 64 ? 64 : TPR0 >= 32 ? 32 : TPR0 >= 16 ? 16 : TPR0 >= 8 ? 8 : TPR0 >= 4 ? 4 : TPR0 >= 2 ? 2 : 1;
  static_assert(THREADS % (BK / AG) == 0, "a thread's A columns must not change between its row groups");
  static_assert(!AC || (sizeof(CT) == 2 && (AM == A_NORM || AM == A_F32 || AM == A_BF16)), "compensated A needs bf16 MFMA");
};

// Raw A registers: bf16 sources keep 8 bf16 (copied to LDS as is; with
// compensation both planes), others 4 floats.
struct U4x2 { uint4 h, l; };
template <int AM, int AC> struct ARaw { using type = float4; };
template <> struct ARaw<A_BF16, 0> { using type = uint4; };
template <> struct ARaw<A_BF16, 1> { using type = U4x2; };

// ---------------------------------------------------------------- kernel
template <typename WT, typename CT, int MB, int WN, int WK, int NBW, int AM, int EM, int UU = 4, int AC = 0>
__global__ __launch_bounds__(64 * WN * WK) void k_gemm(GemmArgs p) {
  using T = GemmTile<WT, CT, MB, WN, WK, NBW, AM, EM, UU, AC>;
  using WL = WLoad<WT>;
  using F = typename Frag<CT>::type;
  using AR = typename ARaw<AM, AC>::type;
  constexpr int NT = T::THREADS, NW = T::NW;
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, U = T::U, GPT = T::GPT;
  constexpr int LROW = T::LROW, TPITCH = T::TPITCH;
  extern __shared__ __align__(16) char smem[];
  char* sA = smem;
  float* sT = reinterpret_cast<float*>(smem);
  float2* sRow = reinterpret_cast<float2*>(smem + (T::SMEM_A > T::SMEM_T ? T::SMEM_A : T::SMEM_T));
  int* sFlag = reinterpret_cast<int*>(sRow + T::NROWST);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wk = wave / WN;

  // ---- XCD-aware tile mapping: the split-K workgroups of one output tile are
  // consecutive logical ids; logical ids [c*G/8, (c+1)*G/8) run on XCD c.
  int bid = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) bid = (bid & 7) * (G >> 3) + (bid >> 3);
  const int s = bid % p.split;
  const int rest = bid / p.split;
  const int nt = rest % p.n_tiles_n;
  const int mt = rest / p.n_tiles_n;
  const int m0 = mt * BM;
  const int kb = s * p.ksplit;
  const int ke = min(p.K, kb + p.ksplit);
  const int nchunks = ke > kb ? (ke - kb + BK - 1) / BK : 0;

  // ---- weight rows of this wave's n-blocks (byte offset of k = 0, or OOB)
  const brsrc wr = make_brsrc(p.w);
  uint32_t wrow[NBW];
#pragma unroll
  for (int j = 0; j < NBW; j++) {
    int jb = wn * NBW + j;                      // n-block index within the tile
    int col = lane & 15;
    int row;
    bool ok;
    if (EM == E_SWIGLU) {
      constexpr int HB = BN / 32 > 0 ? BN / 32 : 1;  // gate n-blocks (first half), then up n-blocks
      int on = nt * (BN / 2) + (jb % HB) * 16 + col;
      ok = on < p.N;
      row = jb < HB ? on : p.n_half + on;
    } else {
      row = nt * BN + jb * 16 + col;
      ok = row < p.N;
    }
    wrow[j] = ok ? (uint32_t)row * (uint32_t)p.ldw * WL::ESZ : BUF_OOB;
  }
  const int kl = (lane >> 4) * 8;               // this lane's offset inside a 32-wide k-step

  using BR = typename WL::raw;
  auto load_b = [&](BR (&br)[U][NBW], int kc) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      int k = kc + (u * WK + wk) * 32 + kl;
#pragma unroll
      for (int j = 0; j < NBW; j++)
        br[u][j] = WL::load(wr, (k < ke && wrow[j] != BUF_OOB) ? wrow[j] + (uint32_t)k * WL::ESZ : BUF_OOB);
    }
  };

  BR b0[U][NBW], b1[U][NBW], b2[U][NBW], b3[U][NBW];

  // ---- per-row normaliser (NORM / MERGE): (value to subtract, 1/std) of
  // every source row of the tile. TPR consecutive threads serve a row; the
  // first LB of each thread's tile partials are requested here, before the
  // first A and W loads, and merged after them (shifted sums, then a fixed
  // butterfly), so they share one memory latency with the weights.
  constexpr int NR = T::NROWST, TPR = T::TPR, LB = 8;
  constexpr bool NORMED = AM == A_NORM || AM == A_MERGE;
  constexpr int NPASS = NORMED ? (NR + NT / TPR - 1) / (NT / TPR) : 1;   // row passes
  float2 rsv[NPASS][NORMED ? LB : 1];
  int rsrc[NPASS];
  const int rr = tid / TPR, jj = tid % TPR;
  const brsrc rsr = make_brsrc(p.rs.part);
  auto load_parts = [&](float2 (&v)[NORMED ? LB : 1], int src, int t0) {
#pragma unroll
    for (int u = 0; u < (NORMED ? LB : 1); u++) {
      int t = t0 + jj + u * TPR;
      uint2 b = bload8(rsr, (src >= 0 && t < p.rs.T) ? ((uint32_t)t * p.rs.M + src) * 8u : BUF_OOB);
      v[u] = make_float2(__uint_as_float(b.x), __uint_as_float(b.y));
    }
  };
  if constexpr (NORMED) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ps++) {
      const int r = ps * (NT / TPR) + rr;
      int src = -1;
      if (r < NR) {
        if (AM == A_NORM) {
          int m = m0 + r;
          src = m < p.M ? m : -1;
        } else {
          int mr = r >> 2, sub = r & 3;         // merged row, 2x2 member
          int m = m0 + mr;
          if (m < p.M && sub < p.merge * p.merge) {
            int per = p.n_merged, im = m / per, mm = m % per;
            int gq = p.vgrid / p.merge;
            int R = mm / gq, C = mm % gq;
            int dy = sub / p.merge, dx = sub % p.merge;
            src = im * p.n_patches + (R * p.merge + dy) * p.vgrid + C * p.merge + dx;
          }
        }
      }
      rsrc[ps] = src;
      load_parts(rsv[ps], src, 0);
    }
  }
  auto row_coeffs = [&]() {
    if constexpr (NORMED) {
#pragma unroll
      for (int ps = 0; ps < NPASS; ps++) {
        const int r = ps * (NT / TPR) + rr;
        const int src = rsrc[ps];
        ShiftSum a;
        for (int t0 = 0;; t0 += LB * TPR) {
#pragma unroll
          for (int u = 0; u < LB; u++) {
            int t = t0 + jj + u * TPR;
            if (src >= 0 && t < p.rs.T) a.add(tile_count(p.rs, t), rsv[ps][u]);
          }
          if (t0 + LB * TPR >= p.rs.T) break;     // uniform: more than LB partials per thread is rare
          load_parts(rsv[ps], src, t0 + LB * TPR);
        }
        float n, mean, m2;
        a.moments(n, mean, m2);
        group_merge(n, mean, m2, TPR);
        if (jj == 0 && r < NR)
          sRow[r] = src >= 0 ? norm_coeffs(make_float2(mean, n > 0.f ? m2 / n : 0.f), p.norm_rms, p.eps)
                             : make_float2(0.f, 0.f);
      }
    }
  };

  // ---- A chunk loader: thread owns AG consecutive k of rows r0 + i*RS
  constexpr int AG = T::AG;
  constexpr int CPR = BK / AG;                  // groups per row
  constexpr int RS = NT / CPR;                  // row stride between a thread's groups
  const int ar0 = tid / CPR;
  const int ac4 = (tid % CPR) * AG;
  const brsrc ars = make_brsrc(p.a);
  constexpr int AESZ = (AM == A_BF16 || AM == A_PATCH) ? 2 : 4;

  auto load_a = [&](AR (&ar)[GPT], int kc) {
    int k = kc + ac4;
#pragma unroll
    for (int i = 0; i < GPT; i++) {
      int r = ar0 + i * RS;
      int m = m0 + r;
      bool ok = r < BM && m < p.M && k < p.K;
      if constexpr (AM == A_BF16 && AC) {
        const uint32_t off = ok ? ((uint32_t)m * p.lda + k) * 2u : BUF_OOB;
        ar[i].h = bload16(ars, off);
        ar[i].l = bload16(make_brsrc(p.a_lo), off);
      } else if constexpr (AM == A_BF16) {
        ar[i] = bload16(ars, ok ? ((uint32_t)m * p.lda + k) * 2u : BUF_OOB);
      } else if constexpr (AM == A_F32 || AM == A_NORM) {
        ar[i] = as_f4(bload16(ars, ok ? ((uint32_t)m * p.lda + k) * 4u : BUF_OOB));
      } else if constexpr (AM == A_PATCH) {
        int im = m / p.n_patches, pi = m % p.n_patches;
        int pr = pi / p.vgrid, pc = pi % p.vgrid;
        int P2 = p.patch * p.patch;
        float t4[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          int kk = k + e;
          int c = kk / P2, rem = kk % P2, ky = rem / p.patch, kx = rem % p.patch;
          uint32_t off = ((((uint32_t)im * p.chans + c) * p.img + pr * p.patch + ky) * p.img + pc * p.patch + kx) * 2u;
          t4[e] = bf2f(bload2(ars, (r < BM && m < p.M && kk < p.K) ? off : BUF_OOB));
        }
        ar[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
      } else if constexpr (AM == A_MERGE) {
        int D = p.lda;
        int per = p.n_merged, im = m / per, mm = m % per;
        int gq = p.vgrid / p.merge;
        int R = mm / gq, C = mm % gq;
        int sub = k / D, d = k % D;
        int dy = sub / p.merge, dx = sub % p.merge;
        int src = im * p.n_patches + (R * p.merge + dy) * p.vgrid + C * p.merge + dx;
        ar[i] = as_f4(bload16(ars, ok ? ((uint32_t)src * D + d) * 4u : BUF_OOB));
      } else {
        ar[i] = make_float4(0.f, 0.f, 0.f, 0.f);   // TIME: computed at store time
      }
    }
  };

  auto store_a = [&](int buf, const AR (&ar)[GPT], int kc) {
    char* base = sA + buf * T::ABUF;
    const int k = kc + ac4;
    float4 ag = make_float4(1.f, 1.f, 1.f, 1.f), ab = make_float4(0.f, 0.f, 0.f, 0.f);
    int sub = 0;
    if constexpr (AM == A_NORM || AM == A_MERGE) {
      int kk = (AM == A_MERGE) ? (k % p.lda) : k;
      if (AM == A_MERGE) sub = k / p.lda;
      if (k < p.K) {
        if (p.g) ag = *reinterpret_cast<const float4*>(p.g + kk);
        if (p.g_plus_one) { ag.x += 1.f; ag.y += 1.f; ag.z += 1.f; ag.w += 1.f; }
        if (p.bsh) ab = *reinterpret_cast<const float4*>(p.bsh + kk);
      }
    }
#pragma unroll
    for (int i = 0; i < GPT; i++) {
      int r = ar0 + i * RS;
      if (r >= BM) break;
      int m = m0 + r;
      bool ok = m < p.M && k < p.K;
      float4 v;
      if constexpr (AM == A_BF16 && AC) {
        // raw copy of both planes
        *reinterpret_cast<uint4*>(base + r * LROW + ac4 * T::ESZ) = ar[i].h;
        *reinterpret_cast<uint4*>(base + T::APLANE + r * LROW + ac4 * T::ESZ) = ar[i].l;
        continue;
      } else if constexpr (AM == A_BF16) {
        // raw copy of 8 bf16 (CT is bf16 for every bf16 source; zeros beyond the edge)
        *reinterpret_cast<uint4*>(base + r * LROW + ac4 * T::ESZ) = ar[i];
        continue;
      } else if constexpr (AM == A_NORM || AM == A_MERGE) {
        v = ar[i];
        float2 rs = sRow[AM == A_MERGE ? r * 4 + sub : r];
        v.x = ok ? (v.x - rs.x) * rs.y * ag.x + ab.x : 0.f;
        v.y = ok ? (v.y - rs.x) * rs.y * ag.y + ab.y : 0.f;
        v.z = ok ? (v.z - rs.x) * rs.y * ag.z + ab.z : 0.f;
        v.w = ok ? (v.w - rs.x) * rs.y * ag.w + ab.w : 0.f;
      } else if constexpr (AM == A_TIME) {
        float t4[4];
        float tm = (float)m / (float)p.tsteps;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          int kk = k + e;
          float val = 0.f;
          if (m < p.M && kk < p.K) {
            int i2 = kk < p.half ? kk : kk - p.half;
            float w = powf(p.freq_base, -(float)i2 / (float)p.half);
            float sn, cs;
            sincosf(p.time_scale * tm * w, &sn, &cs);
            val = kk < p.half ? cs : sn;
          }
          t4[e] = val;
        }
        v = make_float4(t4[0], t4[1], t4[2], t4[3]);
      } else {
        v = ar[i];
      }
      if constexpr (AC) lds_store4_pair(base + r * LROW + ac4 * T::ESZ, T::APLANE, v);
      else lds_store4((CT*)nullptr, base + r * LROW + ac4 * T::ESZ, v);
    }
  };

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < NBW; j++) acc[mb][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // One k-step: every A fragment of the step is requested from LDS before
  // the first MFMA, so the reads overlap instead of each MFMA waiting for
  // its own read.
  auto compute = [&](int buf, const BR (&br)[U][NBW]) {
    const char* base = sA + buf * T::ABUF;
#pragma unroll
    for (int u = 0; u < U; u++) {
      int klocal = (u * WK + wk) * 32 + kl;
      typename WL::frag bf[NBW];
#pragma unroll
      for (int j = 0; j < NBW; j++) bf[j] = WL::cvt(br[u][j]);
      F af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; mb++) lds_frag(af[mb], base + (mb * 16 + (lane & 15)) * LROW + klocal * T::ESZ);
      if constexpr (AC) {
        F al[MB];
#pragma unroll
        for (int mb = 0; mb < MB; mb++) lds_frag(al[mb], base + T::APLANE + (mb * 16 + (lane & 15)) * LROW + klocal * T::ESZ);
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int j = 0; j < NBW; j++) { mma32(acc[mb][j], af[mb], bf[j]); mma32(acc[mb][j], al[mb], bf[j]); }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int j = 0; j < NBW; j++) mma32(acc[mb][j], af[mb], bf[j]);
      }
    }
  };

  // ---- main loop. Chunk c: weights in ring slot c%4 (issued three chunks
  // ahead), activations staged into LDS buffer c%2 from register slot c%2
  // (issued two chunks ahead, stored one chunk ahead). Loads complete in
  // issue order (vmcnt), so each chunk's activations are issued before its
  // weights: waiting for A of chunk c+1 never waits for later weights. Loads
  // past the last chunk read zeros (out-of-range offsets) and are never used.
  AR a0[GPT], a1[GPT];
  load_a(a0, kb); load_b(b0, kb);
  load_a(a1, kb + BK); load_b(b1, kb + BK);
  load_b(b2, kb + 2 * BK);
  // residual inputs of a small unsplit tile are fetched now as well (same
  // element mapping as the epilogue: column tid % BN, rows tid / BN + i * NT / BN)
  constexpr int XPT = (BM * BN + NT - 1) / NT;
  float xpre[XPT <= 4 ? XPT : 1];
  const bool xpref = EM == E_RESID && XPT <= 4 && p.split == 1 && !p.x_init;
  if constexpr (EM == E_RESID && XPT <= 4) {
    if (xpref) {
      const brsrc xr = make_brsrc(p.x);
      const int n = nt * BN + tid % BN;
#pragma unroll
      for (int q = 0; q < XPT; q++) {
        int m = m0 + tid / BN + q * (NT / BN);
        xpre[q] = bloadf(xr, (m < p.M && n < p.N) ? ((uint32_t)m * p.ldx + n) * 4u : BUF_OOB);
      }
    }
  }
  row_coeffs();
  __syncthreads();   // sRow ready
  store_a(0, a0, kb);
  __syncthreads();

#define VLA_GEMM_ITER(C, BCUR, BNEXT3, ARELOAD, ASTORE)                     \
  {                                                                         \
    load_a(ARELOAD, kb + ((C) + 2) * BK);                                   \
    load_b(BNEXT3, kb + ((C) + 3) * BK);                                    \
    if ((C) < nchunks) compute((C) & 1, BCUR);                              \
    store_a(((C) + 1) & 1, ASTORE, kb + ((C) + 1) * BK);                    \
    __syncthreads();                                                        \
  }
  for (int c = 0; c < nchunks; c += 4) {
    VLA_GEMM_ITER(c + 0, b0, b3, a0, a1)
    VLA_GEMM_ITER(c + 1, b1, b0, a1, a0)
    VLA_GEMM_ITER(c + 2, b2, b1, a0, a1)
    VLA_GEMM_ITER(c + 3, b3, b2, a1, a0)
  }
#undef VLA_GEMM_ITER

  // ---- reduce the WK wave slices into the fp32 LDS tile: every slice is
  // written at once (slice w at sT + w * BM * TPITCH), one barrier, then the
  // epilogue threads sum the slices of their elements in slice order
  // (the main loop ended with a barrier: the aliased A buffers are free)
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < NBW; j++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int r = mb * 16 + (lane >> 4) * 4 + i;
        int cidx = (wn * NBW + j) * 16 + (lane & 15);
        sT[(size_t)wk * BM * TPITCH + r * TPITCH + cidx] = acc[mb][j][i];
      }
  __syncthreads();
  // ---- epilogue geometry: NT is a multiple of BN, so each thread keeps one
  // column cc of the tile and visits rows r0e + i * RPT (i < XPT); per-column
  // vectors are loaded once and every thread issues all of its loads before
  // the first wait
  static_assert(NT % BN == 0, "epilogue: each thread owns one column");
  constexpr int RPT = NT / BN;
  constexpr int XPE = (BM + RPT - 1) / RPT;     // elements per thread (threads past BM rows idle)
  const int cc = tid % BN, r0e = tid / BN;
  const int ncol = nt * BN + cc;                // output column (STORE / ROPE / RESID)
  if constexpr (WK > 1) {
    // sum the K slices of this thread's elements (slice order), into slice 0;
    // SWIGLU reads other columns, so every thread finishes before any reads
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT;
      if (r < BM) {
        float v = sT[r * TPITCH + cc];
#pragma unroll
        for (int w = 1; w < WK; w++) v += sT[(size_t)w * BM * TPITCH + r * TPITCH + cc];
        sT[r * TPITCH + cc] = v;
      }
    }
    __syncthreads();
  }

  // residual inputs (unsplit small tiles fetched them before the main loop)
  float xv[EM == E_RESID ? XPE : 1];
  if constexpr (EM == E_RESID) {
    if (!p.x_init) {
      const brsrc xr = make_brsrc(p.x);
#pragma unroll
      for (int i = 0; i < XPE; i++) {
        int m = m0 + r0e + i * RPT;
        if (r0e + i * RPT >= BM) { xv[i] = 0.f; continue; }
        if constexpr (XPT <= 4 && XPE <= XPT) {
          if (xpref) { xv[i] = xpre[i]; continue; }
        }
        xv[i] = bloadf(xr, (m < p.M && ncol < p.N) ? ((uint32_t)m * p.ldx + ncol) * 4u : BUF_OOB);
      }
    }
  }

  // ---- split-K: publish the partial tile; the last arriving workgroup sums
  // all partials in split order. Partials are written with device-scope
  // atomic stores and read with device-coherent (sc1) loads, so the hand-off
  // needs no L2 write-back or invalidate; the counter increment is issued
  // only after every thread's stores have completed.
  if (p.split > 1) {
    const int tile = mt * p.n_tiles_n + nt;
    const size_t tstride = (size_t)p.n_tiles_m * p.n_tiles_n * (BM * BN);
    float* mine = p.part + (size_t)s * tstride + (size_t)tile * (BM * BN);
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT;
      if (r < BM) st_dev(mine + r * BN + cc, sT[r * TPITCH + cc]);
    }
    if (tile_arrive(p.cnt_tile + tile, p.split, sFlag)) return;
    const brsrc pr = make_brsrc(p.part + (size_t)tile * (BM * BN));
    float sum[XPE];
#pragma unroll
    for (int i = 0; i < XPE; i++) sum[i] = 0.f;
    for (int q = 0; q < p.split; q++) {
      float v[XPE];
#pragma unroll
      for (int i = 0; i < XPE; i++)
        v[i] = bloadf<CP_SC1>(pr, r0e + i * RPT < BM ? (uint32_t)(q * tstride + (r0e + i * RPT) * BN + cc) * 4u : BUF_OOB);
#pragma unroll
      for (int i = 0; i < XPE; i++) sum[i] += v[i];
    }
#pragma unroll
    for (int i = 0; i < XPE; i++)
      if (r0e + i * RPT < BM) sT[(r0e + i * RPT) * TPITCH + cc] = sum[i];
    if (tid == 0) p.cnt_tile[tile] = 0u;
    __syncthreads();
  }

  // ---- epilogues
  if constexpr (EM == E_STORE) {
    const bool cok = ncol < p.N;
    const float sc = (p.wscale && cok) ? p.wscale[ncol] : 1.f;
    const float bi = (p.bias && cok) ? p.bias[ncol] : 0.f;
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT, m = m0 + r;
      if (r >= BM || m >= p.M || !cok) continue;
      float v = sT[r * TPITCH + cc] * sc + bi;
      if (p.act == ACT_GELU) v = gelu_erf(v);
      else if (p.act == ACT_SILU) v = silu(v);
      if (p.c_f32) ((float*)p.c)[(size_t)m * p.ldc + ncol] = v;
      else ((uint16_t*)p.c)[(size_t)m * p.ldc + ncol] = f2bf(v);
    }
  } else if constexpr (EM == E_ROPE) {
    const int D = p.head_dim, hd = D >> 1;
    const bool cok = ncol < p.N;
    const bool rot = ncol < p.q_cols + p.k_cols;
    const int d = (ncol < p.q_cols ? ncol : ncol - p.q_cols) % D;
    const int fi = d < hd ? d : d - hd;
    const int pc = d < hd ? cc + hd : cc - hd;           // partner column in the tile
    const int pn = d < hd ? ncol + hd : ncol - hd;
    const float sc = (p.wscale && cok) ? p.wscale[ncol] : 1.f;
    const float sc2 = (p.wscale && cok && rot) ? p.wscale[pn] : 1.f;
    const float theta = exp2f(-2.0f * (float)fi / (float)D * log2f(p.rope_base));
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT, m = m0 + r;
      if (r >= BM || m >= p.M || !cok) continue;
      float v = sT[r * TPITCH + cc] * sc;
      if (rot) {
        float v2 = sT[r * TPITCH + pc] * sc2;
        float sn, cs;
        sincosf((float)(m + p.pos0) * theta, &sn, &cs);
        v = d < hd ? v * cs - v2 * sn : v * cs + v2 * sn;
      }
      if (p.c_f32) ((float*)p.c)[(size_t)m * p.ldc + ncol] = v;
      else ((uint16_t*)p.c)[(size_t)m * p.ldc + ncol] = f2bf(v);
    }
  } else if constexpr (EM == E_SWIGLU) {
    constexpr int BO = BN / 2;
    static_assert(NT % BO == 0, "swiglu epilogue: each thread owns one column");
    constexpr int RPO = NT / BO, XPO = (BM + RPO - 1) / RPO;
    const int co = tid % BO, r0o = tid / BO;
    const int n = nt * BO + co;
    const bool cok = n < p.N;
    const float sg = (p.wscale && cok) ? p.wscale[n] : 1.f;
    const float su = (p.wscale && cok) ? p.wscale[p.n_half + n] : 1.f;
#pragma unroll
    for (int i = 0; i < XPO; i++) {
      int r = r0o + i * RPO, m = m0 + r;
      if (r >= BM || m >= p.M || !cok) continue;
      float gv = sT[r * TPITCH + co] * sg, uv = sT[r * TPITCH + BO + co] * su;
      float a = silu(gv) * uv;
      if (p.c_f32) {
        ((float*)p.c)[(size_t)m * p.ldc + n] = a;
      } else {
        const uint16_t hb = f2bf(a);
        ((uint16_t*)p.c)[(size_t)m * p.ldc + n] = hb;
        if (p.c_lo) ((uint16_t*)p.c_lo)[(size_t)m * p.ldc + n] = f2bf(a - bf2f(hb));
      }
    }
  } else if constexpr (EM == E_RESID) {
    const bool cok = ncol < p.N;
    const float sc = (p.wscale && cok) ? p.wscale[ncol] : 1.f;
    const float bi = (p.bias && cok) ? p.bias[ncol] : 0.f;
    const float ga = (p.gate && cok) ? p.gate[ncol] : 1.f;
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT, m = m0 + r;
      if (r >= BM || m >= p.M || !cok) continue;
      float v = (sT[r * TPITCH + cc] * sc + bi) * ga;
      float xn;
      if (p.x_init) {
        xn = v;
        if (p.addrow) xn += p.addrow[(size_t)(m % p.addrow_rows) * p.N + ncol];
      } else {
        xn = xv[i] + v;
      }
      p.x[(size_t)m * p.ldx + ncol] = xn;
      sT[r * TPITCH + cc] = xn;
    }
    // moments of this tile's columns per row, merged by the stream's next
    // reader: the G = min(BN, 64) lanes holding a row reduce it together
    // (all rows of the tile at once); a wider tile adds its waves' halves
    constexpr int G = BN < 64 ? BN : 64;
    static_assert(BN <= 64, "residual tiles are at most 64 columns wide");
    const int ncols = min(BN, p.N - nt * BN);
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT, m = m0 + r;
      bool live = r < BM && m < p.M && cc < ncols;
      float v = live ? sT[r * TPITCH + cc] : 0.f;
      float sum = v;
#pragma unroll
      for (int o = G >> 1; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, WAVE);
      float mean = sum / (float)ncols;
      float d = live ? v - mean : 0.f;
      float sq = d * d;
#pragma unroll
      for (int o = G >> 1; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, WAVE);
      if (cc == 0 && r < BM && m < p.M) p.rs_out[(size_t)nt * p.M + m] = make_float2(mean, sq);
    }
  }
}

}  // namespace vla
