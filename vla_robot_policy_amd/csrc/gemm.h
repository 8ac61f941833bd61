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
// ring into a double-buffered LDS tile, one barrier per chunk.
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
  int lda;
  RowStats rs;           // NORM/MERGE: row moments of the source rows
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
  int ldc;
  int c_f32;
  int q_cols, k_cols, head_dim, pos0; float rope_base;   // ROPE
  float* x; int ldx;                                      // RESID
  int x_init;                                             // RESID: x = y (+ table) instead of x += y
  const float* addrow; int addrow_rows;                   // RESID: + table[m % rows][n]
  const float* gate;                                      // RESID: per-n gate (NULL = 1)
  float2* rs_out;                                         // RESID: [n_tiles_n][M] tile moments
  // ---- tiling / split-K (filled by the launcher)
  int split, ksplit;
  float* part;
  unsigned* cnt_tile;
  int n_tiles_n, n_tiles_m;
};

// ---------------------------------------------------------------- weight fragments
template <typename WT> struct WLoad;
template <> struct WLoad<uint16_t> {
  using raw = uint4;
  using frag = FragBF16;
  __device__ static raw zero() { return make_uint4(0, 0, 0, 0); }
  __device__ static raw load(const void* w, size_t off) { return *reinterpret_cast<const uint4*>((const uint16_t*)w + off); }
  __device__ static frag cvt(raw r) { FragBF16 f; f.v = __builtin_bit_cast(bf16x8, r); return f; }
};
template <> struct WLoad<uint8_t> {
  using raw = uint2;
  using frag = FragBF16;
  __device__ static raw zero() { return make_uint2(0, 0); }
  __device__ static raw load(const void* w, size_t off) { return *reinterpret_cast<const uint2*>((const uint8_t*)w + off); }
  __device__ static frag cvt(raw r) { return fp8x8_to_frag(r); }
};
struct F32x8 { float4 a, b; };
template <> struct WLoad<float> {
  using raw = F32x8;
  using frag = FragF32;
  __device__ static raw zero() { F32x8 r; r.a = make_float4(0, 0, 0, 0); r.b = r.a; return r; }
  __device__ static raw load(const void* w, size_t off) {
    const float4* p = reinterpret_cast<const float4*>((const float*)w + off);
    F32x8 r; r.a = p[0]; r.b = p[1]; return r;
  }
  __device__ static frag cvt(raw r) { FragF32 f; f.lo = (f32x4){r.a.x, r.a.y, r.a.z, r.a.w}; f.hi = (f32x4){r.b.x, r.b.y, r.b.z, r.b.w}; return f; }
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
template <typename WT, typename CT, int MB, int WN, int WK, int NBW, int AM, int EM, int UU = 4>
struct GemmTile {
  static constexpr int THREADS = 64 * WN * WK;
  static constexpr int NW = WN * WK;             // waves
  static constexpr int BM = 16 * MB;
  static constexpr int BN = 16 * NBW * WN;
  static constexpr int U = UU;                   // 32-wide k-steps per wave per chunk
  static constexpr int BK = 32 * WK * U;         // chunk width
  static constexpr int ESZ = sizeof(CT);
  static constexpr int LROW = BK * ESZ + 16;     // LDS row pitch (bytes), padded
  static constexpr int ABUF = BM * LROW;
  static constexpr int AG = (AM == A_BF16) ? 8 : 4;  // A elements per loader group
  static constexpr int AGROUPS = BM * BK / AG;   // A groups per chunk
  static constexpr int GPT = (AGROUPS + THREADS - 1) / THREADS;  // A groups per thread per chunk
  static constexpr int TPR = (THREADS / (AM == A_MERGE ? 4 * BM : BM)) >= 64 ? 64 : 
                             (THREADS / (AM == A_MERGE ? 4 * BM : BM)) >= 32 ? 32 :
                             (THREADS / (AM == A_MERGE ? 4 * BM : BM)) >= 16 ? 16 :
                             (THREADS / (AM == A_MERGE ? 4 * BM : BM)) >= 8 ? 8 :
                             (THREADS / (AM == A_MERGE ? 4 * BM : BM)) >= 4 ? 4 :
                             (THREADS / (AM == A_MERGE ? 4 * BM : BM)) >= 2 ? 2 : 1;  // threads per normalised row
  static constexpr int MAXL = 32;                // row-moment partials per thread (T <= MAXL * TPR)
  static constexpr int TPITCH = BN + 4;          // fp32 tile pitch (elements)
  static constexpr int SMEM_A = 2 * ABUF;
  static constexpr int SMEM_T = BM * TPITCH * 4;
  static constexpr int NROWST = (AM == A_MERGE) ? 4 * BM : BM;   // normaliser entries
  static constexpr int SMEM = (SMEM_A > SMEM_T ? SMEM_A : SMEM_T) + NROWST * 8 + 64;
  static_assert(THREADS % (BK / AG) == 0, "a thread's A columns must not change between its row groups");
};

// Raw A registers: bf16 sources keep 8 bf16 (copied to LDS as is), others 4 floats.
template <int AM> struct ARaw { using type = float4; };
template <> struct ARaw<A_BF16> { using type = uint4; };

// ---------------------------------------------------------------- kernel
template <typename WT, typename CT, int MB, int WN, int WK, int NBW, int AM, int EM, int UU = 4>
__global__ __launch_bounds__(64 * WN * WK) void k_gemm(GemmArgs p) {
  using T = GemmTile<WT, CT, MB, WN, WK, NBW, AM, EM, UU>;
  using WL = WLoad<WT>;
  using F = typename Frag<CT>::type;
  using AR = typename ARaw<AM>::type;
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

  // ---- weight rows of this wave's n-blocks
  size_t wrow[NBW];
  bool wok[NBW];
#pragma unroll
  for (int j = 0; j < NBW; j++) {
    int jb = wn * NBW + j;                      // n-block index within the tile
    int col = lane & 15;
    if (EM == E_SWIGLU) {
      constexpr int HB = BN / 32 > 0 ? BN / 32 : 1;  // gate n-blocks (first half), then up n-blocks
      int on = nt * (BN / 2) + (jb % HB) * 16 + col;
      wok[j] = on < p.N;
      wrow[j] = (size_t)(jb < HB ? on : p.n_half + on);
    } else {
      int n = nt * BN + jb * 16 + col;
      wok[j] = n < p.N;
      wrow[j] = (size_t)n;
    }
  }
  const int kl = (lane >> 4) * 8;               // this lane's offset inside a 32-wide k-step

  using BR = typename WL::raw;
  auto load_b = [&](BR (&br)[U][NBW], int kc) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      int k = kc + (u * WK + wk) * 32 + kl;
#pragma unroll
      for (int j = 0; j < NBW; j++)
        br[u][j] = (wok[j] && k < ke) ? WL::load(p.w, wrow[j] * (size_t)p.ldw + k) : WL::zero();
    }
  };

  BR b0[U][NBW], b1[U][NBW], b2[U][NBW], b3[U][NBW];

  // ---- per-row normaliser (NORM / MERGE): (mean to subtract, reciprocal std).
  // TPR consecutive threads serve one source row: each merges every TPR-th
  // column tile of it, then the TPR partial results are merged in a fixed
  // butterfly. The partial loads are issued here, before the first A and W
  // loads, and merged after them, so all of them share one memory latency.
  constexpr int NR = T::NROWST, TPR = T::TPR;
  constexpr int MAXL = (AM == A_NORM || AM == A_MERGE) ? T::MAXL : 1;
  constexpr int NPASS = (NR + NT / TPR - 1) / (NT / TPR);   // row passes (1 unless NR > NT / TPR)
  float2 rsv[NPASS][MAXL];
  int rsrc[NPASS];
  const int rr = tid / TPR, jj = tid % TPR;
  if constexpr (AM == A_NORM || AM == A_MERGE) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ps++) {
      const int r = ps * (NT / TPR) + rr;
      int src = -1;
      if (r < NR) {
        if (AM == A_NORM) {
          int m = m0 + r;
          src = m < p.M ? m : -1;
        } else {
          int mr = r >> 2, sub = r & 3;           // merged row, 2x2 member
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
#pragma unroll
      for (int u = 0; u < MAXL; u++) {
        int t = jj + u * TPR;
        rsv[ps][u] = (src >= 0 && t < p.rs.T) ? p.rs.part[(size_t)t * p.rs.M + src] : make_float2(0.f, 0.f);
      }
    }
  }
  auto merge_rows = [&]() {
    if constexpr (AM == A_NORM || AM == A_MERGE) {
#pragma unroll
      for (int ps = 0; ps < NPASS; ps++) {
        const int r = ps * (NT / TPR) + rr;
        const int src = rsrc[ps];
        float n = 0.f, mean = 0.f, m2 = 0.f;
#pragma unroll
        for (int u = 0; u < MAXL; u++) {
          int t = jj + u * TPR;
          if (src >= 0 && t < p.rs.T) moments_merge(n, mean, m2, (float)min(p.rs.tw, p.rs.N - t * p.rs.tw), rsv[ps][u].x, rsv[ps][u].y);
        }
#pragma unroll
        for (int o = TPR >> 1; o >= 1; o >>= 1) {
          float n2 = __shfl_xor(n, o, WAVE), mean2 = __shfl_xor(mean, o, WAVE), m22 = __shfl_xor(m2, o, WAVE);
          moments_merge(n, mean, m2, n2, mean2, m22);
        }
        if (jj == 0 && r < NR) {
          float var = n > 0.f ? m2 / n : 0.f;
          float mu = p.norm_rms ? 0.f : mean;
          float ms = p.norm_rms ? var + mean * mean : var;
          sRow[r] = src >= 0 ? make_float2(mu, rsqrtf(ms + p.eps)) : make_float2(0.f, 0.f);
        }
      }
    }
  };

  // ---- A chunk loader: thread owns AG consecutive k of rows r0 + i*RS
  constexpr int AG = T::AG;
  constexpr int CPR = BK / AG;                  // groups per row
  constexpr int RS = NT / CPR;                  // row stride between a thread's groups
  const int ar0 = tid / CPR;
  const int ac4 = (tid % CPR) * AG;

  auto load_a = [&](AR (&ar)[GPT], int kc) {
    int k = kc + ac4;
#pragma unroll
    for (int i = 0; i < GPT; i++) {
      int r = ar0 + i * RS;
      int m = m0 + r;
      bool ok = r < BM && m < p.M && k < p.K;
      if constexpr (AM == A_BF16) {
        ar[i] = ok ? *reinterpret_cast<const uint4*>((const uint16_t*)p.a + (size_t)m * p.lda + k) : make_uint4(0, 0, 0, 0);
      } else if constexpr (AM == A_F32 || AM == A_NORM) {
        ar[i] = ok ? *reinterpret_cast<const float4*>((const float*)p.a + (size_t)m * p.lda + k) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else if constexpr (AM == A_PATCH) {
        float t4[4] = {0.f, 0.f, 0.f, 0.f};
        if (m < p.M) {
          int im = m / p.n_patches, pi = m % p.n_patches;
          int pr = pi / p.vgrid, pc = pi % p.vgrid;
          int P2 = p.patch * p.patch;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            int kk = k + e;
            if (kk < p.K) {
              int c = kk / P2, rem = kk % P2, ky = rem / p.patch, kx = rem % p.patch;
              size_t off = (((size_t)im * p.chans + c) * p.img + pr * p.patch + ky) * p.img + pc * p.patch + kx;
              t4[e] = bf2f(((const uint16_t*)p.a)[off]);
            }
          }
        }
        ar[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
      } else if constexpr (AM == A_MERGE) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) {
          int D = p.lda;
          int per = p.n_merged, im = m / per, mm = m % per;
          int gq = p.vgrid / p.merge;
          int R = mm / gq, C = mm % gq;
          int sub = k / D, d = k % D;
          int dy = sub / p.merge, dx = sub % p.merge;
          int src = im * p.n_patches + (R * p.merge + dy) * p.vgrid + C * p.merge + dx;
          v = *reinterpret_cast<const float4*>((const float*)p.a + (size_t)src * D + d);
        }
        ar[i] = v;
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
      if constexpr (AM == A_BF16) {
        // raw copy of 8 bf16 (CT is bf16 for every bf16 source)
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
      lds_store4((CT*)nullptr, base + r * LROW + ac4 * T::ESZ, v);
    }
  };

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < NBW; j++) acc[mb][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const BR (&br)[U][NBW]) {
    const char* base = sA + buf * T::ABUF;
#pragma unroll
    for (int u = 0; u < U; u++) {
      int klocal = (u * WK + wk) * 32 + kl;
      typename WL::frag bf[NBW];
#pragma unroll
      for (int j = 0; j < NBW; j++) bf[j] = WL::cvt(br[u][j]);
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        F af;
        lds_frag(af, base + (mb * 16 + (lane & 15)) * LROW + klocal * T::ESZ);
#pragma unroll
        for (int j = 0; j < NBW; j++) mma32(acc[mb][j], af, bf[j]);
      }
    }
  };

  // ---- main loop. Chunk c: weights in ring slot c%4 (issued three chunks
  // ahead), activations staged into LDS buffer c%2 from register slot c%2
  // (issued two chunks ahead, stored one chunk ahead). Loads complete in
  // issue order (vmcnt), so each chunk's activations are issued before its
  // weights: waiting for A of chunk c+1 never waits for later weights.
  AR a0[GPT], a1[GPT];
  if (nchunks > 0) { load_a(a0, kb); load_b(b0, kb); }
  if (nchunks > 1) { load_a(a1, kb + BK); load_b(b1, kb + BK); }
  if (nchunks > 2) load_b(b2, kb + 2 * BK);
  // residual inputs of a small unsplit tile are fetched now as well
  constexpr int XPT = (BM * BN + NT - 1) / NT;
  float xpre[XPT <= 4 ? XPT : 1];
  const bool xpref = EM == E_RESID && XPT <= 4 && p.split == 1 && !p.x_init;
  if constexpr (EM == E_RESID && XPT <= 4) {
    if (xpref) {
#pragma unroll
      for (int q = 0; q < XPT; q++) {
        int e = tid + q * NT;
        int r = e / BN, cc = e % BN;
        int m = m0 + r, n = nt * BN + cc;
        xpre[q] = (e < BM * BN && m < p.M && n < p.N) ? p.x[(size_t)m * p.ldx + n] : 0.f;
      }
    }
  }
  merge_rows();
  __syncthreads();   // sRow ready
  if (nchunks > 0) store_a(0, a0, kb);
  __syncthreads();

#define VLA_GEMM_ITER(C, BCUR, BNEXT3, ARELOAD, ASTORE)                     \
  if ((C) < nchunks) {                                                      \
    if ((C) + 2 < nchunks) load_a(ARELOAD, kb + ((C) + 2) * BK);            \
    if ((C) + 3 < nchunks) load_b(BNEXT3, kb + ((C) + 3) * BK);             \
    compute((C) & 1, BCUR);                                                 \
    if ((C) + 1 < nchunks) store_a(((C) + 1) & 1, ASTORE, kb + ((C) + 1) * BK); \
    __syncthreads();                                                        \
  }
  for (int c = 0; c < nchunks; c += 4) {
    VLA_GEMM_ITER(c + 0, b0, b3, a0, a1)
    VLA_GEMM_ITER(c + 1, b1, b0, a1, a0)
    VLA_GEMM_ITER(c + 2, b2, b1, a0, a1)
    VLA_GEMM_ITER(c + 3, b3, b2, a1, a0)
  }
#undef VLA_GEMM_ITER

  // ---- reduce the WK wave slices into the fp32 LDS tile (fixed order)
#pragma unroll 1
  for (int w = 0; w < WK; w++) {
    if (wk == w) {
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int j = 0; j < NBW; j++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            int r = mb * 16 + (lane >> 4) * 4 + i;
            int cidx = (wn * NBW + j) * 16 + (lane & 15);
            float* d = sT + r * TPITCH + cidx;
            *d = (w == 0) ? acc[mb][j][i] : *d + acc[mb][j][i];
          }
    }
    __syncthreads();
  }

  // ---- split-K: publish the partial tile; the last arriving workgroup sums
  // all partials in split order. Partials are written and read with
  // device-scope atomic accesses (coherent across XCDs without flushing or
  // invalidating the L2); the counter increment is issued only after every
  // thread's stores have completed.
  if (p.split > 1) {
    const int tile = mt * p.n_tiles_n + nt;
    const size_t tstride = (size_t)p.n_tiles_m * p.n_tiles_n * (BM * BN);
    float* mine = p.part + (size_t)s * tstride + (size_t)tile * (BM * BN);
    for (int e = tid; e < BM * BN; e += NT) st_dev(mine + e, sT[(e / BN) * TPITCH + (e % BN)]);
    if (tile_arrive(p.cnt_tile + tile, p.split, sFlag)) return;
    const float* base = p.part + (size_t)tile * (BM * BN);
    for (int e = tid; e < BM * BN; e += NT) {
      float v[SPLIT_MAX];
#pragma unroll
      for (int q = 0; q < SPLIT_MAX; q++) v[q] = q < p.split ? ld_dev(base + (size_t)q * tstride + e) : 0.f;
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < SPLIT_MAX; q++) sum += v[q];
      sT[(e / BN) * TPITCH + (e % BN)] = sum;
    }
    if (tid == 0) p.cnt_tile[tile] = 0u;
    __syncthreads();
  }

  // ---- epilogues
  if constexpr (EM == E_STORE) {
    for (int e = tid; e < BM * BN; e += NT) {
      int r = e / BN, cc = e % BN;
      int m = m0 + r, n = nt * BN + cc;
      if (m >= p.M || n >= p.N) continue;
      float v = sT[r * TPITCH + cc];
      if (p.wscale) v *= p.wscale[n];
      if (p.bias) v += p.bias[n];
      if (p.act == ACT_GELU) v = gelu_erf(v);
      else if (p.act == ACT_SILU) v = silu(v);
      if (p.c_f32) ((float*)p.c)[(size_t)m * p.ldc + n] = v;
      else ((uint16_t*)p.c)[(size_t)m * p.ldc + n] = f2bf(v);
    }
  } else if constexpr (EM == E_ROPE) {
    const int D = p.head_dim, hd = D >> 1;
    const float l2b = log2f(p.rope_base);
    for (int e = tid; e < BM * BN; e += NT) {
      int r = e / BN, cc = e % BN;
      int m = m0 + r, n = nt * BN + cc;
      if (m >= p.M || n >= p.N) continue;
      float v = sT[r * TPITCH + cc];
      if (p.wscale) v *= p.wscale[n];
      if (n < p.q_cols + p.k_cols) {
        int d = (n < p.q_cols ? n : n - p.q_cols) % D;
        int i = d < hd ? d : d - hd;
        int pc = d < hd ? cc + hd : cc - hd;
        int pn = d < hd ? n + hd : n - hd;
        float v2 = sT[r * TPITCH + pc];
        if (p.wscale) v2 *= p.wscale[pn];
        float theta = exp2f(-2.0f * (float)i / (float)D * l2b);
        float sn, cs;
        sincosf((float)(m + p.pos0) * theta, &sn, &cs);
        v = d < hd ? v * cs - v2 * sn : v * cs + v2 * sn;
      }
      if (p.c_f32) ((float*)p.c)[(size_t)m * p.ldc + n] = v;
      else ((uint16_t*)p.c)[(size_t)m * p.ldc + n] = f2bf(v);
    }
  } else if constexpr (EM == E_SWIGLU) {
    constexpr int BO = BN / 2;
    for (int e = tid; e < BM * BO; e += NT) {
      int r = e / BO, cc = e % BO;
      int m = m0 + r, n = nt * BO + cc;
      if (m >= p.M || n >= p.N) continue;
      float gv = sT[r * TPITCH + cc], uv = sT[r * TPITCH + BO + cc];
      if (p.wscale) { gv *= p.wscale[n]; uv *= p.wscale[p.n_half + n]; }
      float a = silu(gv) * uv;
      if (p.c_f32) ((float*)p.c)[(size_t)m * p.ldc + n] = a;
      else ((uint16_t*)p.c)[(size_t)m * p.ldc + n] = f2bf(a);
    }
  } else if constexpr (EM == E_RESID) {
#pragma unroll 1
    for (int q = 0, e = tid; e < BM * BN; q++, e += NT) {
      int r = e / BN, cc = e % BN;
      int m = m0 + r, n = nt * BN + cc;
      if (m >= p.M || n >= p.N) continue;
      float v = sT[r * TPITCH + cc];
      if (p.wscale) v *= p.wscale[n];
      if (p.bias) v += p.bias[n];
      if (p.gate) v *= p.gate[n];
      float* xp = p.x + (size_t)m * p.ldx + n;
      float xn;
      if (p.x_init) {
        xn = v;
        if (p.addrow) xn += p.addrow[(size_t)(m % p.addrow_rows) * p.N + n];
      } else {
        float xo = 0.f;
        bool got = false;
        if constexpr (XPT <= 4) {
#pragma unroll
          for (int qq = 0; qq < XPT; qq++)
            if (xpref && qq == q) { xo = xpre[qq]; got = true; }
        }
        if (!got) xo = *xp;
        xn = xo + v;
      }
      *xp = xn;
      sT[r * TPITCH + cc] = xn;
    }
    __syncthreads();
    // per-row moments of this tile's columns, merged by the next reader
    const int ncols = min(BN, p.N - nt * BN);
    for (int r = wave; r < BM; r += NW) {
      int m = m0 + r;
      if (m >= p.M) continue;          // wave-uniform
      float sum = 0.f;
      for (int cc = lane; cc < ncols; cc += 64) sum += sT[r * TPITCH + cc];
      float mean = wave_sum(sum) / (float)ncols;
      float sq = 0.f;
      for (int cc = lane; cc < ncols; cc += 64) { float d = sT[r * TPITCH + cc] - mean; sq += d * d; }
      float m2 = wave_sum(sq);
      if (lane == 0) p.rs_out[(size_t)nt * p.M + m] = make_float2(mean, m2);
    }
  }
}

}  // namespace vla
