// Weight-streaming GEMM for small M (16..600 rows), y = prologue(A) . W^T,
// with fused prologues (row norms, patch gather, merge gather, sinusoidal
// timestep features) and fused epilogues (bias, GELU/SiLU, RoPE, SwiGLU,
// residual / gated residual with per-tile row moments for the next norm).
//
// Layout: A is [M, K] row-major (token-major activations); W is [N, K]
// row-major (PyTorch Linear). bf16 and fp8 weights are read in whole chunk
// rows (runs of 128-1024 contiguous bytes: a wave's load covers a few rows,
// which HBM serves far better than the 16 rows x 64 bytes of an MFMA
// fragment) and staged through LDS, from where each wave reads its MFMA
// B fragments; fp32 weights (small reference-precision layers) go straight
// to registers in fragment order. A is staged through LDS and shared by the
// workgroup's waves.
// Pipeline: weights stream through a 4-deep register ring (three chunks in
// flight while a fourth is stored), activations through a 2-deep register
// ring, both into double-buffered LDS tiles, one barrier per chunk. Every load is
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
#include <type_traits>
#include "common.h"
#include "rowstats.h"

namespace vla {

enum AMode { A_BF16 = 0, A_F32 = 1, A_NORM = 2, A_PATCH = 3, A_MERGE = 4, A_TIME = 5, A_FP8 = 6, A_I8 = 7 };
// 8-bit activation codes with a per-row scale (W8A8)
constexpr bool a_codes(int am) { return am == A_FP8 || am == A_I8; }
enum EMode { E_STORE = 0, E_ROPE = 1, E_SWIGLU = 2, E_RESID = 3 };
enum ActKind { ACT_NONE = 0, ACT_GELU = 1, ACT_SILU = 2 };

struct GemmArgs {
  int M, N, K;
  // ---- A source
  const void* a;         // BF16/F32/NORM/MERGE: matrix [rows, lda]; PATCH: bf16 images
  const void* a_lo;      // BF16 with compensation: remainder plane, same layout as a
  const float* a_scale;  // FP8 / I8: E4M3FN or int8 codes [rows, lda] in a, one float32 scale per row here
                         // (W8A8: the codes are staged as bytes and widened to bf16 at fragment
                         // load, which is exact, so the bf16 MFMA forms exact products)
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
  int qk_norm; float qk_eps;                              // ROPE: per-head RMSNorm of q and k first
  const float* qn_g; const float* kn_g;                   //   with gains [head_dim]; tiles hold whole heads
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
template <> struct WLoad<int8_t> {
  using raw = uint2;
  using frag = FragBF16;
  static constexpr int ESZ = 1;
  __device__ static raw load(brsrc r, uint32_t off) { return bload8<CP_NT>(r, off); }
  __device__ static frag cvt(raw r) { return int8x8_to_frag(r); }
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
  static constexpr int ESZ = a_codes(AM) ? 1 : (int)sizeof(CT);   // bytes per A element in LDS
#ifndef VLA_LDS_PAD
#define VLA_LDS_PAD 16
#endif
  static constexpr int LROW = BK * ESZ + VLA_LDS_PAD;   // LDS row pitch (bytes), padded
  static constexpr int PLANES = AC ? 2 : 1;      // compensated A: hi and lo planes
  static constexpr int APLANE = BM * LROW;
  static constexpr int ABUF = PLANES * APLANE;
  static constexpr int AG = (AM == A_BF16) ? 8 : a_codes(AM) ? 16 : 4;  // A elements per loader group
  static constexpr int AGROUPS = BM * BK / AG;   // A groups per chunk
  static constexpr int GPT = (AGROUPS + THREADS - 1) / THREADS;  // A groups per thread per chunk
  static constexpr int TPITCH = BN + 4;          // fp32 tile pitch (elements)
  // weights through LDS (bf16 / fp8): [BN][BK] with padded rows; each thread
  // loads NWL 16-byte groups per chunk, LPR groups make one chunk row
  static constexpr bool WLDS = sizeof(WT) <= 2;
  static constexpr int WROW = BK * (int)sizeof(WT) + 16;
  static constexpr int WBUF = WLDS ? BN * WROW : 0;
  static constexpr int LPR = BK * (int)sizeof(WT) / 16;
  static constexpr int NWL = WLDS ? BN * LPR / THREADS : 1;
  static_assert(!WLDS || ((BK * (int)sizeof(WT)) % 16 == 0 && (BN * LPR) % THREADS == 0 && THREADS % LPR == 0),
                "weight chunk rows must split evenly into 16-byte groups over the workgroup");
  static constexpr int SMEM_A = 2 * ABUF + 2 * WBUF;
  static constexpr int SMEM_T = WK * BM * TPITCH * 4;   // one fp32 tile slice per k-wave
  static constexpr int NROWST = (AM == A_MERGE) ? 4 * BM : BM;   // normaliser entries
  static constexpr int SMEM = (SMEM_A > SMEM_T ? SMEM_A : SMEM_T) + NROWST * 8 + 64;
  static_assert(SMEM <= 160 * 1024, "tile exceeds the 160 KiB of LDS of a compute unit");
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
template <> struct ARaw<A_FP8, 0> { using type = uint4; };
template <> struct ARaw<A_I8, 0> { using type = uint4; };

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

  // ---- per-column epilogue vectors, requested now so that their latency
  // hides under the main loop instead of opening the epilogue: the thread
  // serves tile column tid % BN (SwiGLU: tid % (BN / 2)) in every epilogue.
  // Absent vectors read as 0 through an out-of-range offset.
  const int ecol = EM == E_SWIGLU ? nt * (BN / 2) + tid % (BN / 2) : nt * BN + tid % BN;
  const bool ecok = ecol < p.N;
  int ecol2 = ecol;   // RoPE: the partner column; SwiGLU: the up column
  if constexpr (EM == E_ROPE) {
    const int D = p.head_dim, hd = D >> 1;
    const int d = (ecol < p.q_cols ? ecol : ecol - p.q_cols) % D;
    ecol2 = ecol < p.q_cols + p.k_cols ? (d < hd ? ecol + hd : ecol - hd) : ecol;
  }
  if constexpr (EM == E_SWIGLU) ecol2 = p.n_half + ecol;
  const float e_sc = bloadf(make_brsrc(p.wscale), (p.wscale && ecok) ? (uint32_t)ecol * 4u : BUF_OOB);
  const float e_sc2 = (EM == E_ROPE || EM == E_SWIGLU)
                          ? bloadf(make_brsrc(p.wscale), (p.wscale && ecok) ? (uint32_t)ecol2 * 4u : BUF_OOB) : 0.f;
  const float e_bi = (EM == E_STORE || EM == E_RESID)
                         ? bloadf(make_brsrc(p.bias), (p.bias && ecok) ? (uint32_t)ecol * 4u : BUF_OOB) : 0.f;
  const float e_ga = EM == E_RESID ? bloadf(make_brsrc(p.gate), (p.gate && ecok) ? (uint32_t)ecol * 4u : BUF_OOB) : 0.f;
  // QK-norm gains of the column and of its RoPE partner (a tile lies within
  // the query columns or within the key / value columns, so the gain vector
  // is the same for the whole workgroup)
  float e_g1 = 1.f, e_g2 = 1.f;
  if constexpr (EM == E_ROPE) {
    if (p.qk_norm) {
      const int D = p.head_dim, hd = D >> 1;
      const int d1 = (ecol < p.q_cols ? ecol : ecol - p.q_cols) % D, d2 = d1 < hd ? d1 + hd : d1 - hd;
      const brsrc gr = make_brsrc(nt * BN < p.q_cols ? p.qn_g : p.kn_g);
      const bool ok = ecol < p.q_cols + p.k_cols;
      e_g1 = bloadf(gr, ok ? (uint32_t)d1 * 4u : BUF_OOB);
      e_g2 = bloadf(gr, ok ? (uint32_t)d2 * 4u : BUF_OOB);
    }
  }

  // ---- weight row of tile row `row` (byte offset of k = 0, or OOB)
  auto wrow_of = [&](int row) -> uint32_t {
    const int jb = row >> 4, col = row & 15;   // n-block within the tile, row within it
    int wr_;
    bool ok;
    if (EM == E_SWIGLU) {
      constexpr int HB = BN / 32 > 0 ? BN / 32 : 1;  // gate n-blocks (first half), then up n-blocks
      int on = nt * (BN / 2) + (jb % HB) * 16 + col;
      ok = on < p.N;
      wr_ = jb < HB ? on : p.n_half + on;
    } else {
      wr_ = nt * BN + row;
      ok = wr_ < p.N;
    }
    return ok ? (uint32_t)wr_ * (uint32_t)p.ldw * WL::ESZ : BUF_OOB;
  };
  const brsrc wr = make_brsrc(p.w);
  const int kl = (lane >> 4) * 8;               // this lane's offset inside a 32-wide k-step

  // fp32 weights: fragments straight to registers (rows of this wave's n-blocks)
  using BR = typename WL::raw;
  uint32_t wrow[NBW];
#pragma unroll
  for (int j = 0; j < NBW; j++) wrow[j] = T::WLDS ? BUF_OOB : wrow_of((wn * NBW + j) * 16 + (lane & 15));
  auto load_b = [&](BR (&br)[U][NBW], int kc) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      int k = kc + (u * WK + wk) * 32 + kl;
#pragma unroll
      for (int j = 0; j < NBW; j++)
        br[u][j] = WL::load(wr, (k < ke && wrow[j] != BUF_OOB) ? wrow[j] + (uint32_t)k * WL::ESZ : BUF_OOB);
    }
  };

  // bf16 / fp8 weights: whole chunk rows in 16-byte groups; thread tid takes
  // group tid % LPR of rows tid / LPR + i * NT / LPR
  constexpr bool WLDS = T::WLDS;
  constexpr int LPR = T::LPR, NWL = T::NWL, WROW = T::WROW;
  char* sW = smem + 2 * T::ABUF;
  const int wg16 = tid % LPR, wr0 = tid / LPR;
  uint32_t wro[NWL];
#pragma unroll
  for (int i = 0; i < NWL; i++) wro[i] = WLDS ? wrow_of(wr0 + i * (NT / LPR)) : BUF_OOB;
  auto load_w = [&](uint4 (&v)[NWL], int kc) {
    const int k = kc + wg16 * (16 / WL::ESZ);
#pragma unroll
    for (int i = 0; i < NWL; i++) v[i] = bload16<CP_NT>(wr, (k < ke && wro[i] != BUF_OOB) ? wro[i] + (uint32_t)k * WL::ESZ : BUF_OOB);
  };
  auto store_w = [&](int buf, const uint4 (&v)[NWL]) {
    char* base = sW + buf * T::WBUF + wg16 * 16;
#pragma unroll
    for (int i = 0; i < NWL; i++) *reinterpret_cast<uint4*>(base + (wr0 + i * (NT / LPR)) * WROW) = v[i];
  };
  // the weight ring: one register slot per chunk in flight
  using RR = std::conditional_t<WLDS, uint4[NWL], BR[U][NBW]>;
  auto load_ring = [&](RR& r, int kc) {
    if constexpr (WLDS) load_w(r, kc);
    else load_b(r, kc);
  };
  auto store_ring = [&](int buf, const RR& r) {
    if constexpr (WLDS) store_w(buf, r);
  };

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
      } else if constexpr (a_codes(AM)) {
        ar[i] = bload16(ars, ok ? (uint32_t)m * p.lda + k : BUF_OOB);
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
      } else if constexpr (AM == A_BF16 || a_codes(AM)) {
        // raw copy of 8 bf16 or 16 fp8 codes (CT is the source type; zeros beyond the edge)
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
      else if constexpr (!a_codes(AM)) lds_store4((CT*)nullptr, base + r * LROW + ac4 * T::ESZ, v);
    }
  };

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < NBW; j++) acc[mb][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // W8A8 integer: int8 codes of both operands meet in int8 MFMAs with exact
  // int32 accumulation. One 16x16x64 instruction takes two of the 32-wide
  // k-steps: each lane passes its 8 codes of both steps, on the A and the B
  // side alike, so the pairs of k it multiplies are the same.
  constexpr bool I8MMA = AM == A_I8 && std::is_same_v<WT, int8_t> && T::WLDS;
  static_assert(!I8MMA || U % 2 == 0, "int8 MFMAs take the k-steps in pairs");
  i32x4 acci[I8MMA ? MB : 1][I8MMA ? NBW : 1];
  if constexpr (I8MMA) {
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int j = 0; j < NBW; j++) acci[mb][j] = (i32x4){0, 0, 0, 0};
  }

  // One k-step: every A and B fragment of the step is requested from LDS
  // before the first MFMA, so the reads overlap instead of each MFMA waiting
  // for its own read.
  auto compute = [&](int buf, const RR& br) {
    const char* base = sA + buf * T::ABUF;
    const char* wbase = sW + buf * T::WBUF;
    if constexpr (I8MMA) {
      auto pair = [](const char* p0, const char* p1) {
        const uint2 lo = *reinterpret_cast<const uint2*>(p0), hi = *reinterpret_cast<const uint2*>(p1);
        return (i32x4){(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
      };
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const int k0 = (u * WK + wk) * 32 + kl, k1 = ((u + 1) * WK + wk) * 32 + kl;
        i32x4 bi[NBW], ai[MB];
#pragma unroll
        for (int j = 0; j < NBW; j++) {
          const char* wp = wbase + ((wn * NBW + j) * 16 + (lane & 15)) * WROW;
          bi[j] = pair(wp + k0, wp + k1);
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
          const char* ap = base + (mb * 16 + (lane & 15)) * LROW;
          ai[mb] = pair(ap + k0, ap + k1);
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int j = 0; j < NBW; j++) acci[mb][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai[mb], bi[j], acci[mb][j], 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      int klocal = (u * WK + wk) * 32 + kl;
      typename WL::frag bf[NBW];
      if constexpr (WLDS) {
#pragma unroll
        for (int j = 0; j < NBW; j++) {
          const char* wp = wbase + ((wn * NBW + j) * 16 + (lane & 15)) * WROW + klocal * WL::ESZ;
          if constexpr (WL::ESZ == 2) bf[j] = WL::cvt(*reinterpret_cast<const uint4*>(wp));
          else bf[j] = WL::cvt(*reinterpret_cast<const uint2*>(wp));
        }
      } else {
#pragma unroll
        for (int j = 0; j < NBW; j++) bf[j] = WL::cvt(br[u][j]);
      }
      F af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        const char* ap = base + (mb * 16 + (lane & 15)) * LROW + klocal * T::ESZ;
        if constexpr (AM == A_FP8) af[mb] = fp8x8_to_frag(*reinterpret_cast<const uint2*>(ap));
        else if constexpr (AM == A_I8) af[mb] = int8x8_to_frag(*reinterpret_cast<const uint2*>(ap));
        else lds_frag(af[mb], ap);
      }
      if constexpr (AC) {
        F al[MB];
#pragma unroll
        for (int mb = 0; mb < MB; mb++) lds_frag(al[mb], base + T::APLANE + (mb * 16 + (lane & 15)) * LROW + klocal * T::ESZ);
        // every hi product before the lo ones: MFMAs into one accumulator
        // are then MB * NBW instructions apart instead of back to back
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int j = 0; j < NBW; j++) mma32(acc[mb][j], af[mb], bf[j]);
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int j = 0; j < NBW; j++) mma32(acc[mb][j], al[mb], bf[j]);
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
          for (int j = 0; j < NBW; j++) mma32(acc[mb][j], af[mb], bf[j]);
      }
    }
  };

  // ---- main loop. Chunk c: weights in ring slot c%4 (issued three chunks
  // ahead, stored to LDS buffer c%2 one chunk ahead), activations staged into
  // LDS buffer c%2 from register slot c%2 (issued two chunks ahead, stored one
  // chunk ahead). Loads complete in issue order (vmcnt), so each chunk's
  // activations are issued before its weights: waiting for A of chunk c+1
  // never waits for later weights. Loads past the last chunk read zeros
  // (out-of-range offsets) and are never used.
  AR a0[GPT], a1[GPT];
  RR r0, r1, r2, r3;
  load_a(a0, kb); load_ring(r0, kb);
  load_a(a1, kb + BK); load_ring(r1, kb + BK);
  load_ring(r2, kb + 2 * BK);
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
  store_ring(0, r0);
  __syncthreads();

#define VLA_GEMM_ITER(C, RCUR, RNEXT1, RNEXT3, ARELOAD, ASTORE)             \
  {                                                                         \
    load_a(ARELOAD, kb + ((C) + 2) * BK);                                   \
    load_ring(RNEXT3, kb + ((C) + 3) * BK);                                 \
    if ((C) < nchunks) compute((C) & 1, RCUR);                              \
    store_a(((C) + 1) & 1, ASTORE, kb + ((C) + 1) * BK);                    \
    store_ring(((C) + 1) & 1, RNEXT1);                                      \
    __syncthreads();                                                        \
  }
  for (int c = 0; c < nchunks; c += 4) {
    VLA_GEMM_ITER(c + 0, r0, r1, r3, a0, a1)
    VLA_GEMM_ITER(c + 1, r1, r2, r0, a1, a0)
    VLA_GEMM_ITER(c + 2, r2, r3, r1, a0, a1)
    VLA_GEMM_ITER(c + 3, r3, r0, r2, a1, a0)
  }
#undef VLA_GEMM_ITER

  if constexpr (I8MMA) {
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int j = 0; j < NBW; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) acc[mb][j][i] = (float)acci[mb][j][i];
  }

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
  // all partials in split order. Partials move as 16-byte device-coherent
  // (sc1) stores and loads, so the hand-off needs no L2 write-back or
  // invalidate; the counter increment is issued only after every thread's
  // stores have completed. The reducer requests up to four splits' partials
  // at once.
  if (p.split > 1) {
    constexpr int C4 = BN / 4;                  // float4 per tile row
    constexpr int PF4 = (BM * C4 + NT - 1) / NT;
    const int tile = mt * p.n_tiles_n + nt;
    const size_t tstride = (size_t)p.n_tiles_m * p.n_tiles_n * (BM * BN);
    const brsrc pw = make_brsrc(p.part + (size_t)s * tstride + (size_t)tile * (BM * BN));
#pragma unroll
    for (int i = 0; i < PF4; i++) {
      const int e4 = tid + i * NT, r = e4 / C4, c4 = e4 % C4;
      if (r < BM) {
        const float4 v = *reinterpret_cast<const float4*>(sT + r * TPITCH + c4 * 4);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), pw, (uint32_t)(r * BN + c4 * 4) * 4u, 0, CP_SC1);
      }
    }
    if (tile_arrive(p.cnt_tile + tile, p.split, sFlag)) return;
    const brsrc pr = make_brsrc(p.part + (size_t)tile * (BM * BN));
    float4 sum[PF4];
#pragma unroll
    for (int i = 0; i < PF4; i++) sum[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < p.split; q0 += 4) {
      uint4 v[4][PF4];
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < PF4; i++) {
          const int e4 = tid + i * NT, r = e4 / C4, c4 = e4 % C4;
          v[j][i] = bload16<CP_SC1>(pr, (q0 + j < p.split && r < BM) ? (uint32_t)((q0 + j) * tstride + r * BN + c4 * 4) * 4u : BUF_OOB);
        }
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (q0 + j < p.split) {
#pragma unroll
          for (int i = 0; i < PF4; i++) {
            const float4 f = as_f4(v[j][i]);
            sum[i].x += f.x; sum[i].y += f.y; sum[i].z += f.z; sum[i].w += f.w;
          }
        }
    }
#pragma unroll
    for (int i = 0; i < PF4; i++) {
      const int e4 = tid + i * NT, r = e4 / C4, c4 = e4 % C4;
      if (r < BM) *reinterpret_cast<float4*>(sT + r * TPITCH + c4 * 4) = sum[i];
    }
    if (tid == 0) p.cnt_tile[tile] = 0u;
    __syncthreads();
  }

  // ---- W8A8: the per-row scale of the activation codes (the weights'
  // per-column scale is applied by the epilogues)
  if constexpr (a_codes(AM)) {
    const brsrc sr = make_brsrc(p.a_scale);
    float rsc[XPE];
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      const int r = r0e + i * RPT, m = m0 + r;
      rsc[i] = bloadf(sr, (r < BM && m < p.M) ? (uint32_t)m * 4u : BUF_OOB);
    }
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      const int r = r0e + i * RPT;
      if (r < BM) sT[r * TPITCH + cc] *= rsc[i];
    }
    __syncthreads();
  }

  // ---- epilogues (outputs through buffer stores: 32-bit element offsets)
  const brsrc cr = make_brsrc(p.c);
  auto put = [&](uint32_t idx, float v) {
    if (p.c_f32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), cr, idx * 4u, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b16(f2bf(v), cr, idx * 2u, 0, 0);
  };
  if constexpr (EM == E_STORE) {
    const bool cok = ncol < p.N;
    const float sc = p.wscale ? e_sc : 1.f;
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT, m = m0 + r;
      if (r >= BM || m >= p.M || !cok) continue;
      float v = sT[r * TPITCH + cc] * sc + e_bi;
      if (p.act == ACT_GELU) v = gelu_erf(v);
      else if (p.act == ACT_SILU) v = silu(v);
      put((uint32_t)m * p.ldc + ncol, v);
    }
  } else if constexpr (EM == E_ROPE) {
    const int D = p.head_dim, hd = D >> 1;
    const bool cok = ncol < p.N;
    const bool rot = ncol < p.q_cols + p.k_cols;
    const int d = (ncol < p.q_cols ? ncol : ncol - p.q_cols) % D;
    const int fi = d < hd ? d : d - hd;
    const int pc = d < hd ? cc + hd : cc - hd;           // partner column in the tile
    float sc = p.wscale ? e_sc : 1.f;
    float sc2 = p.wscale ? e_sc2 : 1.f;
    // QK-norm: the inverse RMS of every (row, head) of the tile over the
    // head's D columns, from the scaled values; four threads per pair, then
    // a butterfly over them. The tile's heads start at multiples of D.
    float* const qinv = reinterpret_cast<float*>(sRow);   // [BM][BN / D], free after the main loop
    const int nht = BN / D;
    if (p.qk_norm) {
      if (p.wscale) {
#pragma unroll
        for (int i = 0; i < XPE; i++) {
          const int r = r0e + i * RPT;
          if (r < BM) sT[r * TPITCH + cc] *= e_sc;
        }
        __syncthreads();
        sc = sc2 = 1.f;
      }
      const int j4 = tid & 3;
      // head_dim as a compile-time constant: the float4 reads of a row are
      // unrolled and issued together
      auto rows = [&](auto dc) {
        constexpr int DD = decltype(dc)::value, NH = BN / DD, NF = DD / 16;
        for (int pr = tid >> 2; pr < BM * NH; pr += NT / 4) {
          const float* row = sT + (pr / NH) * TPITCH + (pr % NH) * DD;
          float sq = 0.f;
#pragma unroll
          for (int i = 0; i < NF; i++) {
            const float4 x = *reinterpret_cast<const float4*>(row + (j4 + 4 * i) * 4);
            sq += (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w);
          }
          sq += __shfl_xor(sq, 1, WAVE);
          sq += __shfl_xor(sq, 2, WAVE);
          if (j4 == 0) qinv[pr] = rsqrtf(sq / (float)DD + p.qk_eps);
        }
      };
      if (D == 128) rows(std::integral_constant<int, 128>{});
      else rows(std::integral_constant<int, 64>{});
      __syncthreads();
    }
    // the thread's rows step by RPT positions: the first angle and the step
    // come from a double-precision frequency and product reduced to [-pi, pi]
    // in double (a float frequency times a position of several hundred is off
    // by up to 1e-4 rad), each next angle by a rotation through the step
    const double theta = pow((double)p.rope_base, -2.0 * (double)fi / (double)D);
    auto sincos_reduced = [](double a, float* sn_, float* cs_) {
      a -= rint(a * (0.5 / M_PI)) * (2.0 * M_PI);
      sincosf((float)a, sn_, cs_);
    };
    float cs, sn, cd, sd;
    sincos_reduced((double)(m0 + r0e + p.pos0) * theta, &sn, &cs);
    sincos_reduced((double)RPT * theta, &sd, &cd);
#pragma unroll
    for (int i = 0; i < XPE; i++) {
      int r = r0e + i * RPT, m = m0 + r;
      if (r < BM && m < p.M && cok) {
        float v = sT[r * TPITCH + cc] * sc;
        if (rot) {
          float v2 = sT[r * TPITCH + pc] * sc2;
          if (p.qk_norm) {
            const float qs = qinv[r * nht + cc / D];
            v *= qs * e_g1;
            v2 *= qs * e_g2;
          }
          v = d < hd ? v * cs - v2 * sn : v * cs + v2 * sn;
        }
        put((uint32_t)m * p.ldc + ncol, v);
      }
      const float c2 = cs * cd - sn * sd;
      sn = sn * cd + cs * sd;
      cs = c2;
    }
  } else if constexpr (EM == E_SWIGLU) {
    constexpr int BO = BN / 2;
    static_assert(NT % BO == 0, "swiglu epilogue: each thread owns one column");
    constexpr int RPO = NT / BO, XPO = (BM + RPO - 1) / RPO;
    const int co = tid % BO, r0o = tid / BO;
    const int n = nt * BO + co;
    const bool cok = n < p.N;
    const float sg = p.wscale ? e_sc : 1.f;
    const float su = p.wscale ? e_sc2 : 1.f;
    const brsrc clr = make_brsrc(p.c_lo);
#pragma unroll
    for (int i = 0; i < XPO; i++) {
      int r = r0o + i * RPO, m = m0 + r;
      if (r >= BM || m >= p.M || !cok) continue;
      float gv = sT[r * TPITCH + co] * sg, uv = sT[r * TPITCH + BO + co] * su;
      float a = silu(gv) * uv;
      const uint32_t idx = (uint32_t)m * p.ldc + n;
      put(idx, a);
      if (!p.c_f32 && p.c_lo) __builtin_amdgcn_raw_buffer_store_b16(f2bf(a - bf2f(f2bf(a))), clr, idx * 2u, 0, 0);
    }
  } else if constexpr (EM == E_RESID) {
    const bool cok = ncol < p.N;
    const float sc = p.wscale ? e_sc : 1.f;
    const float bi = e_bi;
    const float ga = p.gate ? e_ga : 1.f;
    const brsrc xw = make_brsrc(p.x);
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
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(xn), xw, ((uint32_t)m * p.ldx + ncol) * 4u, 0, 0);
      sT[r * TPITCH + cc] = xn;
    }
    // moments of this tile's columns per row (mean, sum of squared
    // deviations), merged by the stream's next reader: TPRM consecutive
    // threads share a row, each sums a strided set of float4 columns of the
    // LDS tile, then a butterfly over the TPRM lanes; two passes
    static_assert(BN <= 64, "residual tiles are at most 64 columns wide");
    __syncthreads();
    constexpr int C4 = BN / 4;
    constexpr int TPRM0 = NT / BM;
    constexpr int TPRM1 = TPRM0 >= 16 ? 16 : TPRM0 >= 8 ? 8 : TPRM0 >= 4 ? 4 : TPRM0 >= 2 ? 2 : 1;
    constexpr int TPRM = TPRM1 > C4 ? C4 : TPRM1;
    constexpr int F4T = (C4 + TPRM - 1) / TPRM;
    const int ncols = min(BN, p.N - nt * BN);
    const int jq = tid % TPRM;
    for (int r = tid / TPRM; r < BM; r += NT / TPRM) {
      const int m = m0 + r;
      float4 v[F4T];
      float s1 = 0.f;
#pragma unroll
      for (int f = 0; f < F4T; f++) {
        const int c4 = jq + f * TPRM;
        v[f] = c4 < C4 ? *reinterpret_cast<const float4*>(sT + r * TPITCH + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        const int c = 4 * c4;
        s1 += (c < ncols ? v[f].x : 0.f) + (c + 1 < ncols ? v[f].y : 0.f) + (c + 2 < ncols ? v[f].z : 0.f) +
              (c + 3 < ncols ? v[f].w : 0.f);
      }
#pragma unroll
      for (int o = 1; o < TPRM; o <<= 1) s1 += __shfl_xor(s1, o, WAVE);
      const float mean = s1 / (float)ncols;
      float sq = 0.f;
#pragma unroll
      for (int f = 0; f < F4T; f++) {
        const int c = 4 * (jq + f * TPRM);
        const float d0 = c < ncols ? v[f].x - mean : 0.f, d1 = c + 1 < ncols ? v[f].y - mean : 0.f;
        const float d2 = c + 2 < ncols ? v[f].z - mean : 0.f, d3 = c + 3 < ncols ? v[f].w - mean : 0.f;
        sq += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
      }
#pragma unroll
      for (int o = 1; o < TPRM; o <<= 1) sq += __shfl_xor(sq, o, WAVE);
      if (jq == 0 && m < p.M) p.rs_out[(size_t)nt * p.M + m] = make_float2(mean, sq);
    }
  }
}

}  // namespace vla
