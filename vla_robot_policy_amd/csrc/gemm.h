// Weight-streaming GEMM for small M (16..600 rows), y = prologue(A) . W^T,
// with fused prologues (row norms, patch gather, merge gather, sinusoidal
// timestep features) and fused epilogues (bias, GELU/SiLU, RoPE, SwiGLU,
// residual / gated residual with row statistics for the next norm).
//
// Layout: A is [M, K] row-major (token-major activations); W is [N, K]
// row-major (PyTorch Linear); each lane's 16-byte W load is exactly the
// MFMA B-operand fragment, so weights go HBM -> registers without LDS. A is
// staged through LDS once per workgroup and shared by its 4 waves.
// Split-K partial tiles are reduced in a fixed order by the last workgroup
// of each output tile (no float atomics), so results are bitwise
// reproducible run to run.
#pragma once
#include "common.h"

namespace vla {

enum AMode { A_BF16 = 0, A_F32 = 1, A_NORM = 2, A_PATCH = 3, A_MERGE = 4, A_TIME = 5 };
enum EMode { E_STORE = 0, E_ROPE = 1, E_SWIGLU = 2, E_RESID = 3 };
enum ActKind { ACT_NONE = 0, ACT_GELU = 1, ACT_SILU = 2 };

struct GemmArgs {
  int M, N, K;
  // ---- A source
  const void* a;         // BF16/F32/NORM/MERGE: matrix [rows, lda]; PATCH: bf16 images
  int lda;
  const float2* stats;   // NORM/MERGE: per source row (mean, var)
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
  float2* stats_part;                                     // RESID: [n_tiles_n][M] (mean, M2)
  float2* stats_out;                                      // RESID: [M] (mean, var)
  // ---- tiling / split-K (filled by the launcher)
  int split, ksplit;
  float* part;
  unsigned* cnt_tile;
  unsigned* cnt_all;
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

// ---------------------------------------------------------------- kernel
template <typename WT, typename CT, int MB, int WN, int NBW, int AM, int EM>
struct GemmTile {
  static constexpr int WK = 4 / WN;
  static constexpr int BM = 16 * MB;
  static constexpr int BN = 16 * NBW * WN;
  static constexpr int U = 2;                    // 32-wide k-steps per wave per chunk
  static constexpr int BK = 32 * WK * U;         // chunk width
  static constexpr int ESZ = sizeof(CT);
  static constexpr int LROW = BK * ESZ + 16;     // LDS row pitch (bytes), padded
  static constexpr int ABUF = BM * LROW;
  static constexpr int GPT = BM * BK / 4 / 256;  // 4-element A groups per thread per chunk
  static constexpr int TPITCH = BN + 4;          // fp32 tile pitch (elements)
  static constexpr int SMEM_A = 2 * ABUF;
  static constexpr int SMEM_T = BM * TPITCH * 4;
  static constexpr int SMEM = (SMEM_A > SMEM_T ? SMEM_A : SMEM_T) + BM * 8 + 64;
  static_assert(GPT >= 1 && (BM * BK) % 1024 == 0, "A chunk must split evenly over 256 threads");
};

template <typename WT, typename CT, int MB, int WN, int NBW, int AM, int EM>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs p) {
  using T = GemmTile<WT, CT, MB, WN, NBW, AM, EM>;
  using WL = WLoad<WT>;
  using F = typename Frag<CT>::type;
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, WK = T::WK, U = T::U, GPT = T::GPT;
  constexpr int LROW = T::LROW, TPITCH = T::TPITCH;
  extern __shared__ __align__(16) char smem[];
  char* sA = smem;
  float* sT = reinterpret_cast<float*>(smem);
  float2* sRow = reinterpret_cast<float2*>(smem + (T::SMEM_A > T::SMEM_T ? T::SMEM_A : T::SMEM_T));
  int* sFlag = reinterpret_cast<int*>(sRow + BM);

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

  // ---- per-row normaliser (NORM): (mean to subtract, reciprocal std)
  if (AM == A_NORM) {
    for (int r = tid; r < BM; r += 256) {
      int m = m0 + r;
      float2 st = m < p.M ? p.stats[m] : make_float2(0.f, 0.f);
      float mu = p.norm_rms ? 0.f : st.x;
      float var = p.norm_rms ? st.y + st.x * st.x : st.y;
      sRow[r] = make_float2(mu, rsqrtf(var + p.eps));
    }
  }

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

  auto load_b = [&](typename WL::raw (&br)[U][NBW], int kc) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      int k = kc + (u * WK + wk) * 32 + kl;
#pragma unroll
      for (int j = 0; j < NBW; j++)
        br[u][j] = (wok[j] && k < ke) ? WL::load(p.w, wrow[j] * (size_t)p.ldw + k) : WL::zero();
    }
  };

  // ---- A chunk loader: thread owns 4 consecutive k of rows r0 + i*RS
  constexpr int CPR = BK / 4;                   // groups per row
  constexpr int RS = 256 / CPR;                 // row stride between a thread's groups
  const int ar0 = tid / CPR;
  const int ac4 = (tid % CPR) * 4;
  float4 areg[GPT];
  float2 astat[AM == A_MERGE ? GPT : 1];
  float4 ag = make_float4(1.f, 1.f, 1.f, 1.f), ab = make_float4(0.f, 0.f, 0.f, 0.f);

  auto load_a = [&](int kc) {
    int k = kc + ac4;
    if (AM == A_NORM || AM == A_MERGE) {
      int kk = (AM == A_MERGE) ? (k % p.lda) : k;
      if (k < p.K) {
        if (p.g) ag = *reinterpret_cast<const float4*>(p.g + kk);
        else ag = make_float4(1.f, 1.f, 1.f, 1.f);
        if (p.g_plus_one) { ag.x += 1.f; ag.y += 1.f; ag.z += 1.f; ag.w += 1.f; }
        if (p.bsh) ab = *reinterpret_cast<const float4*>(p.bsh + kk);
        else ab = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int i = 0; i < GPT; i++) {
      int r = ar0 + i * RS;
      int m = m0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      bool ok = m < p.M && k < p.K;
      if (AM == A_BF16) {
        if (ok) {
          uint2 u = *reinterpret_cast<const uint2*>((const uint16_t*)p.a + (size_t)m * p.lda + k);
          v = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                          __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
        }
      } else if (AM == A_F32 || AM == A_NORM) {
        if (ok) v = *reinterpret_cast<const float4*>((const float*)p.a + (size_t)m * p.lda + k);
      } else if (AM == A_PATCH) {
        if (m < p.M) {
          int im = m / p.n_patches, pi = m % p.n_patches;
          int pr = pi / p.vgrid, pc = pi % p.vgrid;
          int P2 = p.patch * p.patch;
          float t4[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            int kk = k + e;
            float val = 0.f;
            if (kk < p.K) {
              int c = kk / P2, rem = kk % P2, ky = rem / p.patch, kx = rem % p.patch;
              size_t off = (((size_t)im * p.chans + c) * p.img + pr * p.patch + ky) * p.img + pc * p.patch + kx;
              val = bf2f(((const uint16_t*)p.a)[off]);
            }
            t4[e] = val;
          }
          v = make_float4(t4[0], t4[1], t4[2], t4[3]);
        }
      } else if (AM == A_MERGE) {
        if (ok) {
          int D = p.lda;
          int per = p.n_merged;
          int im = m / per, mm = m % per;
          int gq = p.vgrid / p.merge;
          int R = mm / gq, C = mm % gq;
          int sub = k / D, d = k % D;
          int dy = sub / p.merge, dx = sub % p.merge;
          int src = im * p.n_patches + (R * p.merge + dy) * p.vgrid + C * p.merge + dx;
          v = *reinterpret_cast<const float4*>((const float*)p.a + (size_t)src * D + d);
          astat[i] = p.stats[src];
        } else {
          astat[i] = make_float2(0.f, 1.f);
        }
      }
      areg[i] = v;
    }
  };

  auto store_a = [&](int buf, int kc) {
    char* base = sA + buf * T::ABUF;
#pragma unroll
    for (int i = 0; i < GPT; i++) {
      int r = ar0 + i * RS;
      int m = m0 + r;
      int k = kc + ac4;
      float4 v = areg[i];
      if (AM == A_NORM) {
        float2 rs = sRow[r];
        bool ok = m < p.M && k < p.K;
        v.x = ok ? (v.x - rs.x) * rs.y * ag.x + ab.x : 0.f;
        v.y = ok ? (v.y - rs.x) * rs.y * ag.y + ab.y : 0.f;
        v.z = ok ? (v.z - rs.x) * rs.y * ag.z + ab.z : 0.f;
        v.w = ok ? (v.w - rs.x) * rs.y * ag.w + ab.w : 0.f;
      } else if (AM == A_MERGE) {
        bool ok = m < p.M && k < p.K;
        float mu = astat[i].x, rstd = rsqrtf(astat[i].y + p.eps);
        v.x = ok ? (v.x - mu) * rstd * ag.x + ab.x : 0.f;
        v.y = ok ? (v.y - mu) * rstd * ag.y + ab.y : 0.f;
        v.z = ok ? (v.z - mu) * rstd * ag.z + ab.z : 0.f;
        v.w = ok ? (v.w - mu) * rstd * ag.w + ab.w : 0.f;
      } else if (AM == A_TIME) {
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
      }
      lds_store4((CT*)nullptr, base + r * LROW + ac4 * T::ESZ, v);
    }
  };

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int j = 0; j < NBW; j++) acc[mb][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, typename WL::raw (&br)[U][NBW]) {
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

  __syncthreads();   // sRow ready
  typename WL::raw b0[U][NBW], b1[U][NBW];
  if (nchunks > 0) {
    load_a(kb);
    load_b(b0, kb);
    store_a(0, kb);
  }
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    // even chunk: compute from b0 / buffer 0 while chunk c+1 streams into b1
    int kc1 = kb + (c + 1) * BK;
    if (c + 1 < nchunks) { load_a(kc1); load_b(b1, kc1); }
    compute(0, b0);
    if (c + 1 < nchunks) store_a(1, kc1);
    __syncthreads();
    if (c + 1 >= nchunks) break;
    int kc2 = kb + (c + 2) * BK;
    if (c + 2 < nchunks) { load_a(kc2); load_b(b0, kc2); }
    compute(1, b1);
    if (c + 2 < nchunks) store_a(0, kc2);
    __syncthreads();
  }

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
  // all partials in split order
  if (p.split > 1) {
    const int tile = mt * p.n_tiles_n + nt;
    float* mine = p.part + ((size_t)s * p.n_tiles_m * p.n_tiles_n + tile) * (BM * BN);
    for (int e = tid; e < BM * BN; e += 256) mine[e] = sT[(e / BN) * TPITCH + (e % BN)];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      unsigned old = atomicAdd(p.cnt_tile + tile, 1u);
      sFlag[0] = (old == (unsigned)(p.split - 1));
    }
    __syncthreads();
    if (!sFlag[0]) return;
    __threadfence();
    for (int e = tid; e < BM * BN; e += 256) {
      float sum = 0.f;
      for (int q = 0; q < p.split; q++)
        sum += p.part[((size_t)q * p.n_tiles_m * p.n_tiles_n + tile) * (BM * BN) + e];
      sT[(e / BN) * TPITCH + (e % BN)] = sum;
    }
    if (tid == 0) p.cnt_tile[tile] = 0u;
    __syncthreads();
  }

  // ---- epilogues
  if (EM == E_STORE) {
    for (int e = tid; e < BM * BN; e += 256) {
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
  } else if (EM == E_ROPE) {
    const int D = p.head_dim, hd = D >> 1;
    const float l2b = log2f(p.rope_base);
    for (int e = tid; e < BM * BN; e += 256) {
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
      ((uint16_t*)p.c)[(size_t)m * p.ldc + n] = f2bf(v);
    }
  } else if (EM == E_SWIGLU) {
    constexpr int BO = BN / 2;
    for (int e = tid; e < BM * BO; e += 256) {
      int r = e / BO, cc = e % BO;
      int m = m0 + r, n = nt * BO + cc;
      if (m >= p.M || n >= p.N) continue;
      float gv = sT[r * TPITCH + cc], uv = sT[r * TPITCH + BO + cc];
      if (p.wscale) { gv *= p.wscale[n]; uv *= p.wscale[p.n_half + n]; }
      float a = silu(gv) * uv;
      if (p.c_f32) ((float*)p.c)[(size_t)m * p.ldc + n] = a;
      else ((uint16_t*)p.c)[(size_t)m * p.ldc + n] = f2bf(a);
    }
  } else if (EM == E_RESID) {
    for (int e = tid; e < BM * BN; e += 256) {
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
        xn = *xp + v;
      }
      *xp = xn;
      sT[r * TPITCH + cc] = xn;
    }
    __syncthreads();
    // per-row moments of this tile's columns
    const int ncols = min(BN, p.N - nt * BN);
    for (int r = wave; r < BM; r += 4) {
      int m = m0 + r;
      if (m >= p.M) continue;          // wave-uniform
      float sum = 0.f;
      for (int cc = lane; cc < ncols; cc += 64) sum += sT[r * TPITCH + cc];
      float mean = wave_sum(sum) / (float)ncols;
      float sq = 0.f;
      for (int cc = lane; cc < ncols; cc += 64) { float d = sT[r * TPITCH + cc] - mean; sq += d * d; }
      float m2 = wave_sum(sq);
      if (lane == 0) p.stats_part[(size_t)nt * p.M + m] = make_float2(mean, m2);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      unsigned total = (unsigned)(p.n_tiles_n * p.n_tiles_m);
      unsigned old = atomicAdd(p.cnt_all, 1u);
      sFlag[1] = (old == total - 1);
    }
    __syncthreads();
    if (!sFlag[1]) return;
    __threadfence();
    for (int m = tid; m < p.M; m += 256) {
      float n = 0.f, mean = 0.f, m2 = 0.f;
      for (int t = 0; t < p.n_tiles_n; t++) {
        float2 st = p.stats_part[(size_t)t * p.M + m];
        float nb = (float)min(BN, p.N - t * BN);
        moments_merge(n, mean, m2, nb, st.x, st.y);
      }
      p.stats_out[m] = make_float2(mean, m2 / n);
    }
    if (tid == 0) *p.cnt_all = 0u;
  }
}

}  // namespace vla
