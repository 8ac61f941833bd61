// Flash attention (online softmax) for GQA / MHA, causal or full, on MFMA.
//
// Each wave owns 16 query rows of one query head and walks the keys in
// blocks of 32 staged in LDS (K row-major, V transposed), several blocks per
// stage: a stage's K and V are requested at once (one memory latency for
// all of them) and the next stage is requested before the current one is
// computed. A stage's scores are computed for all its blocks at once
// (independent MFMA chains), followed by one online-softmax update and the
// O MFMAs, so the serial max / exp / rescale chain runs once per stage
// rather than once per 32 keys. The scores are
// computed transposed, S^T = K Q^T, so a lane holds 8 keys of a single query:
// the running max / sum of that query live in the lane (plus a 4-way
// exchange across lane groups), and the exponentiated scores are already in
// the B-operand layout of O^T = V^T P^T. No LDS round trip for P.
// With grouped KV heads one workgroup serves up to 4 query heads that share
// one KV head, so each K/V block is fetched once for all of them.
// When that leaves too few workgroups to fill the chip (batch-1 prefills of
// 100-256 rows), the key-split form (KS) gives each workgroup 16 query rows
// of one head and lets its four waves take one 32-key block of every stage
// each; the four partial results (unnormalised O, running max and sum) are
// combined in LDS in wave order at the end, so the serial chain per wave is
// a quarter as long and four times as many workgroups share the work.
#pragma once
#include <type_traits>

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
  // key split (filled by the launcher): the keys of every tile are shared
  // out to nsplit workgroups of kchunk keys each; each writes its partial
  // (unnormalised O, running max and sum per query) to part, and
  // k_attn_merge combines them in split order
  int nsplit, kchunk;
  float* part;
};

constexpr int ATTN_SPLIT_MAX = 16;

template <typename CT> struct ATraits;
template <> struct ATraits<__bf16> {
  using F = FragBF16;
  static constexpr int ESZ = 2;
  using raw = uint4;                                   // 8 elements
  __device__ static raw rload8(brsrc r, uint32_t elem, bool ok) { return bload16(r, ok ? elem * 2u : BUF_OOB); }
  __device__ static void rstore8(char* dst, const raw& v) { *reinterpret_cast<uint4*>(dst) = v; }
  __device__ static void rput(char* dst, const raw& v, int t) {
    const uint32_t word = (t >> 1) == 0 ? v.x : (t >> 1) == 1 ? v.y : (t >> 1) == 2 ? v.z : v.w;
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(t & 1 ? word >> 16 : word);
  }
  __device__ static F gload(const void* base, size_t off) {
    F f; f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>((const uint16_t*)base + off)); return f;
  }
  __device__ static F lfrag(const char* p) { F f; f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p)); return f; }
  // the fragment's load has completed past this point
  __device__ static void ready(const F& f) {
    const uint4 u = __builtin_bit_cast(uint4, f.v);
    asm volatile("" ::"v"(u.x), "v"(u.y), "v"(u.z), "v"(u.w));
  }
  // V^T fragment: keys {4g..4g+3} at p0 and {16+4g..} at p1 (4 elements each)
  __device__ static F lfrag2(const char* p0, const char* p1) {
    uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
    F f; f.v = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y)); return f;
  }
  __device__ static void store4(void* base, size_t off, float a, float b, float c, float d) {
    uint2 u; u.x = pack_bf2(a, b); u.y = pack_bf2(c, d);
    *reinterpret_cast<uint2*>((uint16_t*)base + off) = u;
  }
};
template <> struct ATraits<float> {
  using F = FragF32;
  static constexpr int ESZ = 4;
  struct raw { float4 a, b; };                         // 8 elements
  __device__ static raw rload8(brsrc r, uint32_t elem, bool ok) {
    raw v;
    v.a = as_f4(bload16(r, ok ? elem * 4u : BUF_OOB));
    v.b = as_f4(bload16(r, ok ? elem * 4u + 16u : BUF_OOB));
    return v;
  }
  __device__ static void rstore8(char* dst, const raw& v) {
    reinterpret_cast<float4*>(dst)[0] = v.a;
    reinterpret_cast<float4*>(dst)[1] = v.b;
  }
  __device__ static void rput(char* dst, const raw& v, int t) {
    const float e = t < 4 ? (t == 0 ? v.a.x : t == 1 ? v.a.y : t == 2 ? v.a.z : v.a.w)
                          : (t == 4 ? v.b.x : t == 5 ? v.b.y : t == 6 ? v.b.z : v.b.w);
    *reinterpret_cast<float*>(dst) = e;
  }
  __device__ static F gload(const void* base, size_t off) {
    const float4* p = reinterpret_cast<const float4*>((const float*)base + off);
    float4 a = p[0], b = p[1];
    F f; f.lo = (f32x4){a.x, a.y, a.z, a.w}; f.hi = (f32x4){b.x, b.y, b.z, b.w}; return f;
  }
  __device__ static void ready(const F& f) {
    asm volatile("" ::"v"(f.lo[0]), "v"(f.lo[1]), "v"(f.lo[2]), "v"(f.lo[3]), "v"(f.hi[0]), "v"(f.hi[1]), "v"(f.hi[2]),
                 "v"(f.hi[3]));
  }
  __device__ static F lfrag(const char* p) {
    float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    F f; f.lo = (f32x4){a.x, a.y, a.z, a.w}; f.hi = (f32x4){b.x, b.y, b.z, b.w}; return f;
  }
  __device__ static F lfrag2(const char* p0, const char* p1) {
    float4 a = *reinterpret_cast<const float4*>(p0), b = *reinterpret_cast<const float4*>(p1);
    F f; f.lo = (f32x4){a.x, a.y, a.z, a.w}; f.hi = (f32x4){b.x, b.y, b.z, b.w}; return f;
  }
  __device__ static void store4(void* base, size_t off, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>((float*)base + off) = make_float4(a, b, c, d);
  }
};

// Blocks of 32 keys staged per round: LDS holds one stage (K [32][DP] and
// V^T [DP][32] per block, padded rows), registers the next one.
template <typename CT, int DP>
struct AttnStage {
  static constexpr int ESZ = ATraits<CT>::ESZ;
  static constexpr int KB = 32;
  static constexpr int KPITCH = DP * ESZ + 16;       // K row pitch (bytes)
  static constexpr int VPITCH = KB * ESZ + 16;       // V^T row pitch (bytes)
  static constexpr int KBYTES = KB * KPITCH, VBYTES = DP * VPITCH;
  static constexpr int NBUF = ESZ == 2 ? 4 : 2;      // blocks per stage
  static constexpr int GROUPS = KB * (DP / 8);        // 8-element groups per block (K, and V)
  static constexpr int GPB = (GROUPS + 255) / 256;    // of them per thread
  static constexpr int SMEM = NBUF * (KBYTES + VBYTES);
};

// DP: head dim padded to a multiple of 32 (64, 96, 128). HPW: query heads per
// workgroup (1, 2 or 4); the 4 waves cover HPW heads x (4 / HPW) row blocks.
// KS: the key-split form (one head, 16 rows, wave w takes block w of each
// stage); bf16 only, HPW 1, head dim 64 or 128, no split across workgroups.
template <typename CT, int DP, int HPW, bool KS = false>
__global__ __launch_bounds__(256) void k_attention(AttnArgs p) {
  using TR = ATraits<CT>;
  using F = typename TR::F;
  using ST = AttnStage<CT, DP>;
  using RAW = typename TR::raw;
  constexpr int ESZ = TR::ESZ;
  static_assert(!KS || (HPW == 1 && ST::NBUF == 4 && DP % 64 == 0), "key-split form: 4 blocks per stage, one head");
  constexpr int RB = KS ? 1 : 4 / HPW;       // 16-row blocks per workgroup
  constexpr int KB = ST::KB, NBUF = ST::NBUF, GPB = ST::GPB;
  constexpr int KPITCH = ST::KPITCH, VPITCH = ST::VPITCH;
  extern __shared__ __align__(16) char smem[];
  char* sK = smem;                            // [NBUF][KB][KPITCH]
  char* sV = smem + NBUF * ST::KBYTES;        // [NBUF][DP][VPITCH]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = p.Hq / p.Hkv;
  const int hsets = group / HPW;             // head subsets per kv head
  const int nrb = (p.Sq + 16 * RB - 1) / (16 * RB);
  int bid = blockIdx.x;
  const int sp = bid % p.nsplit;  bid /= p.nsplit;
  const int tile = bid;
  const int rb = bid % nrb;  bid /= nrb;
  const int hs = bid % hsets; bid /= hsets;
  const int g = bid;                          // kv head
  const int head = g * group + hs * HPW + (KS ? 0 : wave % HPW);
  const int row0 = (rb * RB + (KS ? 0 : wave / HPW)) * 16;     // this wave's first query row
  const int wg_row_end = min(p.Sq, (rb + 1) * RB * 16);
  const int qn = lane & 15, grp = lane >> 4;
  const int qrow = row0 + qn;
  // this workgroup's keys: [kbeg, kend) of the tile's visible keys
  const int kvis = p.causal ? min(p.Sk, wg_row_end) : p.Sk;
  const int kbeg = sp * p.kchunk;
  const int kend = min(kvis, kbeg + p.kchunk);
  const int klim = p.causal ? min(kend, qrow + 1) : kend;   // this lane's visible keys end
  const int kfull = p.causal ? min(kend, row0 + 1) : kend;   // keys every query of the wave sees

  // K / V of one stage (NBUF blocks from key kb0) into registers: thread
  // group e = tid + i * 256 of a block is key e % 32, dims (e / 32) * 8, so
  // that a wave's LDS writes (K rows, V^T columns) fall in distinct banks
  const brsrc kr = make_brsrc(p.k), vr = make_brsrc(p.v);
  RAW rk[NBUF][GPB], rv[NBUF][GPB];
  auto load_stage = [&](int kb0) {
#pragma unroll
    for (int b = 0; b < NBUF; b++)
#pragma unroll
      for (int i = 0; i < GPB; i++) {
        const int e = tid + i * 256, key = e % KB, d8 = (e / KB) * 8;
        const int j = kb0 + b * KB + key;
        const bool ok = e < ST::GROUPS && j < kend && d8 < p.D;
        rk[b][i] = TR::rload8(kr, (uint32_t)j * p.ldk + (uint32_t)g * p.D + d8, ok);
        rv[b][i] = TR::rload8(vr, (uint32_t)j * p.ldv + (uint32_t)g * p.D + d8, ok);
      }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int b = 0; b < NBUF; b++)
#pragma unroll
      for (int i = 0; i < GPB; i++) {
        const int e = tid + i * 256, key = e % KB, d8 = (e / KB) * 8;
        if (e >= ST::GROUPS) continue;
        TR::rstore8(sK + b * ST::KBYTES + key * KPITCH + d8 * ESZ, rk[b][i]);
        char* vd = sV + b * ST::VBYTES + key * ESZ;
#pragma unroll
        for (int t = 0; t < 8; t++) TR::rput(vd + (d8 + t) * VPITCH, rv[b][i], t);
      }
  };
  // Q^T fragments (B operand): query qn, dims ds*32 + grp*8 .. +8. They are
  // requested before the first K / V stage and made ready before the key
  // loop: a load still pending at the loop's entry makes the compiler wait
  // for every outstanding load before the first MFMA of each stage, which
  // would include the next stage's prefetch.
  F qf[DP / 32];
#pragma unroll
  for (int ds = 0; ds < DP / 32; ds++) {
    int d = ds * 32 + grp * 8;
    if (qrow < p.Sq && d < p.D) qf[ds] = TR::gload(p.q, (size_t)qrow * p.ldq + (size_t)head * p.D + d);
    else qf[ds] = zero_frag(F{});
  }
  load_stage(kbeg);
#pragma unroll
  for (int ds = 0; ds < DP / 32; ds++) TR::ready(qf[ds]);

  f32x4 oacc[DP / 16];
#pragma unroll
  for (int i = 0; i < DP / 16; i++) oacc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lrun = 0.f;   // exponent base (raw score units) and this lane's share of l

  for (int kb0 = kbeg; kb0 < kend; kb0 += NBUF * KB) {
    __syncthreads();                          // the previous stage's readers are done
    store_stage();
    __syncthreads();
    if (kb0 + NBUF * KB < kend) load_stage(kb0 + NBUF * KB);   // next stage in flight
    // a stage with at most two live blocks (short key ranges: a chunk's
    // self-attention, one split of a long context) runs a two-block body
    // (the choice is uniform across the workgroup); at head dim 128 the
    // second body would cost registers (one wave per SIMD instead of two)
    auto stage = [&](auto nb_c) {
      constexpr int NB = decltype(nb_c)::value;
      const int bo = KS ? wave : 0;           // the wave's first block of the stage
      // scores of every live block of the stage first: S^T for keys kb0 +
      // 32 b + 16 hb + 4 grp + i of query qn, independent MFMA chains. The
      // last block may run past the last key: those keys are staged as
      // zeros and masked below, so the stage is straight-line code.
      f32x4 s[NB][2];
#pragma unroll
      for (int b = 0; b < NB; b++)
#pragma unroll
        for (int hb = 0; hb < 2; hb++) {
          s[b][hb] = (f32x4){0.f, 0.f, 0.f, 0.f};
          const char* bK = sK + (bo + b) * ST::KBYTES;
#pragma unroll
          for (int ds = 0; ds < DP / 32; ds++) {
            F kf = TR::lfrag(bK + (hb * 16 + qn) * KPITCH + (ds * 32 + grp * 8) * ESZ);
            mma32(s[b][hb], kf, qf[ds]);
          }
        }
      // one online-softmax update for the whole stage, on raw scores; key j is
      // visible to this lane's query iff j < klim. A stage that every query
      // of the wave sees whole skips the mask (a wave-uniform test).
      float bmax = -INFINITY;
      if (kb0 + (bo + NB) * KB <= kfull) {
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
          for (int hb = 0; hb < 2; hb++)
#pragma unroll
            for (int i = 0; i < 4; i++) bmax = fmaxf(bmax, s[b][hb][i]);
      } else {
        const int kl0 = klim - kb0 - bo * KB - grp * 4;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
          for (int hb = 0; hb < 2; hb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const float v = b * KB + hb * 16 + i < kl0 ? s[b][hb][i] : -INFINITY;
              s[b][hb][i] = v;
              bmax = fmaxf(bmax, v);
            }
      }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, WAVE));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, WAVE));
      // The exponent base mref moves only when the running max outgrows it by
      // more than 2^8 (so P stays within 256), and only then are O and l
      // rescaled; both share the base, so O / l is unchanged. Most stages
      // after the first rescale nothing.
      const float mnew = fmaxf(mref, bmax);
      const bool grow = mnew != -INFINITY && (mref == -INFINITY || (mnew - mref) * p.scale_log2 > 8.f);
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float corr = grow ? __builtin_amdgcn_exp2f((mref - mnew) * p.scale_log2) : 1.f;
#pragma unroll
        for (int db = 0; db < DP / 16; db++) oacc[db] = oacc[db] * corr;
        lrun *= corr;
        if (grow) mref = mnew;
      }
      const float base = mref == -INFINITY ? 0.f : mref * p.scale_log2;
      F pf[NB];
      float psum = 0.f;
#pragma unroll
      for (int b = 0; b < NB; b++) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          pv[i] = __builtin_amdgcn_exp2f(fmaf(s[b][0][i], p.scale_log2, -base));
          pv[4 + i] = __builtin_amdgcn_exp2f(fmaf(s[b][1][i], p.scale_log2, -base));
          psum += pv[i] + pv[4 + i];
        }
        frag_from_floats(pf[b], pv);
      }
      lrun += psum;
#pragma unroll
      for (int db = 0; db < DP / 16; db++) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
          const char* vrow = sV + (bo + b) * ST::VBYTES + (db * 16 + qn) * VPITCH;
          F vf = TR::lfrag2(vrow + (grp * 4) * ESZ, vrow + (16 + grp * 4) * ESZ);
          mma32(oacc[db], vf, pf[b]);
        }
      }
    };
    if constexpr (KS) {
      // a block that no query of the wave sees adds nothing: skip it
      const int kwave = p.causal ? min(kend, row0 + 16) : kend;
      if (kb0 + wave * KB < kwave) stage(std::integral_constant<int, 1>{});
    } else if constexpr (NBUF > 2 && DP < 128) {
      if (kend - kb0 <= 2 * KB) stage(std::integral_constant<int, 2>{});
      else stage(std::integral_constant<int, NBUF>{});
    } else {
      stage(std::integral_constant<int, NBUF>{});
    }
  }
  float lsum = lrun;
  lsum += __shfl_xor(lsum, 16, WAVE);
  lsum += __shfl_xor(lsum, 32, WAVE);
  if constexpr (KS) {
    // the four waves' partials of the same 16 queries, combined in LDS: each
    // wave's O^T tile goes in as [query][dim] rows with its (max, sum), then
    // thread t produces dims (t % 16) * DP / 16 .. of query t / 16
    constexpr int OP = DP + 4;                           // row pitch (floats)
    float* mo = reinterpret_cast<float*>(smem);          // [4][16][OP]
    float* ml = mo + 4 * 16 * OP;                        // [4][16][2]
    static_assert((4 * 16 * OP + 4 * 16 * 2) * 4 <= ST::SMEM, "merge tile fits the stage buffers");
    __syncthreads();                                     // every wave is done with the staged K / V
#pragma unroll
    for (int db = 0; db < DP / 16; db++)
      *reinterpret_cast<float4*>(mo + (wave * 16 + qn) * OP + db * 16 + grp * 4) =
          make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    if (grp == 0) {
      ml[(wave * 16 + qn) * 2] = mref == -INFINITY ? -INFINITY : mref * p.scale_log2;
      ml[(wave * 16 + qn) * 2 + 1] = lsum;
    }
    __syncthreads();
    const int q = tid >> 4, c0 = (tid & 15) * (DP / 16);
    float mw[4], fw[4], M = -INFINITY, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) { mw[w] = ml[(w * 16 + q) * 2]; M = fmaxf(M, mw[w]); }
#pragma unroll
    for (int w = 0; w < 4; w++) {
      fw[w] = mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - M);   // a wave that saw no key adds nothing
      L += fw[w] * ml[(w * 16 + q) * 2 + 1];
    }
    const float linv = L > 0.f ? 1.f / L : 0.f;
    const int row = row0 + q;
    if (row < p.Sq) {
#pragma unroll
      for (int i = 0; i < DP / 16; i += 4) {
        const int d = c0 + i;
        if (d >= p.D) continue;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const float4 v = *reinterpret_cast<const float4*>(mo + (w * 16 + q) * OP + d);
          acc.x += fw[w] * v.x; acc.y += fw[w] * v.y; acc.z += fw[w] * v.z; acc.w += fw[w] * v.w;
        }
        TR::store4(p.o, (size_t)row * p.ldo + (size_t)head * p.D + d, acc.x * linv, acc.y * linv, acc.z * linv,
                   acc.w * linv);
      }
    }
    return;
  }
  if (p.nsplit > 1) {
    // partial of this split: [wave][query][DP] unnormalised O, then the
    // running max and sum of each query
    constexpr int PW = 16 * (DP + 2);                   // floats per wave
    float* pt = p.part + ((size_t)(tile * p.nsplit + sp) * 4 + wave) * PW;
#pragma unroll
    for (int db = 0; db < DP / 16; db++) {
      const int d = db * 16 + grp * 4;
      *reinterpret_cast<float4*>(pt + qn * DP + d) = make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    }
    if (grp == 0) { pt[16 * DP + qn] = mref == -INFINITY ? -INFINITY : mref * p.scale_log2; pt[16 * DP + 16 + qn] = lsum; }
    return;
  }
  float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  // O^T[d][q]: the lane's 4 consecutive dims d = 16 db + 4 grp + i of query qrow
  if (qrow < p.Sq) {
#pragma unroll
    for (int db = 0; db < DP / 16; db++) {
      const int d = db * 16 + grp * 4;
      if (d < p.D)
        TR::store4(p.o, (size_t)qrow * p.ldo + (size_t)head * p.D + d, oacc[db][0] * inv, oacc[db][1] * inv,
                   oacc[db][2] * inv, oacc[db][3] * inv);
    }
  }
}

// Merge of a key-split attention: one thread per 4 output dims of one query
// of one head, every split's partial requested at once and combined in split
// order (max, rescaled sums), so results do not depend on timing.
template <typename CT, int DP, int HPW>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs p) {
  using TR = ATraits<CT>;
  constexpr int RB = 4 / HPW, PW = 16 * (DP + 2), ITEMS = 4 * 16 * (DP / 4);
  const int group = p.Hq / p.Hkv, hsets = group / HPW;
  const int nrb = (p.Sq + 16 * RB - 1) / (16 * RB);
  const int per_tile = (ITEMS + 255) / 256;
  const int tile = blockIdx.x / per_tile;
  const int e = (blockIdx.x % per_tile) * 256 + threadIdx.x;
  if (e >= ITEMS) return;
  const int w = e / (16 * (DP / 4)), q = (e / (DP / 4)) % 16, d = (e % (DP / 4)) * 4;
  int t_ = tile;
  const int rb = t_ % nrb; t_ /= nrb;
  const int hs = t_ % hsets;
  const int g = t_ / hsets;
  const int row = (rb * RB + w / HPW) * 16 + q, head = g * group + hs * HPW + (w % HPW);
  if (row >= p.Sq || d >= p.D) return;
  float m[ATTN_SPLIT_MAX], l[ATTN_SPLIT_MAX];
  float4 o[ATTN_SPLIT_MAX];
#pragma unroll
  for (int t = 0; t < ATTN_SPLIT_MAX; t++) {
    if (t < p.nsplit) {
      const float* pt = p.part + ((size_t)(tile * p.nsplit + t) * 4 + w) * PW;
      m[t] = pt[16 * DP + q];
      l[t] = pt[16 * DP + 16 + q];
      o[t] = *reinterpret_cast<const float4*>(pt + q * DP + d);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < ATTN_SPLIT_MAX; t++)
    if (t < p.nsplit) M = fmaxf(M, m[t]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int t = 0; t < ATTN_SPLIT_MAX; t++) {
    if (t < p.nsplit && m[t] != -INFINITY) {           // a split without a visible key adds nothing
      const float f = exp2f(m[t] - M);
      L += f * l[t];
      acc.x += f * o[t].x; acc.y += f * o[t].y; acc.z += f * o[t].z; acc.w += f * o[t].w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  TR::store4(p.o, (size_t)row * p.ldo + (size_t)head * p.D + d, acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

}  // namespace vla
