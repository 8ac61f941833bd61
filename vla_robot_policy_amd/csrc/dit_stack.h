// The DiT layers of one Euler step of the flow sampler's action expert as a
// single persistent kernel, for action chunks of at most 16 rows.
//
// Page "AI Infra如何优化VLA - 模型推理性能提升技术拆解" (section 整体方案 and
// the CUDA Graph section): the action expert is memory-bound and was launch-
// bound before graphs. At 16 rows every GEMM of a layer is a weight stream of
// 3-13 MB, far too little to hide a kernel's launch, argument fetch, first
// load latency and tail; here the eight steps of every layer run in one
// launch, layer after layer:
//
//   0 QKV    u = LN(x)(1 + scale_sa) + shift_sa;  qkv = u Wqkv^T + b
//   1 SAATT  per head: ao = softmax(q k^T / sqrt(d)) v     (no mask)
//   2 SAO    x += gate_sa * (ao Wo^T + b)
//   3 CAQ    u = LN(x)(1 + scale_ca) + shift_ca;  q = u Wcq^T + b
//   4 CAATT  per head: ao = softmax(q Kc^T / sqrt(d)) Vc    (context K/V)
//   5 CAO    x += gate_ca * (ao Wco^T + b)
//   6 UP     u = LN(x)(1 + scale_mlp) + shift_mlp;  h = GELU(u W1^T + b1)
//   7 DOWN   x += gate_mlp * (h W2^T + b2)
//
// Work units: 16 output columns x D input columns of one GEMM (32 columns
// for UP; DOWN is split into mlp / 2D slices of 2D columns, summed in a fixed
// order by the tile's first slice), or one attention head. Unit u of phase p
// of layer l belongs to workgroup (u + base(l, p)) mod G, where the bases
// count every unit before it in the launch, so a workgroup knows its units
// in advance and streams their weights into registers before it waits for
// the previous phase: the HBM latency of the next weights overlaps the
// current phase. The next layer's QKV weights are requested by their owners
// while the current layer's DOWN runs.
// The outputs of QKV and CAQ, which only the attention phases' few
// workgroups read, travel as flagged words (below): the attention polls the
// words of its head, and the load that sees them there is the load that
// brings them. Every other phase hands on by counters: it writes with
// device-coherent (sc1) stores, waits for them, then counts, and the next
// phase polls the counter (counts accumulate over the launch's layers).
// Every other buffer written inside the launch (the fp32 residual stream,
// the attention outputs, the MLP activations) has one copy per layer and
// sublayer and is written once before anything reads it, so once its phase
// is counted it is read with ordinary cached loads: no XCD's private L2 can
// hold an older copy.
// Every wait is bounded and also gives up once another workgroup has
// recorded a time-out: the workgroup then poisons the launch's output with
// NaN and leaves, so a fault can never hang the device. The workgroup that
// completes the last layer's last DOWN tile resets the counters for the next
// launch.
//
// Each LayerNorm is computed by every workgroup that needs it, from the fp32
// residual stream held in registers (two-pass mean / variance), so no
// statistics travel between workgroups. The width D is a template parameter:
// every loop over a row is unrolled without bounds branches.
#pragma once
#include "common.h"

namespace vla {

enum DitPhase { DP_QKV = 0, DP_SAATT, DP_SAO, DP_CAQ, DP_CAATT, DP_CAO, DP_UP, DP_DOWN, DP_N };

constexpr int DS_THREADS = 256;
constexpr int DS_KSW = 10;        // 32-wide k-steps per wave per unit: D <= 4 * 10 * 32
constexpr int DS_MAXU = 2;        // 16 x D GEMM units per workgroup per phase (the kernel unrolls two)
// A workgroup's weight registers hold DS_MAXU units of 16 x D (or one unit
// of UP or DOWN).
constexpr int DS_WSLOTS = DS_MAXU * DS_KSW;
constexpr int DS_DP = 96;         // head dim padded for the attention MFMAs
constexpr int DS_KB = 32;         // keys per attention block
constexpr unsigned DS_SPIN = 1u << 17;   // polls before a wait gives up (a healthy wait is microseconds)
// Phase counters: every phase counts into DS_NC slots 256 bytes apart
// (workgroup w adds to slot w % DS_NC), so arrivals and the next phase's
// polls do not serialise on one address. On the launch's last layer DOWN
// also counts into one more word, whose last arrival resets them all.
constexpr int DS_NC = 16, DS_CSTRIDE = 64;
constexpr int DS_LAST = DP_N * DS_NC * DS_CSTRIDE;   // the last layer's DOWN tiles
__host__ __device__ constexpr int ds_counter_words(int) { return DS_LAST + DS_CSTRIDE; }
// flagged words of the DOWN slice partials: slices 1 .. of every tile
__host__ __device__ constexpr int ds_dpart_words(int D, int mlp) { return (mlp / (2 * D) - 1) * (D / 16) * 256; }

// One layer's weights, as the layer table in device memory holds them.
// The thread index, re-read for every layer: values derived from it are
// recomputed where a phase uses them instead of being hoisted out of the
// layer loop, where they would hold registers across every phase (measured:
// without it the bf16 kernel spills 340 bytes per lane).
__device__ __forceinline__ int ds_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}
// the wave index, known uniform across the wave (a scalar register)
__device__ __forceinline__ int ds_wave() { return __builtin_amdgcn_readfirstlane(ds_tid() >> 6); }

struct DitLayerPtrs {
  const void* w[6];               // qkv, o, cq, co, up, down: [N, K] row-major
  const float* s[6];              // per-row 8-bit weight scales (NULL for bf16)
  const float* b[6];              // biases
};

struct DitLayerArgs {
  int n, D, H, hd, mlp, C;        // action rows (<= 16), width, heads, head dim, MLP width, context tokens
  float eps, scale_log2;          // LayerNorm epsilon; log2(e) / sqrt(hd)
  int l0, l1;                     // the layers this launch runs
  const DitLayerPtrs* tab;        // [layers] weight table
  const float* mod;               // [layers][9][D] modulation of this Euler step
  const uint16_t* ckv;            // context keys: layer l's at ckv + l 2D, row pitch ldc
  const uint16_t* vt;             // context values transposed: layer l's [D][ldvt] at vt + l D ldvt, zero beyond C keys
  int ldc, ldvt;                  // ldvt: a multiple of 32, >= C
  // per-layer buffers, each written once per launch before anything reads it:
  // xs[l] [n, D] is layer l's input (xs[l + 1] its output), x1 = xs[l] + the
  // self-attention branch, x2 = x1 + the cross-attention branch (fp32)
  float* xs;                      // [layers + 1][n][D]
  float* x1;                      // [layers][n][D]
  float* x2;
  uint16_t* aos;                  // [layers][n][D] self-attention output
  uint16_t* aoc;                  // [layers][n][D] cross-attention output
  uint16_t* h;                    // [layers][n][mlp] GELU output
  // flagged words (two bf16 of adjacent columns + flag): [n, 3D / 2], [n, D / 2]
  uint2* qkv;
  uint2* q;                       // cross-attention query
  uint2* dpart;                   // DOWN partials of slices 1..: flagged words [slices - 1][D/16][256]
  const void* wq_next;            // the next launch's first QKV weights (NULL: none), read ahead into the memory-side cache
  unsigned* cnt;                  // ds_counter_words(D) counters (zero between launches)
  int* err;                       // set to 1 when a wait times out
  unsigned spin;                  // polls before a wait gives up (DS_SPIN unless the host asks for fewer)
  unsigned flag0;                 // word flag of layer l0 (layer l: flag0 + l - l0): nonzero, and above every
                                  // flag written since the words were cleared
};

// Layer l of a launch, resolved from the table (uniform across the workgroup).
struct DsLayer {
  const void* w[6];
  const float* s[6];
  const float* b[6];
  const float* mod;
  const uint16_t* ck;
  const uint16_t* cv;
  const float* x_in;
  float* x1;
  float* x2;
  float* x_out;
  uint16_t* aos;
  uint16_t* aoc;
  uint16_t* h;
  const void* wq_next;            // the next layer's QKV weights (NULL on the launch's last layer)
  unsigned flag;
  int l, li;                      // layer, and its index within the launch
  bool last;                      // the launch's last layer
};

__device__ __forceinline__ void st_sc1_f32(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// ---------------------------------------------------------------- flagged words
// A flagged word is 8 bytes: two bf16 of adjacent columns, then the flag of
// the launch that wrote it, stored by one device-coherent 8-byte store (an
// aligned 8-byte store reaches memory whole, so a reader sees the old or
// the new word, never half of each). A consumer polls until every word it
// needs carries the launch's flag; the producer neither waits for its stores
// nor counts. The buffers are cleared before a sampler run and the flags of
// its launches increase, so no word left by an earlier launch can pass.
__device__ __forceinline__ void st_fw(brsrc r, uint32_t word, uint32_t data, uint32_t flag) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, make_uint2(data, flag)), r, word * 8u, 0, CP_SC1);
}

// Poll NCH chunks of two flagged words per thread. word(i) is chunk i's first
// word, -1 for no chunk, -2 for a chunk of zeros (a row beyond the chunk);
// put(i, data) takes its four bf16 once both of its flags are the launch's.
// Every pending chunk is read each round: the pollers are the attention
// phases' few workgroups, with a head's rows each (a few KB). False after
// DS_SPIN rounds.
template <int NCH, typename WordF, typename PutF>
__device__ __forceinline__ bool ds_poll(brsrc r, uint32_t flag, unsigned spin, const int* err, WordF word, PutF put) {
  static_assert(NCH <= 64, "one pending bit per chunk");
  uint4 v[NCH];
  uint64_t pend = 0;
#pragma unroll
  for (int i = 0; i < NCH; i++) {
    const int w = word(i);
    if (w >= 0) pend |= 1ull << i;
    else if (w == -2) put(i, make_uint2(0u, 0u));
    v[i] = bload16<CP_SC1>(r, w >= 0 ? (uint32_t)w * 8u : BUF_OOB);
  }
  for (unsigned spins = 0;; spins++) {
#pragma unroll
    for (int i = 0; i < NCH; i++)
      if ((pend >> i & 1) && v[i].y == flag && v[i].w == flag) {
        put(i, make_uint2(v[i].x, v[i].z));
        pend &= ~(1ull << i);
      }
    if (!pend) return true;
    if (spins >= spin) return false;
    // another workgroup timed out: give up too
    if ((spins & 31) == 31 && __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int i = 0; i < NCH; i++)
      if (pend >> i & 1) v[i] = bload16<CP_SC1>(r, (uint32_t)word(i) * 8u);
  }
}

// ---------------------------------------------------------------- phase geometry
__device__ __forceinline__ int ds_units(const DitLayerArgs& a, int ph) {
  switch (ph) {
    case DP_QKV: return 3 * a.D / 16;
    case DP_SAATT: case DP_CAATT: return a.H;
    case DP_SAO: case DP_CAQ: case DP_CAO: return a.D / 16;
    case DP_UP: return a.mlp / 32;
    default: return (a.D / 16) * (a.mlp / (2 * a.D));
  }
}
// value of the phase counter once the phase is complete
__device__ __forceinline__ int ds_target(const DitLayerArgs& a, int ph) { return ph == DP_DOWN ? a.D / 16 : ds_units(a, ph); }
// units before phase ph of layer l in the launch, modulo the grid
__device__ __forceinline__ int ds_base(const DitLayerArgs& a, int l, int ph) {
  int per = 0, b = 0;
  for (int q = 0; q < DP_N; q++) {
    if (q == ph) b = per;
    per += ds_units(a, q);
  }
  return (int)(((long long)(l - a.l0) * per + b) % gridDim.x);
}
// this workgroup's first unit of phase ph of layer l (>= the phase's units: none)
__device__ __forceinline__ int ds_first(const DitLayerArgs& a, int l, int ph) {
  const int G = gridDim.x;
  return ((int)blockIdx.x - ds_base(a, l, ph) + G) % G;
}

// Wait until the DS_NC slots of a phase counter sum to target (wave 0
// polls, one slot per lane; the workgroup follows). False after `spin`
// polls. One read is in flight at a time: the barrier that follows waits
// for every outstanding read, so reads issued ahead only delay the exit
// (measured: 3.5 us per layer with four in flight).
// Lane 16 reads the error word with the same load: a time-out elsewhere
// ends the wait at once.
__device__ __forceinline__ bool ds_wait(const unsigned* slots, unsigned target, unsigned spin, const int* err, int* sflag) {
  if (ds_wave() == 0) {
    static_assert(DS_NC == 16, "the phase counter slots are one DPP row");
    const int lane = ds_tid();
    const unsigned* p = lane < DS_NC ? slots + lane * DS_CSTRIDE : reinterpret_cast<const unsigned*>(err);
    unsigned spins = 0;
    bool ok = true;
    while (true) {
      unsigned v = lane <= DS_NC ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      // exact: counts stay far below 2^24; uniform (read from lanes 0 and 16)
      const unsigned tot = (unsigned)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(row16_sum((float)(lane < DS_NC ? v : 0u))), 0));
      if (tot >= target) break;
      if (++spins >= spin || __builtin_amdgcn_readlane((int)v, DS_NC)) { ok = false; break; }
      // far from the target, poll less often (fewer reads competing with the
      // phase being waited for)
      if (tot + 8 < target) __builtin_amdgcn_s_sleep(16);
      else __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) sflag[0] = ok;
  }
  __syncthreads();
  return sflag[0] != 0;
}

// Read bytes [i, i + 1) / n of the next launch's QKV weights and drop them
// (the memory-side cache keeps them for that launch's first phase).
template <typename WT, int D>
__device__ __forceinline__ void ds_prefetch_qkv_share(const DitLayerArgs& a, const void* wq, int i, int n) {
  const size_t total = (size_t)3 * D * D * sizeof(WT);
  const size_t share = (total / n + 4095) & ~(size_t)4095;
  const size_t b0 = (size_t)i * share, b1 = b0 + share < total ? b0 + share : total;
  const brsrc nr = make_brsrc(wq);
  uint32_t acc = 0;
  for (size_t off = b0 + (size_t)ds_tid() * 16; off < b1; off += (size_t)DS_THREADS * 16 * 8) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const size_t o = off + (size_t)k * DS_THREADS * 16;
      v[k] = bload16(nr, o < b1 ? (uint32_t)o : BUF_OOB);
    }
#pragma unroll
    for (int k = 0; k < 8; k++) acc ^= v[k].x;
  }
  if (acc == 0x9E3779B9u) a.err[1] = 0;   // keeps the loads; practically never taken
}

// ---------------------------------------------------------------- weight units
template <typename WT> struct DsW;
template <> struct DsW<uint16_t> {
  using raw = uint4;
  static constexpr int ESZ = 2;
  __device__ static raw load(brsrc r, uint32_t off) { return bload16<CP_NT>(r, off); }
  __device__ static FragBF16 frag(raw v) { FragBF16 f; f.v = __builtin_bit_cast(bf16x8, v); return f; }
};
template <> struct DsW<uint8_t> {
  using raw = uint2;
  static constexpr int ESZ = 1;
  __device__ static raw load(brsrc r, uint32_t off) { return bload8<CP_NT>(r, off); }
  __device__ static FragBF16 frag(raw v) { return fp8x8_to_frag(v); }
};
template <> struct DsW<int8_t> {
  using raw = uint2;
  static constexpr int ESZ = 1;
  __device__ static raw load(brsrc r, uint32_t off) { return bload8<CP_NT>(r, off); }
  __device__ static FragBF16 frag(raw v) { return int8x8_to_frag(v); }
};

// A unit is NB blocks of 16 output columns over a k range of KW: 16 columns
// x D for QKV, SAO, CAQ and CAO; 32 columns x D for UP; 16 columns x 2D (one
// of mlp / 2D slices, summed in a fixed order by the tile's last slice) for
// DOWN. The two MLP phases thus have one unit per workgroup at the full
// model's shapes.
struct DsUnit {
  int wi;        // weight index (0..5)
  int N, K;      // output width, row length of W
  int n0, k0;    // first output column, first k of this unit
};

__device__ __forceinline__ DsUnit ds_unit(const DitLayerArgs& a, int ph, int u) {
  DsUnit d;
  d.n0 = 16 * u; d.k0 = 0; d.K = a.D;
  switch (ph) {
    case DP_QKV: d.wi = 0; d.N = 3 * a.D; break;
    case DP_SAO: d.wi = 1; d.N = a.D; break;
    case DP_CAQ: d.wi = 2; d.N = a.D; break;
    case DP_CAO: d.wi = 3; d.N = a.D; break;
    case DP_UP: d.wi = 4; d.N = a.mlp; d.n0 = 32 * u; break;
    default: {   // DOWN: tile u % (D/16), slice u / (D/16) of 2D columns
      const int nt = a.D / 16;
      d.wi = 5; d.N = a.D; d.K = a.mlp;
      d.n0 = 16 * (u % nt); d.k0 = (u / nt) * 2 * a.D;
    }
  }
  return d;
}

// The wave's k-steps of a unit: steps s = wave + 4 i (i < NS) of KST for each
// of the NB column blocks, into register slots OFF + b NS + i.
template <typename WT, int OFF, int NB, int NS, int KST>
__device__ __forceinline__ void ds_load_unit(const void* w, const DsUnit& d, typename DsW<WT>::raw (&r)[DS_WSLOTS]) {
  static_assert(OFF + NB * NS <= DS_WSLOTS, "unit exceeds the weight registers");
  const int lane = ds_tid() & 63, wave = ds_wave();
  const brsrc wr = make_brsrc(w);
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const int col = d.n0 + b * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < NS; i++) {
      int s = wave + 4 * i;
      int k = d.k0 + s * 32 + (lane >> 4) * 8;
      bool ok = s < KST && col < d.N;
      r[OFF + b * NS + i] = DsW<WT>::load(wr, ok ? ((uint32_t)col * d.K + k) * DsW<WT>::ESZ : BUF_OOB);
    }
  }
}

// Zero register slots OFF .. OFF + N - 1.
template <typename WT, int OFF, int N>
__device__ __forceinline__ void ds_zero_slots(typename DsW<WT>::raw (&r)[DS_WSLOTS]) {
#pragma unroll
  for (int i = OFF; i < OFF + N && i < DS_WSLOTS; i++) r[i] = typename DsW<WT>::raw{};
}

// NB 16 x 16 tiles of one unit: A [16][KW] bf16 in LDS (pitch apitch),
// weights in register slots OFF ..; the wave's partial sums over its k-steps.
template <typename WT, int OFF, int NB, int NS, int KST>
__device__ __forceinline__ void ds_mma(const char* rA, int apitch, const typename DsW<WT>::raw (&w)[DS_WSLOTS], f32x4 (&acc)[NB]) {
  const int lane = ds_tid() & 63, wave = ds_wave();
#pragma unroll
  for (int b = 0; b < NB; b++) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; i++) {
    int s = wave + 4 * i;
    if (s < KST) {
      FragBF16 af;
      af.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rA + (lane & 15) * apitch + (s * 32 + (lane >> 4) * 8) * 2));
#pragma unroll
      for (int b = 0; b < NB; b++) mma32(acc[b], af, DsW<WT>::frag(w[OFF + b * NS + i]));
    }
  }
}

// ---------------------------------------------------------------- attention of one head (<= 16 queries)
// Cross-attention: the four waves take interleaved blocks of 32 context
// keys: S^T = K Q^T per block, online softmax per lane, O^T = V^T P^T. Q
// comes from LDS (staged from its flagged words); the K and V^T fragments
// are 16-byte loads straight from memory: K rows are contiguous in the head
// dimension, and the values are stored transposed (one row of keys per head
// column). The K rows of a block are taken in the order that leaves lane
// group g the scores of keys 8g .. 8g + 7 (keys 8g + i from the first
// 16-row half, 8g + 4 + i from the second), so the lane's P fragment and the
// V^T fragment it multiplies cover 8 consecutive keys. With more than one
// block the waves' partial (max, sum, O) are combined in LDS; with one block
// wave 0 writes the output itself (device-coherent bf16 stores).

// Key of row r (< 16) of half hb of a block: lane group r / 4 holds rows
// 4 (r / 4) .. + 3 of each half.
__device__ __forceinline__ int ds_key_of_row(int hb, int r) { return 8 * (r >> 2) + 4 * hb + (r & 3); }

// The fragments of one 32-key block: K for the two 16-key halves and the
// three 32-wide steps of the (padded) head dimension; V^T for the six
// 16-column blocks, keys 8g .. 8g + 7 of lane group g.
struct DsAttFr {
  uint4 k[2][DS_DP / 32];
  uint4 v[DS_DP / 16];
};

__device__ __forceinline__ void ds_att_frags(brsrc kr, brsrc vr, int blk, int nblk, int nk, int ldk, int ldvt, int hd,
                                             DsAttFr& f) {
  const int lane = ds_tid() & 63, qn = lane & 15, grp = lane >> 4;
  const int kb = blk * DS_KB;
  const bool live = blk < nblk;
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int ds = 0; ds < DS_DP / 32; ds++) {
      const int key = kb + ds_key_of_row(hb, qn), d = ds * 32 + grp * 8;
      const uint32_t off = (live && key < nk && d < hd) ? ((uint32_t)key * ldk + d) * 2u : BUF_OOB;
      f.k[hb][ds] = bload16(kr, off);
    }
  // keys up to the block's end lie within the zero-padded rows of V^T
#pragma unroll
  for (int db = 0; db < DS_DP / 16; db++) {
    const int d = db * 16 + qn;
    f.v[db] = bload16(vr, (live && d < hd) ? ((uint32_t)d * ldvt + kb + 8 * grp) * 2u : BUF_OOB);
  }
}

// `f` holds this wave's first block when `have0` (requested before the
// caller's wait); each later round is requested before the current one is
// computed.
// qs: Q rows [16][DS_DP] bf16 in LDS, zero beyond nq rows and hd columns;
// the output goes to columns oc .. oc + hd of O's rows (ldo bf16 columns).
__device__ __forceinline__ void ds_attention(const char* qs, const uint16_t* Kp, const uint16_t* Vt, int ldk, int ldvt,
                                             uint16_t* O, int ldo, int oc, int nq, int nk, int hd, float scale_log2,
                                             char* lds_o, DsAttFr& f, bool have0) {
  const int tid = ds_tid(), lane = tid & 63, wave = ds_wave();
  const int qn = lane & 15, grp = lane >> 4;
  const brsrc kr = make_brsrc(Kp), vr = make_brsrc(Vt), orr = make_brsrc(O);
  const int nblk = (nk + DS_KB - 1) / DS_KB;

  FragBF16 qf[DS_DP / 32];
#pragma unroll
  for (int ds = 0; ds < DS_DP / 32; ds++)
    qf[ds].v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qs + (qn * DS_DP + ds * 32 + grp * 8) * 2));
  if (!have0) ds_att_frags(kr, vr, wave, nblk, nk, ldk, ldvt, hd, f);
  f32x4 oacc[DS_DP / 16];
#pragma unroll
  for (int i = 0; i < DS_DP / 16; i++) oacc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  for (int r0 = 0; r0 < nblk; r0 += 4) {
    const int blk = r0 + wave;
    if (blk < nblk) {
      const int kb = blk * DS_KB;
      // this block's fragments; the next round's are requested before use
      FragBF16 kf[2][DS_DP / 32], vf[DS_DP / 16];
#pragma unroll
      for (int hb = 0; hb < 2; hb++)
#pragma unroll
        for (int ds = 0; ds < DS_DP / 32; ds++) kf[hb][ds].v = __builtin_bit_cast(bf16x8, f.k[hb][ds]);
#pragma unroll
      for (int db = 0; db < DS_DP / 16; db++) vf[db].v = __builtin_bit_cast(bf16x8, f.v[db]);
      if (r0 + 4 < nblk) ds_att_frags(kr, vr, blk + 4, nblk, nk, ldk, ldvt, hd, f);
      f32x4 s[2];
#pragma unroll
      for (int hb = 0; hb < 2; hb++) {
        s[hb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS_DP / 32; ds++) mma32(s[hb], kf[hb][ds], qf[ds]);
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int hb = 0; hb < 2; hb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int j = kb + ds_key_of_row(hb, grp * 4 + i);
          float v = j < nk ? s[hb][i] * scale_log2 : -INFINITY;
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
      FragBF16 pf;
      frag_from_floats(pf, pv);
#pragma unroll
      for (int db = 0; db < DS_DP / 16; db++) {
        oacc[db] = oacc[db] * corr;
        mma32(oacc[db], vf[db], pf);
      }
    }
  }
  float lsum = lrun;
  lsum += __shfl_xor(lsum, 16, WAVE);
  lsum += __shfl_xor(lsum, 32, WAVE);
  if (nblk <= 1) {
    // one block: wave 0 holds the whole result, O^T[d][q] with d = 16 db +
    // 4 g + i in lane (q, g)
    if (wave == 0 && qn < nq) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int db = 0; db < DS_DP / 16; db++) {
        const int d = db * 16 + grp * 4;
        if (d < hd) {
          uint2 pk;
          pk.x = pack_bf2(oacc[db][0] * inv, oacc[db][1] * inv);
          pk.y = pack_bf2(oacc[db][2] * inv, oacc[db][3] * inv);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, pk), orr, (uint32_t)(qn * ldo + oc + d) * 2u, 0,
                                                CP_SC1);
        }
      }
    }
    return;
  }
  // combine the four waves: per query (max, sum) and O^T partials in LDS
  float* sml = reinterpret_cast<float*>(lds_o);                  // [4][16][2]
  float* so = sml + 4 * 16 * 2;                                  // [4][16][DP]
  __syncthreads();
  if (grp == 0) { sml[(wave * 16 + qn) * 2] = mrun; sml[(wave * 16 + qn) * 2 + 1] = lsum; }
#pragma unroll
  for (int db = 0; db < DS_DP / 16; db++)
#pragma unroll
    for (int i = 0; i < 4; i++) so[(wave * 16 + qn) * DS_DP + db * 16 + grp * 4 + i] = oacc[db][i];
  __syncthreads();
  for (int e = tid; e < 16 * DS_DP / 4; e += DS_THREADS) {
    const int q = e / (DS_DP / 4), d = (e % (DS_DP / 4)) * 4;
    if (q >= nq || d >= hd) continue;
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) { mw[w] = sml[(w * 16 + q) * 2]; M = fmaxf(M, mw[w]); }
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; w++) {
      float fw = (mw[w] == -INFINITY) ? 0.f : exp2f(mw[w] - M);
      L += fw * sml[(w * 16 + q) * 2 + 1];
      float4 o = *reinterpret_cast<const float4*>(so + (w * 16 + q) * DS_DP + d);
      acc.x += fw * o.x; acc.y += fw * o.y; acc.z += fw * o.z; acc.w += fw * o.w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint2 pk;
    pk.x = pack_bf2(acc.x * inv, acc.y * inv);
    pk.y = pack_bf2(acc.z * inv, acc.w * inv);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, pk), orr, (uint32_t)(q * ldo + oc + d) * 2u, 0, CP_SC1);
  }
}

// Self-attention of one head over the chunk's n <= 16 rows, from LDS: Q and
// K rows [16][DS_DP] and V transposed [DS_DP][16], zero beyond n rows and hd
// columns. Wave 0 computes S^T = K Q^T, the softmax and O^T = V^T P^T as
// one 32-key block whose keys 16..31 are absent (their P is zero), with the
// arithmetic of the cross-attention's single-block case.
__device__ __forceinline__ void ds_self_att(const char* st, uint16_t* O, int ldo, int oc, int n, int hd, float scale_log2) {
  if (ds_wave() != 0) return;
  const int lane = ds_tid() & 63, qn = lane & 15, grp = lane >> 4;
  const char* qs = st;
  const char* ks = st + 16 * DS_DP * 2;
  const char* vt = st + 2 * 16 * DS_DP * 2;
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < DS_DP / 32; ds++) {
    FragBF16 qf, kf;
    qf.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qs + (qn * DS_DP + ds * 32 + grp * 8) * 2));
    kf.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks + (qn * DS_DP + ds * 32 + grp * 8) * 2));
    mma32(s, kf, qf);
  }
  // lane (query qn, group g) holds the scores of keys 4g .. 4g + 3
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float v = grp * 4 + i < n ? s[i] * scale_log2 : -INFINITY;
    s[i] = v;
    m = fmaxf(m, v);
  }
  m = fmaxf(m, __shfl_xor(m, 16, WAVE));
  m = fmaxf(m, __shfl_xor(m, 32, WAVE));
  float pv[8], l = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    pv[i] = exp2f(s[i] - m);
    pv[4 + i] = 0.f;
    l += pv[i];
  }
  l += __shfl_xor(l, 16, WAVE);
  l += __shfl_xor(l, 32, WAVE);
  FragBF16 pf;
  frag_from_floats(pf, pv);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const brsrc orr = make_brsrc(O);
#pragma unroll
  for (int db = 0; db < DS_DP / 16; db++) {
    const uint2 v2 = *reinterpret_cast<const uint2*>(vt + ((db * 16 + qn) * 16 + 4 * grp) * 2);
    FragBF16 vf;
    vf.v = __builtin_bit_cast(bf16x8, make_uint4(v2.x, v2.y, 0u, 0u));
    f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
    mma32(o, vf, pf);
    const int d = db * 16 + grp * 4;
    if (qn < n && d < hd) {
      uint2 pk;
      pk.x = pack_bf2(o[0] * inv, o[1] * inv);
      pk.y = pack_bf2(o[2] * inv, o[3] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, pk), orr, (uint32_t)(qn * ldo + oc + d) * 2u, 0,
                                            CP_SC1);
    }
  }
}

// True when every thread of the workgroup passed (sflag[2] is cleared at the
// kernel's start and set only by a failure, after which the workgroup leaves).
__device__ __forceinline__ bool ds_all(bool ok, int* sflag) {
  if (!ok) sflag[2] = 1;
  __syncthreads();
  return sflag[2] == 0;
}

// ---------------------------------------------------------------- the layer kernel
// LDS: [region A: bf16 A operand (16 x D, 16 x 2D for DOWN), or attention
// partials then the head's staged Q, K, V^T] [4 waves x 2 blocks x 256 fp32
// wave sums] [flags]
constexpr int DS_ATT_PART = (4 * 16 * 2 + 4 * 16 * DS_DP) * 4;
constexpr int DS_ATT_STAGE = 3 * 16 * DS_DP * 2;
__host__ __device__ constexpr int ds_region_a(int D) {
  return 16 * (4 * D + 16) > DS_ATT_PART + DS_ATT_STAGE ? 16 * (4 * D + 16) : DS_ATT_PART + DS_ATT_STAGE;
}
__host__ __device__ constexpr int ds_smem_bytes(int D) { return ds_region_a(D) + 2 * 4 * 256 * 4 + 64; }

// Layer l of the launch from the weight table and the per-layer buffers.
template <int D>
__device__ __forceinline__ DsLayer ds_layer(const DitLayerArgs& a, int l) {
  DsLayer y;
  const DitLayerPtrs* t = a.tab + l;
#pragma unroll
  for (int i = 0; i < 6; i++) { y.w[i] = t->w[i]; y.s[i] = t->s[i]; y.b[i] = t->b[i]; }
  const size_t nd = (size_t)a.n * D;
  y.mod = a.mod + (size_t)l * 9 * D;
  y.ck = a.ckv + (size_t)l * 2 * D;
  y.cv = a.vt + (size_t)l * D * a.ldvt;
  y.x_in = a.xs + (size_t)l * nd;
  y.x_out = a.xs + (size_t)(l + 1) * nd;
  y.x1 = a.x1 + (size_t)l * nd;
  y.x2 = a.x2 + (size_t)l * nd;
  y.aos = a.aos + (size_t)l * nd;
  y.aoc = a.aoc + (size_t)l * nd;
  y.h = a.h + (size_t)l * a.n * a.mlp;
  y.last = l + 1 == a.l1;
  y.wq_next = y.last ? nullptr : a.tab[l + 1].w[0];
  y.flag = a.flag0 + (unsigned)(l - a.l0);
  y.l = l;
  y.li = l - a.l0;
  return y;
}

// One phase of a layer for this workgroup, specialised per phase so that
// each phase's registers are allocated for that phase alone. False when the
// workgroup must leave the kernel (a wait timed out). `wdown` holds the
// workgroup's DOWN unit: a workgroup that also has an UP unit requests it
// together with the UP weights (it is idle long before UP starts), so its
// DOWN phase does not begin with a weight fetch queued ahead of its wait.
// `wqkv` holds its QKV units: those of the next layer are requested during
// this layer's DOWN, before its wait.
template <typename WT, int D, int PH>
__device__ __forceinline__ bool ds_phase(const DitLayerArgs& a, const DsLayer& y, int prev_err, char* rA, float* red,
                                         int* sflag, int& finished_tiles, typename DsW<WT>::raw (&wdown)[DS_WSLOTS],
                                         bool& have_down, typename DsW<WT>::raw (&wqkv)[DS_WSLOTS], bool& have_qkv) {
  using WR = typename DsW<WT>::raw;
  const int tid = ds_tid(), lane = tid & 63, wave = ds_wave();
  const int G = gridDim.x;
  const int n = a.n;
  constexpr int APITCH = D * 2 + 16;
  constexpr int ntile = D / 16;
  // unit geometry: NB column blocks of 16 over a k extent KW (a unit of UP
  // or DOWN fills all weight registers; the other GEMMs take up to two units)
  constexpr int NB = PH == DP_UP ? 2 : 1;
  constexpr int KW = PH == DP_DOWN ? 2 * D : D;
  constexpr int KST = KW / 32;                       // 32-wide k-steps of a unit
  constexpr int NSW = (KST + 3) / 4;                 // of them per wave
  constexpr int MAXU = 2 * NB * NSW <= DS_WSLOTS ? 2 : 1;
  const int U = ds_units(a, PH);
  const int first = ds_first(a, y.l, PH);
  // the next layer's QKV units of this workgroup, into wqkv, requested when
  // UP starts: early enough to arrive long before the next QKV, and not
  // queued ahead of the DOWN epilogue's loads (loads complete in order).
  // Every slot is written on every path (zeros where there is no unit), so
  // the registers are free between a layer's QKV and its UP.
  auto preload_qkv = [&]() {
    constexpr int KSTQ = D / 32, NSWQ = (KSTQ + 3) / 4;
    const int fq = y.last ? 0 : ds_first(a, y.l + 1, DP_QKV), uq = ds_units(a, DP_QKV);
    const bool one = !y.last && fq < uq, two = one && fq + G < uq;
    if (one) ds_load_unit<WT, 0, 1, NSWQ, KSTQ>(y.wq_next, ds_unit(a, DP_QKV, fq), wqkv);
    else ds_zero_slots<WT, 0, NSWQ>(wqkv);
    if (two) ds_load_unit<WT, NSWQ, 1, NSWQ, KSTQ>(y.wq_next, ds_unit(a, DP_QKV, fq + G), wqkv);
    else ds_zero_slots<WT, NSWQ, DS_WSLOTS - NSWQ>(wqkv);
    have_qkv = one;
  };
  if (first >= U) {                                  // no work in this phase
    if constexpr (PH == DP_UP) {
      // nor in DOWN, on the launch's last layer: read a share of the next
      // launch's first QKV weights into the memory-side cache
      const int fd = ds_first(a, y.l, DP_DOWN), ud = ds_units(a, DP_DOWN);
      if (y.last && fd >= ud && a.wq_next) ds_prefetch_qkv_share<WT, D>(a, a.wq_next, fd - ud, G - ud);
      // wdown is written on every path through UP (its DOWN unit loads it)
      ds_zero_slots<WT, 0, DS_WSLOTS>(wdown);
      have_down = false;
      preload_qkv();
    }
    return true;
  }
  const int nu = (U - first + G - 1) / G;           // at most MAXU (checked by the launcher)
  constexpr bool is_att = PH == DP_SAATT || PH == DP_CAATT;

  constexpr bool norm = PH == DP_QKV || PH == DP_CAQ || PH == DP_UP;
  // Everything that does not depend on the previous phase is requested
  // before its wait: the first context K / V block of a cross-attention
  // head, a LayerNorm's shift / scale, the weights of the GEMM units. Each
  // kind of phase keeps its own registers across its own wait.
  // a wait timed out: record it, poison this workgroup's outputs
  auto fail = [&]() -> bool {
    if (tid == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float* xo = a.xs + (size_t)a.l1 * n * D;
    for (int e = tid; e < n * D; e += DS_THREADS) st_sc1_f32(xo + e, __builtin_nanf(""));
    return false;
  };
  // every phase but the attentions waits for the previous phase's counter
  // (QKV: the previous layer's DOWN; none on the launch's first layer).
  // Counts accumulate over the launch's layers. After a failed earlier
  // launch of the run, the first wait leaves.
  auto wait_prev = [&]() -> bool {
    if (PH == DP_QKV && y.li == 0) return true;
    const int pp = PH == DP_QKV ? DP_DOWN : PH - 1;
    const unsigned target = (unsigned)((PH == DP_QKV ? y.li : y.li + 1) * ds_target(a, pp));
    if (!prev_err && ds_wait(a.cnt + pp * DS_NC * DS_CSTRIDE, target, a.spin, a.err, sflag)) return true;
    return fail();
  };
  // LayerNorm geometry: wave w normalises rows 4w .. 4w + 3; lane l holds
  // float4 column groups l + 64 k (k < KG) of them
  constexpr int KG = (D / 4 + 63) / 64;

  if constexpr (is_att) {
    DsAttFr f;
    constexpr bool cross = PH == DP_CAATT;
    if (cross)
      ds_att_frags(make_brsrc(y.ck + first * a.hd), make_brsrc(y.cv + (size_t)first * a.hd * a.ldvt), wave,
                   (a.C + DS_KB - 1) / DS_KB, a.C, a.ldc, a.ldvt, a.hd, f);
    // the head's rows are staged after the partials: Q [16][DS_DP], and for
    // the self-attention K [16][DS_DP] and V^T [DS_DP][16], zero beyond n
    // rows (written by the poll) and hd columns (written here)
    char* st = rA + DS_ATT_PART;
    uint16_t* st16 = reinterpret_cast<uint16_t*>(st);
    const int hd = a.hd, hq = hd / 4, pad = DS_DP - hd;
    for (int e = tid; e < 16 * pad; e += DS_THREADS) {
      const int r = e / pad, c = hd + e % pad;
      st16[r * DS_DP + c] = 0;
      if (!cross) {
        st16[16 * DS_DP + r * DS_DP + c] = 0;
        st16[2 * 16 * DS_DP + c * 16 + r] = 0;
      }
    }
    if (prev_err) return fail();
    // ---- one head per unit
    for (int j = 0; j < nu; j++) {
      const int hh = first + j * G;
      if (j) __syncthreads();   // the previous head's staged rows and partials have been read
      bool ok;
      if constexpr (cross) {
        constexpr int NCH = (16 * DS_DP / 4 + DS_THREADS - 1) / DS_THREADS;
        ok = ds_poll<NCH>(
            make_brsrc(a.q), y.flag, a.spin, a.err,
            [&](int i) -> int {
              const int e = tid + i * DS_THREADS;
              if (e >= 16 * hq) return -1;
              const int r = e / hq, c = 4 * (e % hq);
              return r < n ? (r * D + hh * hd + c) / 2 : -2;
            },
            [&](int i, uint2 v) {
              const int e = tid + i * DS_THREADS, r = e / hq, c = 4 * (e % hq);
              *reinterpret_cast<uint2*>(st + (r * DS_DP + c) * 2) = v;
            });
      } else {
        constexpr int NCH = (3 * 16 * DS_DP / 4 + DS_THREADS - 1) / DS_THREADS;
        ok = ds_poll<NCH>(
            make_brsrc(a.qkv), y.flag, a.spin, a.err,
            [&](int i) -> int {
              const int e = tid + i * DS_THREADS;
              if (e >= 3 * 16 * hq) return -1;
              const int mtx = e / (16 * hq), rem = e % (16 * hq), r = rem / hq, c = 4 * (rem % hq);
              return r < n ? (r * 3 * D + mtx * D + hh * hd + c) / 2 : -2;
            },
            [&](int i, uint2 v) {
              const int e = tid + i * DS_THREADS;
              const int mtx = e / (16 * hq), rem = e % (16 * hq), r = rem / hq, c = 4 * (rem % hq);
              if (mtx < 2) {
                *reinterpret_cast<uint2*>(st + (mtx * 16 * DS_DP + r * DS_DP + c) * 2) = v;
              } else {
                uint16_t* vt = st16 + 2 * 16 * DS_DP;
                vt[(c + 0) * 16 + r] = (uint16_t)v.x;
                vt[(c + 1) * 16 + r] = (uint16_t)(v.x >> 16);
                vt[(c + 2) * 16 + r] = (uint16_t)v.y;
                vt[(c + 3) * 16 + r] = (uint16_t)(v.y >> 16);
              }
            });
      }
      if (!ds_all(ok, sflag)) return fail();
      if constexpr (cross)
        ds_attention(st, y.ck + hh * hd, y.cv + (size_t)hh * hd * a.ldvt, a.ldc, a.ldvt, y.aoc, D, hh * hd, n, a.C, hd,
                     a.scale_log2, rA, f, j == 0);
      else
        ds_self_att(st, y.aos, D, hh * hd, n, hd, a.scale_log2);
    }
  } else {
    const int mi = PH == DP_QKV ? 0 : PH == DP_CAQ ? 3 : 6;   // shift, scale at mod[mi], mod[mi + 1]
    // shift and 1 + scale of the lane's column groups (requested before the wait)
    float4 shv[norm ? KG : 1], gv[norm ? KG : 1];
    if constexpr (norm) {
      const brsrc mr = make_brsrc(y.mod + (size_t)mi * D);
#pragma unroll
      for (int k = 0; k < KG; k++) {
        const int cg = lane + 64 * k;
        shv[k] = as_f4(bload16(mr, cg < D / 4 ? (uint32_t)cg * 16u : BUF_OOB));
        gv[k] = as_f4(bload16(mr, cg < D / 4 ? (uint32_t)(D + 4 * cg) * 4u : BUF_OOB));
      }
    }
    // per-column epilogue vectors of each unit (bias, 8-bit weight scale,
    // residual gate): inputs of the launch, requested before anything waits
    float pb[MAXU][NB], ps[MAXU][NB], pg[MAXU][NB];
    {
      const int wi = ds_unit(a, PH, first).wi;
      const bool scaled = y.s[wi] != nullptr;
      const brsrc br = make_brsrc(y.b[wi]), sr = make_brsrc(y.s[wi]);
      const brsrc gr = make_brsrc(y.mod + (size_t)(PH == DP_SAO ? 2 : PH == DP_CAO ? 5 : 8) * D);
#pragma unroll
      for (int j = 0; j < MAXU; j++) {
        const DsUnit d = ds_unit(a, PH, first + j * G);
#pragma unroll
        for (int b = 0; b < NB; b++) {
          const int col = d.n0 + b * 16 + (tid & 15);
          const uint32_t off = (j < nu && col < d.N) ? (uint32_t)col * 4u : BUF_OOB;
          pb[j][b] = bloadf(br, off);
          ps[j][b] = scaled ? bloadf(sr, off) : 1.f;
          pg[j][b] = norm ? 0.f : bloadf(gr, off);
        }
      }
    }
    // LayerNorm input rows: wave w holds rows 4w .. 4w + 3, lane l the float4
    // column groups l + 64 k. The first layer's QKV input is final at launch,
    // so its rows are requested ahead of its weights (loads complete in
    // order); the other LayerNorms read theirs after the wait.
    float4 xv[norm ? 4 : 1][norm ? KG : 1];
    const bool x_early = PH == DP_QKV && y.li == 0;
    auto load_x = [&]() {
      const brsrc xr = make_brsrc(PH == DP_QKV ? y.x_in : PH == DP_CAQ ? y.x1 : y.x2);
#pragma unroll
      for (int rr = 0; rr < 4; rr++)
#pragma unroll
        for (int k = 0; k < KG; k++) {
          const int r = 4 * wave + rr, cg = lane + 64 * k;
          xv[rr][k] = as_f4(bload16(xr, (cg < D / 4 && r < n) ? ((uint32_t)r * D + 4 * cg) * 4u : BUF_OOB));
        }
    };
    if (x_early) load_x();
    WR wreg[DS_WSLOTS];
    auto& wuse = [&]() -> WR (&)[DS_WSLOTS] {
      if constexpr (PH == DP_DOWN) return wdown;
      else if constexpr (PH == DP_QKV) return wqkv;
      else return wreg;
    }();
    const bool preloaded = (PH == DP_DOWN && have_down) || (PH == DP_QKV && have_qkv);
    if (!preloaded) {
      ds_load_unit<WT, 0, NB, NSW, KST>(y.w[ds_unit(a, PH, first).wi], ds_unit(a, PH, first), wuse);
      if constexpr (MAXU > 1)
        if (nu > 1) ds_load_unit<WT, NB * NSW, NB, NSW, KST>(y.w[ds_unit(a, PH, first).wi], ds_unit(a, PH, first + G), wuse);
    }
    if constexpr (PH == DP_DOWN) have_down = false;
    if constexpr (PH == DP_QKV) have_qkv = false;
    if constexpr (PH == DP_UP) {
      // every slot of wdown is written here (zeros without a DOWN unit), so
      // the registers are free between a layer's DOWN and the next UP
      const int fd = ds_first(a, y.l, DP_DOWN), ud = ds_units(a, DP_DOWN);
      constexpr int KSTD = 2 * D / 32, NSWD = (KSTD + 3) / 4;
      static_assert(NSWD <= DS_WSLOTS, "a DOWN unit exceeds the weight registers");
      if (fd < ud) ds_load_unit<WT, 0, 1, NSWD, KSTD>(y.w[5], ds_unit(a, DP_DOWN, fd), wdown);
      else ds_zero_slots<WT, 0, DS_WSLOTS>(wdown);
      have_down = fd < ud;
      preload_qkv();
      if (fd >= ud && y.last && a.wq_next) {
        // a workgroup with UP but no DOWN work is idle from here to UP's
        // wait: on the launch's last layer it reads its share of the next
        // launch's first QKV weights, so that launch's first phase finds
        // them in the memory-side cache (HBM is quiet here; the UP weights
        // were requested earlier and, needed only after the
        // cross-attention, have time to arrive)
        ds_prefetch_qkv_share<WT, D>(a, a.wq_next, fd - ud, G - ud);
      }
    }
    if (!wait_prev()) return false;
    // ---- the A operand [16][KW] (bf16) in region A
    float xpre[MAXU];
    if constexpr (!norm) {
      // SAO, CAO: the attention output; DOWN: the unit's slice of h (a
      // workgroup's units share their k range). Rows beyond n are zeros.
      const DsUnit d0 = ds_unit(a, PH, first);
      const uint16_t* src = PH == DP_DOWN ? y.h : PH == DP_SAO ? y.aos : y.aoc;
      const int lds = PH == DP_DOWN ? a.mlp : D;
      const brsrc sr = make_brsrc(src);
      constexpr int apitch = KW * 2 + 16;
      constexpr int AS = (16 * KW / 8 + DS_THREADS - 1) / DS_THREADS;   // 16-byte groups per thread
      uint4 av[AS];
#pragma unroll
      for (int i = 0; i < AS; i++) {
        const int e8 = tid + i * DS_THREADS, r = (e8 * 8) / KW, c = (e8 * 8) % KW;
        av[i] = bload16(sr, (e8 < 16 * KW / 8 && r < n) ? ((uint32_t)r * lds + d0.k0 + c) * 2u : BUF_OOB);
      }
      // the residual input at this thread's epilogue element of each unit,
      // requested with the A operand rather than after the product
      const brsrc xr = make_brsrc(PH == DP_SAO ? y.x_in : PH == DP_CAO ? y.x1 : y.x2);
#pragma unroll
      for (int j = 0; j < MAXU; j++) {
        const int r = tid >> 4, col = ds_unit(a, PH, first + j * G).n0 + (tid & 15);
        xpre[j] = bloadf(xr, (j < nu && r < n) ? (uint32_t)(r * D + col) * 4u : BUF_OOB);
      }
#pragma unroll
      for (int i = 0; i < AS; i++) {
        const int e8 = tid + i * DS_THREADS, r = (e8 * 8) / KW, c = (e8 * 8) % KW;
        if (e8 < 16 * KW / 8) *reinterpret_cast<uint4*>(rA + r * apitch + c * 2) = av[i];
      }
    }
    if constexpr (norm) {
      // two-pass mean / variance of each of the wave's 4 rows (wave-wide
      // sums), then u = LN(x)(1 + scale) + shift in bf16 into LDS. Rows
      // beyond n read zeros and give finite values that no output uses.
      if (!x_early) load_x();
      float mean[4], rstd[4];
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        float s1 = 0.f;
#pragma unroll
        for (int k = 0; k < KG; k++) s1 += (xv[rr][k].x + xv[rr][k].y) + (xv[rr][k].z + xv[rr][k].w);
        mean[rr] = s1;
      }
#pragma unroll
      for (int rr = 0; rr < 4; rr++) mean[rr] = wave_sum_rows(mean[rr]);
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        mean[rr] *= 1.f / (float)D;
        float s2 = 0.f;
#pragma unroll
        for (int k = 0; k < KG; k++) {
          if (lane + 64 * k < D / 4) {
            const float d0 = xv[rr][k].x - mean[rr], d1 = xv[rr][k].y - mean[rr];
            const float d2 = xv[rr][k].z - mean[rr], d3 = xv[rr][k].w - mean[rr];
            s2 += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
          }
        }
        rstd[rr] = s2;
      }
#pragma unroll
      for (int rr = 0; rr < 4; rr++) rstd[rr] = wave_sum_rows(rstd[rr]);
#pragma unroll
      for (int rr = 0; rr < 4; rr++) rstd[rr] = rsqrtf(rstd[rr] * (1.f / (float)D) + a.eps);
#pragma unroll
      for (int k = 0; k < KG; k++) {
        const int cg = lane + 64 * k;
        if (cg < D / 4) {
          const float4 g = make_float4(1.f + gv[k].x, 1.f + gv[k].y, 1.f + gv[k].z, 1.f + gv[k].w);
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            const float4 xx = xv[rr][k];
            const float m = mean[rr], rs = rstd[rr];
            uint2 pk;
            pk.x = pack_bf2((xx.x - m) * rs * g.x + shv[k].x, (xx.y - m) * rs * g.y + shv[k].y);
            pk.y = pack_bf2((xx.z - m) * rs * g.z + shv[k].z, (xx.w - m) * rs * g.w + shv[k].w);
            *reinterpret_cast<uint2*>(rA + (4 * wave + rr) * APITCH + cg * 8) = pk;
          }
        }
      }
    }
    bool timed_out = false;   // a DOWN partial never arrived
    auto unit = [&](int j) {
      const DsUnit d = ds_unit(a, PH, first + j * G);
      constexpr int apitch = KW * 2 + 16;
      __syncthreads();
      // ---- NB 16 x 16 tiles: wave w covers k-steps w, w + 4, ...
      f32x4 acc[NB];
      if (j == 0) ds_mma<WT, 0, NB, NSW, KST>(rA, apitch, wuse, acc);
      else if constexpr (MAXU > 1) ds_mma<WT, NB * NSW, NB, NSW, KST>(rA, apitch, wuse, acc);
#pragma unroll
      for (int b = 0; b < NB; b++)
#pragma unroll
        for (int i = 0; i < 4; i++) red[(wave * NB + b) * 256 + ((lane >> 4) * 4 + i) * 16 + (lane & 15)] = acc[b][i];
      __syncthreads();
      // ---- epilogue: thread = (row tid / 16, column tid % 16 of each block)
      const int r = tid >> 4, cc = tid & 15;
#pragma unroll
      for (int b = 0; b < NB; b++) {
        const int col = d.n0 + b * 16 + cc;
        float v = red[(0 * NB + b) * 256 + tid] + red[(1 * NB + b) * 256 + tid] + red[(2 * NB + b) * 256 + tid] +
                  red[(3 * NB + b) * 256 + tid];
        if (y.s[d.wi]) v *= ps[j][b];
        if (PH == DP_DOWN) {
          // slices 1.. publish their partial as flagged words and are done;
          // the tile's slice-0 unit adds them to its own in slice order
          const int tile = d.n0 / 16, slice = d.k0 / KW, nsl = a.mlp / KW;
          const brsrc pr = make_brsrc(a.dpart);
          if (slice > 0) {
            st_fw(pr, (uint32_t)((slice - 1) * ntile + tile) * 256u + tid, __float_as_uint(v), y.flag);
            return;
          }
          for (int q = 1; q < nsl; q++) {
            const uint32_t off = ((uint32_t)((q - 1) * ntile + tile) * 256u + tid) * 8u;
            uint2 w = bload8<CP_SC1>(pr, off);
            for (unsigned spins = 0; w.y != y.flag; spins++) {
              if (spins >= a.spin ||
                  ((spins & 31) == 31 && __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                timed_out = true;
                break;
              }
              __builtin_amdgcn_s_sleep(1);
              w = bload8<CP_SC1>(pr, off);
            }
            v += __uint_as_float(w.x);
          }
          finished_tiles++;
        }
        v += pb[j][b];
        if (PH == DP_QKV || PH == DP_CAQ || PH == DP_UP) {
          if (PH == DP_UP) v = gelu_erf(v);
          const uint32_t bits = f2bf(v);
          if constexpr (PH == DP_UP) {
            if (r < n && col < d.N)
              __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bits, make_brsrc(y.h), (uint32_t)(r * a.mlp + col) * 2u, 0, CP_SC1);
          } else {
            // even columns store the flagged word of their pair (the odd
            // column is the next lane, same row)
            uint2* out = PH == DP_QKV ? a.qkv : a.q;
            const int ldo = PH == DP_QKV ? 3 * D : D;
            const uint32_t odd = (uint32_t)__shfl_xor((int)bits, 1, WAVE);
            if (!(cc & 1) && r < n && col < d.N)
              st_fw(make_brsrc(out), (uint32_t)(r * ldo + col) / 2u, bits | (odd << 16), y.flag);
          }
        } else {
          // gated residual: x += gate * v
          if (r < n) {
            float* xd = PH == DP_SAO ? y.x1 : PH == DP_CAO ? y.x2 : y.x_out;
            st_sc1_f32(xd + (size_t)r * D + col, xpre[j] + pg[j][b] * v);
          }
        }
      }
    };
    unit(0);
    if constexpr (MAXU > 1)
      if (nu > 1) unit(1);
    if constexpr (PH == DP_DOWN)
      if (!ds_all(!timed_out, sflag)) return fail();
  }
  // ---- count this phase's finished units once every store has completed
  // (QKV and CAQ write flagged words and do not count)
  if constexpr (PH == DP_QKV || PH == DP_CAQ) {
    __syncthreads();   // region A is free for the next phase
    return true;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    sflag[1] = 0;
    unsigned add = PH == DP_DOWN ? (unsigned)finished_tiles : (unsigned)nu;
    if (add) {
      unsigned* slot = a.cnt + PH * DS_NC * DS_CSTRIDE + ((int)blockIdx.x % DS_NC) * DS_CSTRIDE;
      __hip_atomic_fetch_add(slot, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // the last layer's last DOWN tile: every unit of every phase is done
      // and no workgroup polls any more, so the counters can be cleared
      // (release: this workgroup's slot count lands before its reset count)
      if (PH == DP_DOWN && y.last) {
        const unsigned old = __hip_atomic_fetch_add(a.cnt + DS_LAST, add, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        sflag[1] = old + add == (unsigned)ds_target(a, DP_DOWN);
      }
    }
  }
  __syncthreads();
  if (sflag[1] && tid <= DP_N * DS_NC)
    __hip_atomic_store(a.cnt + tid * DS_CSTRIDE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The weight table of the launches: up to DS_TAB_CHUNK layers per fill.
constexpr int DS_TAB_CHUNK = 12;
struct DitTableArgs {
  DitLayerPtrs p[DS_TAB_CHUNK];
  int n;
  DitLayerPtrs* out;
};

template <typename WT, int D>
__global__ __launch_bounds__(DS_THREADS, 1) void k_dit_layers(DitLayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  char* rA = smem;
  float* red = reinterpret_cast<float*>(rA + ds_region_a(D));
  int* sflag = reinterpret_cast<int*>(red + 2 * 4 * 256);
  typename DsW<WT>::raw wdown[DS_WSLOTS], wqkv[DS_WSLOTS];
  bool have_down = false, have_qkv = false;

  // A failed earlier launch of this run: its flag is requested now and
  // acted on at this launch's first wait, where the workgroup poisons the
  // stream and leaves (the first QKV waits for nothing, so it needs no check).
  if (ds_tid() == 0) sflag[2] = 0;
  __syncthreads();
  const int prev_err = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int l = a.l0; l < a.l1; l++) {
    const DsLayer y = ds_layer<D>(a, l);
    int ft = 0;   // DOWN tiles of this layer this workgroup completed
    if (!ds_phase<WT, D, DP_QKV>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_SAATT>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_SAO>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_CAQ>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_CAATT>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_CAO>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_UP>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
    if (!ds_phase<WT, D, DP_DOWN>(a, y, prev_err, rA, red, sflag, ft, wdown, have_down, wqkv, have_qkv)) return;
  }
}

}  // namespace vla
