// libvla host runtime: argument validation, workspace planning, kernel
// selection and launch, and the captured whole-step graph (C ABI in vla.h).
//
// Every entry point is written once as a "schedule" over a Ctx. The schedule
// runs twice: in plan mode (no device pointers, nothing launched) it sizes
// the workspace — fixed buffers by bump allocation and the shared split-K
// scratch as the maximum over all GEMMs — and in launch mode it enqueues the
// kernels on the caller's stream. Both passes allocate in the same order, so
// the buffers land at the same offsets.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "../../include/vla.h"
#include "gemm.h"
#include "attention.h"
#include "kernels.h"
#include "tail.h"
#include "dit_stack.h"

using namespace vla;

namespace {

thread_local std::string g_err;

vla_status fail(vla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define VLA_TRY(expr)                    \
  do {                                   \
    vla_status _s = (expr);              \
    if (_s != VLA_OK) return _s;         \
  } while (0)

#define VLA_HIP(expr)                                                                         \
  do {                                                                                        \
    hipError_t _e = (expr);                                                                   \
    if (_e != hipSuccess) return fail(VLA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(_e));  \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// One recorded kernel launch of a schedule (kept by step plans so a single
// kernel can be relaunched on its own for timing).
struct LaunchRec {
  std::string label;
  const void* fn;
  dim3 grid, block;
  size_t smem;
  std::vector<std::vector<char>> args;
};

struct ArgRef {
  const void* p;
  size_t n;
};
template <typename T>
ArgRef arg(const T& v) { return ArgRef{&v, sizeof(T)}; }

// The first STATUS_BYTES of every workspace hold its status words (word 0:
// set by the DiT layer kernel when one of its bounded waits gives up); the
// buffers of a schedule start after them.
constexpr size_t STATUS_BYTES = 256;

struct Ctx {
  bool plan;               // plan mode: size buffers, launch nothing
  char* base;              // workspace base (launch mode)
  size_t cap;
  size_t off = STATUS_BYTES;
  int* status = nullptr;   // the workspace's status words (launch mode)
  hipStream_t st = nullptr;
  // shared GEMM scratch (requirements gathered in plan mode): split-K
  // partial tiles and their counters
  size_t need_part = 0, need_tiles = 0;
  float* part = nullptr;
  unsigned* cnt_tile = nullptr;
  int kernels = 0;         // launches issued (or that would be issued)
  const char* label = "";  // name of the operation being launched
  std::vector<LaunchRec>* recs = nullptr;

  // A planning pass hands out addresses in a reserved range that is never
  // dereferenced, not null: code that tests a buffer's presence then takes
  // the same branch when planning as when running, so the plan sizes the
  // scratch for the launches that really run.
  static constexpr uintptr_t PLAN_BASE = (uintptr_t)1 << 44;
  template <typename T>
  T* take(size_t n) {
    off = align_up(off, 256);
    T* p = reinterpret_cast<T*>(plan ? (char*)PLAN_BASE + off : base + off);
    off += n * sizeof(T);
    return p;
  }
  // Lay out the GEMM scratch (sized by a plan pass `q`) after the fixed buffers.
  void take_scratch(const Ctx& q) {
    need_part = q.need_part; need_tiles = q.need_tiles;
    part = take<float>(std::max<size_t>(need_part, 1));
    cnt_tile = take<unsigned>(need_tiles + 1);
  }
};

vla_status launch(Ctx& c, const void* fn, dim3 grid, dim3 block, size_t smem, std::initializer_list<ArgRef> args) {
  c.kernels++;
  if (c.plan) return VLA_OK;
  void* ptrs[16];
  int i = 0;
  for (const ArgRef& a : args) ptrs[i++] = const_cast<void*>(a.p);
  VLA_HIP(hipLaunchKernel(fn, grid, block, ptrs, smem, c.st));
  if (c.recs) {
    LaunchRec r;
    r.label = c.label;
    r.fn = fn; r.grid = grid; r.block = block; r.smem = smem;
    for (const ArgRef& a : args) r.args.emplace_back((const char*)a.p, (const char*)a.p + a.n);
    c.recs->push_back(std::move(r));
  }
  return VLA_OK;
}

vla_status zero_counters(Ctx& c) {
  if (c.plan) return VLA_OK;
  unsigned* p = c.cnt_tile;
  unsigned v = 0;
  int n = (int)(c.need_tiles + 1);
  c.label = "fill";
  return launch(c, k_fill_ref(), dim3((n + 255) / 256), dim3(256), 0, {arg(p), arg(v), arg(n)});
}

// Kernels that need more than 64 KiB of dynamic LDS are opted in once.
vla_status allow_smem(const KernelRef& k) {
  static std::mutex mu;
  static std::set<const void*> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count(k.fn)) return VLA_OK;
  VLA_HIP(hipFuncSetAttribute(k.fn, hipFuncAttributeMaxDynamicSharedMemorySize, k.smem));
  done.insert(k.fn);
  return VLA_OK;
}

// ------------------------------------------------------------------ GEMM launcher
struct GemmOp {
  int wdtype;   // vla_dtype of W
  int am, em;
  int ac = 0;   // compensated (hi + lo) bf16 activations
  int pk = 0;   // W in the packed layout of vla_pack_weights
};

// Row tile (16-row blocks) by M: one tile up to 112 rows; 64-row tiles up to
// 256 rows (twice the workgroups of 128-row tiles, a quarter of the LDS
// traffic per MFMA of narrower ones); 128-row tiles beyond, except for
// compensated narrow tiles, whose two A planes only fit in LDS at 64 rows.
// Narrow tiles: 16 columns with 4 waves splitting K when M <= 16, else 64
// columns with 4 waves side by side. Wide tiles (RoPE pairs, gate/up pairs):
// 128 columns with 8 waves side by side; compensated, 4 x 2 waves (column
// blocks x k-steps) with two 16-column blocks per wave.
// Measured at the workloads' shapes (cold last-level cache, per launch):
// 64-column tiles for 16-row GEMMs with very many columns (the adaLN
// modulations: 166 vs 271 us with 16-column tiles), 128-column tiles for
// taller ones (the cross-attention K/V: 82 vs 108 us), and two k-waves of
// 32 columns with a two-way split for small residual GEMMs (the ViT output
// projection: 12.0 vs 14.2 us).
// Backbone shapes of 65-112 rows (measured at 104): the RoPE tile with two
// k-steps per wave and four activation chunks in flight (QKV 21.1 -> 20.1
// us), the O projection on 32-column tiles of two k-waves (18.5 -> 16.0 us),
// the compensated down projection with one k-step per wave and four
// activation chunks in flight (37.2 -> 32.2 us). Packed weights (pk) take the
// same tiles (and give the same bits).
void pick_tile(int M, int N, int K, int am, int em, int ac, int wdtype, int& mb, int& wn, int& wk, int& nbw,
               int& u, int& aq, int& split_hint, int& target_wgs) {
  if (am == A_BF16R) am = A_BF16;   // the same staging; the row scale is an epilogue step
  bool wide = em == E_ROPE || em == E_SWIGLU;
  mb = M <= 16 ? 1 : M <= 64 ? 4 : M <= 112 ? 7 : (M <= 256 || (ac && !wide)) ? 4 : 8;
  u = ac ? 2 : 4;
  nbw = 1;
  split_hint = 0;
  target_wgs = 0;
  const bool plain_store = em == E_STORE && am == A_BF16 && wdtype != VLA_F32;
  // 17..64 rows from bf16 activations (the action expert at a 50-row chunk):
  // few column tiles, so the K loop is shared out to more workgroups
  // (O projection 15.3 -> 11.0 us, MLP down 21.6 -> 14.1 us at 1280 wide)
  const bool mid_rows = M > 16 && M <= 64 && am == A_BF16 && wdtype != VLA_F32 && !ac;
  if (wide && ac) { wn = 4; wk = 2; nbw = 2; u = 1; }   // two column blocks per wave: half the A reads
  else if (wide) { wn = 8; wk = 1; }
  else if (mb == 1) {
    if (plain_store && N >= 16 * 1024) { wn = 4; wk = 1; }
    else { wn = 1; wk = 4; }
  }
  else if (ac) { wn = 4; wk = 2; }     // compensated residual GEMMs: two k-waves per column block
  else if (plain_store && N >= 64 * 1024) { wn = 8; wk = 1; }
  else if (em == E_RESID && am == A_BF16 && wdtype == VLA_BF16 && mb == 4 && M > 64 && K <= 1024 &&
           ((N + 63) / 64) * ((M + 63) / 64) < 128) {
    wn = 2; wk = 2; u = 2; split_hint = 2;
  }
  else if (mid_rows && em == E_RESID) { wn = 2; wk = 2; u = 2; target_wgs = 160; }
  else if (mid_rows && em == E_STORE) { wn = 4; wk = 1; target_wgs = 80; }
  else { wn = 4; wk = 1; }
  aq = 2;
  if (mb == 7 && am == A_BF16 && wdtype != VLA_F32) {
    if (em == E_ROPE && !ac) { u = 2; aq = 4; }
    else if (em == E_RESID && !ac) { wn = 2; wk = 2; nbw = 1; u = 2; split_hint = 0; target_wgs = 0; }
    else if (em == E_RESID && ac) { u = 1; aq = 4; }
    // compensated gate/up: 256 weight rows per tile over three k-splits, so
    // 228 workgroups each stage a third of the A rows (47.0 -> 44.7 us at
    // 104 rows, packed weights)
    else if (em == E_SWIGLU && ac && wdtype == VLA_BF16) { wn = 8; wk = 1; nbw = 2; u = 2; }
  }
  // 193..256 rows of bf16 weights: 128-row tiles for the MLP and the long-K
  // residual GEMMs (at 256 rows, packed weights: gate/up 105 -> 90 us, down
  // 76 -> 61 us, O projection 26.4 -> 23.9 us)
  if (M > 192 && M <= 256 && am == A_BF16 && wdtype == VLA_BF16) {
    if (ac && em == E_SWIGLU) { mb = 8; wn = 8; wk = 1; nbw = 2; u = 2; }
    else if (ac && em == E_RESID) { mb = 8; wn = 2; wk = 2; nbw = 2; u = 1; split_hint = 3; target_wgs = 0; }
    else if (!ac && em == E_RESID && N >= 2048 && K > 1024) { mb = 8; wn = 4; wk = 1; nbw = 1; u = 4; split_hint = 0; target_wgs = 0; }
    // narrow long-K residual (the vision MLP's down projection, 1024 wide
    // over K 4096): 64 x 64 tiles of two k-waves over four k-splits
    // (15.9 -> 14.4 us)
    else if (!ac && em == E_RESID && N < 2048 && K > 1024) { mb = 4; wn = 4; wk = 2; nbw = 1; u = 2; split_hint = 4; target_wgs = 0; }
  }
  // fp8 weights over more than 256 rows: two column blocks per wave, so each
  // A fragment read from LDS feeds two MFMAs (gate/up at 560 rows 121 -> 103
  // us, QKV 43 -> 41 us; the cross K/V GEMM at 560 rows, 256 columns per
  // tile, 394 -> 268 us)
  if (mb == 8 && am == A_BF16 && wdtype == VLA_FP8_E4M3 && !ac && (em == E_SWIGLU || em == E_ROPE)) {
    wn = 4; wk = 1; nbw = 2; u = 2; split_hint = 1;
  }
  if (mb == 8 && am == A_BF16 && wdtype == VLA_FP8_E4M3 && !ac && em == E_STORE && N >= 16 * 1024) {
    wn = 8; wk = 1; nbw = 2; u = 2; split_hint = 1;
  }
  // 65..112 rows, plain stores: the wide cross K/V GEMM takes two column
  // blocks per wave (82 -> 67 us at 104 rows), narrow ones more workgroups
  // (the 2560 -> 1280 projector 17.6 -> 13.8 us with five k-splits)
  if (mb == 7 && em == E_STORE && am == A_BF16 && !ac && (wdtype == VLA_BF16 || wdtype == VLA_FP8_E4M3)) {
    if (N >= 64 * 1024) { wn = 4; wk = 1; nbw = 2; u = 2; }
    else target_wgs = 100;
  }
  // 17..64 rows, plain stores over K of 4096 or more (the merger's two
  // Linears at 64 rows): four k-splits (16.3 -> 12.4 us, 16.7 -> 13.5 us)
  if (mid_rows && em == E_STORE && K >= 4096) split_hint = 4;
}

// Launch one GEMM. For a residual epilogue, *produced receives the column
// tiling of the row moments the kernel leaves in a.rs_out.
vla_status gemm(Ctx& c, GemmArgs a, GemmOp op, RowStats* produced = nullptr) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return fail(VLA_ERR_SHAPE, "gemm: empty shape %d x %d x %d", a.M, a.N, a.K);
  int mb, wn, wk, nbw, u, aq, split_hint, target_wgs;
  pick_tile(a.M, a.N, a.K, op.am, op.em, op.ac, op.wdtype, mb, wn, wk, nbw, u, aq, split_hint, target_wgs);
  const int BM = 16 * mb, BN = 16 * nbw * wn, BK = 32 * wk * u;
  const int bn_out = op.em == E_SWIGLU ? BN / 2 : BN;
  a.n_tiles_n = (a.N + bn_out - 1) / bn_out;
  a.n_tiles_m = (a.M + BM - 1) / BM;
  const int tiles = a.n_tiles_n * a.n_tiles_m;
  // Split K when one workgroup would stream more than ~192 KiB of weights,
  // or when a large GEMM has too few tiles to cover the CUs; never beyond
  // one round of resident workgroups (512-thread tiles hold one workgroup
  // per CU, 256-thread tiles two), never for small latency-bound GEMMs.
  const int threads = 64 * wn * wk;
  const int slots = 256 * (threads >= 512 ? 1 : 2);
  const double wbytes = op.wdtype == VLA_F32 ? 4.0 : op.wdtype == VLA_BF16 ? 2.0 : 1.0;
  const double per_wg = (double)BN * a.K * wbytes;
  const double total = per_wg * tiles / (double)a.n_tiles_m;
  int split = std::max(1, (int)std::ceil(per_wg / (192.0 * 1024.0)));
  if (total >= 16.0 * 1024 * 1024 && tiles * split < 200) split = (200 + tiles - 1) / tiles;
  split = std::min(split, std::max(1, slots / tiles));
  // two-k-wave residual tiles: up to 240 workgroups (the down projection at
  // 104 rows: 39.8 us with 6 splits vs 48.4 us with 4)
  if (threads >= 512 && op.em == E_RESID) split = std::min(split, std::max(1, 240 / tiles));
  if (split_hint) split = split_hint;
  if (target_wgs && tiles < target_wgs) split = std::max(split, target_wgs / tiles);
  split = std::min(split, std::max(1, (a.K + BK - 1) / BK));
  split = std::min(split, SPLIT_MAX);
  int ksplit = (int)align_up((size_t)((a.K + split - 1) / split), (size_t)BK);
  split = (a.K + ksplit - 1) / ksplit;
  a.split = split;
  a.ksplit = ksplit;
  // weight-type / alignment requirements of the 8-element fragment loads
  if (a.ldw % 8 != 0 || a.ldw < a.K) return fail(VLA_ERR_SHAPE, "gemm: weight pitch %d must be >= K=%d and a multiple of 8", a.ldw, a.K);
  if ((op.wdtype == VLA_FP8_E4M3 || op.wdtype == VLA_INT8) && (a.K % 16 != 0 || a.ldw % 16 != 0))
    return fail(VLA_ERR_SHAPE, "gemm: 8-bit weights need K %d and pitch %d to be multiples of 16", a.K, a.ldw);
  const int ag = a_bf16(op.am) ? 8 : a_codes(op.am) ? 16 : 4;   // activation elements per 16-byte load
  if (a_codes(op.am) && !a.a_scale && !c.plan) return fail(VLA_ERR_INVALID_ARG, "gemm: 8-bit activations without row scales");
  if (op.am == A_BF16R && ((!a.rsq && !c.plan) || a.rsq_t < 1 || a.rsq_t > a.rsq_ld || a.rsq_ld % 4))
    return fail(VLA_ERR_INVALID_ARG, "gemm: deferred RMSNorm rows without their per-tile sums of squares");
  if ((a_bf16(op.am) || op.am == A_F32 || op.am == A_NORM || a_codes(op.am)) && (a.lda % ag != 0 || a.K % ag != 0))
    return fail(VLA_ERR_SHAPE, "gemm: activation pitch %d and K %d must be multiples of %d", a.lda, a.K, ag);
  // the epilogues store 4 consecutive columns at once and read the
  // per-column vectors as float4
  if (a.N % 4 != 0 || (op.em == E_RESID ? a.ldx % 4 != 0 : a.ldc % 4 != 0))
    return fail(VLA_ERR_SHAPE, "gemm: N %d and the output pitch must be multiples of 4", a.N);
  for (const void* v : {(const void*)a.bias, (const void*)a.wscale, (const void*)a.gate, (const void*)a.c, (const void*)a.x,
                        (const void*)a.rope_cos, (const void*)a.rope_sin, (const void*)a.addrow, (const void*)a.xg,
                        (const void*)a.xg_lo, (const void*)a.xg_gain})
    if (reinterpret_cast<uintptr_t>(v) & 15) return fail(VLA_ERR_INVALID_ARG, "gemm: output or epilogue vector not 16-byte aligned");
  // buffer-load offsets are 32-bit: operands up to 2 GiB
  const double wrows = op.em == E_SWIGLU ? (double)a.n_half + a.N : (double)a.N;
  if (wrows * a.ldw * wbytes >= (double)BUF_LIMIT) return fail(VLA_ERR_SHAPE, "gemm: weight matrix beyond 2 GiB");
  if (op.pk && (std::ceil(wrows / 16.0) * std::ceil(a.K / 32.0) * 512.0 * wbytes >= (double)BUF_LIMIT ||
                (op.em == E_SWIGLU && a.n_half % 16)))
    return fail(VLA_ERR_SHAPE, "gemm: packed weight matrix beyond 2 GiB, or gate/up halves not on 16-row blocks");
  if ((double)a.M * a.lda * 4.0 >= (double)BUF_LIMIT)
    return fail(VLA_ERR_SHAPE, "gemm: activation matrix beyond 2 GiB");
  if ((op.em == E_RESID ? (double)a.M * a.ldx * 4.0 : (double)a.M * a.ldc * (a.c_f32 ? 4.0 : 2.0)) >= (double)BUF_LIMIT)
    return fail(VLA_ERR_SHAPE, "gemm: output matrix beyond 2 GiB");
  if (op.ac && (op.wdtype != VLA_BF16 || (op.am != A_NORM && op.am != A_F32 && !a_bf16(op.am))))
    return fail(VLA_ERR_UNSUPPORTED, "gemm: compensated activations need bf16 weights");
  if ((a.xg || a.rsq_out) && op.em != E_RESID)
    return fail(VLA_ERR_INVALID_ARG, "gemm: gained bf16 rows and row scales come from a residual epilogue");
  if (op.ac && a_bf16(op.am) && !a.a_lo && !c.plan) return fail(VLA_ERR_INVALID_ARG, "gemm: compensated bf16 source without its remainder plane");
  if (op.em == E_RESID) {
    if (!a.rs_out && !c.plan) return fail(VLA_ERR_INVALID_ARG, "gemm: residual epilogue without a row-moment output");
    if (a.n_tiles_n > (a.N + 15) / 16) return fail(VLA_ERR_SHAPE, "gemm: residual tiling finer than 16 columns");
    if (produced) { produced->T = a.n_tiles_n; produced->tw = BN; produced->N = a.N; produced->M = a.M; }
  }
  size_t part_f = split > 1 ? (size_t)split * tiles * BM * BN : 0;
  c.need_part = std::max(c.need_part, part_f);
  if (a.rsq_out && (a.n_tiles_n > a.rsq_ld || a.rsq_ld % 4))
    return fail(VLA_ERR_SHAPE, "gemm: %d column tiles of sums of squares in rows of %d", a.n_tiles_n, a.rsq_ld);
  c.need_tiles = std::max(c.need_tiles, (size_t)tiles);
  KernelRef k{};
  bool found = false;
  const GemmPick g{op.am, op.em, mb, wn, wk, nbw, u, op.ac, aq, op.pk};
  if (op.wdtype == VLA_BF16) found = gemm_lookup_bf16(g, &k);
  else if (op.wdtype == VLA_FP8_E4M3) found = gemm_lookup_fp8(g, &k);
  else if (op.wdtype == VLA_INT8) found = gemm_lookup_int8(g, &k);
  else if (op.wdtype == VLA_F32 && !op.pk) found = gemm_lookup_f32(g, &k);
  if (!found)
    return fail(VLA_ERR_UNSUPPORTED, "gemm: no kernel for wdtype %d am %d em %d tile %d/%d/%d/%d u %d ac %d aq %d packed %d",
                op.wdtype, op.am, op.em, mb, wn, wk, nbw, u, op.ac, aq, op.pk);
  if (c.plan) { c.kernels++; return VLA_OK; }
  a.part = c.part;
  a.cnt_tile = c.cnt_tile;
  if (k.smem > 64 * 1024) VLA_TRY(allow_smem(k));
  return launch(c, k.fn, dim3(tiles * split), dim3(k.threads), (size_t)k.smem, {arg(a)});
}

// Whether a GEMM of this shape and kind has an instantiated tile (the
// deferred-norm forms exist for the backbone's tiles only).
bool gemm_has(int M, int N, int K, GemmOp op) {
  int mb, wn, wk, nbw, u, aq, split_hint, target_wgs;
  pick_tile(M, N, K, op.am, op.em, op.ac, op.wdtype, mb, wn, wk, nbw, u, aq, split_hint, target_wgs);
  KernelRef k{};
  const GemmPick g{op.am, op.em, mb, wn, wk, nbw, u, op.ac, aq, op.pk};
  if (op.wdtype == VLA_BF16) return gemm_lookup_bf16(g, &k);
  if (op.wdtype == VLA_FP8_E4M3) return gemm_lookup_fp8(g, &k);
  if (op.wdtype == VLA_INT8) return gemm_lookup_int8(g, &k);
  return false;
}

GemmArgs gargs() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.split = 1;
  return a;
}

// ------------------------------------------------------------------ attention
vla_status attention(Ctx& c, AttnArgs a, bool f32) {
  if (a.Hkv <= 0 || a.Hq % a.Hkv != 0) return fail(VLA_ERR_SHAPE, "attention: %d query heads not a multiple of %d kv heads", a.Hq, a.Hkv);
  int dp = a.D <= 64 ? 64 : a.D <= 96 ? 96 : a.D <= 128 ? 128 : 0;
  if (dp == 0 || a.D % 8 != 0) return fail(VLA_ERR_SHAPE, "attention: head_dim %d unsupported", a.D);
  // 8-element loads of q, k, v rows and 4-element stores of o rows
  if (a.ldq % 8 || a.ldk % 8 || a.ldv % 8 || a.ldo % 4)
    return fail(VLA_ERR_SHAPE, "attention: row pitches %d/%d/%d/%d not multiples of 8/8/8/4", a.ldq, a.ldk, a.ldv, a.ldo);
  int group = a.Hq / a.Hkv;
  int hpw = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  int rb = 4 / hpw;
  int nrb = (a.Sq + 16 * rb - 1) / (16 * rb);
  int tiles = a.Hkv * (group / hpw) * nrb;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)a.D));
  // Few tiles with long key loops (cross-attention of a small chunk to a
  // long context): share each tile's keys out to several workgroups of at
  // least two 32-key blocks, up to about 192 workgroups, and merge their
  // partials in a second launch. Short loops gain nothing from a split.
  const int kblocks = (a.Sk + 31) / 32;
  int nsplit = 1;
  if (kblocks >= 12 && tiles <= 64) nsplit = std::min({kblocks / 2, 192 / tiles, ATTN_SPLIT_MAX});
  // Otherwise, with fewer tiles than about three quarters of the compute
  // units and at least two key blocks (the batch-1 prefills: 56 tiles for
  // 104 rows of 32/8 heads, 64 for the encoder's 256 rows of 16 heads), the
  // key-split form: 16 rows of one head per workgroup, the four waves on
  // different key blocks, merged in LDS.
  int ks = 0;
  if (nsplit == 1 && !f32 && (dp == 64 || dp == 128) && kblocks >= 2 && tiles < 192) {
    ks = 1;
    hpw = 1;
    rb = 1;
    nrb = (a.Sq + 15) / 16;
    tiles = a.Hq * nrb;
  }
  KernelRef k{}, km{};
  if (!attn_lookup(f32 ? 1 : 0, dp, hpw, ks, &k, &km)) return fail(VLA_ERR_UNSUPPORTED, "attention: no kernel for D %d", a.D);
  a.kchunk = ((kblocks + nsplit - 1) / nsplit) * 32;
  a.nsplit = nsplit = (a.Sk + a.kchunk - 1) / a.kchunk;
  if (nsplit > 1) {
    const size_t pw = 16 * (size_t)(dp + 2);
    c.need_part = std::max(c.need_part, (size_t)tiles * nsplit * 4 * pw);
    a.part = c.part;
  }
  if (!c.plan && k.smem > 64 * 1024) VLA_TRY(allow_smem(k));
  VLA_TRY(launch(c, k.fn, dim3(tiles * nsplit), dim3(256), (size_t)k.smem, {arg(a)}));
  if (nsplit == 1) return VLA_OK;
  const int per_tile = (4 * 16 * (dp / 4) + 255) / 256;
  return launch(c, km.fn, dim3(tiles * per_tile), dim3(256), 0, {arg(a)});
}

vla_status stage_rows(Ctx& c, float* x, int ldx, int M, int N, const void* src, int src_f32, int ld_src, int r0, int r1,
                      float2* stats) {
  if (N % 4 || ldx % 4 || (src && ld_src % 4))
    return fail(VLA_ERR_SHAPE, "stage rows: width %d and pitches %d, %d must be multiples of 4", N, ldx, ld_src);
  return launch(c, k_stage_rows_ref(), dim3((M + 3) / 4), dim3(256), 0,
                {arg(x), arg(ldx), arg(M), arg(N), arg(src), arg(src_f32), arg(ld_src), arg(r0), arg(r1), arg(stats)});
}

vla_status rmsnorm_out(Ctx& c, const float* x, int ldx, int M, int N, RowStats rs, const float* gain, float eps,
                       void* out, int ldo, int out_f32) {
  if (N % 4 || ldx % 4 || ldo % 4)
    return fail(VLA_ERR_SHAPE, "rmsnorm out: width %d and pitches %d, %d must be multiples of 4", N, ldx, ldo);
  return launch(c, k_rmsnorm_out_ref(), dim3((M + 3) / 4), dim3(256), 0,
                {arg(x), arg(ldx), arg(M), arg(N), arg(rs), arg(gain), arg(eps), arg(out), arg(ldo), arg(out_f32)});
}

// A residual stream: fp32 rows, their per-tile moment buffer (sized for the
// finest column tiling, 16 columns) and the tiling its last writer used.
struct Stream {
  float* x = nullptr;
  float2* part = nullptr;
  RowStats rs{};
};

Stream take_stream(Ctx& c, int M, int N) {
  Stream st;
  st.x = c.take<float>((size_t)M * N);
  st.part = c.take<float2>((size_t)((N + 15) / 16) * M);   // finest tiling: 16 columns
  st.rs.part = st.part;
  st.rs.M = M;
  st.rs.N = N;
  st.rs.T = 1;
  st.rs.tw = N;
  return st;
}

// Copy rows [r0, r1) from src into the stream (when src is given) and write
// the moments of every row as one tile.
vla_status stage_stream(Ctx& c, Stream& st, int M, int N, const void* src, int src_f32, int r0, int r1) {
  st.rs.T = 1;
  st.rs.tw = N;
  return stage_rows(c, st.x, N, M, N, src, src_f32, N, r0, r1, st.part);
}

// Normalise M rows of x once, into bf16 (and the remainder plane when out_lo).
vla_status norm_rows(Ctx& c, const float* x, int ldx, int M, int K, RowStats rs, int rms, float eps, const float* g,
                     int g_plus_one, const float* bsh, uint16_t* out, uint16_t* out_lo, int ldo, int merge = 0,
                     int vgrid = 0, int n_patches = 0) {
  if (K % 4 != 0 || ldx % 4 != 0 || ldo % 4 != 0) return fail(VLA_ERR_SHAPE, "norm: row length %d must be a multiple of 4", K);
  if (merge && (vgrid % merge || n_patches != vgrid * vgrid || M % n_patches || ldo != merge * merge * K))
    return fail(VLA_ERR_SHAPE, "norm: merge %d of a %d-patch grid does not tile", merge, vgrid);
  NormArgs a{};
  a.x = x; a.ldx = ldx; a.M = M; a.K = K; a.rs = rs; a.rms = rms; a.eps = eps;
  a.g = g; a.g_plus_one = g_plus_one; a.bsh = bsh; a.out = out; a.out_lo = out_lo; a.ldo = ldo;
  a.merge = merge; a.vgrid = vgrid; a.n_patches = n_patches;
  return launch(c, k_norm_rows_ref(), dim3(M), dim3(256), 0, {arg(a)});
}

// W8A8: the normalised rows as E4M3FN codes with one scale per row (K <= 4096)
vla_status norm_rows8(Ctx& c, const float* x, int ldx, int M, int K, RowStats rs, int rms, float eps, const float* g,
                      uint8_t* out8, float* oscale, int ldo, int int8) {
  if (K % 4 != 0 || K > 4096 || ldx % 4 != 0 || ldo % 4 != 0) return fail(VLA_ERR_SHAPE, "norm (fp8 out): row length %d", K);
  NormArgs a{};
  a.x = x; a.ldx = ldx; a.M = M; a.K = K; a.rs = rs; a.rms = rms; a.eps = eps;
  a.g = g; a.out8 = out8; a.oscale = oscale; a.ldo = ldo; a.out8_int8 = int8;
  return launch(c, k_norm_rows_ref(), dim3(M), dim3(256), 0, {arg(a)});
}

// W8A8: E4M3FN or int8 codes of bf16 or fp32 rows with one scale per row (K <= 16384)
vla_status quant_rows(Ctx& c, const void* x, int x_f32, int ldx, int M, int K, uint8_t* out, int ldo, float* scale,
                      int int8) {
  if (K % 8 != 0 || K > 16384 || ldx % 8 != 0 || ldo % 8 != 0) return fail(VLA_ERR_SHAPE, "quant rows: row length %d", K);
  return launch(c, k_quant_rows_ref(), dim3(M), dim3(256), 0,
                {arg(x), arg(x_f32), arg(ldx), arg(K), arg(out), arg(ldo), arg(scale), arg(int8)});
}

vla_status convert_rows(Ctx& c, const float* x, int ldx, int M, int N, void* out, int ldo, int out_f32) {
  return launch(c, k_convert_rows_ref(), dim3((M + 3) / 4), dim3(256), 0,
                {arg(x), arg(ldx), arg(M), arg(N), arg(out), arg(ldo), arg(out_f32)});
}

bool dtype_ok(int t) { return t == VLA_F32 || t == VLA_BF16 || t == VLA_FP8_E4M3 || t == VLA_INT8; }
// 8-bit weights (E4M3FN or int8 codes) carry one float32 scale per output row
bool scaled8(int t) { return t == VLA_FP8_E4M3 || t == VLA_INT8; }

// ------------------------------------------------------------------ backbone
vla_status check_block_cfg(const vla_block_cfg* cfg) {
  if (!cfg) return fail(VLA_ERR_INVALID_ARG, "null block cfg");
  if (cfg->flags & ~(VLA_BLOCK_QK_NORM | VLA_BLOCK_A8 | VLA_BLOCK_PACKED))
    return fail(VLA_ERR_UNSUPPORTED, "block cfg flags 0x%x: unknown bits", cfg->flags);
  if (cfg->flags & VLA_BLOCK_PACKED) {
    if (cfg->wdtype == VLA_F32)
      return fail(VLA_ERR_UNSUPPORTED, "block cfg: packed weights need bf16, fp8 or int8 weights and bf16 activations");
    if (cfg->flags & VLA_BLOCK_A8) return fail(VLA_ERR_UNSUPPORTED, "block cfg: packed weights with 8-bit activations");
    // the up rows of the gate/up matrix start a new 16-row block
    if (cfg->intermediate % 16)
      return fail(VLA_ERR_UNSUPPORTED, "block cfg: packed weights need intermediate %d to be a multiple of 16", cfg->intermediate);
  }
  if (cfg->flags & VLA_BLOCK_A8) {
    if (!scaled8(cfg->wdtype) || cfg->adtype != VLA_BF16)
      return fail(VLA_ERR_UNSUPPORTED, "block cfg: 8-bit activations need fp8 or int8 weights and bf16 activations");
    const int qd = cfg->n_q_heads * cfg->head_dim;
    if (cfg->hidden > 4096 || cfg->hidden % 16 || qd > 16384 || qd % 16 || cfg->intermediate > 16384 || cfg->intermediate % 16)
      return fail(VLA_ERR_UNSUPPORTED, "block cfg: 8-bit activations need hidden <= 4096 and Linear inputs <= 16384 wide, multiples of 16");
  }
  if (!dtype_ok(cfg->wdtype) || (cfg->adtype != VLA_F32 && cfg->adtype != VLA_BF16))
    return fail(VLA_ERR_INVALID_ARG, "block cfg: bad dtype (w %d, act %d)", cfg->wdtype, cfg->adtype);
  if ((cfg->wdtype == VLA_F32) != (cfg->adtype == VLA_F32))
    return fail(VLA_ERR_UNSUPPORTED, "block cfg: fp32 weights need fp32 activations and vice versa");
  if (cfg->hidden <= 0 || cfg->hidden % 8 || cfg->intermediate <= 0 || cfg->intermediate % 8)
    return fail(VLA_ERR_SHAPE, "block cfg: hidden %d / intermediate %d must be positive multiples of 8", cfg->hidden, cfg->intermediate);
  if (scaled8(cfg->wdtype) && (cfg->hidden % 16 || cfg->intermediate % 16))
    return fail(VLA_ERR_SHAPE, "block cfg: fp8 weights need hidden %d / intermediate %d to be multiples of 16", cfg->hidden, cfg->intermediate);
  if (cfg->n_kv_heads <= 0 || cfg->n_q_heads <= 0 || cfg->n_q_heads % cfg->n_kv_heads)
    return fail(VLA_ERR_SHAPE, "block cfg: n_q_heads %d not a multiple of n_kv_heads %d", cfg->n_q_heads, cfg->n_kv_heads);
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return fail(VLA_ERR_SHAPE, "block cfg: head_dim %d not in {64, 128}", cfg->head_dim);
  if (!(cfg->eps >= 0.f) || !(cfg->rope_base > 1.f)) return fail(VLA_ERR_INVALID_ARG, "block cfg: bad eps / rope_base");
  // QK-norm runs in the RoPE epilogue of the 128-column QKV tiles: a tile
  // holds whole heads and lies within the query or the key / value columns
  if ((cfg->flags & VLA_BLOCK_QK_NORM) && (cfg->n_q_heads * cfg->head_dim) % 128)
    return fail(VLA_ERR_UNSUPPORTED, "block cfg: QK-norm needs n_q_heads * head_dim %d to be a multiple of 128",
                cfg->n_q_heads * cfg->head_dim);
  return VLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

vla_status check_block_weights(const vla_block_cfg* cfg, const vla_block_weights* w) {
  if (!w) return fail(VLA_ERR_INVALID_ARG, "null block weights");
  if (!w->attn_norm || !w->w_qkv || !w->w_o || !w->mlp_norm || !w->w_gate_up || !w->w_down)
    return fail(VLA_ERR_INVALID_ARG, "block weights: null tensor pointer");
  for (const void* v : {(const void*)w->attn_norm, w->w_qkv, (const void*)w->s_qkv, w->w_o, (const void*)w->s_o,
                        (const void*)w->mlp_norm, w->w_gate_up, (const void*)w->s_gate_up, w->w_down,
                        (const void*)w->s_down, (const void*)w->q_norm, (const void*)w->k_norm})
    if (!aligned16(v)) return fail(VLA_ERR_INVALID_ARG, "block weights: tensor not 16-byte aligned");
  if (scaled8(cfg->wdtype) && (!w->s_qkv || !w->s_o || !w->s_gate_up || !w->s_down))
    return fail(VLA_ERR_INVALID_ARG, "block weights: fp8 weights need scales");
  if ((cfg->flags & VLA_BLOCK_QK_NORM) && (!w->q_norm || !w->k_norm))
    return fail(VLA_ERR_INVALID_ARG, "block weights: QK-norm needs q_norm and k_norm");
  return VLA_OK;
}

struct BackboneBufs {
  Stream xs;       // [S, H] residual stream
  void* qkv;       // [S, Nqkv]
  void* ao;        // [S, q_dim]
  void* act;       // [S, I]
  uint16_t* xn;    // [S, H] normalised rows (bf16 activations)
  uint16_t* xn_lo; // [S, H] their remainder plane (compensated MLP)
  float* rsq;      // [S][rsq_ld] per-column-tile sums of squares of the stream's rows (deferred RMSNorm)
  int rsq_ld;
  uint16_t* act_lo;// [S, I] remainder plane of the SwiGLU output (compensated MLP)
  uint8_t* q8;     // [S, max(H, q_dim, I)] E4M3FN codes of the next Linear's input (fp8 activations)
  float* q8s;      // [S] their row scales
  float* rope_cos; // [S, head_dim / 2] RoPE tables of the pass (positions 0 .. S-1)
  float* rope_sin;
};

// bf16 backbones carry the MLP's activations (the normalised input of gate/up
// and the SwiGLU output feeding down) as compensated hi + lo bf16 pairs: the
// two MLP operands dominate the rounding error of a deep stack.
bool mlp_compensated(const vla_block_cfg& cfg) { return cfg.wdtype == VLA_BF16; }

BackboneBufs take_backbone_bufs(Ctx& c, const vla_block_cfg& cfg, int S) {
  size_t es = cfg.adtype == VLA_F32 ? 4 : 2;
  const bool comp = mlp_compensated(cfg);
  int nqkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim;
  BackboneBufs b;
  b.xs = take_stream(c, S, cfg.hidden);
  // W8A8 keeps q, k, v, the attention (fp32 kernel) and the SwiGLU product
  // in fp32 until they are quantised: rounding to bf16 before an fp8 code is
  // chosen moves about one value in thirty to a neighbouring code
  const size_t eq = (cfg.flags & VLA_BLOCK_A8) ? 4 : es;
  b.qkv = c.take<char>((size_t)S * nqkv * eq);
  b.ao = c.take<char>((size_t)S * cfg.n_q_heads * cfg.head_dim * eq);
  b.act = c.take<char>((size_t)S * cfg.intermediate * eq);
  b.xn = b.xn_lo = b.act_lo = nullptr;
  b.q8 = nullptr; b.q8s = nullptr;
  b.rope_cos = c.take<float>((size_t)S * (cfg.head_dim / 2));
  b.rope_sin = c.take<float>((size_t)S * (cfg.head_dim / 2));
  b.rsq = nullptr;
  b.rsq_ld = (((cfg.hidden + 15) / 16) + 3) / 4 * 4;   // the finest residual tiling: 16 columns
  if (cfg.adtype != VLA_F32) {
    b.xn = c.take<uint16_t>((size_t)S * cfg.hidden);
    b.rsq = c.take<float>((size_t)S * b.rsq_ld);
  }
  if (cfg.flags & VLA_BLOCK_A8) {
    const int w = std::max({cfg.hidden, cfg.n_q_heads * cfg.head_dim, cfg.intermediate});
    b.q8 = c.take<uint8_t>((size_t)S * w);
    b.q8s = c.take<float>((size_t)S);
  }
  if (comp) {
    b.xn_lo = c.take<uint16_t>((size_t)S * cfg.hidden);
    b.act_lo = c.take<uint16_t>((size_t)S * cfg.intermediate);
  }
  return b;
}

vla_status sched_layers(Ctx& c, const vla_block_cfg& cfg, const vla_block_weights* layers, int n_layers, BackboneBufs& b,
                        int S) {
  const int H = cfg.hidden, D = cfg.head_dim, qd = cfg.n_q_heads * D, kd = cfg.n_kv_heads * D;
  const int nqkv = qd + 2 * kd, I = cfg.intermediate;
  const bool f32 = cfg.adtype == VLA_F32;
  const int wt = cfg.wdtype;
  const size_t es = f32 ? 4 : 2;
  const int comp = mlp_compensated(cfg) ? 1 : 0;
  const int pk = (cfg.flags & VLA_BLOCK_PACKED) ? 1 : 0;   // W in the packed layout of vla_pack_weights
  // W8A8: each Linear reads its input as per-row E4M3FN codes (the norms
  // write codes, the attention and SwiGLU outputs are quantised by a row pass)
  const bool a8 = (cfg.flags & VLA_BLOCK_A8) != 0;
  const int i8 = wt == VLA_INT8 ? 1 : 0;              // the activation codes follow the weights' format
  const int am_bf = a8 ? (i8 ? A_I8 : A_FP8) : A_BF16;
  // Deferred RMSNorm (bf16 activations): each residual epilogue also writes
  // bf16(x g) with the gain of the norm that reads the stream next (and its
  // remainder plane for the compensated gate/up) and each column tile's sum
  // of squares of every row; the QKV and gate/up GEMMs sum a row's tiles
  // and scale their output rows by its 1 / rms. Only layer 0's attention
  // norm, whose stream comes from the staging pass, runs as a pass of its
  // own.
  const bool defer = !f32 && !a8 && gemm_has(S, nqkv, H, {wt, A_BF16R, E_ROPE, 0, pk}) &&
                     gemm_has(S, I, H, {wt, A_BF16R, E_SWIGLU, comp, pk});
  {  // cos / sin of every position's RoPE angles, once for the pass
    c.label = "llm.rope_table";
    const int ne = S * (D / 2);
    VLA_TRY(launch(c, k_rope_table_ref(), dim3((ne + 255) / 256), dim3(256), 0,
                   {arg(b.rope_cos), arg(b.rope_sin), arg(S), arg(D), arg(cfg.rope_base)}));
  }
  for (int l = 0; l < n_layers; l++) {
    const vla_block_weights& w = layers[l];
    {  // RMSNorm -> fused QKV -> RoPE
      if (a8) {
        c.label = "llm.attn_norm";
        VLA_TRY(norm_rows8(c, b.xs.x, H, S, H, b.xs.rs, 1, cfg.eps, w.attn_norm, b.q8, b.q8s, H, i8));
      } else if (!f32 && (!defer || l == 0)) {
        c.label = "llm.attn_norm";
        VLA_TRY(norm_rows(c, b.xs.x, H, S, H, b.xs.rs, 1, cfg.eps, w.attn_norm, 0, nullptr, b.xn, nullptr, H));
      }
    c.label = "llm.qkv";
      GemmArgs a = gargs();
      a.M = S; a.N = nqkv; a.K = H;
      const bool rq = defer && l > 0;   // b.xn holds bf16(x g) from the previous layer's down projection
      if (f32) { a.a = b.xs.x; a.lda = H; a.rs = b.xs.rs; a.norm_rms = 1; a.eps = cfg.eps; a.g = w.attn_norm; }
      else if (a8) { a.a = b.q8; a.a_scale = b.q8s; a.lda = H; }
      else { a.a = b.xn; a.lda = H; }
      if (rq) { a.rsq = b.rsq; a.rsq_ld = b.rsq_ld; a.rsq_t = b.xs.rs.T; a.eps = cfg.eps; }
      a.w = w.w_qkv; a.ldw = H; a.wscale = w.s_qkv;
      a.c = b.qkv; a.ldc = nqkv; a.c_f32 = f32 || a8;
      a.q_cols = qd; a.k_cols = kd; a.head_dim = D; a.pos0 = 0; a.rope_cos = b.rope_cos; a.rope_sin = b.rope_sin;
      if (cfg.flags & VLA_BLOCK_QK_NORM) { a.qk_norm = 1; a.qk_eps = cfg.eps; a.qn_g = w.q_norm; a.kn_g = w.k_norm; }
      VLA_TRY(gemm(c, a, {wt, f32 ? A_NORM : rq ? A_BF16R : am_bf, E_ROPE, 0, pk}));
    }
    {  // causal GQA attention
    c.label = "llm.attn";
      AttnArgs a{};
      const size_t eq = f32 || a8 ? 4 : 2;
      a.q = b.qkv; a.ldq = nqkv;
      a.k = b.qkv ? (const char*)b.qkv + qd * eq : nullptr; a.ldk = nqkv;
      a.v = b.qkv ? (const char*)b.qkv + (qd + kd) * eq : nullptr; a.ldv = nqkv;
      a.o = b.ao; a.ldo = qd;
      a.Sq = S; a.Sk = S; a.Hq = cfg.n_q_heads; a.Hkv = cfg.n_kv_heads; a.D = D; a.causal = 1;
      VLA_TRY(attention(c, a, f32 || a8));
    }
    {  // O-proj + residual (+ row statistics)
      if (a8) {
        c.label = "llm.o_quant";
        VLA_TRY(quant_rows(c, b.ao, 1, qd, S, qd, b.q8, qd, b.q8s, i8));
      }
    c.label = "llm.o";
      GemmArgs a = gargs();
      a.M = S; a.N = H; a.K = qd;
      if (a8) { a.a = b.q8; a.a_scale = b.q8s; a.lda = qd; }
      else { a.a = b.ao; a.lda = qd; }
      a.w = w.w_o; a.ldw = qd; a.wscale = w.s_o;
      a.x = b.xs.x; a.ldx = H; a.rs_out = b.xs.part;
      if (defer) { a.xg = b.xn; a.xg_lo = comp ? b.xn_lo : nullptr; a.xg_gain = w.mlp_norm; a.rsq_out = b.rsq; a.rsq_ld = b.rsq_ld; }
      VLA_TRY(gemm(c, a, {wt, f32 ? A_F32 : am_bf, E_RESID, 0, pk}, &b.xs.rs));
    }
    {  // RMSNorm -> gate/up -> SiLU(gate) * up
      if (a8) {
        c.label = "llm.mlp_norm";
        VLA_TRY(norm_rows8(c, b.xs.x, H, S, H, b.xs.rs, 1, cfg.eps, w.mlp_norm, b.q8, b.q8s, H, i8));
      } else if (!f32 && !defer) {
        c.label = "llm.mlp_norm";
        VLA_TRY(norm_rows(c, b.xs.x, H, S, H, b.xs.rs, 1, cfg.eps, w.mlp_norm, 0, nullptr, b.xn, b.xn_lo, H));
      }
    c.label = "llm.gate_up";
      GemmArgs a = gargs();
      a.M = S; a.N = I; a.K = H;
      if (f32) { a.a = b.xs.x; a.lda = H; a.rs = b.xs.rs; a.norm_rms = 1; a.eps = cfg.eps; a.g = w.mlp_norm; }
      else if (a8) { a.a = b.q8; a.a_scale = b.q8s; a.lda = H; }
      else { a.a = b.xn; a.a_lo = b.xn_lo; a.lda = H; }
      if (defer) { a.rsq = b.rsq; a.rsq_ld = b.rsq_ld; a.rsq_t = b.xs.rs.T; a.eps = cfg.eps; }
      a.w = w.w_gate_up; a.ldw = H; a.wscale = w.s_gate_up; a.n_half = I;
      a.c = b.act; a.c_lo = b.act_lo; a.ldc = I; a.c_f32 = f32 || a8;
      VLA_TRY(gemm(c, a, {wt, f32 ? A_NORM : defer ? A_BF16R : am_bf, E_SWIGLU, comp, pk}));
    }
    {  // down + residual (+ row statistics)
      if (a8) {
        c.label = "llm.down_quant";
        VLA_TRY(quant_rows(c, b.act, 1, I, S, I, b.q8, I, b.q8s, i8));
      }
    c.label = "llm.down";
      GemmArgs a = gargs();
      a.M = S; a.N = H; a.K = I;
      if (a8) { a.a = b.q8; a.a_scale = b.q8s; a.lda = I; }
      else { a.a = b.act; a.a_lo = b.act_lo; a.lda = I; }
      a.w = w.w_down; a.ldw = I; a.wscale = w.s_down;
      a.x = b.xs.x; a.ldx = H; a.rs_out = b.xs.part;
      if (defer && l + 1 < n_layers) { a.xg = b.xn; a.xg_gain = layers[l + 1].attn_norm; a.rsq_out = b.rsq; a.rsq_ld = b.rsq_ld; }
      VLA_TRY(gemm(c, a, {wt, f32 ? A_F32 : am_bf, E_RESID, comp, pk}, &b.xs.rs));
    }
  }
  return VLA_OK;
}

// The scratch is laid out after the fixed buffers; plan mode sizes it from
// what the GEMMs asked for (a schedule is run once to learn the maxima).
template <typename Sched>
vla_status two_pass(void* ws, size_t ws_bytes, hipStream_t st, size_t* need_out, Sched sched) {
  // pass 0: learn scratch maxima
  Ctx p0;
  p0.plan = true;
  VLA_TRY(sched(p0));
  size_t fixed = p0.off;
  Ctx p1;
  p1.plan = true;
  p1.off = fixed;
  p1.take_scratch(p0);
  size_t need = p1.off;
  if (need_out) { *need_out = need; return VLA_OK; }
  if (!ws) return fail(VLA_ERR_INVALID_ARG, "null workspace");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(VLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(VLA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  Ctx c;
  c.plan = false; c.base = (char*)ws; c.cap = ws_bytes; c.st = st;
  c.status = (int*)ws;
  c.off = fixed;
  c.take_scratch(p0);
  c.off = STATUS_BYTES;   // fixed buffers are taken again by the schedule after the status words
  VLA_TRY(zero_counters(c));
  return sched(c);
}


// ------------------------------------------------------------------ DiT
vla_status check_dit(const vla_dit* d) {
  if (!d) return fail(VLA_ERR_INVALID_ARG, "null dit");
  const vla_dit_cfg& c = d->cfg;
  if (c.flags != 0) return fail(VLA_ERR_UNSUPPORTED, "dit cfg flags must be 0");
  if (c.wdtype != VLA_BF16 && !scaled8(c.wdtype)) return fail(VLA_ERR_UNSUPPORTED, "dit: weights must be bf16, fp8 or int8");
  if (c.head_dim != 80 && c.head_dim != 64) return fail(VLA_ERR_SHAPE, "dit: head_dim %d not in {64, 80}", c.head_dim);
  if (c.heads <= 0 || c.hidden != c.heads * c.head_dim) return fail(VLA_ERR_SHAPE, "dit: hidden %d != heads*head_dim", c.hidden);
  if (c.hidden % 8 || c.mlp % 8 || c.tdim % 8 || c.ctx_dim % 8 || c.layers <= 0 || c.mlp <= 0)
    return fail(VLA_ERR_SHAPE, "dit: widths must be positive multiples of 8");
  if (scaled8(c.wdtype) && (c.hidden % 16 || c.mlp % 16 || c.tdim % 16 || c.ctx_dim % 16))
    return fail(VLA_ERR_SHAPE, "dit: fp8 weights need widths that are multiples of 16");
  if (!d->layers || !d->w_ada || !d->b_ada || !d->w_ckv || !d->b_ckv || !d->w_t1 || !d->b_t1 || !d->w_t2 || !d->b_t2 ||
      !d->w_f || !d->b_f || !d->w_in || !d->b_in || !d->w_out || !d->b_out)
    return fail(VLA_ERR_INVALID_ARG, "dit: null tensor pointer");
  for (int l = 0; l < c.layers; l++) {
    const vla_dit_layer& L = d->layers[l];
    if (!L.w_qkv || !L.b_qkv || !L.w_o || !L.b_o || !L.w_cq || !L.b_cq || !L.w_co || !L.b_co || !L.w_up || !L.b_up ||
        !L.w_down || !L.b_down)
      return fail(VLA_ERR_INVALID_ARG, "dit layer %d: null tensor pointer", l);
    if (scaled8(c.wdtype) && (!L.s_qkv || !L.s_o || !L.s_cq || !L.s_co || !L.s_up || !L.s_down))
      return fail(VLA_ERR_INVALID_ARG, "dit layer %d: fp8 weights need scales", l);
  }
  if (scaled8(c.wdtype) && (!d->s_ada || !d->s_ckv || !d->s_t1 || !d->s_t2 || !d->s_f || !d->s_in || !d->s_out))
    return fail(VLA_ERR_INVALID_ARG, "dit: fp8 weights need scales");
  return VLA_OK;
}

// Compute units of the current device (one persistent workgroup each); 256
// when it cannot be queried (sizing a workspace without a device).
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

// The persistent layer kernel covers chunks of at most 16 rows, widths with
// an instantiated kernel, and MLPs whose width is a multiple of 2D (DOWN
// units span 2D), with enough workgroups for its units.
bool dit_stack_ok(const vla_dit_cfg& cf, int n, int G) {
  const int D = cf.hidden;
  if (n < 1 || n > 16 || cf.head_dim > DS_DP || cf.head_dim % 8 || D % 32 || D > 4 * DS_KSW * 32) return false;
  KernelRef k{};
  if (!dit_layer_lookup(cf.wdtype, D, &k)) return false;   // widths with an instantiated layer kernel
  if (cf.mlp % (2 * D)) return false;
  // up to two 16 x D units per workgroup in QKV, SAO, CAQ, CAO; one 32 x D
  // unit of UP and one 16 x 2D unit of DOWN
  if (3 * D / 16 > DS_MAXU * G || cf.heads > DS_MAXU * G) return false;
  return cf.mlp / 32 <= G && (D / 16) * (cf.mlp / (2 * D)) <= G;
}

struct DitIO {
  const void* ctx; int ctx_len;
  const float* x0; int n, A, K;
  float* actions; float* velocities;
};

// The sampler's buffers (all but the context's cross-attention K/V) and the
// state its parts hand on: the residual stream's row-statistics tiling.
struct DitState {
  uint16_t* phi = nullptr;   // sinusoidal features of the time grid [K, tdim]
  uint16_t* t1 = nullptr; uint16_t* sc = nullptr; float* mod = nullptr; float* fmod = nullptr;
  Stream xs{};
  // the layers kernel's per-layer buffers: layer l reads lx[l] (lx[0] is
  // xs.x) and writes lx[l + 1] through x1[l], x2[l]; aos, ao, h likewise
  float* lx = nullptr;
  float* x1 = nullptr; float* x2 = nullptr;
  DitLayerPtrs* tab = nullptr;   // the layers' weights, in device memory
  uint16_t* qkv = nullptr; uint16_t* ao = nullptr; uint16_t* q = nullptr; uint16_t* h = nullptr;
  int* derr = nullptr;
  uint16_t* aos = nullptr;   // the layer kernel's self-attention output
  // the layer kernel's flagged words (two bf16 + a flag each): QKV output
  // and cross-attention query, one block
  uint2* fw = nullptr; size_t fw_words = 0;
  uint2* fqkv = nullptr; uint2* fq = nullptr; uint2* fdp = nullptr;
  uint16_t* u = nullptr;   // modulated LayerNorm rows of the launch-per-operation path (bf16)
  // the launch-per-operation path normalises into u (8-bit / bf16 weights)
  // rather than in the GEMM prologue (fp32 weights); decided from the
  // configuration, never from u itself, which a planning pass leaves null
  bool urows = false;
  bool stack = false;
  int G = 0;
  unsigned spin = DS_SPIN;   // poll limit of the layer kernel's bounded waits
};

// Poll limit of the layer kernel's bounded waits: DS_SPIN, or fewer when the
// environment variable VLA_DIT_SPIN_LIMIT asks for it (a test of the
// time-out path makes every wait give up almost at once; nothing hangs).
unsigned dit_spin_limit() {
  const char* e = getenv("VLA_DIT_SPIN_LIMIT");
  if (!e || !*e) return DS_SPIN;
  const long v = strtol(e, nullptr, 10);
  return v >= 1 && v < (long)DS_SPIN ? (unsigned)v : DS_SPIN;
}

// Buffers of the sampler; clears the layer kernel's counters.
vla_status dit_begin(Ctx& c, const vla_dit& d, const DitIO& io, DitState& s) {
  const vla_dit_cfg& cf = d.cfg;
  const int D = cf.hidden, L = cf.layers, K = io.K, n = io.n;
  const int mod_w = L * 9 * D;
  s.phi = c.take<uint16_t>((size_t)K * cf.tdim);
  s.t1 = c.take<uint16_t>((size_t)K * D);
  s.sc = c.take<uint16_t>((size_t)K * D);
  s.mod = c.take<float>((size_t)K * mod_w);
  s.fmod = c.take<float>((size_t)K * 2 * D);
  s.xs = take_stream(c, n, D);
  s.G = cu_count();
  s.stack = dit_stack_ok(cf, n, s.G);
  s.spin = dit_spin_limit();
  if (s.stack) {
    const size_t nd = (size_t)n * D;
    s.lx = c.take<float>((size_t)(L + 1) * nd);
    s.xs.x = s.lx;
    s.x1 = c.take<float>((size_t)L * nd);
    s.x2 = c.take<float>((size_t)L * nd);
    s.aos = c.take<uint16_t>((size_t)L * nd);
    s.ao = c.take<uint16_t>((size_t)L * nd);
    s.h = c.take<uint16_t>((size_t)L * n * cf.mlp);
    s.tab = c.take<DitLayerPtrs>((size_t)L);
    const size_t wq = (size_t)n * 3 * D / 2, wd = (size_t)n * D / 2, wp = (size_t)ds_dpart_words(D, cf.mlp);
    s.fw_words = wq + wd + wp;
    s.fw = c.take<uint2>(s.fw_words);
    s.fqkv = s.fw; s.fq = s.fqkv + wq; s.fdp = s.fq + wd;
  } else {
    s.qkv = c.take<uint16_t>((size_t)n * 3 * D);
    s.q = c.take<uint16_t>((size_t)n * D);
    s.ao = c.take<uint16_t>((size_t)n * D);
    s.h = c.take<uint16_t>((size_t)n * cf.mlp);
  }
  s.derr = c.status;      // word 0 of the workspace's status block
  s.urows = !s.stack && cf.wdtype != VLA_F32;
  s.u = s.urows ? c.take<uint16_t>((size_t)n * D) : nullptr;
  if (s.stack) {
    // phase counters of the layer kernel live in the shared counter array
    // (every kernel leaves its counters at zero)
    const int nclr = ds_counter_words(D);
    c.need_tiles = std::max(c.need_tiles, (size_t)nclr);
    c.label = "dit.clear";
    unsigned z = 0;
    VLA_TRY(launch(c, k_fill_ref(), dim3((nclr + 255) / 256), dim3(256), 0, {arg(c.cnt_tile), arg(z), arg(nclr)}));
    int one = 1;
    VLA_TRY(launch(c, k_fill_ref(), dim3(1), dim3(256), 0, {arg(s.derr), arg(z), arg(one)}));
    // flagged words start at flag 0; the run's layers use flags 1, 2, ...
    const int nfw = (int)(s.fw_words * 2);
    VLA_TRY(launch(c, k_fill_ref(), dim3((nfw + 255) / 256), dim3(256), 0, {arg(s.fw), arg(z), arg(nfw)}));
    // the layers' weight table, DS_TAB_CHUNK layers per fill
    c.label = "dit.table";
    const bool sc = scaled8(cf.wdtype);
    for (int l0 = 0; l0 < L; l0 += DS_TAB_CHUNK) {
      DitTableArgs t{};
      t.n = std::min(DS_TAB_CHUNK, L - l0);
      t.out = s.tab ? s.tab + l0 : nullptr;
      for (int i = 0; i < t.n; i++) {
        const vla_dit_layer& w = d.layers[l0 + i];
        const void* ws[6] = {w.w_qkv, w.w_o, w.w_cq, w.w_co, w.w_up, w.w_down};
        const float* ss[6] = {w.s_qkv, w.s_o, w.s_cq, w.s_co, w.s_up, w.s_down};
        const float* bs[6] = {w.b_qkv, w.b_o, w.b_cq, w.b_co, w.b_up, w.b_down};
        for (int j = 0; j < 6; j++) { t.p[i].w[j] = ws[j]; t.p[i].s[j] = sc ? ss[j] : nullptr; t.p[i].b[j] = bs[j]; }
      }
      VLA_TRY(launch(c, k_dit_table_ref(), dim3(1), dim3(64), 0, {arg(t)}));
    }
  }
  return VLA_OK;
}

// Conditioning of every step from the fixed time grid: SiLU(c_k), the adaLN
// modulations of every layer and the final-layer modulation.
vla_status dit_conditioning(Ctx& c, const vla_dit& d, const DitIO& io, DitState& s) {
  const vla_dit_cfg& cf = d.cfg;
  const int D = cf.hidden, L = cf.layers, K = io.K, wt = cf.wdtype;
  const int mod_w = L * 9 * D;
  {  // phi(t_k) once for the whole grid, then Linear -> SiLU
    c.label = "dit.time_embed";
    const int half = cf.tdim / 2, ne = K * half;
    VLA_TRY(launch(c, k_time_embed_ref(), dim3((ne + 255) / 256), dim3(256), 0,
                   {arg(s.phi), arg(K), arg(half), arg(cf.time_scale), arg(cf.freq_base)}));
    c.label = "dit.time_fc1";
    GemmArgs a = gargs();
    a.M = K; a.N = D; a.K = cf.tdim;
    a.a = s.phi; a.lda = cf.tdim;
    a.w = d.w_t1; a.ldw = cf.tdim; a.wscale = d.s_t1; a.bias = d.b_t1; a.act = ACT_SILU;
    a.c = s.t1; a.ldc = D;
    VLA_TRY(gemm(c, a, {wt, A_BF16, E_STORE}));
  }
  {  // Linear -> SiLU: SiLU(c_k) for every step
    c.label = "dit.time_fc2";
    GemmArgs a = gargs();
    a.M = K; a.N = D; a.K = D;
    a.a = s.t1; a.lda = D;
    a.w = d.w_t2; a.ldw = D; a.wscale = d.s_t2; a.bias = d.b_t2; a.act = ACT_SILU;
    a.c = s.sc; a.ldc = D;
    VLA_TRY(gemm(c, a, {wt, A_BF16, E_STORE}));
  }
  {  // adaLN modulations of every layer for every step (one launch)
    c.label = "dit.adaln";
    GemmArgs a = gargs();
    a.M = K; a.N = mod_w; a.K = D;
    a.a = s.sc; a.lda = D;
    a.w = d.w_ada; a.ldw = D; a.wscale = d.s_ada; a.bias = d.b_ada;
    a.c = s.mod; a.ldc = mod_w; a.c_f32 = 1;
    VLA_TRY(gemm(c, a, {wt, A_BF16, E_STORE}));
  }
  {  // final-layer modulation
    c.label = "dit.final_mod";
    GemmArgs a = gargs();
    a.M = K; a.N = 2 * D; a.K = D;
    a.a = s.sc; a.lda = D;
    a.w = d.w_f; a.ldw = D; a.wscale = d.s_f; a.bias = d.b_f;
    a.c = s.fmod; a.ldc = 2 * D; a.c_f32 = 1;
    VLA_TRY(gemm(c, a, {wt, A_BF16, E_STORE}));
  }
  return VLA_OK;
}

// Keys per row of the transposed context values the layer kernel reads.
int dit_vt_pitch(int C) { return (C + 31) / 32 * 32; }
size_t dit_vt_elems(const vla_dit_cfg& cf, int C) { return (size_t)cf.layers * cf.hidden * dit_vt_pitch(C); }

// Cross-attention K/V of every layer from a context (one launch), and for
// the layer kernel (vt not null) the values transposed.
vla_status dit_cross_kv(Ctx& c, const vla_dit& d, const void* ctx, int C, uint16_t* ckv, uint16_t* vt, bool transpose) {
  const vla_dit_cfg& cf = d.cfg;
  const int D = cf.hidden, L = cf.layers;
  c.label = "dit.cross_kv";
  GemmArgs a = gargs();
  a.M = C; a.N = L * 2 * D; a.K = cf.ctx_dim;
  a.a = ctx; a.lda = cf.ctx_dim;
  a.w = d.w_ckv; a.ldw = cf.ctx_dim; a.wscale = d.s_ckv; a.bias = d.b_ckv;
  a.c = ckv; a.ldc = L * 2 * D;
  VLA_TRY(gemm(c, a, {cf.wdtype, A_BF16, E_STORE}));
  if (!transpose) return VLA_OK;
  c.label = "dit.cross_vt";
  const int Cp = dit_vt_pitch(C);
  const size_t nt = (size_t)L * (Cp / 8) * D;
  return launch(c, k_ctx_vt_ref(), dim3((unsigned)((nt + 255) / 256)), dim3(256), 0,
                {arg((const uint16_t*)ckv), arg(C), arg(L), arg(D), arg(Cp), arg(vt)});
}

// a_0 = x0 -> x = a_0 W_in^T + b_in (+ row statistics)
vla_status dit_in_proj(Ctx& c, const vla_dit& d, const DitIO& io, DitState& s) {
  const vla_dit_cfg& cf = d.cfg;
  KernelRef tail{};
  euler_tail_lookup(cf.wdtype, &tail);
  TailArgs t{};
  t.n = io.n; t.D = cf.hidden; t.A = io.A; t.K = io.K; t.eps = cf.eps;
  t.a_in = io.x0; t.a_out = io.actions;
  t.w_in = d.w_in; t.s_in = d.s_in; t.b_in = d.b_in; t.x_out = s.xs.x; t.rs_out = s.xs.part;
  s.xs.rs.T = 1; s.xs.rs.tw = cf.hidden;
  c.label = "dit.in_proj";
  return launch(c, tail.fn, dim3(io.n), dim3(256), (size_t)(cf.hidden + io.A) * sizeof(float), {arg(t)});
}

// Euler steps k0 .. k1-1 of the K-step sampler, cross-attending to `ckv`
// (the layer kernel: keys from ckv, values from their transpose vt).
vla_status dit_steps(Ctx& c, const vla_dit& d, const DitIO& io, DitState& s, const uint16_t* ckv, const uint16_t* vt,
                     int k0, int k1) {
  const vla_dit_cfg& cf = d.cfg;
  const int D = cf.hidden, L = cf.layers, K = io.K, n = io.n, A = io.A, C = io.ctx_len;
  const int wt = cf.wdtype;
  const int mod_w = L * 9 * D;
  float* x = s.xs.x;
  Stream& xs = s.xs;
  KernelRef tail{};
  euler_tail_lookup(wt, &tail);
  const size_t tail_smem = (size_t)(D + A) * sizeof(float);
  KernelRef lk{};
  if (s.stack && !dit_layer_lookup(wt, D, &lk)) return fail(VLA_ERR_UNSUPPORTED, "dit: no layer kernel for wdtype %d", wt);
  if (s.stack && !c.plan && lk.smem > 64 * 1024) VLA_TRY(allow_smem(lk));
  for (int k = k0; k < k1; k++) {
    if (s.stack) {  // every layer of the step in one persistent launch
      c.label = "dit.layers";
      DitLayerArgs a{};
      a.n = n; a.D = D; a.H = cf.heads; a.hd = cf.head_dim; a.mlp = cf.mlp; a.C = C;
      a.eps = cf.eps; a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cf.head_dim));
      a.l0 = 0; a.l1 = L;
      a.tab = s.tab;
      a.mod = s.mod ? s.mod + (size_t)k * mod_w : nullptr;
      a.ckv = ckv; a.ldc = L * 2 * D;
      a.vt = vt; a.ldvt = dit_vt_pitch(C);
      a.xs = s.lx; a.x1 = s.x1; a.x2 = s.x2; a.aos = s.aos; a.aoc = s.ao; a.h = s.h;
      a.qkv = s.fqkv; a.q = s.fq; a.dpart = s.fdp;
      a.wq_next = k + 1 < K ? d.layers[0].w_qkv : nullptr;
      a.cnt = c.cnt_tile; a.err = s.derr; a.spin = s.spin;
      a.flag0 = 1u + (unsigned)(k * L);   // increasing over the run, whose start cleared the words
      VLA_TRY(launch(c, lk.fn, dim3(s.G), dim3(lk.threads), (size_t)lk.smem, {arg(a)}));
    }
    for (int l = 0; l < L && !s.stack; l++) {
      const vla_dit_layer& w = d.layers[l];
      const float* m = s.mod ? s.mod + (size_t)k * mod_w + (size_t)l * 9 * D : nullptr;
      auto mv = [&](int j) { return m ? m + (size_t)j * D : nullptr; };
      // The modulated LayerNorm u = LN(x)(1 + scale) + shift of a sublayer's
      // input: bf16 / fp8 weights take u from one row-norm launch (each of
      // the GEMM's workgroups would otherwise normalise every row again);
      // fp32 weights normalise in the GEMM's prologue.
      auto modln = [&](GemmArgs& a, int sh, int sc, const char* label) -> vla_status {
        if (s.urows) {
          c.label = label;
          VLA_TRY(norm_rows(c, x, D, n, D, xs.rs, 0, cf.eps, mv(sc), 1, mv(sh), s.u, nullptr, D));
          a.a = s.u; a.lda = D;
        } else {
          a.a = x; a.lda = D; a.rs = xs.rs; a.norm_rms = 0; a.eps = cf.eps; a.g = mv(sc); a.g_plus_one = 1; a.bsh = mv(sh);
        }
        return VLA_OK;
      };
      const int am_norm = s.urows ? A_BF16 : A_NORM;
      {  // adaLN(LN) -> self-attn QKV
        GemmArgs a = gargs();
        VLA_TRY(modln(a, 0, 1, "dit.sa_norm"));
        c.label = "dit.sa_qkv";
        a.M = n; a.N = 3 * D; a.K = D;
        a.w = w.w_qkv; a.ldw = D; a.wscale = w.s_qkv; a.bias = w.b_qkv;
        a.c = s.qkv; a.ldc = 3 * D;
        VLA_TRY(gemm(c, a, {wt, am_norm, E_STORE}));
      }
      {
        c.label = "dit.sa_attn";
        AttnArgs a{};
        a.q = s.qkv; a.ldq = 3 * D;
        a.k = s.qkv ? s.qkv + D : nullptr; a.ldk = 3 * D;
        a.v = s.qkv ? s.qkv + 2 * D : nullptr; a.ldv = 3 * D;
        a.o = s.ao; a.ldo = D;
        a.Sq = n; a.Sk = n; a.Hq = cf.heads; a.Hkv = cf.heads; a.D = cf.head_dim; a.causal = 0;
        VLA_TRY(attention(c, a, false));
      }
      {  // O-proj, gated residual
      c.label = "dit.sa_o";
        GemmArgs a = gargs();
        a.M = n; a.N = D; a.K = D;
        a.a = s.ao; a.lda = D;
        a.w = w.w_o; a.ldw = D; a.wscale = w.s_o; a.bias = w.b_o; a.gate = mv(2);
        a.x = x; a.ldx = D; a.rs_out = xs.part;
        VLA_TRY(gemm(c, a, {wt, A_BF16, E_RESID}, &xs.rs));
      }
      {  // adaLN(LN) -> cross-attn query
        GemmArgs a = gargs();
        VLA_TRY(modln(a, 3, 4, "dit.ca_norm"));
        c.label = "dit.ca_q";
        a.M = n; a.N = D; a.K = D;
        a.w = w.w_cq; a.ldw = D; a.wscale = w.s_cq; a.bias = w.b_cq;
        a.c = s.q; a.ldc = D;
        VLA_TRY(gemm(c, a, {wt, am_norm, E_STORE}));
      }
      {
        c.label = "dit.ca_attn";
        AttnArgs a{};
        a.q = s.q; a.ldq = D;
        a.k = ckv ? ckv + (size_t)l * 2 * D : nullptr; a.ldk = L * 2 * D;
        a.v = ckv ? ckv + (size_t)l * 2 * D + D : nullptr; a.ldv = L * 2 * D;
        a.o = s.ao; a.ldo = D;
        a.Sq = n; a.Sk = C; a.Hq = cf.heads; a.Hkv = cf.heads; a.D = cf.head_dim; a.causal = 0;
        VLA_TRY(attention(c, a, false));
      }
      {  // cross-attn out, gated residual
      c.label = "dit.ca_o";
        GemmArgs a = gargs();
        a.M = n; a.N = D; a.K = D;
        a.a = s.ao; a.lda = D;
        a.w = w.w_co; a.ldw = D; a.wscale = w.s_co; a.bias = w.b_co; a.gate = mv(5);
        a.x = x; a.ldx = D; a.rs_out = xs.part;
        VLA_TRY(gemm(c, a, {wt, A_BF16, E_RESID}, &xs.rs));
      }
      {  // adaLN(LN) -> MLP up -> GELU
        GemmArgs a = gargs();
        VLA_TRY(modln(a, 6, 7, "dit.mlp_norm"));
        c.label = "dit.mlp_up";
        a.M = n; a.N = cf.mlp; a.K = D;
        a.w = w.w_up; a.ldw = D; a.wscale = w.s_up; a.bias = w.b_up; a.act = ACT_GELU;
        a.c = s.h; a.ldc = cf.mlp;
        VLA_TRY(gemm(c, a, {wt, am_norm, E_STORE}));
      }
      {  // MLP down, gated residual
      c.label = "dit.mlp_down";
        GemmArgs a = gargs();
        a.M = n; a.N = D; a.K = cf.mlp;
        a.a = s.h; a.lda = cf.mlp;
        a.w = w.w_down; a.ldw = cf.mlp; a.wscale = w.s_down; a.bias = w.b_down; a.gate = mv(8);
        a.x = x; a.ldx = D; a.rs_out = xs.part;
        VLA_TRY(gemm(c, a, {wt, A_BF16, E_RESID}, &xs.rs));
      }
    }
    {  // velocity head + Euler update (+ input projection for the next step)
      TailArgs t{};
      t.n = n; t.D = D; t.A = A; t.K = K; t.eps = cf.eps;
      t.x = s.stack ? s.lx + (size_t)L * n * D : x;   // the last layer's output
      t.shift = s.fmod ? s.fmod + (size_t)k * 2 * D : nullptr;
      t.scale = s.fmod ? s.fmod + (size_t)k * 2 * D + D : nullptr;
      t.w_out = d.w_out; t.s_out = d.s_out; t.b_out = d.b_out;
      t.a_in = io.actions; t.a_out = io.actions;
      t.v_out = io.velocities ? io.velocities + (size_t)k * n * A : nullptr;
      if (k + 1 < K) { t.w_in = d.w_in; t.s_in = d.s_in; t.b_in = d.b_in; t.x_out = x; t.rs_out = xs.part; }
      c.label = "dit.tail";
      VLA_TRY(launch(c, tail.fn, dim3(n), dim3(256), tail_smem, {arg(t)}));
      xs.rs.T = 1; xs.rs.tw = D;
    }
  }
  return VLA_OK;
}

vla_status sched_dit(Ctx& c, const vla_dit& d, const DitIO& io) {
  DitState s;
  VLA_TRY(dit_begin(c, d, io, s));
  uint16_t* ckv = c.take<uint16_t>((size_t)io.ctx_len * d.cfg.layers * 2 * d.cfg.hidden);
  uint16_t* vt = s.stack ? c.take<uint16_t>(dit_vt_elems(d.cfg, io.ctx_len)) : nullptr;
  VLA_TRY(dit_conditioning(c, d, io, s));
  VLA_TRY(dit_cross_kv(c, d, io.ctx, io.ctx_len, ckv, vt, s.stack));
  VLA_TRY(dit_in_proj(c, d, io, s));
  return dit_steps(c, d, io, s, ckv, vt, 0, io.K);
}

// ------------------------------------------------------------------ ViT
vla_status check_vit(const vla_vit* v) {
  if (!v) return fail(VLA_ERR_INVALID_ARG, "null vit");
  const vla_vit_cfg& c = v->cfg;
  if (c.flags & ~VLA_BLOCK_PACKED) return fail(VLA_ERR_UNSUPPORTED, "vit cfg flags: only VLA_BLOCK_PACKED");
  if (c.wdtype != VLA_BF16) return fail(VLA_ERR_UNSUPPORTED, "vit: weights must be bf16");
  if (c.patch <= 0 || c.image % c.patch || c.merge <= 0 || (c.image / c.patch) % c.merge)
    return fail(VLA_ERR_SHAPE, "vit: image %d / patch %d / merge %d do not tile", c.image, c.patch, c.merge);
  if (c.head_dim != 64 || c.hidden != c.heads * c.head_dim) return fail(VLA_ERR_SHAPE, "vit: head_dim must be 64 and hidden = heads*64");
  if (c.hidden % 8 || c.mlp % 8 || c.out_dim % 8) return fail(VLA_ERR_SHAPE, "vit: widths must be multiples of 8");
  if (!v->layers || !v->w_pe || !v->b_pe || !v->pos || !v->mln_g || !v->mln_b || !v->w_m1 || !v->b_m1 || !v->w_m2 || !v->b_m2)
    return fail(VLA_ERR_INVALID_ARG, "vit: null tensor pointer");
  for (int l = 0; l < c.layers; l++) {
    const vla_vit_layer& L = v->layers[l];
    if (!L.ln1_g || !L.ln1_b || !L.w_qkv || !L.b_qkv || !L.w_o || !L.b_o || !L.ln2_g || !L.ln2_b || !L.w_up || !L.b_up ||
        !L.w_down || !L.b_down)
      return fail(VLA_ERR_INVALID_ARG, "vit layer %d: null tensor pointer", l);
  }
  return VLA_OK;
}

// Writes the merged tokens (fp32) to out rows [0, n_img * n_merged) with pitch ldo.
vla_status sched_vit(Ctx& c, const vla_vit& v, const void* images, int n_img, float* out, int ldo, float* vit_out) {
  const vla_vit_cfg& cf = v.cfg;
  const int grid = cf.image / cf.patch, np = grid * grid, S = n_img * np, D = cf.hidden;
  const int pdim = cf.channels * cf.patch * cf.patch, pitch = (int)align_up(pdim, 8);
  const int nm = np / (cf.merge * cf.merge), Mm = n_img * nm, MD = D * cf.merge * cf.merge;
  const int pk = (cf.flags & VLA_BLOCK_PACKED) ? 1 : 0;   // the layers' four Linears packed by vla_pack_weights
  Stream zst = take_stream(c, S, D);
  float* z = zst.x;
  uint16_t* qkv = c.take<uint16_t>((size_t)S * 3 * D);
  uint16_t* ao = c.take<uint16_t>((size_t)S * D);
  uint16_t* h = c.take<uint16_t>((size_t)S * cf.mlp);
  uint16_t* m1 = c.take<uint16_t>((size_t)Mm * MD);
  uint16_t* mz = c.take<uint16_t>((size_t)Mm * MD);   // LayerNormed patches, 2x2 groups concatenated
  uint16_t* zn = c.take<uint16_t>((size_t)S * D);      // LayerNorm-ed rows (bf16)
  uint16_t* prow = c.take<uint16_t>((size_t)S * pitch);   // patch rows, zero-padded to the weights' pitch
  {  // patchify -> Linear + bias + position table (+ row statistics)
    c.label = "vit.patch_rows";
    const size_t ne = (size_t)S * (pitch / 8);
    VLA_TRY(launch(c, k_patch_rows_ref(), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0,
                   {arg((const uint16_t*)images), arg(n_img), arg(cf.channels), arg(cf.image), arg(cf.patch), arg(grid),
                    arg(pitch), arg(prow)}));
    c.label = "vit.patch_embed";
    GemmArgs a = gargs();
    // K runs over the pitch: the pad columns are zero in the patch rows and
    // in w_pe alike
    a.M = S; a.N = D; a.K = pitch;
    a.a = prow; a.lda = pitch;
    a.w = v.w_pe; a.ldw = pitch; a.bias = v.b_pe;
    a.x = z; a.ldx = D; a.x_init = 1; a.addrow = v.pos; a.addrow_rows = np; a.rs_out = zst.part;
    VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_RESID}, &zst.rs));
  }
  for (int l = 0; l < cf.layers; l++) {
    const vla_vit_layer& w = v.layers[l];
    {
      c.label = "vit.ln1";
      VLA_TRY(norm_rows(c, z, D, S, D, zst.rs, 0, cf.eps, w.ln1_g, 0, w.ln1_b, zn, nullptr, D));
      c.label = "vit.qkv";
      GemmArgs a = gargs();
      a.M = S; a.N = 3 * D; a.K = D;
      a.a = zn; a.lda = D;
      a.w = w.w_qkv; a.ldw = D; a.bias = w.b_qkv;
      a.c = qkv; a.ldc = 3 * D;
      VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_STORE, 0, pk}));
    }
    {
      c.label = "vit.attn";
      AttnArgs a{};
      a.q = qkv; a.ldq = 3 * D;
      a.k = qkv ? qkv + D : nullptr; a.ldk = 3 * D;
      a.v = qkv ? qkv + 2 * D : nullptr; a.ldv = 3 * D;
      a.o = ao; a.ldo = D;
      // images are independent sequences: one attention call per image
      for (int i = 0; i < n_img; i++) {
        AttnArgs ai = a;
        if (qkv) {
          ai.q = qkv + (size_t)i * np * 3 * D;
          ai.k = qkv + (size_t)i * np * 3 * D + D;
          ai.v = qkv + (size_t)i * np * 3 * D + 2 * D;
          ai.o = ao + (size_t)i * np * D;
        }
        ai.Sq = np; ai.Sk = np; ai.Hq = cf.heads; ai.Hkv = cf.heads; ai.D = cf.head_dim; ai.causal = 0;
        VLA_TRY(attention(c, ai, false));
      }
    }
    {
      c.label = "vit.o";
      GemmArgs a = gargs();
      a.M = S; a.N = D; a.K = D;
      a.a = ao; a.lda = D;
      a.w = w.w_o; a.ldw = D; a.bias = w.b_o;
      a.x = z; a.ldx = D; a.rs_out = zst.part;
      VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_RESID, 0, pk}, &zst.rs));
    }
    {
      c.label = "vit.ln2";
      VLA_TRY(norm_rows(c, z, D, S, D, zst.rs, 0, cf.eps, w.ln2_g, 0, w.ln2_b, zn, nullptr, D));
      c.label = "vit.up";
      GemmArgs a = gargs();
      a.M = S; a.N = cf.mlp; a.K = D;
      a.a = zn; a.lda = D;
      a.w = w.w_up; a.ldw = D; a.bias = w.b_up; a.act = ACT_GELU;
      a.c = h; a.ldc = cf.mlp;
      VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_STORE, 0, pk}));
    }
    {
      c.label = "vit.down";
      GemmArgs a = gargs();
      a.M = S; a.N = D; a.K = cf.mlp;
      a.a = h; a.lda = cf.mlp;
      a.w = w.w_down; a.ldw = cf.mlp; a.bias = w.b_down;
      a.x = z; a.ldx = D; a.rs_out = zst.part;
      VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_RESID, 0, pk}, &zst.rs));
    }
  }
  if (vit_out) { c.label = "vit.out"; VLA_TRY(convert_rows(c, z, D, S, D, vit_out, D, 1)); }
  {  // LN of every patch, written straight into its 2x2 group of the merged rows
    c.label = "mrg.ln";
    VLA_TRY(norm_rows(c, z, D, S, D, zst.rs, 0, cf.eps, v.mln_g, 0, v.mln_b, mz, nullptr, MD, cf.merge, grid, np));
  }
  {  // Linear -> GELU
    c.label = "mrg.fc1";
    GemmArgs a = gargs();
    a.M = Mm; a.N = MD; a.K = MD;
    a.a = mz; a.lda = MD;
    a.w = v.w_m1; a.ldw = MD; a.bias = v.b_m1; a.act = ACT_GELU;
    a.c = m1; a.ldc = MD;
    VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_STORE}));
  }
  {  // Linear -> visual tokens (fp32)
    c.label = "mrg.fc2";
    GemmArgs a = gargs();
    a.M = Mm; a.N = cf.out_dim; a.K = MD;
    a.a = m1; a.lda = MD;
    a.w = v.w_m2; a.ldw = MD; a.bias = v.b_m2;
    a.c = out; a.ldc = ldo; a.c_f32 = 1;
    VLA_TRY(gemm(c, a, {VLA_BF16, A_BF16, E_STORE}));
  }
  return VLA_OK;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

const char* vla_last_error(void) { return g_err.c_str(); }

size_t vla_packed_bytes(int32_t wdtype, int32_t N, int32_t K) {
  if ((wdtype != VLA_BF16 && !scaled8(wdtype)) || N < 1 || K < 1) return 0;
  const size_t esz = wdtype == VLA_BF16 ? 2 : 1;
  return (size_t)((N + 15) / 16) * (size_t)((K + 31) / 32) * 512 * esz;
}

vla_status vla_pack_weights(int32_t wdtype, const void* w, int32_t N, int32_t K, int32_t ldw, void* packed,
                            hipStream_t stream) {
  if (wdtype != VLA_BF16 && !scaled8(wdtype)) return fail(VLA_ERR_UNSUPPORTED, "pack weights: dtype %d (bf16, fp8 or int8)", wdtype);
  if (!w || !packed) return fail(VLA_ERR_INVALID_ARG, "pack weights: null pointer");
  if ((reinterpret_cast<uintptr_t>(packed) & 15) != 0) return fail(VLA_ERR_INVALID_ARG, "pack weights: output not 16-byte aligned");
  if (N < 1 || K < 1 || ldw < K) return fail(VLA_ERR_SHAPE, "pack weights: N %d, K %d, pitch %d", N, K, ldw);
  const size_t chunks = vla_packed_bytes(wdtype, N, K) / (wdtype == VLA_BF16 ? 16 : 8);
  if (vla_packed_bytes(wdtype, N, K) >= (size_t)BUF_LIMIT) return fail(VLA_ERR_SHAPE, "pack weights: matrix beyond 2 GiB");
  Ctx c;
  c.plan = false; c.st = stream;
  c.label = "pack_weights";
  const int esz = wdtype == VLA_BF16 ? 2 : 1;
  return launch(c, k_pack_weights_ref(), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                {arg(w), arg(N), arg(K), arg(ldw), arg(esz), arg(packed)});
}

vla_status vla_workspace_status(const void* ws, hipStream_t stream) {
  if (!ws) return fail(VLA_ERR_INVALID_ARG, "null workspace");
  VLA_HIP(hipStreamSynchronize(stream));
  int word = 0;
  VLA_HIP(hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost));
  if (word != 0)
    return fail(VLA_ERR_TIMEOUT, "a bounded wait of the DiT layer kernel gave up in the last pass on this workspace; "
                                 "its actions and velocities hold NaN");
  return VLA_OK;
}
int32_t vla_abi_version(void) { return VLA_ABI_VERSION; }

static vla_status block_sched(Ctx& c, const vla_block_cfg* cfg, const vla_block_weights* w, const void* x_in, void* x_out,
                              int seq) {
  BackboneBufs b = take_backbone_bufs(c, *cfg, seq);
  const int f32 = cfg->adtype == VLA_F32;
  c.label = "llm.stage";
  VLA_TRY(stage_stream(c, b.xs, seq, cfg->hidden, x_in, f32, 0, seq));
  VLA_TRY(sched_layers(c, *cfg, w, 1, b, seq));
  c.label = "llm.out";
  return convert_rows(c, b.xs.x, cfg->hidden, seq, cfg->hidden, x_out, cfg->hidden, f32);
}

vla_status vla_block_forward(const vla_block_cfg* cfg, const vla_block_weights* w, const void* x_in, void* x_out,
                             int32_t seq, void* ws, size_t ws_bytes, hipStream_t stream) {
  VLA_TRY(check_block_cfg(cfg));
  VLA_TRY(check_block_weights(cfg, w));
  if (!x_in || !x_out) return fail(VLA_ERR_INVALID_ARG, "null input/output");
  if (seq < 1 || seq > 4096) return fail(VLA_ERR_SHAPE, "seq %d outside [1, 4096]", seq);
  return two_pass(ws, ws_bytes, stream, nullptr, [&](Ctx& c) { return block_sched(c, cfg, w, x_in, x_out, seq); });
}

size_t vla_block_workspace_bytes(const vla_block_cfg* cfg, int32_t seq) {
  if (check_block_cfg(cfg) != VLA_OK || seq < 1 || seq > 4096) return 0;
  vla_block_weights dummy{};
  size_t need = 0;
  if (two_pass(nullptr, 0, nullptr, &need, [&](Ctx& c) { return block_sched(c, cfg, &dummy, nullptr, nullptr, seq); }) != VLA_OK)
    return 0;
  return need;
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free block
// Scratch of vla_block_forward_static: a file-scope device array, one copy
// per GPU (each GPU the library runs on holds it until the process ends).
// On the host the array's name is only a stand-in for the symbol; its
// device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept here, and only that address is ever handed to
// kernels.
static __device__ __align__(256) char scratch[VLA_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // by device ordinal

vla_status scratch_ptr(void** out) {
  int dev = 0;
  VLA_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    VLA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0)
      return fail(VLA_ERR_HIP, "static scratch: unusable device address %p", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VLA_OK;
}
}  // namespace

extern "C" {

vla_status vla_block_forward_static(const vla_block_cfg* cfg, const vla_block_weights* w, const void* x_in, void* x_out,
                                    int32_t seq, hipStream_t stream) {
  VLA_TRY(check_block_cfg(cfg));
  VLA_TRY(check_block_weights(cfg, w));
  if (!x_in || !x_out) return fail(VLA_ERR_INVALID_ARG, "null input/output");
  if (seq < 1 || seq > 4096) return fail(VLA_ERR_SHAPE, "seq %d outside [1, 4096]", seq);
  auto sched = [&](Ctx& c) { return block_sched(c, cfg, w, x_in, x_out, seq); };
  size_t need = 0;
  VLA_TRY(two_pass(nullptr, 0, nullptr, &need, sched));
  if (need > (size_t)VLA_STATIC_SCRATCH_BYTES)
    return fail(VLA_ERR_WORKSPACE, "block at seq %d needs %zu bytes of scratch, above the static array's %zu", seq, need,
                (size_t)VLA_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  VLA_TRY(scratch_ptr(&ws));
  // the pass starts with a fill kernel that zeroes its split-K counters;
  // every other buffer of the block is written before it is read
  return two_pass(ws, (size_t)VLA_STATIC_SCRATCH_BYTES, stream, nullptr, sched);
}

static vla_status check_backbone(const vla_backbone* bb) {
  if (!bb) return fail(VLA_ERR_INVALID_ARG, "null backbone");
  VLA_TRY(check_block_cfg(&bb->cfg));
  if (bb->n_layers < 1 || !bb->layers) return fail(VLA_ERR_INVALID_ARG, "backbone: no layers");
  for (int l = 0; l < bb->n_layers; l++) VLA_TRY(check_block_weights(&bb->cfg, &bb->layers[l]));
  return VLA_OK;
}

static vla_status backbone_sched(Ctx& c, const vla_backbone* bb, const void* embeds, int seq, void* out) {
  const vla_block_cfg& cfg = bb->cfg;
  BackboneBufs b = take_backbone_bufs(c, cfg, seq);
  const int f32 = cfg.adtype == VLA_F32;
  c.label = "llm.stage";
  VLA_TRY(stage_stream(c, b.xs, seq, cfg.hidden, embeds, f32, 0, seq));
  VLA_TRY(sched_layers(c, cfg, bb->layers, bb->n_layers, b, seq));
  c.label = "llm.final_norm";
  if (bb->final_norm) return rmsnorm_out(c, b.xs.x, cfg.hidden, seq, cfg.hidden, b.xs.rs, bb->final_norm, cfg.eps, out, cfg.hidden, f32);
  return convert_rows(c, b.xs.x, cfg.hidden, seq, cfg.hidden, out, cfg.hidden, f32);
}

vla_status vla_backbone_prefill(const vla_backbone* bb, const void* embeds, int32_t seq, void* hidden_out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  VLA_TRY(check_backbone(bb));
  if (!embeds || !hidden_out) return fail(VLA_ERR_INVALID_ARG, "null input/output");
  if (seq < 1 || seq > 4096) return fail(VLA_ERR_SHAPE, "seq %d outside [1, 4096]", seq);
  return two_pass(ws, ws_bytes, stream, nullptr, [&](Ctx& c) { return backbone_sched(c, bb, embeds, seq, hidden_out); });
}

size_t vla_backbone_workspace_bytes(const vla_backbone* bb, int32_t seq) {
  if (!bb || check_block_cfg(&bb->cfg) != VLA_OK || seq < 1 || seq > 4096 || bb->n_layers < 1) return 0;
  std::vector<vla_block_weights> dummy(bb->n_layers);
  vla_backbone b2 = *bb;
  b2.layers = dummy.data();
  size_t need = 0;
  if (two_pass(nullptr, 0, nullptr, &need, [&](Ctx& c) { return backbone_sched(c, &b2, nullptr, seq, nullptr); }) != VLA_OK)
    return 0;
  return need;
}

static vla_status check_dit_call(const vla_dit* d, int ctx_len, int chunk, int A, int K) {
  if (ctx_len < 1 || ctx_len > 4096) return fail(VLA_ERR_SHAPE, "ctx_len %d outside [1, 4096]", ctx_len);
  if (chunk < 1 || chunk > 64) return fail(VLA_ERR_SHAPE, "chunk %d outside [1, 64]", chunk);
  if (A < 1 || A > 256) return fail(VLA_ERR_SHAPE, "action_dim %d outside [1, 256]", A);
  if (K < 1 || K > 64) return fail(VLA_ERR_SHAPE, "K %d outside [1, 64]", K);
  (void)d;
  return VLA_OK;
}

vla_status vla_flow_euler_sample(const vla_dit* dit, const void* ctx, int32_t ctx_len, const float* x0, int32_t chunk,
                                 int32_t action_dim, int32_t K, float* actions_out, float* velocities_out, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  VLA_TRY(check_dit(dit));
  VLA_TRY(check_dit_call(dit, ctx_len, chunk, action_dim, K));
  if (!ctx || !x0 || !actions_out) return fail(VLA_ERR_INVALID_ARG, "null input/output");
  DitIO io{ctx, ctx_len, x0, chunk, action_dim, K, actions_out, velocities_out};
  return two_pass(ws, ws_bytes, stream, nullptr, [&](Ctx& c) { return sched_dit(c, *dit, io); });
}

size_t vla_dit_workspace_bytes(const vla_dit* dit, int32_t ctx_len, int32_t chunk, int32_t action_dim, int32_t K) {
  if (!dit || check_dit_call(dit, ctx_len, chunk, action_dim, K) != VLA_OK) return 0;
  std::vector<vla_dit_layer> dummy(dit->cfg.layers > 0 ? dit->cfg.layers : 1);
  vla_dit d2 = *dit;
  d2.layers = dummy.data();
  DitIO io{nullptr, ctx_len, nullptr, chunk, action_dim, K, nullptr, nullptr};
  size_t need = 0;
  if (two_pass(nullptr, 0, nullptr, &need, [&](Ctx& c) { return sched_dit(c, d2, io); }) != VLA_OK) return 0;
  return need;
}

vla_status vla_vit_encode(const vla_vit* vit, const void* images, int32_t n_images, float* tokens_out, float* vit_out,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  VLA_TRY(check_vit(vit));
  if (!images || !tokens_out) return fail(VLA_ERR_INVALID_ARG, "null input/output");
  if (n_images < 1 || n_images > 16) return fail(VLA_ERR_SHAPE, "n_images %d outside [1, 16]", n_images);
  return two_pass(ws, ws_bytes, stream, nullptr,
                  [&](Ctx& c) { return sched_vit(c, *vit, images, n_images, tokens_out, vit->cfg.out_dim, vit_out); });
}

size_t vla_vit_workspace_bytes(const vla_vit* vit, int32_t n_images) {
  if (!vit || n_images < 1 || n_images > 16) return 0;
  std::vector<vla_vit_layer> dummy(vit->cfg.layers > 0 ? vit->cfg.layers : 1);
  vla_vit v2 = *vit;
  v2.layers = dummy.data();
  size_t need = 0;
  if (two_pass(nullptr, 0, nullptr, &need,
               [&](Ctx& c) { return sched_vit(c, v2, nullptr, n_images, nullptr, v2.cfg.out_dim, nullptr); }) != VLA_OK)
    return 0;
  return need;
}

}  // extern "C"

// ================================================================== step plan
// Events of a fused cycle: fork (both branches start after the work the
// caller queued), context ready, action branch done.
struct FusedEvents { hipEvent_t fork = nullptr, ctx_ready = nullptr, done = nullptr; };

struct vla_step_plan {
  // deep copies of the host-side descriptors
  vla_vit vit{};
  bool has_vit = false;
  std::vector<vla_vit_layer> vit_layers;
  vla_backbone bb{};
  std::vector<vla_block_weights> bb_layers;
  vla_dit dit{};
  std::vector<vla_dit_layer> dit_layers;
  const void* w_proj = nullptr; const float* s_proj = nullptr; const float* b_proj = nullptr;
  vla_step_shape shape{};
  vla_step_io io{};
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int nodes = 0;
  std::vector<LaunchRec> recs;   // the captured launches, in order
  // Split-K and phase counters of the plan's own shape. Every kernel leaves
  // the counters it uses at zero, so a pass can start without clearing them
  // only when the last pass on this workspace had the same layout.
  unsigned* cnt = nullptr;
  int ncnt = 0;
  vla_step_shape zeroed{};       // layout whose counters are known to be zero
  bool zeroed_valid = false;
  // graphs of other shapes (vla_step_run_shape), least recently used evicted
  struct Entry {
    vla_step_shape shape{};
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int nodes = 0;
    unsigned* cnt = nullptr;
    int ncnt = 0;
    uint64_t used = 0;
  };
  std::vector<Entry> cache;
  uint64_t tick = 0;
  vla_step_cache_stats stats{};
  int64_t cycles = 0;            // passes run (eager or replayed)
  // V-AEFusion plans (n_stale >= 0): the action branch's stream, the
  // cycle's events, and one graph per parity of the cycle count
  int n_stale = -1;
  hipStream_t aux = nullptr;
  FusedEvents fev{};
  hipGraph_t fgraph[2] = {nullptr, nullptr};
  hipGraphExec_t fexec[2] = {nullptr, nullptr};
};

namespace {

// Vision encoder, backbone with final norm and projector of one step: the
// context rows the action expert attends to.
vla_status vlm_sched(Ctx& c, const vla_step_plan& P, const vla_step_shape& sh, uint16_t*& ctx, int& S) {
  const vla_block_cfg& cfg = P.bb.cfg;
  const int H = cfg.hidden;
  const bool vit = P.has_vit && sh.n_images > 0;
  int n_vis = 0;
  if (vit) {
    const int grid = P.vit.cfg.image / P.vit.cfg.patch;
    n_vis = sh.n_images * (grid * grid) / (P.vit.cfg.merge * P.vit.cfg.merge);
  }
  S = n_vis + sh.n_text;
  BackboneBufs b = take_backbone_bufs(c, cfg, S);
  uint16_t* hid = c.take<uint16_t>((size_t)S * H);
  ctx = c.take<uint16_t>((size_t)S * P.dit.cfg.ctx_dim);
  if (vit) VLA_TRY(sched_vit(c, P.vit, P.io.images, sh.n_images, b.xs.x, H, nullptr));
  c.label = "llm.stage";
  VLA_TRY(stage_stream(c, b.xs, S, H, P.io.text, 0, n_vis, S));
  VLA_TRY(sched_layers(c, cfg, P.bb.layers, P.bb.n_layers, b, S));
  c.label = "llm.final_norm";
  VLA_TRY(rmsnorm_out(c, b.xs.x, H, S, H, b.xs.rs, P.bb.final_norm, cfg.eps, hid, H, 0));
  c.label = "llm.hidden_out";
  if (P.io.hidden_out) VLA_TRY(rmsnorm_out(c, b.xs.x, H, S, H, b.xs.rs, P.bb.final_norm, cfg.eps, P.io.hidden_out, H, 0));
  {  // projector to the action expert's context width
    c.label = "proj";
    GemmArgs a = gargs();
    a.M = S; a.N = P.dit.cfg.ctx_dim; a.K = H;
    a.a = hid; a.lda = H;
    a.w = P.w_proj; a.ldw = H; a.wscale = P.s_proj; a.bias = P.b_proj;
    a.c = ctx; a.ldc = P.dit.cfg.ctx_dim;
    VLA_TRY(gemm(c, a, {cfg.wdtype, A_BF16, E_STORE}));
  }
  return VLA_OK;
}

// The sampler's buffers and clearing fills come first: a layer kernel that
// timed out in the previous pass may have left phase counters set in the
// counter array the VLM's split-K GEMMs share, and the fills reset them
// before any GEMM of this pass runs.
vla_status step_sched(Ctx& c, const vla_step_plan& P, const vla_step_shape& sh) {
  const int grid = P.has_vit ? P.vit.cfg.image / P.vit.cfg.patch : 0;
  const int n_vis = P.has_vit && sh.n_images > 0 ? sh.n_images * grid * grid / (P.vit.cfg.merge * P.vit.cfg.merge) : 0;
  DitIO io{nullptr, n_vis + sh.n_text, P.io.noise, sh.chunk, sh.action_dim, sh.steps, P.io.actions, P.io.velocities};
  DitState ds;
  VLA_TRY(dit_begin(c, P.dit, io, ds));
  uint16_t* ctx = nullptr;
  int S = 0;
  VLA_TRY(vlm_sched(c, P, sh, ctx, S));
  io.ctx = ctx;
  uint16_t* ckv = c.take<uint16_t>((size_t)io.ctx_len * P.dit.cfg.layers * 2 * P.dit.cfg.hidden);
  uint16_t* vt = ds.stack ? c.take<uint16_t>(dit_vt_elems(P.dit.cfg, io.ctx_len)) : nullptr;
  VLA_TRY(dit_conditioning(c, P.dit, io, ds));
  VLA_TRY(dit_cross_kv(c, P.dit, io.ctx, io.ctx_len, ckv, vt, ds.stack));
  VLA_TRY(dit_in_proj(c, P.dit, io, ds));
  return dit_steps(c, P.dit, io, ds, ckv, vt, 0, io.K);
}

// One V-AEFusion cycle on two contexts. `cv` (the caller's stream) runs the
// vision encoder, backbone, projector and the cross-attention K/V of this
// cycle into ckv[parity]; `ca` (the action branch) computes the conditioning,
// the input projection and the first n_stale Euler steps against ckv[parity^1],
// the previous cycle's, while the VLM runs, then the remaining steps against
// ckv[parity] once it is ready. Both cross-K/V buffers come first in the
// layout, so every cycle finds them at the same addresses.
vla_status fused_sched(Ctx& cv, Ctx& ca, const vla_step_plan& P, const vla_step_shape& sh, int n_stale, int parity,
                       const FusedEvents* ev, bool clear) {
  const vla_dit_cfg& cf = P.dit.cfg;
  const int grid = P.has_vit ? P.vit.cfg.image / P.vit.cfg.patch : 0;
  const int n_vis = P.has_vit && sh.n_images > 0 ? sh.n_images * grid * grid / (P.vit.cfg.merge * P.vit.cfg.merge) : 0;
  const int C = n_vis + sh.n_text;
  const size_t ckv_elems = (size_t)C * cf.layers * 2 * cf.hidden;
  uint16_t* ckv2 = cv.take<uint16_t>(2 * ckv_elems);
  uint16_t* cur = ckv2 ? ckv2 + (size_t)parity * ckv_elems : nullptr;
  uint16_t* prev = ckv2 ? ckv2 + (size_t)(parity ^ 1) * ckv_elems : nullptr;
  // the layer kernel's transposed values, double-buffered the same way
  const size_t vt_elems = dit_stack_ok(cf, sh.chunk, cu_count()) ? dit_vt_elems(cf, C) : 0;
  uint16_t* vt2 = vt_elems ? cv.take<uint16_t>(2 * vt_elems) : nullptr;
  uint16_t* cur_vt = vt2 ? vt2 + (size_t)parity * vt_elems : nullptr;
  uint16_t* prev_vt = vt2 ? vt2 + (size_t)(parity ^ 1) * vt_elems : nullptr;
  const bool live = !cv.plan;
  if (live) {
    VLA_HIP(hipEventRecord(ev->fork, cv.st));
    VLA_HIP(hipStreamWaitEvent(ca.st, ev->fork, 0));
  }
  if (clear) { VLA_TRY(zero_counters(cv)); VLA_TRY(zero_counters(ca)); }
  DitIO io{nullptr, C, P.io.noise, sh.chunk, sh.action_dim, sh.steps, P.io.actions, P.io.velocities};
  DitState ds;
  VLA_TRY(dit_begin(ca, P.dit, io, ds));
  VLA_TRY(dit_conditioning(ca, P.dit, io, ds));
  VLA_TRY(dit_in_proj(ca, P.dit, io, ds));
  // the stale steps share the GPU with the VLM: the layer kernel takes the
  // fewest workgroups it can run on, leaving the other compute units free
  const int g_all = ds.G;
  if (ds.stack) {
    int g = g_all;
    while (g > 1 && dit_stack_ok(cf, sh.chunk, g - 16)) g -= 16;
    ds.G = g;
  }
  VLA_TRY(dit_steps(ca, P.dit, io, ds, prev, prev_vt, 0, n_stale));
  ds.G = g_all;
  uint16_t* ctx = nullptr;
  int S = 0;
  VLA_TRY(vlm_sched(cv, P, sh, ctx, S));
  VLA_TRY(dit_cross_kv(cv, P.dit, ctx, S, cur, cur_vt, vt_elems > 0));
  if (live) {
    VLA_HIP(hipEventRecord(ev->ctx_ready, cv.st));
    VLA_HIP(hipStreamWaitEvent(ca.st, ev->ctx_ready, 0));
  }
  VLA_TRY(dit_steps(ca, P.dit, io, ds, cur, cur_vt, n_stale, sh.steps));
  if (live) {
    VLA_HIP(hipEventRecord(ev->done, ca.st));
    VLA_HIP(hipStreamWaitEvent(cv.st, ev->done, 0));
  }
  return VLA_OK;
}

// Workspace of a fused plan: [VLM buffers][action buffers][VLM scratch]
// [action scratch]; each branch has its own split-K scratch and counters.
struct FusedLayout {
  size_t off_b = 0, scr_a = 0, scr_b = 0, need = 0;
  Ctx a0, b0;   // plan passes: sizes and scratch needs of each branch
};

vla_status fused_layout(const vla_step_plan& P, FusedLayout& L) {
  L.a0.plan = true;
  L.b0.plan = true;
  VLA_TRY(fused_sched(L.a0, L.b0, P, P.shape, 0, 0, nullptr, false));
  size_t off = align_up(L.a0.off, 256);
  L.off_b = off;
  off += align_up(L.b0.off, 256);
  Ctx t;
  t.plan = true; t.off = off;
  t.take_scratch(L.a0);
  L.scr_a = off;
  off = align_up(t.off, 256);
  Ctx u;
  u.plan = true; u.off = off - L.off_b;
  L.scr_b = u.off;
  u.take_scratch(L.b0);
  L.need = L.off_b + u.off;
  return VLA_OK;
}

// Both branches report into the workspace's status words (only the action
// branch runs the DiT layer kernel).
void fused_ctxs(const vla_step_plan& P, const FusedLayout& L, hipStream_t sv, hipStream_t sa, Ctx& cv, Ctx& ca) {
  cv.plan = false; cv.base = (char*)P.ws; cv.cap = P.ws_bytes; cv.st = sv;
  cv.status = ca.status = (int*)P.ws;
  cv.off = L.scr_a; cv.take_scratch(L.a0); cv.off = STATUS_BYTES;
  ca.plan = false; ca.base = (char*)P.ws + L.off_b; ca.cap = P.ws_bytes - L.off_b; ca.st = sa;
  ca.off = L.scr_b; ca.take_scratch(L.b0); ca.off = STATUS_BYTES;
}

vla_status check_step(const vla_model* m, const vla_step_shape* s) {
  if (!m || !s) return fail(VLA_ERR_INVALID_ARG, "null model/shape");
  VLA_TRY(check_backbone(m->backbone));
  if (m->backbone->cfg.adtype != VLA_BF16) return fail(VLA_ERR_UNSUPPORTED, "step: backbone activations must be bf16");
  if (!m->backbone->final_norm) return fail(VLA_ERR_INVALID_ARG, "step: backbone final_norm required");
  VLA_TRY(check_dit(m->dit));
  if (m->dit->cfg.wdtype != m->backbone->cfg.wdtype) return fail(VLA_ERR_UNSUPPORTED, "step: backbone and DiT weight dtypes differ");
  if (!m->w_proj || !m->b_proj) return fail(VLA_ERR_INVALID_ARG, "step: null projector");
  if (scaled8(m->backbone->cfg.wdtype) && !m->s_proj) return fail(VLA_ERR_INVALID_ARG, "step: 8-bit projector needs scales");
  if (s->n_images < 0 || s->n_text < 0) return fail(VLA_ERR_SHAPE, "step: negative token counts");
  if (s->n_images > 0) {
    VLA_TRY(check_vit(m->vit));
    if (m->vit->cfg.out_dim != m->backbone->cfg.hidden) return fail(VLA_ERR_SHAPE, "step: vit out_dim != backbone hidden");
    if (s->n_images > 16) return fail(VLA_ERR_SHAPE, "step: n_images %d > 16", s->n_images);
  }
  int n_vis = 0;
  if (s->n_images > 0) {
    int g = m->vit->cfg.image / m->vit->cfg.patch;
    n_vis = s->n_images * g * g / (m->vit->cfg.merge * m->vit->cfg.merge);
  }
  int S = n_vis + s->n_text;
  if (S < 1 || S > 4096) return fail(VLA_ERR_SHAPE, "step: sequence %d outside [1, 4096]", S);
  VLA_TRY(check_dit_call(m->dit, S, s->chunk, s->action_dim, s->steps));
  return VLA_OK;
}

void fill_plan(vla_step_plan& P, const vla_model* m, const vla_step_shape* s) {
  P.shape = *s;
  P.has_vit = s->n_images > 0;
  if (P.has_vit) {
    P.vit = *m->vit;
    P.vit_layers.assign(m->vit->layers, m->vit->layers + m->vit->cfg.layers);
    P.vit.layers = P.vit_layers.data();
  }
  P.bb = *m->backbone;
  P.bb_layers.assign(m->backbone->layers, m->backbone->layers + m->backbone->n_layers);
  P.bb.layers = P.bb_layers.data();
  P.dit = *m->dit;
  P.dit_layers.assign(m->dit->layers, m->dit->layers + m->dit->cfg.layers);
  P.dit.layers = P.dit_layers.data();
  P.w_proj = m->w_proj; P.s_proj = m->s_proj; P.b_proj = m->b_proj;
}

}  // namespace

extern "C" {

vla_status vla_quantize_rows(const void* x, int32_t x_dtype, int32_t code_dtype, int32_t rows, int32_t K, int32_t ldx,
                             void* codes, int32_t ldc, float* scales, hipStream_t stream) {
  if (!x || !codes || !scales) return fail(VLA_ERR_INVALID_ARG, "quantize rows: null pointer");
  if (x_dtype != VLA_BF16 && x_dtype != VLA_F32) return fail(VLA_ERR_UNSUPPORTED, "quantize rows: input dtype %d", x_dtype);
  if (!scaled8(code_dtype)) return fail(VLA_ERR_UNSUPPORTED, "quantize rows: code dtype %d", code_dtype);
  if (rows < 0 || K < 8 || K > 16384 || K % 8 || ldx < K || ldx % 8 || ldc < K || ldc % 8)
    return fail(VLA_ERR_SHAPE, "quantize rows: K %d (a multiple of 8 in [8, 16384]) with pitches %d, %d", K, ldx, ldc);
  if (rows == 0) return VLA_OK;
  Ctx c;
  c.plan = false; c.st = stream;
  c.label = "quantize_rows";
  return quant_rows(c, x, x_dtype == VLA_F32 ? 1 : 0, ldx, rows, K, (uint8_t*)codes, ldc, scales,
                    code_dtype == VLA_INT8 ? 1 : 0);
}

size_t vla_step_workspace_bytes(const vla_model* model, const vla_step_shape* shape) {
  if (check_step(model, shape) != VLA_OK) return 0;
  vla_step_plan P;
  fill_plan(P, model, shape);
  size_t need = 0;
  if (two_pass(nullptr, 0, nullptr, &need, [&](Ctx& c) { return step_sched(c, P, P.shape); }) != VLA_OK) return 0;
  return need;
}

vla_status vla_step_plan_create(const vla_model* model, const vla_step_shape* shape, const vla_step_io* io, void* ws,
                                size_t ws_bytes, vla_step_plan** out) {
  if (!out) return fail(VLA_ERR_INVALID_ARG, "null plan out pointer");
  *out = nullptr;
  VLA_TRY(check_step(model, shape));
  if (!io || !io->text || !io->noise || !io->actions || (shape->n_images > 0 && !io->images))
    return fail(VLA_ERR_INVALID_ARG, "step io: null buffer");
  vla_step_plan* P = new vla_step_plan();
  fill_plan(*P, model, shape);
  P->io = *io;
  size_t need = 0;
  vla_status s = two_pass(nullptr, 0, nullptr, &need, [&](Ctx& c) { return step_sched(c, *P, P->shape); });
  if (s != VLA_OK) { delete P; return s; }
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) { delete P; return fail(VLA_ERR_INVALID_ARG, "workspace null or not 256-byte aligned"); }
  if (ws_bytes < need) { delete P; return fail(VLA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need); }
  P->ws = ws;
  P->ws_bytes = ws_bytes;
  *out = P;
  return VLA_OK;
}

size_t vla_step_fused_workspace_bytes(const vla_model* model, const vla_step_shape* shape) {
  if (check_step(model, shape) != VLA_OK) return 0;
  vla_step_plan P;
  fill_plan(P, model, shape);
  FusedLayout L;
  if (fused_layout(P, L) != VLA_OK) return 0;
  return L.need;
}

vla_status vla_step_plan_create_fused(const vla_model* model, const vla_step_shape* shape, const vla_step_io* io,
                                      int32_t n_stale, void* ws, size_t ws_bytes, vla_step_plan** out) {
  if (!out) return fail(VLA_ERR_INVALID_ARG, "null plan out pointer");
  *out = nullptr;
  VLA_TRY(check_step(model, shape));
  if (n_stale < 0 || n_stale > shape->steps) return fail(VLA_ERR_SHAPE, "n_stale %d outside [0, %d]", n_stale, shape->steps);
  if (!io || !io->text || !io->noise || !io->actions || (shape->n_images > 0 && !io->images))
    return fail(VLA_ERR_INVALID_ARG, "step io: null buffer");
  vla_step_plan* P = new vla_step_plan();
  fill_plan(*P, model, shape);
  P->io = *io;
  P->n_stale = n_stale;
  FusedLayout L;
  vla_status s = fused_layout(*P, L);
  if (s != VLA_OK) { delete P; return s; }
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) { delete P; return fail(VLA_ERR_INVALID_ARG, "workspace null or not 256-byte aligned"); }
  if (ws_bytes < L.need) { delete P; return fail(VLA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.need); }
  P->ws = ws;
  P->ws_bytes = ws_bytes;
  *out = P;
  return VLA_OK;
}

}  // extern "C"

namespace {

bool same_shape(const vla_step_shape& a, const vla_step_shape& b) {
  return a.n_images == b.n_images && a.n_text == b.n_text && a.chunk == b.chunk && a.action_dim == b.action_dim &&
         a.steps == b.steps;
}

// A shape the plan's buffers can serve: every count at most the plan's
// (inputs and outputs are used as packed prefixes), the same action width,
// and a workspace need that fits what the plan was given.
vla_status check_sub_shape(const vla_step_plan& P, const vla_step_shape& s) {
  vla_model m{P.has_vit ? &P.vit : nullptr, &P.bb, P.w_proj, P.s_proj, P.b_proj, &P.dit};
  VLA_TRY(check_step(&m, &s));
  const vla_step_shape& M = P.shape;
  if (s.n_images > M.n_images || s.n_text > M.n_text || s.chunk > M.chunk || s.steps > M.steps)
    return fail(VLA_ERR_SHAPE, "step shape (%d images, %d text, chunk %d, %d steps) exceeds the plan's (%d, %d, %d, %d)",
                s.n_images, s.n_text, s.chunk, s.steps, M.n_images, M.n_text, M.chunk, M.steps);
  if (s.action_dim != M.action_dim)
    return fail(VLA_ERR_SHAPE, "step action_dim %d != the plan's %d", s.action_dim, M.action_dim);
  size_t need = 0;
  VLA_TRY(two_pass(nullptr, 0, nullptr, &need, [&](Ctx& c) { return step_sched(c, P, s); }));
  if (need > P.ws_bytes) return fail(VLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required by this shape", P.ws_bytes, need);
  return VLA_OK;
}

struct Captured {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int nodes = 0;
  unsigned* cnt = nullptr;
  int ncnt = 0;
};

// Record one pass of shape `sh` into a graph (nothing runs). The counters
// must be zero when the graph starts; the caller arranges that.
vla_status capture_pass(const vla_step_plan& P, const vla_step_shape& sh, std::vector<LaunchRec>* recs, Captured& out) {
  hipStream_t cs = nullptr;
  VLA_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  vla_status s = VLA_OK;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) { (void)hipStreamDestroy(cs); return fail(VLA_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e)); }
  {
    Ctx p0;
    p0.plan = true;
    s = step_sched(p0, P, sh);
    if (s == VLA_OK) {
      size_t fixed = p0.off;
      Ctx c;
      c.plan = false; c.base = (char*)P.ws; c.cap = P.ws_bytes; c.st = cs;
      c.status = (int*)P.ws;
      c.off = fixed;
      c.take_scratch(p0);
      c.off = STATUS_BYTES;
      if (recs) recs->clear();
      c.recs = recs;
      s = step_sched(c, P, sh);
      out.nodes = c.kernels;
      out.cnt = c.cnt_tile;
      out.ncnt = (int)(c.need_tiles + 1);
    }
  }
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (s != VLA_OK) { if (g) (void)hipGraphDestroy(g); return s; }
  if (e != hipSuccess) return fail(VLA_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) { (void)hipGraphDestroy(g); return fail(VLA_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e)); }
  out.graph = g;
  out.exec = ex;
  return VLA_OK;
}

// Eager pass of shape `sh` (clears that layout's counters first).
vla_status run_eager(vla_step_plan& P, const vla_step_shape& sh, hipStream_t stream) {
  P.zeroed_valid = false;
  VLA_TRY(two_pass(P.ws, P.ws_bytes, stream, nullptr, [&](Ctx& c) { return step_sched(c, P, sh); }));
  P.zeroed = sh;
  P.zeroed_valid = true;
  return VLA_OK;
}

// Before a graph of shape `sh` starts: when the last pass on the workspace
// had another layout, its buffers may cover this layout's counters, so clear
// them with a fill kernel on the stream.
vla_status ready_counters(vla_step_plan& P, const vla_step_shape& sh, unsigned* cnt, int ncnt, hipStream_t stream) {
  if (P.zeroed_valid && same_shape(P.zeroed, sh)) return VLA_OK;
  Ctx c;
  c.plan = false; c.st = stream;
  unsigned z = 0;
  c.label = "fill";
  VLA_TRY(launch(c, k_fill_ref(), dim3((ncnt + 255) / 256), dim3(256), 0, {arg(cnt), arg(z), arg(ncnt)}));
  P.zeroed = sh;
  P.zeroed_valid = true;
  return VLA_OK;
}

// The action branch's stream and the cycle's events (default priority),
// made on the first pass of a fused plan and kept until it is destroyed.
vla_status fused_ready(vla_step_plan& P) {
  if (!P.aux) VLA_HIP(hipStreamCreateWithFlags(&P.aux, hipStreamNonBlocking));
  hipEvent_t* evs[3] = {&P.fev.fork, &P.fev.ctx_ready, &P.fev.done};
  for (hipEvent_t* e : evs)
    if (!*e) VLA_HIP(hipEventCreateWithFlags(e, hipEventDisableTiming));
  return VLA_OK;
}

// One eager cycle of a fused plan (the first cycle has no previous context:
// none of its steps is stale).
vla_status run_fused(vla_step_plan& P, hipStream_t stream) {
  VLA_TRY(fused_ready(P));
  FusedLayout L;
  VLA_TRY(fused_layout(P, L));
  Ctx cv, ca;
  fused_ctxs(P, L, stream, P.aux, cv, ca);
  const int n = P.cycles == 0 ? 0 : P.n_stale;
  VLA_TRY(fused_sched(cv, ca, P, P.shape, n, (int)(P.cycles & 1), &P.fev, true));
  P.cycles++;
  return VLA_OK;
}

// Record the fused cycle of one parity into a graph (nothing runs): the
// action branch forks from the capturing stream and joins it again.
vla_status capture_fused(vla_step_plan& P, int parity, std::vector<LaunchRec>* recs, hipGraph_t& g_out,
                         hipGraphExec_t& ex_out, int& nodes) {
  FusedLayout L;
  VLA_TRY(fused_layout(P, L));
  hipStream_t cs = nullptr;
  VLA_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) { (void)hipStreamDestroy(cs); return fail(VLA_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e)); }
  Ctx cv, ca;
  fused_ctxs(P, L, cs, P.aux, cv, ca);
  if (recs) recs->clear();
  cv.recs = recs; ca.recs = recs;
  vla_status s = fused_sched(cv, ca, P, P.shape, P.n_stale, parity, &P.fev, false);
  nodes = cv.kernels + ca.kernels;
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (s != VLA_OK) { if (g) (void)hipGraphDestroy(g); return s; }
  if (e != hipSuccess) return fail(VLA_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) { (void)hipGraphDestroy(g); return fail(VLA_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e)); }
  g_out = g;
  ex_out = ex;
  return VLA_OK;
}

bool captured(const vla_step_plan* p) { return p->exec || p->fexec[0]; }

void drop(vla_step_plan::Entry& en) {
  if (en.exec) (void)hipGraphExecDestroy(en.exec);
  if (en.graph) (void)hipGraphDestroy(en.graph);
  en.exec = nullptr; en.graph = nullptr;
}

}  // namespace

extern "C" {

vla_status vla_step_run(vla_step_plan* plan, hipStream_t stream) {
  if (!plan) return fail(VLA_ERR_INVALID_ARG, "null plan");
  if (plan->n_stale >= 0) return run_fused(*plan, stream);
  VLA_TRY(run_eager(*plan, plan->shape, stream));
  plan->cycles++;
  return VLA_OK;
}

vla_status vla_step_capture(vla_step_plan* plan, hipStream_t stream) {
  if (!plan) return fail(VLA_ERR_INVALID_ARG, "null plan");
  if (captured(plan)) return fail(VLA_ERR_STATE, "plan already captured");
  // warm-up pass; it leaves the counters at zero, so the captured pass
  // launches no clearing node
  VLA_TRY(vla_step_run(plan, stream));
  VLA_HIP(hipStreamSynchronize(stream));
  if (plan->n_stale >= 0) {
    for (int p = 0; p < 2; p++) {
      vla_status s = capture_fused(*plan, p, p == 0 ? &plan->recs : nullptr, plan->fgraph[p], plan->fexec[p], plan->nodes);
      if (s != VLA_OK) {
        if (plan->fexec[0]) (void)hipGraphExecDestroy(plan->fexec[0]);
        if (plan->fgraph[0]) (void)hipGraphDestroy(plan->fgraph[0]);
        plan->fexec[0] = nullptr; plan->fgraph[0] = nullptr;
        return s;
      }
    }
    return VLA_OK;
  }
  Captured cp;
  VLA_TRY(capture_pass(*plan, plan->shape, &plan->recs, cp));
  plan->graph = cp.graph;
  plan->exec = cp.exec;
  plan->nodes = cp.nodes;
  plan->cnt = cp.cnt;
  plan->ncnt = cp.ncnt;
  return VLA_OK;
}

vla_status vla_step_replay(vla_step_plan* plan, hipStream_t stream) {
  if (!plan) return fail(VLA_ERR_INVALID_ARG, "null plan");
  if (!captured(plan)) return fail(VLA_ERR_STATE, "plan not captured");
  if (plan->n_stale >= 0) {
    VLA_HIP(hipGraphLaunch(plan->fexec[plan->cycles & 1], stream));
    plan->cycles++;
    return VLA_OK;
  }
  VLA_TRY(ready_counters(*plan, plan->shape, plan->cnt, plan->ncnt, stream));
  VLA_HIP(hipGraphLaunch(plan->exec, stream));
  plan->cycles++;
  return VLA_OK;
}

vla_status vla_step_run_shape(vla_step_plan* plan, const vla_step_shape* shape, hipStream_t stream) {
  if (!plan || !shape) return fail(VLA_ERR_INVALID_ARG, "null plan/shape");
  if (plan->n_stale >= 0) return fail(VLA_ERR_UNSUPPORTED, "a fused plan runs its own shape only");
  const vla_step_shape sh = *shape;
  plan->tick++;
  // shapes already captured were validated when they were first seen
  if (plan->exec && same_shape(sh, plan->shape)) {
    VLA_TRY(vla_step_replay(plan, stream));   // counts the cycle
    plan->stats.hits++;
    return VLA_OK;
  }
  for (auto& en : plan->cache) {
    if (!same_shape(en.shape, sh)) continue;
    VLA_TRY(ready_counters(*plan, sh, en.cnt, en.ncnt, stream));
    VLA_HIP(hipGraphLaunch(en.exec, stream));
    en.used = plan->tick;
    plan->stats.hits++;
    plan->cycles++;
    return VLA_OK;
  }
  // miss: an eager pass produces this call's outputs, then the shape is
  // captured for the next calls
  VLA_TRY(check_sub_shape(*plan, sh));
  VLA_TRY(run_eager(*plan, sh, stream));
  plan->cycles++;
  VLA_HIP(hipStreamSynchronize(stream));
  Captured cp;
  VLA_TRY(capture_pass(*plan, sh, nullptr, cp));
  plan->stats.misses++;
  if ((int)plan->cache.size() >= VLA_STEP_GRAPH_CACHE) {
    auto lru = std::min_element(plan->cache.begin(), plan->cache.end(),
                                [](const vla_step_plan::Entry& x, const vla_step_plan::Entry& y) { return x.used < y.used; });
    drop(*lru);
    plan->cache.erase(lru);
    plan->stats.evictions++;
  }
  vla_step_plan::Entry en;
  en.shape = sh;
  en.graph = cp.graph; en.exec = cp.exec; en.nodes = cp.nodes;
  en.cnt = cp.cnt; en.ncnt = cp.ncnt;
  en.used = plan->tick;
  plan->cache.push_back(en);
  plan->stats.entries = (int32_t)plan->cache.size();
  return VLA_OK;
}

vla_status vla_step_cache_info(const vla_step_plan* plan, vla_step_cache_stats* out) {
  if (!plan || !out) return fail(VLA_ERR_INVALID_ARG, "null plan/out");
  *out = plan->stats;
  out->entries = (int32_t)plan->cache.size();
  return VLA_OK;
}

int32_t vla_step_graph_nodes(const vla_step_plan* plan) { return plan && captured(plan) ? plan->nodes : 0; }

int64_t vla_step_cycles(const vla_step_plan* plan) { return plan ? plan->cycles : 0; }

vla_status vla_step_status(vla_step_plan* plan, hipStream_t stream) {
  if (!plan) return fail(VLA_ERR_INVALID_ARG, "null plan");
  const vla_status s = vla_workspace_status(plan->ws, stream);
  // a timed-out layer kernel leaves its counters set: clear them before the next graph
  if (s == VLA_ERR_TIMEOUT) plan->zeroed_valid = false;
  return s;
}

const char* vla_step_kernel_label(const vla_step_plan* plan, int32_t index) {
  if (!plan || index < 0 || index >= (int32_t)plan->recs.size()) return nullptr;
  return plan->recs[index].label.c_str();
}

vla_status vla_step_launch_kernel(vla_step_plan* plan, int32_t index, hipStream_t stream) {
  if (!plan) return fail(VLA_ERR_INVALID_ARG, "null plan");
  if (!captured(plan)) return fail(VLA_ERR_STATE, "plan not captured");
  if (index < 0 || index >= (int32_t)plan->recs.size()) return fail(VLA_ERR_INVALID_ARG, "kernel index %d out of range", index);
  if (plan->n_stale < 0) VLA_TRY(ready_counters(*plan, plan->shape, plan->cnt, plan->ncnt, stream));
  LaunchRec& r = plan->recs[index];
  void* ptrs[16];
  for (size_t i = 0; i < r.args.size(); i++) ptrs[i] = r.args[i].data();
  VLA_HIP(hipLaunchKernel(r.fn, r.grid, r.block, ptrs, r.smem, stream));
  return VLA_OK;
}

void vla_step_plan_destroy(vla_step_plan* plan) {
  if (!plan) return;
  for (auto& en : plan->cache) drop(en);
  if (plan->exec) (void)hipGraphExecDestroy(plan->exec);
  if (plan->graph) (void)hipGraphDestroy(plan->graph);
  for (int p = 0; p < 2; p++) {
    if (plan->fexec[p]) (void)hipGraphExecDestroy(plan->fexec[p]);
    if (plan->fgraph[p]) (void)hipGraphDestroy(plan->fgraph[p]);
  }
  if (plan->fev.fork) (void)hipEventDestroy(plan->fev.fork);
  if (plan->fev.ctx_ready) (void)hipEventDestroy(plan->fev.ctx_ready);
  if (plan->fev.done) (void)hipEventDestroy(plan->fev.done);
  if (plan->aux) (void)hipStreamDestroy(plan->aux);
  delete plan;
}

}  // extern "C"
