/*
 * libvla — batch-1 forward pass of a Vision-Language-Action policy on one
 * AMD Instinct MI355X (gfx950): ViT encoder + 2x2 merger -> pre-norm GQA
 * decoder backbone (prefill) -> projector -> DiT action expert inside a
 * K-step flow-matching Euler loop, optionally captured as one hipGraph.
 *
 * Sources (pages, by title and section):
 *   [R]  "AI Infra如何优化VLA - 模型推理性能提升技术拆解" (StarVLA on RTX 4090):
 *        整体方案 (model structure, the ten operator types), 自研推理框架
 *        (weights handed over directly as tensors), CUDA Graph (three graphs,
 *        static I/O buffers refreshed by copy before replay), 算子开发 (RMSNorm
 *        chain, half-split RoPE), 算子融合 (fused GELU / SwiGLU MLP, fused QKV).
 *   [A]  "开源 APXInf 把 VLA 推理压到 26 毫秒": capture the whole inference
 *        graph on the first call and replay it every control cycle; FP8
 *        weights.
 *   [X]  "跨XPU平台表征视觉-语言-动作模型：机器人部署中的约束与加速": section
 *        5.3 V-AEFusion and Figure 9 (the action expert's first denoising
 *        steps run on the previous cycle's features, alongside the VLM).
 *
 * Conventions for every entry point
 *   - Activations are row-major [rows, features] (token-major). A Linear
 *     weight is row-major [N_out, K_in] (PyTorch convention, y = x W^T + b).
 *     bf16 tensors are raw bfloat16 bit patterns (uint16); fp8 tensors are
 *     OCP E4M3FN codes (uint8) with one float32 scale per output row; norm
 *     gains, biases, positional tables and modulation vectors are float32.
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned (the widest
 *     single access any kernel makes; hipMalloc and torch allocations are
 *     256-byte aligned and satisfy it), owned by the caller. The library never allocates device memory in a run, capture or
 *     replay call; scratch space is the caller's workspace (ws, ws_bytes),
 *     whose required size the matching *_workspace_bytes() returns. The
 *     workspace content need not be initialised.
 *   - Calls are asynchronous on the given stream (0 = the null stream);
 *     results are valid once the caller has synchronised that stream.
 *   - Errors: a negative vla_status; vla_last_error() returns a message
 *     for the calling thread. Nothing is launched when argument validation
 *     fails. VLA_ERR_HIP wraps a HIP runtime error (launch or graph API).
 */
#ifndef VLA_H
#define VLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VLA_ABI_VERSION 3   /* 2: vla_block_weights gained q_norm, k_norm; 3: packed weights */

typedef enum {
  VLA_OK = 0,
  VLA_ERR_INVALID_ARG = -1, /* null pointer, bad enum, misaligned buffer   */
  VLA_ERR_SHAPE = -2,       /* shape outside the supported set            */
  VLA_ERR_UNSUPPORTED = -3, /* valid but not implemented combination      */
  VLA_ERR_WORKSPACE = -4,   /* ws_bytes below the required size           */
  VLA_ERR_HIP = -5,         /* HIP runtime error                          */
  VLA_ERR_STATE = -6,       /* plan used out of order / already captured  */
  VLA_ERR_TIMEOUT = -7      /* a device-side bounded wait gave up (see vla_workspace_status) */
} vla_status;

/* VLA_INT8 ([A]: INT8 where FP8 units are missing): int8 weight codes in
 * [-127, 127] with one float32 scale per output row, like FP8_E4M3. */
typedef enum { VLA_F32 = 0, VLA_BF16 = 1, VLA_FP8_E4M3 = 2, VLA_INT8 = 3 } vla_dtype;

/* ------------------------------------------------------------------ block
 * One pre-norm decoder block ([R] 整体方案, 算子开发, 算子融合):
 *   [Q|K|V] = RMSNorm(x, attn_norm) W_qkv^T, RoPE (half-split, base
 *   rope_base, positions 0..seq-1) on Q and K, causal GQA attention (query
 *   head h reads KV head h / (n_q_heads / n_kv_heads)), h = x + O W_o^T,
 *   out = h + (SiLU(n W_gate^T) * (n W_up^T)) W_down^T with n = RMSNorm(h,
 *   mlp_norm). RMSNorm(x, g) = x / sqrt(mean(x^2) + eps) * g. No biases.
 * With flags & VLA_BLOCK_QK_NORM (QK-norm; section 算子开发 counts RMSNorm
 * calls on Q and K besides the pre-norms), every query and key head vector
 * is RMS-normalised over head_dim before RoPE: Q_h <- Q_h / sqrt(mean(Q_h^2)
 * + eps) * q_norm, K_g likewise with k_norm; it needs n_q_heads * head_dim
 * to be a multiple of 128.
 * With flags & VLA_BLOCK_A8 (W8A8; [A]: FP8 weights and activations, INT8
 * where FP8 units are missing), the input rows of the four Linears (the two
 * normalised rows, the attention output and the SwiGLU product) become 8-bit
 * codes in the weights' format with one scale per row: E4M3FN with s =
 * max|row| / 448 (nearest value, ties to the even code), or int8 with s =
 * max|row| / 127 (nearest integer, halves to even), decided from float32.
 * y = (codes . W codes^T) * s_row * s_channel, with exact code products
 * (int8: exact int32 sums on the int8 MFMA; E4M3FN: the fp8 MFMA's float32
 * accumulation, within about 1e-4 relative of exact sums at K = 1024); q,
 * k, v, the attention and the SwiGLU product stay
 * float32 until quantised. Needs FP8_E4M3 or INT8 weights, BF16 activations,
 * hidden <= 4096, and the Linear inputs (hidden, n_q_heads * head_dim,
 * intermediate) multiples of 16 and at most 16384 wide;
 * VLA_ERR_UNSUPPORTED otherwise.
 * With flags & VLA_BLOCK_PACKED, w_qkv, w_o, w_gate_up and w_down are the
 * packed copies vla_pack_weights writes of the row-major matrices above
 * (each packed on its own, N and K as listed; scales unchanged). Needs BF16,
 * FP8_E4M3 or INT8 weights without VLA_BLOCK_A8, and intermediate a
 * multiple of 16; VLA_ERR_UNSUPPORTED otherwise. Results are bitwise those
 * of the row-major weights.
 * Supported: head_dim in {64, 128}; hidden, intermediate multiples of 8
 * (of 16 for FP8_E4M3 weights); n_q_heads % n_kv_heads == 0; wdtype F32 with adtype F32, or wdtype
 * BF16 / FP8_E4M3 with adtype BF16.
 */
#define VLA_BLOCK_QK_NORM 1
#define VLA_BLOCK_A8 2
#define VLA_BLOCK_PACKED 4
typedef struct {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, intermediate;
  float rope_base, eps;
  int32_t wdtype;  /* vla_dtype of the Linear weights                  */
  int32_t adtype;  /* vla_dtype of x_in / x_out / embeddings: F32, BF16 */
  int32_t flags;   /* VLA_BLOCK_QK_NORM | VLA_BLOCK_A8 | VLA_BLOCK_PACKED */
} vla_block_cfg;

typedef struct {
  const float* attn_norm; /* [hidden]                                             */
  const void* w_qkv;      /* [(Hq + 2 Hkv) head_dim, hidden]: rows of W_q, W_k, W_v */
  const float* s_qkv;     /* fp8 only: [(Hq + 2 Hkv) head_dim]                     */
  const void* w_o;        /* [hidden, Hq head_dim]                                 */
  const float* s_o;
  const float* mlp_norm;  /* [hidden]                                             */
  const void* w_gate_up;  /* [2 intermediate, hidden]: rows of W_gate, then W_up   */
  const float* s_gate_up;
  const void* w_down;     /* [hidden, intermediate]                                */
  const float* s_down;
  const float* q_norm;    /* [head_dim], VLA_BLOCK_QK_NORM only (else ignored)     */
  const float* k_norm;    /* [head_dim], VLA_BLOCK_QK_NORM only                    */
} vla_block_weights;

/* x_in, x_out: [seq, hidden] in cfg->adtype (may alias). */
vla_status vla_block_forward(const vla_block_cfg* cfg, const vla_block_weights* w, const void* x_in, void* x_out,
                             int32_t seq, void* ws, size_t ws_bytes, hipStream_t stream);
size_t vla_block_workspace_bytes(const vla_block_cfg* cfg, int32_t seq);

/* vla_block_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same operation, arguments (minus ws,
 * ws_bytes), layouts and results as vla_block_forward; the scratch is a
 * static device array of VLA_STATIC_SCRATCH_BYTES (64 MiB) inside the
 * library, one per GPU, held from the library's load until the process
 * ends. The call allocates nothing (no hipMalloc / hipFree, no other
 * allocating routine). Every call on a GPU shares that GPU's array and
 * leaves its contents behind; each pass first zeroes the counters it needs
 * with a fill kernel, so nothing has to be cleared by the caller, but calls
 * that overlap on one GPU (other streams, other host threads) race on the
 * array: order them on one stream. Errors as vla_block_forward, and
 * VLA_ERR_WORKSPACE when vla_block_workspace_bytes(cfg, seq) exceeds the
 * array (about seq 560 for the 2560-wide bf16 block). */
#define VLA_STATIC_SCRATCH_BYTES (64u << 20)
vla_status vla_block_forward_static(const vla_block_cfg* cfg, const vla_block_weights* w, const void* x_in, void* x_out,
                                    int32_t seq, hipStream_t stream);

/* ------------------------------------------------------------------ weight packing
 * [R] 自研推理框架: weights reach the engine as ready device tensors, laid
 * out once at load time for the kernels that read them. A packed matrix
 * holds the same values as the row-major W[N, K] (pitch ldw elements),
 * regrouped so that one 64-lane wave load is one MFMA operand block: blocks
 * of 16 rows x 32 k, ordered [row block][k block] (row block nb, k block kb
 * at element offset (nb * ceil(K/32) + kb) * 512), lane l of a block holding
 * the 8 consecutive values of row 16 nb + l % 16 at k = 32 kb + 8 (l / 16)
 * .. + 7. Rows beyond N and k beyond K are zero. 8-bit scales stay per row
 * and unpacked.
 * vla_packed_bytes: size of the packed copy, ceil(N/16) * ceil(K/32) * 512
 * elements of the weight type (a multiple of 512 bytes, so packed matrices
 * placed back to back keep their alignment); 0 for an unsupported dtype
 * (only BF16, FP8_E4M3, INT8 pack) or N, K < 1.
 * vla_pack_weights: one kernel on stream, reading w (device, [N, ldw],
 * ldw >= K) and writing packed (device, vla_packed_bytes(wdtype, N, K)
 * bytes, 16-byte aligned, caller-owned, must not overlap w). Asynchronous:
 * w must stay valid until the stream reaches the kernel. Errors:
 * VLA_ERR_UNSUPPORTED (dtype), VLA_ERR_INVALID_ARG (null or misaligned
 * pointer), VLA_ERR_SHAPE (N, K < 1, ldw < K, or more than 2 GiB packed). */
size_t vla_packed_bytes(int32_t wdtype, int32_t N, int32_t K);
vla_status vla_pack_weights(int32_t wdtype, const void* w, int32_t N, int32_t K, int32_t ldw, void* packed,
                            hipStream_t stream);

/* ------------------------------------------------------------------ backbone
 * The decoder prefill ([R] 整体方案; CUDA Graph: "36 layers to the final
 * RMSNorm"): n_layers blocks over the embeddings, then RMSNorm(final_norm)
 * when final_norm is not NULL. `layers` is a HOST array of n_layers weight
 * records (device pointers inside); it is read during the call only.
 */
typedef struct {
  vla_block_cfg cfg;
  int32_t n_layers;
  const vla_block_weights* layers; /* host array [n_layers]      */
  const float* final_norm;         /* [hidden] or NULL           */
} vla_backbone;

/* embeds, hidden_out: [seq, hidden] in cfg.adtype. 1 <= seq <= 4096. */
vla_status vla_backbone_prefill(const vla_backbone* bb, const void* embeds, int32_t seq, void* hidden_out, void* ws,
                                size_t ws_bytes, hipStream_t stream);
size_t vla_backbone_workspace_bytes(const vla_backbone* bb, int32_t seq);

/* ------------------------------------------------------------------ DiT + Euler
 * The action expert ([R] 整体方案: flow-matching Euler denoising from noise).
 * With t_k = k/K and a_0 = x0:  a_{k+1} = a_k + v(a_k, t_k, ctx) / K; the
 * output is a_K. The velocity v:
 *   x = a W_in^T + b_in;  phi(t) = [cos(time_scale t w_i), sin(time_scale t
 *   w_i)], w_i = freq_base^(-i/(tdim/2)); c = W_t2 SiLU(W_t1 phi + b_t1) +
 *   b_t2;  per layer m = W_ada SiLU(c) + b_ada = 9 vectors [shift, scale,
 *   gate] x [self-attn, cross-attn, MLP]; each sublayer adds
 *   gate * f(LN(x)(1 + scale) + shift) (LN without affine, eps); self-attn
 *   is full multi-head attention over the action rows; cross-attn reads
 *   K/V = ctx W^T + b of every context row; MLP is Linear-GELU(erf)-Linear;
 *   finally v = (LN(x)(1 + scale_f) + shift_f) W_out^T + b_out with
 *   [shift_f, scale_f] = W_f SiLU(c) + b_f. Every Linear has a bias.
 * Supported: head_dim 80 or 64 (hidden = heads * head_dim); hidden, mlp,
 * tdim, ctx_dim multiples of 8 (of 16 for FP8_E4M3 weights); 1 <= chunk <= 64; 1 <= K <= 64; 1 <= ctx_len <= 4096.
 */
typedef struct {
  int32_t hidden, heads, head_dim, mlp, layers, tdim, ctx_dim;
  float eps, time_scale, freq_base;
  int32_t wdtype; /* BF16 or FP8_E4M3      */
  int32_t flags;  /* must be 0             */
} vla_dit_cfg;

typedef struct {
  const void* w_qkv; const float* s_qkv; const float* b_qkv; /* self-attn [3 hidden, hidden]: W_q, W_k, W_v rows */
  const void* w_o; const float* s_o; const float* b_o;       /* [hidden, hidden]                                */
  const void* w_cq; const float* s_cq; const float* b_cq;    /* cross-attn query [hidden, hidden]               */
  const void* w_co; const float* s_co; const float* b_co;    /* cross-attn out   [hidden, hidden]               */
  const void* w_up; const float* s_up; const float* b_up;    /* [mlp, hidden]                                   */
  const void* w_down; const float* s_down; const float* b_down; /* [hidden, mlp]                                */
} vla_dit_layer;

typedef struct {
  vla_dit_cfg cfg;
  const vla_dit_layer* layers;  /* host array [cfg.layers]                                            */
  /* per-layer tensors stacked over layers so each is one launch per policy step:              */
  const void* w_ada; const float* s_ada; const float* b_ada; /* [layers*9*hidden, hidden]                 */
  const void* w_ckv; const float* s_ckv; const float* b_ckv; /* [layers*2*hidden, ctx_dim]: per layer W_k then W_v */
  const void* w_t1; const float* s_t1; const float* b_t1;    /* [hidden, tdim]                            */
  const void* w_t2; const float* s_t2; const float* b_t2;    /* [hidden, hidden]                          */
  const void* w_f; const float* s_f; const float* b_f;       /* [2 hidden, hidden]: shift rows, scale rows */
  const void* w_in; const float* s_in; const float* b_in;    /* [hidden, action_dim]                      */
  const void* w_out; const float* s_out; const float* b_out; /* [action_dim, hidden]                      */
} vla_dit;

/* ctx: [ctx_len, ctx_dim] bf16; x0, actions_out:
 * float32 [chunk, action_dim] (may alias); velocities_out: optional float32
 * [K, chunk, action_dim] record of every v (NULL to skip). */
vla_status vla_flow_euler_sample(const vla_dit* dit, const void* ctx, int32_t ctx_len, const float* x0, int32_t chunk,
                                 int32_t action_dim, int32_t K, float* actions_out, float* velocities_out, void* ws,
                                 size_t ws_bytes, hipStream_t stream);
size_t vla_dit_workspace_bytes(const vla_dit* dit, int32_t ctx_len, int32_t chunk, int32_t action_dim, int32_t K);

/* ------------------------------------------------------------------ vision
 * ViT + merger ([R] CUDA Graph: PatchEmbed -> ViT blocks -> Merger; 算子融合:
 * GELU MLPs). Patch (r, c) of image i is token i*grid^2 + r*grid + c with
 * features in (channel, row, column) order; z = P W_pe^T + b_pe + pos; each
 * layer: z += MHA(LN(z)) W_o^T + b_o (non-causal, biased q/k/v), z += W_2
 * GELU(W_1 LN(z) + b_1) + b_2. Merger: u = LN(z; mln); merged token (R, C)
 * concatenates u of patches (2R+dy, 2C+dx) for (dy, dx) in raster order;
 * out = GELU(u W_m1^T + b_m1) W_m2^T + b_m2.
 * w_pe rows have a pitch of round_up(channels*patch^2, 8) elements; the pad
 * columns must be zero.
 * With flags & VLA_BLOCK_PACKED, every layer's w_qkv, w_o, w_up and w_down
 * are the packed copies vla_pack_weights (BF16) writes of the row-major
 * matrices below; the results are the same bits. Other flags:
 * VLA_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t image, patch, channels, hidden, heads, head_dim, mlp, layers, merge, out_dim;
  float eps;
  int32_t wdtype; /* BF16 */
  int32_t flags;  /* 0 or VLA_BLOCK_PACKED */
} vla_vit_cfg;

typedef struct {
  const float* ln1_g; const float* ln1_b;
  const void* w_qkv; const float* b_qkv;  /* [3 hidden, hidden]: W_q, W_k, W_v rows */
  const void* w_o; const float* b_o;      /* [hidden, hidden]                      */
  const float* ln2_g; const float* ln2_b;
  const void* w_up; const float* b_up;    /* [mlp, hidden]                         */
  const void* w_down; const float* b_down;/* [hidden, mlp]                         */
} vla_vit_layer;

typedef struct {
  vla_vit_cfg cfg;
  const vla_vit_layer* layers;            /* host array [cfg.layers]                  */
  const void* w_pe; const float* b_pe;    /* [hidden, pitch] (see above), [hidden]    */
  const float* pos;                       /* [grid^2, hidden]                         */
  const float* mln_g; const float* mln_b; /* [hidden]                                 */
  const void* w_m1; const float* b_m1;    /* [4 hidden, 4 hidden] (merge 2)           */
  const void* w_m2; const float* b_m2;    /* [out_dim, 4 hidden]                      */
} vla_vit;

/* images: bf16 [n_images, channels, image, image]; tokens_out: float32
 * [n_images * grid^2 / merge^2, out_dim]; vit_out: optional float32
 * [n_images * grid^2, hidden] (the encoder output before the merger). */
vla_status vla_vit_encode(const vla_vit* vit, const void* images, int32_t n_images, float* tokens_out, float* vit_out,
                          void* ws, size_t ws_bytes, hipStream_t stream);
size_t vla_vit_workspace_bytes(const vla_vit* vit, int32_t n_images);

/* W8A8 activation quantiser ([A]: FP8 or INT8 activations): each of `rows`
 * rows x[r, 0..K) (x_dtype VLA_BF16 or VLA_F32, row pitch ldx elements)
 * becomes K codes (row pitch ldc bytes) and one float32 scale s[r] =
 * max|x[r]| / qmax. code_dtype VLA_FP8_E4M3: qmax 448, codes[r, k] is
 * x[r, k] * (448 / max|x[r]|) in float32, clamped to +-448 and rounded to
 * the nearest E4M3FN value, ties to the even code; a negative value that
 * rounds to zero keeps its sign (0x80). code_dtype VLA_INT8: qmax 127, the
 * nearest integer (halves to even) clipped to +-127. A zero row gets zero
 * codes and scale 0. K a multiple of 8 in [8, 16384]; pitches multiples of
 * 8. This is the pass a VLA_BLOCK_A8 block runs on the attention output and
 * the SwiGLU product (both float32). */
vla_status vla_quantize_rows(const void* x, int32_t x_dtype, int32_t code_dtype, int32_t rows, int32_t K, int32_t ldx,
                             void* codes, int32_t ldc, float* scales, hipStream_t stream);

/* ------------------------------------------------------------------ whole step
 * The full policy step ([R] 整体方案: vision -> LLM (with projection layers)
 * -> action head; [A]: capture once, replay per control cycle): sequence =
 * [visual tokens of each image; text embeddings], backbone with final norm,
 * ctx = hidden W_proj^T + b_proj (all rows), then the Euler sampler.
 * A plan binds the model and the caller's static I/O buffers; the caller
 * refreshes the inputs in place (device copies) before each replay ([R]
 * CUDA Graph). Every pointer handed to the plan must stay valid at the same
 * address until vla_step_plan_destroy.
 */
typedef struct {
  const vla_vit* vit;           /* NULL: no vision encoder (all tokens given as text) */
  const vla_backbone* backbone; /* final_norm required                               */
  const void* w_proj; const float* s_proj; const float* b_proj; /* [ctx_dim, hidden], bias [ctx_dim] */
  const vla_dit* dit;
} vla_model;

typedef struct {
  int32_t n_images, n_text, chunk, action_dim, steps;
} vla_step_shape;

typedef struct {
  const void* images;   /* bf16 [n_images, C, image, image] or NULL when n_images == 0 */
  const void* text;     /* [n_text, hidden] in the backbone's adtype                  */
  const float* noise;   /* [chunk, action_dim]                                        */
  float* actions;       /* [chunk, action_dim]                                        */
  void* hidden_out;     /* optional [seq, hidden] copy of the backbone output (adtype) */
  float* velocities;    /* optional [steps, chunk, action_dim]                        */
} vla_step_io;

typedef struct vla_step_plan vla_step_plan;

size_t vla_step_workspace_bytes(const vla_model* model, const vla_step_shape* shape);
/* Validates, copies the host-side descriptors, and binds io and ws. Host
 * memory only; nothing is launched. */
vla_status vla_step_plan_create(const vla_model* model, const vla_step_shape* shape, const vla_step_io* io, void* ws,
                                size_t ws_bytes, vla_step_plan** out);
/* One eager pass of the step (kernel launches on `stream`). */
vla_status vla_step_run(vla_step_plan* plan, hipStream_t stream);
/* Capture one pass into a hipGraph and instantiate it (one eager warm-up
 * pass is launched first). VLA_ERR_STATE if already captured. */
vla_status vla_step_capture(vla_step_plan* plan, hipStream_t stream);
/* Replay the captured graph (VLA_ERR_STATE if not captured). After a pass of
 * another shape (vla_step_run_shape) it first clears the counters the graph
 * expects at zero, with one small fill kernel. */
vla_status vla_step_replay(vla_step_plan* plan, hipStream_t stream);
/* Kernel nodes in the captured graph (0 before capture). */
int32_t vla_step_graph_nodes(const vla_step_plan* plan);
/* Name of the operation of captured kernel `index` (0 <= index < nodes),
 * e.g. "llm.gate_up", "dit.mlp_down"; NULL when out of range. */
const char* vla_step_kernel_label(const vla_step_plan* plan, int32_t index);
/* Launch captured kernel `index` once more, on its own, on `stream` (for
 * timing one kernel with events). It reads and writes the plan's workspace
 * as in the graph, so intermediate buffers hold arbitrary values afterwards;
 * the next vla_step_run / vla_step_replay recomputes everything from the
 * inputs. Valid only after vla_step_capture. The DiT layer kernel hands QKV
 * and the cross query to its attention phases as words tagged with the
 * launch's position in the sampler run; launched again right after itself,
 * it can take its previous run's words, which hold the same values (its
 * inputs are unchanged), without waiting. To time that kernel, launch its
 * captured launches in graph order, as a replay would. */
vla_status vla_step_launch_kernel(vla_step_plan* plan, int32_t index, hipStream_t stream);

/* Shape-keyed graphs ([R] CUDA Graph: when the sequence length changes, the
 * LLM graph falls back to an eager pass and is captured again, the cached
 * length being what a call is matched against). One pass of `shape`, which
 * may be smaller than the plan's: n_images, n_text, chunk and steps at most
 * the plan's, action_dim equal to it. The plan's buffers serve as packed
 * prefixes for that shape: images [n_images, C, image, image], text
 * [n_text, hidden], noise and actions [chunk, action_dim], hidden_out
 * [seq, hidden], velocities [steps, chunk, action_dim].
 *   - A shape seen before replays its graph (the plan's own shape replays the
 *     vla_step_capture graph when there is one); asynchronous like a replay.
 *   - A new shape runs one eager pass, whose outputs are this call's, then
 *     synchronises `stream` and captures the shape into a graph (nothing of
 *     the capture runs). At most VLA_STEP_GRAPH_CACHE such graphs are kept;
 *     adding one more destroys the least recently used.
 * Every shape shares the plan's workspace, so passes of any shapes must be
 * ordered on one stream. Errors: VLA_ERR_SHAPE (outside the plan's shape),
 * VLA_ERR_WORKSPACE (the shape needs more workspace than the plan holds),
 * VLA_ERR_HIP; the cache is unchanged after an error. */
#define VLA_STEP_GRAPH_CACHE 8
vla_status vla_step_run_shape(vla_step_plan* plan, const vla_step_shape* shape, hipStream_t stream);

typedef struct {
  int32_t entries;    /* graphs held for shapes other than the plan's own      */
  int32_t hits;       /* vla_step_run_shape calls that replayed a graph         */
  int32_t misses;     /* calls that ran eagerly and captured a new shape        */
  int32_t evictions;  /* graphs destroyed to make room                          */
} vla_step_cache_stats;
vla_status vla_step_cache_info(const vla_step_plan* plan, vla_step_cache_stats* out);

/* V-AEFusion plans ([X] 5.3, Figure 9). Every pass of such a plan is one
 * control cycle c. The action expert's first n_stale Euler steps of cycle c
 * cross-attend to the context of cycle c-1 and run alongside the vision
 * encoder, backbone and projector of cycle c (a second stream in an eager
 * pass, a second branch of the captured graph); the remaining steps wait for
 * cycle c's context. The first cycle of a plan has no previous context, so
 * none of its steps is stale. 0 <= n_stale <= steps.
 *   - The workspace (vla_step_fused_workspace_bytes) holds the cross-
 *     attention K/V of the last two contexts and separate scratch for the
 *     two branches; the caller's buffers are as for vla_step_plan_create.
 *   - vla_step_run runs one cycle eagerly. vla_step_capture runs one cycle
 *     as its warm-up, then captures one graph per parity of the cycle count;
 *     vla_step_replay replays the graph of the next cycle. The first pass
 *     creates a non-blocking stream and three events (default priority),
 *     kept until vla_step_plan_destroy.
 *   - vla_step_run_shape returns VLA_ERR_UNSUPPORTED.
 * Errors as for vla_step_plan_create; VLA_ERR_SHAPE for n_stale outside
 * [0, steps]. */
size_t vla_step_fused_workspace_bytes(const vla_model* model, const vla_step_shape* shape);
vla_status vla_step_plan_create_fused(const vla_model* model, const vla_step_shape* shape, const vla_step_io* io,
                                      int32_t n_stale, void* ws, size_t ws_bytes, vla_step_plan** out);
/* Passes run by a plan so far (eager, replayed or through
 * vla_step_run_shape): the cycle count of a fused plan. */
int64_t vla_step_cycles(const vla_step_plan* plan);

void vla_step_plan_destroy(vla_step_plan* plan);

/* ------------------------------------------------------------------ status
 * Device-side failures. For chunks of at most 16 rows the action expert runs
 * one persistent kernel per DiT layer whose workgroups hand results to each
 * other through device counters and tagged words. Every such wait is bounded
 * (2^17 polls, far beyond a healthy wait of microseconds); when one gives up,
 * the kernel sets word 0 of the workspace's status block (the workspace's
 * first 256 bytes, cleared at the start of every sampler pass), fills the
 * layer's output rows with NaN and leaves, and every later layer launch of
 * the pass sees the word and leaves at once with NaN outputs. The failure is
 * therefore never a hang; it shows as NaN actions and velocities and as this
 * status. Every host call of the pass still returns VLA_OK (the calls are
 * asynchronous), so a caller that must know asks here after the pass.
 *
 * vla_workspace_status: synchronises `stream`, then reads word 0 of the
 * workspace `ws` of the last pass (vla_flow_euler_sample, or a step plan's
 * workspace): VLA_OK, or VLA_ERR_TIMEOUT when a wait gave up in that pass.
 * vla_step_status: the same for a plan's workspace; after VLA_ERR_TIMEOUT
 * the plan's next replay first clears its counters with a fill kernel.
 * The environment variable VLA_DIT_SPIN_LIMIT (a positive poll count below
 * 2^17) lowers the bound for later passes, so that the time-out path can be
 * exercised: with a limit of 1 a wait gives up after one unsuccessful poll. */
vla_status vla_workspace_status(const void* ws, hipStream_t stream);
vla_status vla_step_status(vla_step_plan* plan, hipStream_t stream);

/* ------------------------------------------------------------------ misc */
const char* vla_last_error(void);
int32_t vla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VLA_H */
