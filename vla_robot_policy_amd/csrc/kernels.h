// Host-visible lookup of the kernel instantiations compiled into libvla.
#pragma once
#include <stddef.h>

namespace vla {

struct KernelRef {
  const void* fn;
  int smem;     // dynamic LDS bytes
  int threads;  // workgroup size
};

// GEMM: one lookup per weight type; am / em from gemm.h, tile (mb, wn, wk,
// nbw), u k-steps per chunk, ac = compensated (hi + lo) bf16 activations,
// aq = activation chunks in flight (2 or 4), pk = packed weights.
struct GemmPick {
  int am, em, mb, wn, wk, nbw, u, ac, aq, pk;
};
bool gemm_lookup_f32(const GemmPick& g, KernelRef* out);
bool gemm_lookup_bf16(const GemmPick& g, KernelRef* out);
bool gemm_lookup_fp8(const GemmPick& g, KernelRef* out);
bool gemm_lookup_int8(const GemmPick& g, KernelRef* out);

// Attention: f32 (1) or bf16 (0) elements, padded head dim, heads per workgroup.
// the attention kernel and the merge of its key-split partials
bool attn_lookup(int f32, int dp, int hpw, int ks, KernelRef* out, KernelRef* merge);

// Misc kernels.
const void* k_fill_ref();
const void* k_stage_rows_ref();
const void* k_rmsnorm_out_ref();
const void* k_time_embed_ref();
const void* k_rope_table_ref();
const void* k_pack_weights_ref();
const void* k_ctx_vt_ref();
const void* k_patch_rows_ref();
const void* k_dit_table_ref();
const void* k_norm_rows_ref();
const void* k_quant_rows_ref();
const void* k_convert_rows_ref();
bool euler_tail_lookup(int wt, KernelRef* out);

// Persistent DiT layer kernel (wt 1 = bf16, 2 = fp8) for width D.
bool dit_layer_lookup(int wt, int D, KernelRef* out);

}  // namespace vla
