// Attention kernel instantiations. This file is compiled with MFMA
// accumulators in ordinary vector registers (-mllvm -amdgpu-mfma-vgpr-form,
// set by the build): the softmax reads every score tile the MFMAs produce
// and rescales the output tile, which would otherwise cost an
// accumulator-register move per value on a path with one wave per SIMD.
#include "attention.h"
#include "kernels.h"

namespace vla {

#define VLA_ATTN_CASE(CT, F32V, DPV, HPWV)          \
  if (f32 == F32V && dp == DPV && hpw == HPWV) {    \
    out->fn = (const void*)&k_attention<CT, DPV, HPWV>; \
    out->smem = AttnStage<CT, DPV>::SMEM; out->threads = 256; \
    if (merge) { merge->fn = (const void*)&k_attn_merge<CT, DPV, HPWV>; merge->smem = 0; merge->threads = 256; } \
    return true;                                    \
  }

bool attn_lookup(int f32, int dp, int hpw, int ks, KernelRef* out, KernelRef* merge) {
  if (ks) {   // key-split form: bf16, one head per workgroup, no merge launch
    if (f32 || hpw != 1 || (dp != 64 && dp != 128)) return false;
    out->fn = dp == 64 ? (const void*)&k_attention<__bf16, 64, 1, true> : (const void*)&k_attention<__bf16, 128, 1, true>;
    out->smem = dp == 64 ? AttnStage<__bf16, 64>::SMEM : AttnStage<__bf16, 128>::SMEM;
    out->threads = 256;
    return true;
  }
  VLA_ATTN_CASE(__bf16, 0, 64, 1) VLA_ATTN_CASE(__bf16, 0, 64, 2) VLA_ATTN_CASE(__bf16, 0, 64, 4)
  VLA_ATTN_CASE(__bf16, 0, 96, 1) VLA_ATTN_CASE(__bf16, 0, 96, 2) VLA_ATTN_CASE(__bf16, 0, 96, 4)
  VLA_ATTN_CASE(__bf16, 0, 128, 1) VLA_ATTN_CASE(__bf16, 0, 128, 2) VLA_ATTN_CASE(__bf16, 0, 128, 4)
  VLA_ATTN_CASE(float, 1, 64, 1) VLA_ATTN_CASE(float, 1, 64, 2) VLA_ATTN_CASE(float, 1, 64, 4)
  VLA_ATTN_CASE(float, 1, 128, 1) VLA_ATTN_CASE(float, 1, 128, 2) VLA_ATTN_CASE(float, 1, 128, 4)
  return false;
}

}  // namespace vla
