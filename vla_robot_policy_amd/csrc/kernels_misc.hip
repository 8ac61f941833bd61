// Attention, staging, norm, conversion and Euler-tail kernel instantiations.
#include "attention.h"
#include "kernels.h"
#include "misc.h"

namespace vla {

// x (fp32 rows) -> out rows in fp32 or bf16.
__global__ __launch_bounds__(256) void k_convert_rows(const float* x, int ldx, int M, int N, void* out, int ldo,
                                                    int out_f32) {
  int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (r >= M) return;
  for (int c = lane; c < N; c += 64) {
    float v = x[(size_t)r * ldx + c];
    if (out_f32) ((float*)out)[(size_t)r * ldo + c] = v;
    else ((uint16_t*)out)[(size_t)r * ldo + c] = f2bf(v);
  }
}

#define VLA_ATTN_CASE(CT, F32V, DPV, HPWV)          \
  if (f32 == F32V && dp == DPV && hpw == HPWV) {    \
    out->fn = (const void*)&k_attention<CT, DPV, HPWV>; \
    out->smem = AttnStage<CT, DPV>::SMEM; out->threads = 256; \
    if (merge) { merge->fn = (const void*)&k_attn_merge<CT, DPV, HPWV>; merge->smem = 0; merge->threads = 256; } \
    return true;                                    \
  }

bool attn_lookup(int f32, int dp, int hpw, KernelRef* out, KernelRef* merge) {
  VLA_ATTN_CASE(__bf16, 0, 64, 1) VLA_ATTN_CASE(__bf16, 0, 64, 2) VLA_ATTN_CASE(__bf16, 0, 64, 4)
  VLA_ATTN_CASE(__bf16, 0, 96, 1) VLA_ATTN_CASE(__bf16, 0, 96, 2) VLA_ATTN_CASE(__bf16, 0, 96, 4)
  VLA_ATTN_CASE(__bf16, 0, 128, 1) VLA_ATTN_CASE(__bf16, 0, 128, 2) VLA_ATTN_CASE(__bf16, 0, 128, 4)
  VLA_ATTN_CASE(float, 1, 64, 1) VLA_ATTN_CASE(float, 1, 64, 2) VLA_ATTN_CASE(float, 1, 64, 4)
  VLA_ATTN_CASE(float, 1, 128, 1) VLA_ATTN_CASE(float, 1, 128, 2) VLA_ATTN_CASE(float, 1, 128, 4)
  return false;
}

const void* k_fill_ref() { return (const void*)&k_fill_u32; }
const void* k_stage_rows_ref() { return (const void*)&k_stage_rows; }
const void* k_rmsnorm_out_ref() { return (const void*)&k_rmsnorm_out; }
const void* k_norm_rows_ref() { return (const void*)&k_norm_rows; }
const void* k_quant_rows_ref() { return (const void*)&k_quant_rows; }
const void* k_convert_rows_ref() { return (const void*)&k_convert_rows; }

bool euler_tail_lookup(int wt, KernelRef* out) {
  out->smem = 0;
  out->threads = 256;
  if (wt == 0) { out->fn = (const void*)&k_euler_tail<float>; return true; }
  if (wt == 1) { out->fn = (const void*)&k_euler_tail<uint16_t>; return true; }
  if (wt == 2) { out->fn = (const void*)&k_euler_tail<uint8_t>; return true; }
  if (wt == 3) { out->fn = (const void*)&k_euler_tail<int8_t>; return true; }
  return false;
}

}  // namespace vla
