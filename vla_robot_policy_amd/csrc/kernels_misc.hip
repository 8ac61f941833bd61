// Staging, norm, conversion and Euler-tail kernel instantiations.
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


const void* k_fill_ref() { return (const void*)&k_fill_u32; }
const void* k_stage_rows_ref() { return (const void*)&k_stage_rows; }
const void* k_rmsnorm_out_ref() { return (const void*)&k_rmsnorm_out; }
const void* k_time_embed_ref() { return (const void*)&k_time_embed; }
const void* k_rope_table_ref() { return (const void*)&k_rope_table; }
const void* k_pack_weights_ref() { return (const void*)&k_pack_weights; }
const void* k_ctx_vt_ref() { return (const void*)&k_ctx_vt; }
const void* k_patch_rows_ref() { return (const void*)&k_patch_rows; }
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
