// Instantiations of the persistent DiT layers kernel (bf16, fp8 and int8
// weights) for the supported widths, and its weight-table fill.
#include "dit_stack.h"
#include "kernels.h"

namespace vla {
#define VLA_DIT_WIDTHS(X) X(160) X(512) X(768) X(1024) X(1280)
#define VLA_DIT_INST(D)                                                  \
  template __global__ void k_dit_layers<uint16_t, D>(DitLayerArgs);       \
  template __global__ void k_dit_layers<uint8_t, D>(DitLayerArgs);        \
  template __global__ void k_dit_layers<int8_t, D>(DitLayerArgs);
VLA_DIT_WIDTHS(VLA_DIT_INST)

bool dit_layer_lookup(int wt, int D, KernelRef* out) {
  out->fn = nullptr;
#define VLA_DIT_CASE(DV)                                                       \
  if (D == DV) {                                                               \
    if (wt == 1) out->fn = (const void*)&k_dit_layers<uint16_t, DV>;            \
    else if (wt == 2) out->fn = (const void*)&k_dit_layers<uint8_t, DV>;        \
    else if (wt == 3) out->fn = (const void*)&k_dit_layers<int8_t, DV>;         \
  }
  VLA_DIT_WIDTHS(VLA_DIT_CASE)
  if (!out->fn) return false;
  out->smem = ds_smem_bytes(D);
  out->threads = DS_THREADS;
  return true;
}

__global__ __launch_bounds__(64) void k_dit_table(DitTableArgs a) {
  if ((int)threadIdx.x < a.n) a.out[threadIdx.x] = a.p[threadIdx.x];
}
const void* k_dit_table_ref() { return (const void*)&k_dit_table; }
}  // namespace vla
