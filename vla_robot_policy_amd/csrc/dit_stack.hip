// Instantiations of the persistent DiT layer kernel (bf16, fp8 and int8 weights)
// for the supported widths.
#include "dit_stack.h"
#include "kernels.h"

namespace vla {
#define VLA_DIT_WIDTHS(X) X(160) X(512) X(768) X(1024) X(1280)
#define VLA_DIT_INST(D)                                                  \
  template __global__ void k_dit_layer<uint16_t, D>(DitLayerArgs);       \
  template __global__ void k_dit_layer<uint8_t, D>(DitLayerArgs);        \
  template __global__ void k_dit_layer<int8_t, D>(DitLayerArgs);
VLA_DIT_WIDTHS(VLA_DIT_INST)

bool dit_layer_lookup(int wt, int D, KernelRef* out) {
  out->fn = nullptr;
#define VLA_DIT_CASE(DV)                                                       \
  if (D == DV) {                                                               \
    if (wt == 1) out->fn = (const void*)&k_dit_layer<uint16_t, DV>;            \
    else if (wt == 2) out->fn = (const void*)&k_dit_layer<uint8_t, DV>;        \
    else if (wt == 3) out->fn = (const void*)&k_dit_layer<int8_t, DV>;         \
  }
  VLA_DIT_WIDTHS(VLA_DIT_CASE)
  if (!out->fn) return false;
  out->smem = ds_smem_bytes(D);
  out->threads = DS_THREADS;
  return true;
}
}  // namespace vla
