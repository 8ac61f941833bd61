// Instantiations of the persistent DiT layer kernel (bf16 and fp8 weights).
#include "dit_stack.h"
#include "kernels.h"

namespace vla {
template __global__ void k_dit_layer<uint16_t>(DitLayerArgs);
template __global__ void k_dit_layer<uint8_t>(DitLayerArgs);

bool dit_layer_lookup(int wt, int D, KernelRef* out) {
  if (wt == 1) out->fn = (const void*)&k_dit_layer<uint16_t>;
  else if (wt == 2) out->fn = (const void*)&k_dit_layer<uint8_t>;
  else return false;
  out->smem = ds_smem_bytes(D);
  out->threads = DS_THREADS;
  return true;
}
}  // namespace vla
