// GEMM instantiations for fp32 weights and activations (fp32 MFMA).
#include "gemm_inst.h"

namespace vla {
bool gemm_lookup_f32(const GemmPick& g, KernelRef* out) {
  VLA_GEMM_NARROW(float, float, A_F32, E_STORE)
  VLA_GEMM_NARROW(float, float, A_F32, E_RESID)
  VLA_GEMM_WIDE(float, float, A_NORM, E_ROPE)
  VLA_GEMM_WIDE(float, float, A_NORM, E_SWIGLU)
  return false;
}
}  // namespace vla
