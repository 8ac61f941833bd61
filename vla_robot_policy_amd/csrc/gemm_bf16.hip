// GEMM instantiations for bf16 weights (bf16 MFMA, fp32 accumulate).
#include "gemm_inst.h"

namespace vla {
bool gemm_lookup_bf16(int am, int em, int mb, int wn, int wk, int nbw, int u, int ac, KernelRef* out) {
  VLA_GEMM_NARROW(uint16_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_CASE(uint16_t, __bf16, A_BF16, E_STORE, 1, 4, 1, 1)
  VLA_GEMM_WIDE(uint16_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_CASE_X(uint16_t, __bf16, A_BF16, E_RESID, 4, 2, 2, 1, 2, 0)
  VLA_GEMM_NARROW(uint16_t, __bf16, A_BF16, E_RESID)
  VLA_GEMM_NARROW(uint16_t, __bf16, A_NORM, E_STORE)
  VLA_GEMM_WIDE(uint16_t, __bf16, A_BF16, E_ROPE)
  VLA_GEMM_WIDE(uint16_t, __bf16, A_BF16, E_SWIGLU)
  VLA_GEMM_WIDE_AC(uint16_t, __bf16, A_BF16, E_SWIGLU)
  VLA_GEMM_NARROW_AC(uint16_t, __bf16, A_BF16, E_RESID)
  VLA_GEMM_NARROW(uint16_t, __bf16, A_PATCH, E_RESID)
  VLA_GEMM_NARROW(uint16_t, __bf16, A_MERGE, E_STORE)
  return false;
}
}  // namespace vla
