// GEMM instantiations for int8 weights with per-row scales: codes are
// widened to bf16 in registers (exact, |code| <= 127), bf16 MFMA, fp32
// accumulate, scale applied per output column in the epilogue. W8A8 integer
// (A_I8): int8 activation codes (per-row scales) are staged as bytes and
// widened the same way; both scales are applied to the fp32 tile.
#include "gemm_inst.h"

namespace vla {
bool gemm_lookup_int8(const GemmPick& g, KernelRef* out) {
  VLA_GEMM_NARROW(int8_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_CASE(int8_t, __bf16, A_BF16, E_STORE, 1, 4, 1, 1)
  VLA_GEMM_WIDE(int8_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_NARROW(int8_t, __bf16, A_BF16, E_RESID)
  VLA_GEMM_CASE_X(int8_t, __bf16, A_BF16, E_RESID, 4, 2, 2, 1, 2, 0)
  VLA_GEMM_NARROW(int8_t, __bf16, A_NORM, E_STORE)
  VLA_GEMM_WIDE(int8_t, __bf16, A_BF16, E_ROPE)
  VLA_GEMM_WIDE(int8_t, __bf16, A_BF16, E_SWIGLU)
  VLA_GEMM_WIDE(int8_t, __bf16, A_I8, E_ROPE)
  VLA_GEMM_WIDE(int8_t, __bf16, A_I8, E_SWIGLU)
  VLA_GEMM_NARROW(int8_t, __bf16, A_I8, E_RESID)
  VLA_GEMM_BACKBONE_M7(int8_t, 0)
  VLA_GEMM_BACKBONE_M7(int8_t, 1)
  VLA_GEMM_PACKED_ROWS(int8_t, 1)
  VLA_GEMM_PACKED_ROWS(int8_t, 4)
  VLA_GEMM_PACKED_ROWS(int8_t, 7)
  VLA_GEMM_PACKED_ROWS(int8_t, 8)
  VLA_GEMM_PACKED_RESID(int8_t)
  return false;
}
}  // namespace vla
