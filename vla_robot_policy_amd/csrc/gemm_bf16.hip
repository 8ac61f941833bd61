// GEMM instantiations for bf16 weights (bf16 MFMA, fp32 accumulate).
#include "gemm_inst.h"

namespace vla {
bool gemm_lookup_bf16(const GemmPick& g, KernelRef* out) {
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
  // compensated MLP tiles: down at 65-112 rows with one k-step per wave and
  // four activation chunks in flight; the packed gate/up and down tiles
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 7, 4, 2, 1, 1, 1, 4, 0)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 7, 4, 2, 1, 1, 1, 4, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 1, 4, 2, 2, 1, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 4, 4, 2, 2, 1, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 7, 4, 2, 2, 1, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 8, 4, 2, 2, 1, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 1, 1, 4, 1, 2, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 4, 4, 2, 1, 2, 1, 2, 1)
  VLA_GEMM_BACKBONE_M7(uint16_t, 0)
  VLA_GEMM_BACKBONE_M7(uint16_t, 1)
  VLA_GEMM_PACKED_ROWS(uint16_t, 1)
  VLA_GEMM_PACKED_ROWS(uint16_t, 4)
  VLA_GEMM_PACKED_ROWS(uint16_t, 7)
  VLA_GEMM_PACKED_ROWS(uint16_t, 8)
  VLA_GEMM_PACKED_RESID(uint16_t)
  // compensated gate/up of 256 weight rows per tile at 65..112 and 193..256
  // rows, compensated down of 128 x 64 tiles at 193..256 rows
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 7, 8, 1, 2, 2, 1, 2, 0)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 7, 8, 1, 2, 2, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 8, 8, 1, 2, 2, 1, 2, 0)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_SWIGLU, 8, 8, 1, 2, 2, 1, 2, 1)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 8, 2, 2, 2, 1, 1, 2, 0)
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 8, 2, 2, 2, 1, 1, 2, 1)
  // wide plain stores at 65..112 rows: two column blocks per wave
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_STORE, 7, 4, 1, 2, 2, 0, 2, 0)
  // narrow long-K residual at 193..256 rows: two k-waves of 64 columns
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16, E_RESID, 4, 4, 2, 1, 2, 0, 2, 0)
  VLA_GEMM_PACKED_STORE(uint16_t)
  VLA_GEMM_BF16R_BF16(0)
  VLA_GEMM_BF16R_BF16(1)
  return false;
}
}  // namespace vla
