// GEMM instantiations for fp8 (OCP E4M3FN) weights with per-row scales:
// codes are widened to bf16 in registers (exact), bf16 MFMA, fp32 accumulate,
// scale applied per output column in the epilogue. W8A8 (A_FP8): activation
// codes (per-row scales) are staged as bytes and meet the weight codes in
// the fp8 MFMA (16x16x32, fp32 accumulation; its internal sums are coarser
// than fp32: about 5e-5 relative at K = 1024, far below the quantisation
// error of the codes themselves); both scales are applied to the fp32 tile.
#include "gemm_inst.h"

namespace vla {
bool gemm_lookup_fp8(const GemmPick& g, KernelRef* out) {
  VLA_GEMM_NARROW(uint8_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_CASE(uint8_t, __bf16, A_BF16, E_STORE, 1, 4, 1, 1)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_NARROW(uint8_t, __bf16, A_BF16, E_RESID)
  VLA_GEMM_CASE_X(uint8_t, __bf16, A_BF16, E_RESID, 4, 2, 2, 1, 2, 0)
  VLA_GEMM_NARROW(uint8_t, __bf16, A_NORM, E_STORE)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_BF16, E_ROPE)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_BF16, E_SWIGLU)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_FP8, E_ROPE)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_FP8, E_SWIGLU)
  VLA_GEMM_NARROW(uint8_t, __bf16, A_FP8, E_RESID)
  VLA_GEMM_BACKBONE_M7(uint8_t, 0)
  VLA_GEMM_BACKBONE_M7(uint8_t, 1)
  VLA_GEMM_PACKED_ROWS(uint8_t, 1)
  VLA_GEMM_PACKED_ROWS(uint8_t, 4)
  VLA_GEMM_PACKED_ROWS(uint8_t, 7)
  VLA_GEMM_PACKED_ROWS(uint8_t, 8)
  VLA_GEMM_PACKED_RESID(uint8_t)
  // more than 256 rows: two 16-column blocks per wave for gate/up and QKV
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16, E_SWIGLU, 8, 4, 1, 2, 2, 0, 2, 0)
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16, E_SWIGLU, 8, 4, 1, 2, 2, 0, 2, 1)
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16, E_ROPE, 8, 4, 1, 2, 2, 0, 2, 0)
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16, E_ROPE, 8, 4, 1, 2, 2, 0, 2, 1)
  // wide plain stores: 256 columns per tile beyond 256 rows, two column
  // blocks per wave at 65..112 rows
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16, E_STORE, 8, 8, 1, 2, 2, 0, 2, 0)
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16, E_STORE, 7, 4, 1, 2, 2, 0, 2, 0)
  VLA_GEMM_BF16R_FP8(0)
  VLA_GEMM_BF16R_FP8(1)
  return false;
}
}  // namespace vla
