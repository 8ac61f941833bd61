// GEMM instantiations for fp8 (OCP E4M3FN) weights with per-row scales:
// codes are widened to bf16 in registers (exact), bf16 MFMA, fp32 accumulate,
// scale applied per output column in the epilogue. W8A8 (A_FP8): activation
// codes (per-row scales) are staged as bytes and widened to bf16 like the
// weights, so the bf16 MFMA forms exact code products with full fp32
// accumulation; both scales are applied to the fp32 tile. (The fp8 MFMA's
// internal accumulation is coarser: 5e-5 relative error at K = 1024 against
// 2e-7 this way, and a per-token requantisation in every layer amplifies it.)
#include "gemm_inst.h"

namespace vla {
bool gemm_lookup_fp8(int am, int em, int mb, int wn, int wk, int nbw, int u, int ac, KernelRef* out) {
  VLA_GEMM_NARROW(uint8_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_CASE(uint8_t, __bf16, A_BF16, E_STORE, 1, 4, 1, 1)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_BF16, E_STORE)
  VLA_GEMM_NARROW(uint8_t, __bf16, A_BF16, E_RESID)
  VLA_GEMM_CASE_X(uint8_t, __bf16, A_BF16, E_RESID, 4, 2, 2, 1, 2, 0)
  VLA_GEMM_NARROW(uint8_t, __bf16, A_NORM, E_STORE)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_BF16, E_ROPE)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_BF16, E_SWIGLU)
  VLA_GEMM_CASE(uint8_t, __bf16, A_TIME, E_STORE, 1, 1, 4, 1)
  VLA_GEMM_CASE(uint8_t, __bf16, A_TIME, E_STORE, 4, 4, 1, 1)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_FP8, E_ROPE)
  VLA_GEMM_WIDE(uint8_t, __bf16, A_FP8, E_SWIGLU)
  VLA_GEMM_NARROW(uint8_t, __bf16, A_FP8, E_RESID)
  return false;
}
}  // namespace vla
