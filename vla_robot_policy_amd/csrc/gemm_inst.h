// Explicit GEMM instantiations and their lookup (included once per weight type).
#pragma once
#include "gemm.h"
#include "kernels.h"

#define VLA_GEMM_CASE(WT, CT, AMV, EMV, MBV, WNV, NBWV)                                      \
  if (am == AMV && em == EMV && mb == MBV && wn == WNV && nbw == NBWV) {                     \
    out->fn = (const void*)&k_gemm<WT, CT, MBV, WNV, NBWV, AMV, EMV>;                        \
    out->smem = GemmTile<WT, CT, MBV, WNV, NBWV, AMV, EMV>::SMEM;                            \
    return true;                                                                             \
  }

// narrow tiles (BN = 16 for one 16-row block, else 64) and wide tiles (BN = 128)
#define VLA_GEMM_NARROW(WT, CT, AMV, EMV)  \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 1, 1, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 4, 4, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 7, 4, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 16, 4, 1)
#define VLA_GEMM_WIDE(WT, CT, AMV, EMV)    \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 1, 4, 2) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 4, 4, 2) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 7, 4, 2) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 16, 4, 2)
