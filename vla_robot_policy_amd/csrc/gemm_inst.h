// Explicit GEMM instantiations and their lookup (included once per weight type).
#pragma once
#include "gemm.h"
#include "kernels.h"

#define VLA_GEMM_CASE_U(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, UV)                              \
  if (am == AMV && em == EMV && mb == MBV && wn == WNV && wk == WKV && nbw == NBWV) {                \
    out->fn = (const void*)&k_gemm<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV>;                    \
    out->smem = GemmTile<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV>::SMEM;                        \
    out->threads = GemmTile<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV>::THREADS;                  \
    return true;                                                                                  \
  }
#define VLA_GEMM_CASE(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV) VLA_GEMM_CASE_U(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, 4)

// narrow tiles (16 columns for 16-row tiles, else 64) and wide tiles (128 columns)
#define VLA_GEMM_NARROW(WT, CT, AMV, EMV)     \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 1, 1, 4, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 4, 4, 1, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 7, 4, 1, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 8, 4, 1, 1)
#define VLA_GEMM_WIDE(WT, CT, AMV, EMV)       \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 1, 8, 1, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 4, 8, 1, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 7, 8, 1, 1) \
  VLA_GEMM_CASE(WT, CT, AMV, EMV, 8, 8, 1, 1)
