// Explicit GEMM instantiations and their lookup (included once per weight type).
#pragma once
#include "gemm.h"
#include "kernels.h"

#define VLA_GEMM_CASE_X(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, UV, ACV)                                     \
  if (am == AMV && em == EMV && mb == MBV && wn == WNV && wk == WKV && nbw == NBWV && u == UV && ac == ACV) { \
    out->fn = (const void*)&k_gemm<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV, ACV>;                          \
    out->smem = GemmTile<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV, ACV>::SMEM;                              \
    out->threads = GemmTile<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV, ACV>::THREADS;                        \
    return true;                                                                                             \
  }
#define VLA_GEMM_CASE(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV) VLA_GEMM_CASE_X(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, 4, 0)

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
// compensated-A variants (two k-steps per chunk: half the LDS of the plain
// tiles); 128-row narrow tiles would not fit in LDS with both A planes
#define VLA_GEMM_NARROW_AC(WT, CT, AMV, EMV)            \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 1, 1, 4, 1, 2, 1) \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 4, 4, 2, 1, 2, 1) \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 7, 4, 2, 1, 2, 1)
// wide compensated tiles: 4 x 2 waves with two 16-column blocks each, one
// 32-wide k-step per wave per chunk
#define VLA_GEMM_WIDE_AC(WT, CT, AMV, EMV)              \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 1, 4, 2, 2, 1, 1) \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 4, 4, 2, 2, 1, 1) \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 7, 4, 2, 2, 1, 1) \
  VLA_GEMM_CASE_X(WT, CT, AMV, EMV, 8, 4, 2, 2, 1, 1)
