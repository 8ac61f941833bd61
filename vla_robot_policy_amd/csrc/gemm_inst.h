// Explicit GEMM instantiations and their lookup (included once per weight type).
#pragma once
#include "gemm.h"
#include "kernels.h"

#define VLA_GEMM_CASE_F(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, UV, ACV, AQV, PKV)                               \
  if (g.am == AMV && g.em == EMV && g.mb == MBV && g.wn == WNV && g.wk == WKV && g.nbw == NBWV && g.u == UV &&      \
      g.ac == ACV && g.aq == AQV && g.pk == PKV) {                                                                  \
    out->fn = (const void*)&k_gemm<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV, ACV, AQV, PKV>;                      \
    out->smem = GemmTile<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV, ACV, AQV, PKV>::SMEM;                          \
    out->threads = GemmTile<WT, CT, MBV, WNV, WKV, NBWV, AMV, EMV, UV, ACV, AQV, PKV>::THREADS;                    \
    return true;                                                                                                   \
  }
#define VLA_GEMM_CASE_X(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, UV, ACV) \
  VLA_GEMM_CASE_F(WT, CT, AMV, EMV, MBV, WNV, WKV, NBWV, UV, ACV, 2, 0)
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

// Backbone tiles of the 65-112-row shapes (measured at 104 rows: QKV 21.1 ->
// 20.1 us, O projection 18.5 -> 16.0, down 37.2 -> 32.2; with packed
// weights 18.9, 15.5 and 30.7, gate/up 49.9 -> 47.0), and the packed-weight
// counterparts of every backbone tile (PK = 1) for all row tilings.
#define VLA_GEMM_BACKBONE_M7(WT, PKV)                                            \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_ROPE, 7, 8, 1, 1, 2, 0, 4, PKV)        \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_RESID, 7, 2, 2, 1, 2, 0, 2, PKV)
#define VLA_GEMM_PACKED_ROWS(WT, MBV)                                            \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_ROPE, MBV, 8, 1, 1, 4, 0, 2, 1)        \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_SWIGLU, MBV, 8, 1, 1, 4, 0, 2, 1)      \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_RESID, MBV, 4, 1, 1, 4, 0, 2, 1)
// the other residual tiles of the row-major picks, so that packed weights
// give the same tiles and the same bits: 16 rows over four k-waves, and two
// k-waves of 32 columns for 17..64 rows
#define VLA_GEMM_PACKED_RESID(WT)                                                \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_RESID, 1, 1, 4, 1, 4, 0, 2, 1)         \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_RESID, 4, 2, 2, 1, 2, 0, 2, 1)

// Packed-weight plain-store tiles (the vision encoder's QKV and MLP
// up-projection with packed weights), for every row class, and the packed
// narrow long-K residual tile of 193-256 rows (its MLP down-projection)
#define VLA_GEMM_PACKED_STORE(WT)                                                \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_STORE, 1, 1, 4, 1, 4, 0, 2, 1)         \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_STORE, 4, 4, 1, 1, 4, 0, 2, 1)         \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_STORE, 7, 4, 1, 1, 4, 0, 2, 1)         \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_STORE, 8, 4, 1, 1, 4, 0, 2, 1)         \
  VLA_GEMM_CASE_F(WT, __bf16, A_BF16, E_RESID, 4, 4, 2, 1, 2, 0, 2, 1)
// Deferred-RMSNorm (A_BF16R) counterparts of the backbone's QKV and gate/up
// tiles, row-major (PKV 0) and packed (PKV 1): 1-16, 17-64 and 113-256
// (64-row tiles), 65-112 and beyond 256 rows; the compensated gate/up of
// bf16 weights with its 256-weight-row tiles at 65-112 and 193-256 rows
#define VLA_GEMM_BF16R_BF16(PKV)                                                        \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_ROPE, 1, 8, 1, 1, 4, 0, 2, PKV)         \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_ROPE, 4, 8, 1, 1, 4, 0, 2, PKV)         \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_ROPE, 7, 8, 1, 1, 2, 0, 4, PKV)         \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_ROPE, 8, 8, 1, 1, 4, 0, 2, PKV)         \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_SWIGLU, 1, 4, 2, 2, 1, 1, 2, PKV)       \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_SWIGLU, 4, 4, 2, 2, 1, 1, 2, PKV)       \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_SWIGLU, 7, 8, 1, 2, 2, 1, 2, PKV)       \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_SWIGLU, 8, 8, 1, 2, 2, 1, 2, PKV)       \
  VLA_GEMM_CASE_F(uint16_t, __bf16, A_BF16R, E_SWIGLU, 8, 4, 2, 2, 1, 1, 2, PKV)
// fp8 weights (plain bf16 activations): the same row classes
#define VLA_GEMM_BF16R_FP8(PKV)                                                         \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_ROPE, 1, 8, 1, 1, 4, 0, 2, PKV)          \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_ROPE, 4, 8, 1, 1, 4, 0, 2, PKV)          \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_ROPE, 7, 8, 1, 1, 2, 0, 4, PKV)          \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_ROPE, 8, 4, 1, 2, 2, 0, 2, PKV)          \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_SWIGLU, 1, 8, 1, 1, 4, 0, 2, PKV)        \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_SWIGLU, 4, 8, 1, 1, 4, 0, 2, PKV)        \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_SWIGLU, 7, 8, 1, 1, 4, 0, 2, PKV)        \
  VLA_GEMM_CASE_F(uint8_t, __bf16, A_BF16R, E_SWIGLU, 8, 4, 1, 2, 2, 0, 2, PKV)
