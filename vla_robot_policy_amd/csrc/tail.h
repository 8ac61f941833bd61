// Arguments of the fused Euler-tail kernel (shared by host and device code).
#pragma once
#include <hip/hip_runtime.h>
#include "rowstats.h"

namespace vla {

struct TailArgs {
  int n, D, A, K;             // action rows, DiT width, action dim, Euler steps
  // velocity head (skipped when w_out == NULL)
  const float* x; float eps;                     // residual stream (its rows are normalised here)
  const float* shift; const float* scale;   // final modulation of this step [D] each
  const void* w_out; const float* s_out; const float* b_out;   // [A, D], per-row scale, [A]
  const float* a_in;          // current actions [n, A]
  float* a_out;               // updated actions [n, A] (may equal a_in)
  float* v_out;               // optional velocity record [n, A]
  // input projection of the (updated) actions (skipped when w_in == NULL)
  const void* w_in; const float* s_in; const float* b_in;      // [D, A], per-row scale, [D]
  float* x_out; float2* rs_out;                  // new stream, its moments as one tile
};

// Arguments of the row-normalisation kernel.
struct NormArgs {
  const float* x; int ldx;    // [M, ldx] fp32 rows
  int M, K;                   // rows, row length (a multiple of 4)
  RowStats rs;                // the writer's tile moments of x
  int rms; float eps;         // 1: RMSNorm, 0: LayerNorm
  const float* g; int g_plus_one; const float* bsh;   // gain (NULL = 1), 1 + g, shift (NULL = 0)
  uint16_t* out; uint16_t* out_lo; int ldo;            // bf16 result, optional remainder plane
  uint8_t* out8; float* oscale;                        // instead: 8-bit codes [M, ldo] and row scales (K <= 4096)
  int out8_int8;                                       //   int8 codes (else E4M3FN)
  // merge > 0: the rows are patches of images of vgrid x vgrid patches
  // (n_patches each, raster order); patch row r is written as segment
  // (dy * merge + dx) of merged row (image, R, C), where (merge R + dy,
  // merge C + dx) is its grid position (segments K wide, ldo = merge^2 K)
  int merge, vgrid, n_patches;
};

}  // namespace vla
