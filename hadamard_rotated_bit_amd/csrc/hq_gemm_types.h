// Types shared by the GEMM kernels and their callers (kept apart from the
// launcher declarations so that the kernels' sources change only with them).
#pragma once

#include <stdint.h>

namespace hq {

// Rows per group of the E2M3 code layout (see CodeFmt in hq_internal.h).
// 32-row groups (each 1-KB stage load of the FP6 GEMM reading one contiguous
// range) measured no faster than 4-row groups.
constexpr int F6_GROUP = 4;

// Dequant epilogue of the GEMMs: y = s_x s_w acc + b + mu c (+ U L2), stored
// as bf16 or fp32 at Y with row pitch ldy.
struct GemmEpi {
  const float* s_x;       // [M]
  const float* mu;        // [M]
  const float* s_w;       // [N]
  const float* c;         // [N]
  const float* bias;      // [N]
  const float* U;         // [M, rank] or NULL
  const uint16_t* l2_hi;  // [N, rank]
  const uint16_t* l2_lo;
  int l2_lo_zero;         // l2_lo is all zero (L2 given in bf16 is its own hi
                          // part): its products are skipped
  int rank;
  void* Y;                // [M, ldy]
  int y_bf16;
  int64_t ldy;
  int prescaled;          // accumulators already carry s_x s_w (group-wise GEMM)
};

}  // namespace hq
