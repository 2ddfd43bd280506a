// Internal interface between the host entry point lf_attn_project
// (lf_attn_host.cpp) and the projection kernel (lf_proj.hip).  Not part of
// the public ABI.
#pragma once

#include <stdint.h>

#include "lf_attn.h"

namespace lf {

// Input projections: y[p][m][c] = x[m] . w[p*C + c] + bias[p*C + c].
struct ProjParams {
  const void* x;      // [M, C]
  const void* w;      // [N, C], N = P * C
  const float* bias;  // [N] or null
  void* out;          // [P, M, C]
  int32_t M, C, N, dtype;
  // projections computed at global tokens only: bit p set -> out[p][m] is
  // computed where mask[m] == 2 and zero elsewhere (mask [M] int8; null and
  // 0 for the plain projections)
  const int8_t* mask;
  uint32_t global_only;
};

// Launches the projection GEMM (bf16 or f16).  Returns the hipError_t value.
int launch_project(const ProjParams& pp, void* stream);

// Tile configuration the launch uses for M tokens and N stacked features on
// a device with `cus` compute units: 0 = 128 x 128, 1 = 128 x 192,
// 2 = 256 x 288, 3 = 256 x 256 (tokens x features).
int proj_tile_config(int M, int N, int cus);

}  // namespace lf
