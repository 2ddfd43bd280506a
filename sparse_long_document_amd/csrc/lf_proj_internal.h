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
};

// Launches the projection GEMM (bf16 or f16).  Returns the hipError_t value.
int launch_project(const ProjParams& pp, void* stream);

}  // namespace lf
