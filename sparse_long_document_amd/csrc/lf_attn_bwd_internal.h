// Internal interface of the backward's launches, between the host entry
// point (lf_attn_host.cpp) and the device code (lf_attn_bwd.hip).  Not part
// of the public ABI.
#pragma once

#include <stdint.h>

#include "lf_attn_internal.h"

namespace lf {

// Workgroups of the backward's global-token launch: one workgroup per (b,
// h, block of 32 global slots, group of four chunks) for GQ and again for
// GK, then the GKV units four per workgroup; 0 without global work.
inline int64_t bwd_glob_workgroups(int64_t n_gkv, int64_t B, int64_t H, int64_t gslots, int64_t chunks) {
  if (n_gkv <= 0) return 0;
  return (n_gkv + 3) / 4 + 2 * B * H * gslots * ((chunks + 3) / 4);
}

// One launch of the backward on a stream (the band or the global-token
// kernel).
typedef void (*BwdLaunch)(const BwdParams& bp, void* stream);

// Enqueues band(bp, stream) on the caller's stream and glob(bp, aux) on the
// library's second stream of the current device, forked from `stream`
// after the work already on it (the preparation) and joined back into it,
// so that the two launches run at the same time; also under graph capture
// once the second stream exists (it is created at the first call outside
// capture).  Without it both go on `stream`, band first.  Returns the
// hipError_t value as int.
int launch_backward_pair(const BwdParams& bp, void* stream, BwdLaunch band, BwdLaunch glob);

}  // namespace lf
