// Stand-ins for the device-side entry points, for the host-only build of
// lf_attn_host.cpp under the address and undefined-behaviour sanitizers
// (build.py, build_host_sanitized).  That build checks the argument
// validation and workspace layout code on the CPU; nothing here launches
// anything: every launch reports that no device is present.
#include <hip/hip_runtime_api.h>

#include "lf_attn.h"
#include "lf_attn_internal.h"
#include "lf_proj_internal.h"

namespace lf {

int launch_forward(const KernelParams&, int, int, void*) { return (int)hipErrorNoDevice; }
int launch_backward(const BwdParams&, void*) { return (int)hipErrorNoDevice; }
int launch_project(const ProjParams&, void*) { return (int)hipErrorNoDevice; }
int64_t resident_workgroups(int, int) { return 0; }

}  // namespace lf

// The no-allocation entry point's own code is device code (its scratch is a
// device array); here it keeps its argument checks, which are the host's.
extern "C" lf_status lf_attn_forward_noalloc(const lf_attn_params* p, const void* q, const void* k,
                                             const void* v, const void* q_g, const void* k_g, const void* v_g,
                                             const int8_t* mask, void* out, int32_t* row_nnz, void*) {
  size_t need = 0;
  const lf_status st = lf::check_forward_args(p, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, &need);
  if (st != LF_OK) return st;
  if (need > (size_t)LF_NOALLOC_SCRATCH_BYTES) return LF_ERR_WORKSPACE;
  return LF_ERR_HIP;
}
