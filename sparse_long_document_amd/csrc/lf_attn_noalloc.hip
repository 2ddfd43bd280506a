// The forward for callers that cannot allocate device memory: the same
// kernels as lf_attn_forward, with the workspace (status word, arrival
// counters, partial records of the global rows) in a static device array of
// this library instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "lf_attn.h"
#include "lf_attn_internal.h"

namespace {

// Each device that runs the library holds its own copy of this array until
// the process ends.  In host code its name only stands for the device
// symbol: the device address is what hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[LF_NOALLOC_SCRATCH_BYTES];

// Zeroes `n` 32-bit words: the part of the scratch that must start each
// call at zero (a kernel, not hipMemsetAsync, so that a caller may record
// the call into a HIP graph).
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of this device's scratch, looked up once per device
// (with that device current); null if the runtime refuses.
void* scratch_ptr(int dev) {
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  g_scratch[dev].store(ptr, std::memory_order_release);  // concurrent first calls store the same address
  return ptr;
}

}  // namespace

extern "C" lf_status lf_attn_forward_noalloc(const lf_attn_params* p, const void* q, const void* k,
                                             const void* v, const void* q_g, const void* k_g, const void* v_g,
                                             const int8_t* mask, void* out, int32_t* row_nnz, void* stream) {
  // every argument check first, before any HIP call
  size_t need = 0;
  const lf_status st = lf::check_forward_args(p, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, &need);
  if (st != LF_OK) return st;
  if (need > (size_t)LF_NOALLOC_SCRATCH_BYTES) return LF_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LF_ERR_HIP;
  void* ws = scratch_ptr(dev);
  if (!ws) return LF_ERR_HIP;
  // The status word and the arrival counters start every call at zero (a
  // completed launch leaves its counters at zero, but the previous call may
  // have used another layout or set a status bit); the partial records are
  // written before they are read.  Status word: the first 256 bytes; the
  // counters follow it, B*H of them.
  const int words = (256 + p->B * p->H * 4 + 3) / 4;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(clear_words, dim3((words + 255) / 256 < 64 ? (words + 255) / 256 : 64), dim3(256), 0, s,
                     static_cast<uint32_t*>(ws), words);
  if (hipGetLastError() != hipSuccess) return LF_ERR_HIP;
  return lf::forward_with_workspace(p, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, ws,
                                    (size_t)LF_NOALLOC_SCRATCH_BYTES, stream);
}
