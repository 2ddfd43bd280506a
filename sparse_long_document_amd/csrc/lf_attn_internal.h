// Internal interface between the host entry points (lf_attn_host.cpp) and
// the device code (lf_attn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lf_attn.h"

namespace lf {

// Tiling constants shared by the host planner and the kernels.
constexpr int kTileQ = 64;         // query rows of one band workgroup (two halves of 32)
constexpr int kBlockK = 32;        // keys per inner block (M of the 32x32 MFMA)
constexpr int kWaves = 4;          // waves per workgroup: query half x key parity
constexpr int kThreads = 64 * kWaves;
// Keys per split of a global row: the short chunk when the whole launch is
// resident at once (splits then end sooner), else the long one (fewer splits,
// fewer records to merge).  The workspace is sized for the short one.
constexpr int kGlobalChunkShort = 512;
constexpr int kGlobalChunkLong = 1024;
// Floats per partial record of a global-row split at head dim D: m, l,
// count, pad, O[D].
constexpr int partial_stride(int D) { return 4 + D; }

// Everything one launch needs, passed by value as the kernel argument.
struct KernelParams {
  const void* q;
  const void* k;
  const void* v;
  const void* qg;
  const void* kg;
  const void* vg;
  const int8_t* mask;
  void* out;
  int32_t* row_nnz;    // may be null
  float* lse;          // may be null: natural log-sum-exp of each row's scores [B][H][n]
  int32_t* status;     // device status word
  int32_t* tickets;    // [B*H] arrival counters of the global-row splits
  float* partials;     // [B][H][max_global][S][partial_stride(D)]
  int32_t B, n, H, w, causal, max_global, use_globals;
  float c;             // score scale * log2(e)
  int32_t tiles_per_b; // band workgroups per batch row
  int32_t n_band;      // band workgroups in the launch
  int32_t n_glob;      // global-row workgroups in the launch
  int32_t S;           // splits of a global row
  int32_t chunk;       // keys per split
  int32_t uni_dil;     // the dilation of every head when all heads share one, else 0
  int32_t tiles_per_head;  // band tiles of each head of a batch row when uni_dil > 0
  int32_t dil[LF_MAX_HEADS];
  int32_t tile0[LF_MAX_HEADS + 1];  // first band tile of each head within a batch row
};

// Backward: keys or rows per global-work unit.
constexpr int kBwdChunk = 128;

// Everything the backward launches need.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* qg;
  const void* kg;
  const void* vg;
  const int8_t* mask;
  const void* out;
  const void* dout;
  const float* lse;    // [B][H][n] natural log-sum-exp saved by the forward
  float* dq;
  float* dk;
  float* dv;
  float* dqg;
  float* dkg;
  float* dvg;
  float* dneg;         // [B][H][n] workspace: -<dout, out> per row
  float* lneg;         // [B][H][n] workspace: -lse / scale per row (0 where lse is not finite)
  int32_t* glist;      // [B][gstride] workspace: global positions, ascending
  int32_t* gcount;     // [B] workspace: entries of glist in use
  int32_t* status;     // device status word
  int32_t B, n, H, w, causal, max_global, use_globals, dtype;
  float c;             // score scale * log2(e)
  float scale;
  int32_t bt_per_b;    // band tiles (128 rows of one residue class) per batch row, all heads
  int32_t n_bt;        // B * bt_per_b: the band launch runs a dq and a dk/dv workgroup per tile
  int32_t n_gkv;       // units of the global rows' key work: B * H * ceil(n / 32)
  int32_t n_gq;        // units of the global rows' query work
  int32_t n_gk;        // units of the global keys' work of local rows
  int32_t gslots;      // ceil(max_global / 32)
  int32_t chunks;      // ceil(n / kBwdChunk)
  int32_t gstride;     // max(max_global, 1)
  int32_t dil[LF_MAX_HEADS];
  int32_t btile0[LF_MAX_HEADS + 1];  // first band tile of each head within a batch row
};

// Rows of one band tile of the backward (four waves of 32).
constexpr int kBwdBandRows = 128;

// Launches the backward (preparation with the global lists and row sums,
// the band kernel, then the global-token kernel when there is global work)
// for bf16 or f16 elements.  Returns the hipError_t value as int.
int launch_backward(const BwdParams& bp, void* stream);
int launch_backward_f16(const BwdParams& bp, void* stream);

// Launches the forward kernel of head dim D (32, 64 or 128) for dtype.
// Returns the hipError_t value as int.
int launch_forward(const KernelParams& kp, int dtype, int D, void* stream);

// Workgroups of that forward kernel that the current device holds at once
// (compute units times workgroups per unit), or 0 if the runtime cannot say.
int64_t resident_workgroups(int dtype, int D);

// The units behind the two: lf_attn_kernels.hip compiled once per head dim
// D (LF_KD = D) into namespace d<D>, for bf16 and fp32 elements, and once
// more with LF_HALF_F16 for f16 elements (lf_attn_kernels*.hip).
#define LF_FORWARD_UNITS(ns)                                          \
  namespace ns {                                                      \
  int launch(const KernelParams& kp, int dtype, void* stream);        \
  int64_t resident(int dtype);                                        \
  int launch_f16(const KernelParams& kp, void* stream);               \
  int64_t resident_f16();                                             \
  }
LF_FORWARD_UNITS(d32)
LF_FORWARD_UNITS(d64)
LF_FORWARD_UNITS(d128)
#undef LF_FORWARD_UNITS

// Every argument check of lf_attn_forward except those of the workspace (no
// HIP call); on LF_OK, *workspace_bytes gets the workspace size needed.
lf_status check_forward_args(const lf_attn_params* p, const void* q, const void* k, const void* v,
                             const void* q_g, const void* k_g, const void* v_g, const int8_t* mask,
                             const void* out, const int32_t* row_nnz, size_t* workspace_bytes);

// lf_attn_forward on a caller-provided workspace that is already large
// enough and cleared (arguments validated as by lf_attn_forward).
lf_status forward_with_workspace(const lf_attn_params* p, const void* q, const void* k, const void* v,
                                 const void* q_g, const void* k_g, const void* v_g, const int8_t* mask,
                                 void* out, int32_t* row_nnz, void* workspace, size_t workspace_bytes,
                                 void* stream);

}  // namespace lf
