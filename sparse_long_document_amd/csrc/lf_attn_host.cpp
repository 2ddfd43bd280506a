// Host side of the C ABI declared in include/lf_attn.h: argument
// validation (before any HIP call), workspace layout, launch planning.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "lf_attn.h"
#include "lf_attn_internal.h"
#include "lf_attn_bwd_internal.h"
#include "lf_proj_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int use_globals = 0;
  int S = 0;
  int64_t tiles_per_b = 0;
  int dil[LF_MAX_HEADS];
  int tile0[LF_MAX_HEADS + 1];
  size_t elem = 0;
  size_t tensor_bytes = 0;
  size_t ws_tickets_off = 0;
  size_t ws_partials_off = 0;
  size_t ws_bytes = 0;
};

// Validates the parameter block and derives the launch plan.  No HIP calls.
lf_status make_plan(const lf_attn_params* p, Plan& pl) {
  if (!p) return LF_ERR_INVALID_ARG;
  if (p->B <= 0 || p->n <= 0 || p->H <= 0 || p->D <= 0) return LF_ERR_INVALID_ARG;
  if (p->window < 0) return LF_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return LF_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale) || p->scale < 0.f) return LF_ERR_INVALID_ARG;
  if (p->max_global < 0) return LF_ERR_INVALID_ARG;
  if (p->D != 32 && p->D != 64 && p->D != 128) return LF_ERR_UNSUPPORTED;
  if (p->dtype != LF_F32 && p->dtype != LF_BF16 && p->dtype != LF_F16) return LF_ERR_UNSUPPORTED;
  if (p->H > LF_MAX_HEADS || p->max_global > LF_MAX_GLOBAL || p->n > LF_MAX_SEQ) return LF_ERR_UNSUPPORTED;
  const int64_t tokens = (int64_t)p->B * p->n;
  if (tokens > INT32_MAX) return LF_ERR_UNSUPPORTED;

  pl.elem = p->dtype == LF_F32 ? 4 : 2;
  pl.tensor_bytes = (size_t)tokens * p->H * p->D * pl.elem;
  // The kernels address one batch row of a tensor with 32-bit byte offsets.
  if ((int64_t)p->n * p->H * p->D * pl.elem > (int64_t)LF_MAX_ROW_BYTES) return LF_ERR_UNSUPPORTED;

  int64_t tiles = 0;
  for (int h = 0; h < p->H; ++h) {
    const int d = p->dilation ? p->dilation[h] : 1;
    if (d < 1) return LF_ERR_INVALID_ARG;
    pl.dil[h] = d;
    pl.tile0[h] = (int)tiles;
    // positions r, r+d, ... < n: residues r < n % d have n/d + 1 of them
    const int64_t qn = p->n / d, rm = p->n % d;
    const int64_t T1 = (qn + 1 + lf::kTileQ - 1) / lf::kTileQ;
    const int64_t T0 = (qn + lf::kTileQ - 1) / lf::kTileQ;
    tiles += rm * T1 + (d - rm) * T0;
    if (tiles > (int64_t)1 << 26) return LF_ERR_UNSUPPORTED;
  }
  pl.tile0[p->H] = (int)tiles;
  pl.tiles_per_b = tiles;
  if (tiles * p->B > (int64_t)1 << 30) return LF_ERR_UNSUPPORTED;

  pl.use_globals = (p->causal == 0 && p->max_global > 0) ? 1 : 0;
  // records are laid out for the split count of the short chunk, the most
  pl.S = (p->n + lf::kGlobalChunkShort - 1) / lf::kGlobalChunkShort;
  const size_t bh = (size_t)p->B * p->H;
  pl.ws_tickets_off = kAlign;
  pl.ws_partials_off = pl.ws_tickets_off + align_up(bh * sizeof(int32_t), kAlign);
  size_t partial_bytes = 0;
  if (pl.use_globals)
    partial_bytes = bh * (size_t)p->max_global * (size_t)pl.S * lf::partial_stride(p->D) * sizeof(float);
  pl.ws_bytes = pl.ws_partials_off + align_up(partial_bytes, kAlign);
  return LF_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

size_t lf_attn_workspace_bytes(const lf_attn_params* p) {
  Plan pl;
  if (make_plan(p, pl) != LF_OK) return 0;
  return pl.ws_bytes;
}

lf_status lf_attn_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < kAlign) return LF_ERR_WORKSPACE;
  const hipError_t e = hipMemsetAsync(workspace, 0, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LF_OK : LF_ERR_HIP;
}

}  // extern "C"

namespace {

// Every argument check of the forward (no HIP call); with_ws = false skips
// the checks of the workspace (a library-owned one cannot overlap the
// caller's buffers).
lf_status check_forward(const lf_attn_params* p, Plan& pl, const void* q, const void* k, const void* v,
                        const void* q_g, const void* k_g, const void* v_g, const int8_t* mask, const void* out,
                        const int32_t* row_nnz, const float* lse, const void* workspace, size_t workspace_bytes,
                        bool with_ws) {
  const lf_status st = make_plan(p, pl);
  if (st != LF_OK) return st;
  if (!q || !k || !v || !mask || !out) return LF_ERR_INVALID_ARG;
  if (!q_g) q_g = q;
  if (!k_g) k_g = k;
  if (!v_g) v_g = v;
  const size_t tb = pl.tensor_bytes;
  const size_t mb = (size_t)p->B * p->n;
  const size_t nb = (size_t)p->B * p->H * p->n * sizeof(int32_t);
  const void* ins[6] = {q, k, v, q_g, k_g, v_g};
  for (const void* in : ins)
    if (overlaps(out, tb, in, tb)) return LF_ERR_INVALID_ARG;
  if (overlaps(out, tb, mask, mb)) return LF_ERR_INVALID_ARG;
  if (row_nnz) {
    for (const void* in : ins)
      if (overlaps(row_nnz, nb, in, tb)) return LF_ERR_INVALID_ARG;
    if (overlaps(row_nnz, nb, out, tb) || overlaps(row_nnz, nb, mask, mb)) return LF_ERR_INVALID_ARG;
  }
  if (lse) {
    const size_t lb = (size_t)p->B * p->H * p->n * sizeof(float);
    for (const void* in : ins)
      if (overlaps(lse, lb, in, tb)) return LF_ERR_INVALID_ARG;
    if (overlaps(lse, lb, out, tb) || overlaps(lse, lb, mask, mb)) return LF_ERR_INVALID_ARG;
    if (row_nnz && overlaps(lse, lb, row_nnz, nb)) return LF_ERR_INVALID_ARG;
  }
  if (!with_ws) return LF_OK;
  if (!workspace || workspace_bytes < pl.ws_bytes) return LF_ERR_WORKSPACE;
  // the kernel writes tickets and partial records into the workspace: it
  // may overlap no input and no output
  for (const void* in : ins)
    if (overlaps(workspace, pl.ws_bytes, in, tb)) return LF_ERR_INVALID_ARG;
  if (overlaps(workspace, pl.ws_bytes, mask, mb) || overlaps(workspace, pl.ws_bytes, out, tb))
    return LF_ERR_INVALID_ARG;
  if (row_nnz && overlaps(workspace, pl.ws_bytes, row_nnz, nb)) return LF_ERR_INVALID_ARG;
  if (lse && overlaps(workspace, pl.ws_bytes, lse, (size_t)p->B * p->H * p->n * sizeof(float)))
    return LF_ERR_INVALID_ARG;
  return LF_OK;
}

lf_status forward_impl(const lf_attn_params* p, const void* q, const void* k, const void* v, const void* q_g,
                       const void* k_g, const void* v_g, const int8_t* mask, void* out, int32_t* row_nnz,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  const lf_status st =
      check_forward(p, pl, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, lse, workspace, workspace_bytes, true);
  if (st != LF_OK) return st;
  if (!q_g) q_g = q;
  if (!k_g) k_g = k;
  if (!v_g) v_g = v;

  lf::KernelParams kp;
  std::memset(&kp, 0, sizeof(kp));
  kp.q = q;
  kp.k = k;
  kp.v = v;
  kp.qg = q_g;
  kp.kg = k_g;
  kp.vg = v_g;
  kp.mask = mask;
  kp.out = out;
  kp.row_nnz = row_nnz;
  kp.lse = lse;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  kp.status = reinterpret_cast<int32_t*>(ws);
  kp.tickets = reinterpret_cast<int32_t*>(ws + pl.ws_tickets_off);
  kp.partials = reinterpret_cast<float*>(ws + pl.ws_partials_off);
  kp.B = p->B;
  kp.n = p->n;
  kp.H = p->H;
  kp.w = p->window;
  kp.causal = p->causal;
  kp.max_global = p->max_global;
  kp.use_globals = pl.use_globals;
  const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / std::sqrt((double)p->D);
  kp.c = (float)(scale * 1.4426950408889634);  // log2(e)
  kp.tiles_per_b = (int32_t)pl.tiles_per_b;
  kp.n_band = (int32_t)(pl.tiles_per_b * p->B);
  // Global-row splits: short chunks when band tiles and short splits are all
  // resident at once, long ones otherwise (both fit the workspace).
  int chunk = lf::kGlobalChunkLong;
  if (pl.use_globals) {
    const int64_t resident = lf::resident_workgroups(p->dtype, p->D);
    const int64_t short_splits = (int64_t)p->B * p->H * pl.S;
    if (resident > 0 && (int64_t)kp.n_band + short_splits <= resident) chunk = lf::kGlobalChunkShort;
  }
  kp.chunk = chunk;
  kp.S = (p->n + chunk - 1) / chunk;
  kp.n_glob = pl.use_globals ? p->B * p->H * kp.S : 0;
  for (int h = 0; h < p->H; ++h) {
    kp.dil[h] = pl.dil[h];
    kp.tile0[h] = pl.tile0[h];
  }
  kp.tile0[p->H] = pl.tile0[p->H];
  kp.uni_dil = pl.dil[0];
  for (int h = 1; h < p->H; ++h)
    if (pl.dil[h] != pl.dil[0]) kp.uni_dil = 0;
  kp.tiles_per_head = kp.uni_dil > 0 ? pl.tile0[1] - pl.tile0[0] : 0;
  const int e = lf::launch_forward(kp, p->dtype, p->D, stream);
  return e == 0 ? LF_OK : LF_ERR_HIP;
}

}  // namespace

namespace lf {

lf_status check_forward_args(const lf_attn_params* p, const void* q, const void* k, const void* v,
                             const void* q_g, const void* k_g, const void* v_g, const int8_t* mask,
                             const void* out, const int32_t* row_nnz, size_t* workspace_bytes) {
  Plan pl;
  const lf_status st =
      check_forward(p, pl, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, nullptr, nullptr, 0, false);
  if (st == LF_OK && workspace_bytes) *workspace_bytes = pl.ws_bytes;
  return st;
}

// The forward with a workspace the caller has already sized and cleared
// (used by the no-allocation entry point).
lf_status forward_with_workspace(const lf_attn_params* p, const void* q, const void* k, const void* v,
                                 const void* q_g, const void* k_g, const void* v_g, const int8_t* mask,
                                 void* out, int32_t* row_nnz, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return forward_impl(p, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, nullptr, workspace, workspace_bytes, stream);
}

}  // namespace lf

extern "C" {

lf_status lf_attn_forward(const lf_attn_params* p, const void* q, const void* k, const void* v,
                          const void* q_g, const void* k_g, const void* v_g, const int8_t* mask, void* out,
                          int32_t* row_nnz, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(p, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, nullptr, workspace, workspace_bytes, stream);
}

lf_status lf_attn_forward_lse(const lf_attn_params* p, const void* q, const void* k, const void* v,
                              const void* q_g, const void* k_g, const void* v_g, const int8_t* mask, void* out,
                              int32_t* row_nnz, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!lse) return LF_ERR_INVALID_ARG;
  return forward_impl(p, q, k, v, q_g, k_g, v_g, mask, out, row_nnz, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

struct BwdLayout {
  size_t gcount_off = 0, glist_off = 0, dsum_off = 0, lse2_off = 0, bytes = 0;
  int gstride = 1;
};

BwdLayout bwd_layout(const lf_attn_params* p) {
  BwdLayout L;
  L.gstride = p->max_global > 0 ? p->max_global : 1;
  L.gcount_off = kAlign;
  L.glist_off = L.gcount_off + align_up((size_t)p->B * sizeof(int32_t), kAlign);
  L.dsum_off = L.glist_off + align_up((size_t)p->B * L.gstride * sizeof(int32_t), kAlign);
  L.lse2_off = L.dsum_off + align_up((size_t)p->B * p->H * p->n * sizeof(float), kAlign);
  L.bytes = L.lse2_off + align_up((size_t)p->B * p->H * p->n * sizeof(float), kAlign);
  return L;
}

}  // namespace

extern "C" {

size_t lf_attn_backward_workspace_bytes(const lf_attn_params* p) {
  Plan pl;
  if (make_plan(p, pl) != LF_OK || p->D != LF_BWD_HEAD_DIM) return 0;
  return bwd_layout(p).bytes;
}

lf_status lf_attn_backward(const lf_attn_params* p, const void* q, const void* k, const void* v,
                           const void* q_g, const void* k_g, const void* v_g, const int8_t* mask,
                           const void* out, const void* dout, const float* lse, float* dq, float* dk, float* dv,
                           float* dq_g, float* dk_g, float* dv_g, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Plan pl;
  const lf_status st = make_plan(p, pl);
  if (st != LF_OK) return st;
  if (p->dtype != LF_BF16 && p->dtype != LF_F16) return LF_ERR_UNSUPPORTED;
  if (p->D != LF_BWD_HEAD_DIM) return LF_ERR_UNSUPPORTED;
  if (!q || !k || !v || !mask || !out || !dout || !lse) return LF_ERR_INVALID_ARG;
  if (!dq || !dk || !dv || !dq_g || !dk_g || !dv_g) return LF_ERR_INVALID_ARG;
  if (!q_g) q_g = q;
  if (!k_g) k_g = k;
  if (!v_g) v_g = v;
  const size_t tb = pl.tensor_bytes;
  const size_t gb = tb / pl.elem * sizeof(float);
  const size_t mb = (size_t)p->B * p->n;
  const size_t lb = (size_t)p->B * p->H * p->n * sizeof(float);
  const BwdLayout L = bwd_layout(p);
  // band tiles: kBwdBandRows consecutive rows of one residue class of one
  // head (positions r, r + d, ...: n / d + 1 of them for r < n % d, else n / d)
  int64_t tiles = 0;
  lf::BwdParams bp;
  std::memset(&bp, 0, sizeof(bp));
  for (int h = 0; h < p->H; ++h) {
    const int d = pl.dil[h];
    const int64_t qn = p->n / d, rm = p->n % d, R = lf::kBwdBandRows;
    bp.dil[h] = d;
    bp.btile0[h] = (int32_t)tiles;
    tiles += rm * ((qn + 1 + R - 1) / R) + (d - rm) * ((qn + R - 1) / R);
  }
  bp.btile0[p->H] = (int32_t)tiles;
  const int64_t gslots = (p->max_global + 31) / 32;
  const int64_t chunks = (p->n + lf::kBwdChunk - 1) / lf::kBwdChunk;
  const int64_t bhn = (int64_t)p->B * p->H;
  const int64_t n_gkv = pl.use_globals ? bhn * ((p->n + 31) / 32) : 0;
  const int64_t n_gq = pl.use_globals ? bhn * gslots * chunks : 0;
  if (2 * (int64_t)p->B * tiles > INT32_MAX || lf::bwd_glob_workgroups(n_gkv, p->B, p->H, gslots, chunks) > INT32_MAX)
    return LF_ERR_UNSUPPORTED;
  if ((int64_t)p->B + ((int64_t)p->B * p->n * p->H + 15) / 16 > INT32_MAX) return LF_ERR_UNSUPPORTED;

  const void* ins[10] = {q, k, v, q_g, k_g, v_g, out, dout, mask, lse};
  const size_t in_bytes[10] = {tb, tb, tb, tb, tb, tb, tb, tb, mb, lb};
  float* outs[6] = {dq, dk, dv, dq_g, dk_g, dv_g};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlaps(outs[i], gb, ins[j], in_bytes[j])) return LF_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], gb, outs[j], gb)) return LF_ERR_INVALID_ARG;
  }
  if (!workspace || workspace_bytes < L.bytes) return LF_ERR_WORKSPACE;
  for (int i = 0; i < 6; ++i)
    if (overlaps(workspace, L.bytes, outs[i], gb)) return LF_ERR_INVALID_ARG;
  for (int j = 0; j < 10; ++j)
    if (overlaps(workspace, L.bytes, ins[j], in_bytes[j])) return LF_ERR_INVALID_ARG;

  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.qg = q_g;
  bp.kg = k_g;
  bp.vg = v_g;
  bp.mask = mask;
  bp.out = out;
  bp.dout = dout;
  bp.lse = lse;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.dqg = dq_g;
  bp.dkg = dk_g;
  bp.dvg = dv_g;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  bp.status = reinterpret_cast<int32_t*>(ws);
  bp.gcount = reinterpret_cast<int32_t*>(ws + L.gcount_off);
  bp.glist = reinterpret_cast<int32_t*>(ws + L.glist_off);
  bp.dneg = reinterpret_cast<float*>(ws + L.dsum_off);
  bp.lneg = reinterpret_cast<float*>(ws + L.lse2_off);
  bp.B = p->B;
  bp.n = p->n;
  bp.H = p->H;
  bp.w = p->window;
  bp.causal = p->causal;
  bp.max_global = p->max_global;
  bp.use_globals = pl.use_globals;
  bp.dtype = p->dtype;
  const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / std::sqrt((double)p->D);
  bp.scale = (float)scale;
  bp.c = (float)(scale * 1.4426950408889634);
  bp.bt_per_b = (int32_t)tiles;
  bp.n_bt = (int32_t)(p->B * tiles);
  bp.n_gkv = (int32_t)n_gkv;
  bp.n_gq = (int32_t)n_gq;
  bp.n_gk = (int32_t)n_gq;
  bp.gslots = (int32_t)gslots;
  bp.chunks = (int32_t)chunks;
  bp.gstride = L.gstride;
  const int e = lf::launch_backward(bp, stream);
  return e == 0 ? LF_OK : LF_ERR_HIP;
}

static lf_status project_impl(int32_t M, int32_t C, int32_t P, int32_t dtype, const void* x, const void* w,
                              const float* bias, const int8_t* mask, uint32_t global_only, void* out, void* stream) {
  if (M <= 0 || C <= 0 || P <= 0) return LF_ERR_INVALID_ARG;
  if (!x || !w || !out) return LF_ERR_INVALID_ARG;
  if (dtype != LF_BF16 && dtype != LF_F16) return LF_ERR_UNSUPPORTED;
  if (C % 64 != 0 || P > LF_MAX_PROJ) return LF_ERR_UNSUPPORTED;
  if (global_only >> P) return LF_ERR_INVALID_ARG;  // a projection beyond P
  if (global_only && !mask) return LF_ERR_INVALID_ARG;
  const int64_t N = (int64_t)P * C;
  if (N > INT32_MAX || (N + 127) / 128 > 65535) return LF_ERR_UNSUPPORTED;
  const size_t xb = (size_t)M * C * 2, wb = (size_t)N * C * 2, ob = (size_t)P * xb, bb = (size_t)N * 4;
  // x and w are addressed through 32-bit buffer offsets; 16-byte loads and
  // stores need 16-byte aligned bases
  if (xb > (size_t)INT32_MAX || wb > (size_t)INT32_MAX) return LF_ERR_UNSUPPORTED;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)out | (uintptr_t)bias) & 15u) return LF_ERR_UNSUPPORTED;
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, w, wb) || (bias && overlaps(out, ob, bias, bb)) ||
      (global_only && overlaps(out, ob, mask, (size_t)M)))
    return LF_ERR_INVALID_ARG;
  lf::ProjParams pp;
  pp.x = x;
  pp.w = w;
  pp.bias = bias;
  pp.out = out;
  pp.M = M;
  pp.C = C;
  pp.N = (int32_t)N;
  pp.dtype = dtype;
  pp.mask = global_only ? mask : nullptr;
  pp.global_only = global_only;
  const int e = lf::launch_project(pp, stream);
  return e == 0 ? LF_OK : LF_ERR_HIP;
}

lf_status lf_attn_project(int32_t M, int32_t C, int32_t P, int32_t dtype, const void* x, const void* w,
                          const float* bias, void* out, void* stream) {
  return project_impl(M, C, P, dtype, x, w, bias, nullptr, 0u, out, stream);
}

lf_status lf_attn_project_global_only(int32_t M, int32_t C, int32_t P, int32_t dtype, const void* x,
                                      const void* w, const float* bias, const int8_t* mask,
                                      uint32_t global_only, void* out, void* stream) {
  return project_impl(M, C, P, dtype, x, w, bias, mask, global_only, out, stream);
}

lf_status lf_attn_device_status(const void* workspace, void* stream, int32_t* status) {
  if (!workspace || !status) return LF_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return LF_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LF_ERR_HIP;
  return LF_OK;
}

const char* lf_status_str(int32_t s) {
  switch (s) {
    case LF_OK: return "ok";
    case LF_ERR_INVALID_ARG: return "invalid argument";
    case LF_ERR_UNSUPPORTED: return "unsupported configuration";
    case LF_ERR_WORKSPACE: return "workspace missing or too small";
    case LF_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
