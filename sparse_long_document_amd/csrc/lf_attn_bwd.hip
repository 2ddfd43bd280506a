// Backward of the Longformer combined attention on gfx950: gradients of q,
// k, v, q_g, k_g, v_g (fp32) from the upstream gradient of the output, the
// forward's output and its saved row log-sum-exp.
//
// The layer is the one the forward computes (sliding window with per-head
// dilation and optional causality, symmetric global attention with its own
// projections: segmentfault Longformer summary, "Sliding window", "Dilated
// sliding window", "Global attention", "Linear projections for global
// attention"; mask values 0/1/2 from the allenai README, "Usage").  Its
// gradient is the chain rule through each row's softmax over its key set
// S(i): with p the row's probabilities, dp_j = <dout_i, v_j> and
// D_i = <dout_i, out_i>, de_j = p_j (dp_j - D_i); dq_i = s sum_j de_j k_j,
// dk_j += s de_j q_i, dv_j += p_j dout_i.
//
// Work is split so that every gradient row has one owner and no atomics,
// except where a few rows collect from the whole sequence:
//   role Q  (local rows):   one wave per 32 query rows of one residue class
//                           of one head; walks the rows' window key blocks
//                           and the global key blocks; writes dq.
//   role KV (local keys):   one wave per 32 keys of one residue class; walks
//                           the query blocks whose windows hold those keys;
//                           writes dk, dv of non-global keys.
//   role GK (global keys):  one wave per 32 global tokens and 512 rows;
//                           adds every local row's dk, dv to the global
//                           tokens' rows (atomic fp32 adds; the rows were
//                           zeroed by the preparation kernel).
//   role GQ (global rows):  one wave per 32 global rows and 512 keys; adds
//                           to dq_g (atomic fp32 adds onto zeroed rows).
//   role GKV (their keys):  one wave per 32 tokens; walks the global rows;
//                           writes dk_g, dv_g.
// Each block step is three or four 32x32x16 MFMA chains: scores and dP from
// row-major fragments loaded straight from HBM, then the gradient product,
// whose transposed operand is read column-wise from rows staged in LDS.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "lf_attn_internal.h"

namespace lf {
namespace {

#if LF_HALF_F16
typedef _Float16 e16;
#else
typedef __bf16 e16;
#endif
typedef e16 e16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsRow = 72;           // staged row: 64 head dims + 16 B of padding
constexpr int kSentinel = -(1 << 29); // residue index of a key outside the row's class
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;              // MI355X: accelerator complex dies, one L2 each
constexpr int kXcdGroup = 32;         // consecutive units kept on one XCD

__device__ __forceinline__ f32x16 mma(e16x8 a, e16x8 b, f32x16 c) {
#if LF_HALF_F16
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}

// Row of accumulator register r of lane half hl in a 32x32 MFMA result.
__device__ __forceinline__ int acc_row(int r, int hl) { return 8 * (r >> 2) + (r & 3) + 4 * hl; }

__device__ __forceinline__ int eff_mask(int8_t m, int use_g) {
  return m == 1 ? 1 : (m == 2 ? (use_g ? 2 : 1) : 0);
}

struct BwdShared {
  e16 st[2][32][kLdsRow];  // rows staged for the column-wise operand
  int4 info[32];           // current block's slots: position, residue index, mask type
  float2 stat[32];         // current block's query rows: log2-domain lse, D
  int opos[32];            // positions of the wave's own 32 keys
};

// Slot code from a block description: a token's raw mask byte (0..255), or
// 256 + a type decided without the mask.  The type is taken when the block
// is used, so that the mask byte's load is waited for one step later.
__device__ __forceinline__ int slot_type(int pos, int code, int use_g) {
  return pos < 0 ? 0 : (code >= 256 ? code - 256 : eff_mask((int8_t)code, use_g));
}

__device__ __forceinline__ e16x8 ld8(const e16* p) { return *reinterpret_cast<const e16x8*>(p); }

__device__ __forceinline__ e16x8 zero8() {
  e16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (e16)0.f;
  return z;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = 0.f;
  return z;
}

// Row fragment: lane (c, hl) holds head dims 16 s + 8 hl .. + 7 of row c, the
// operand layout of the 32x32x16 MFMA with the row as M (A) or N (B).
__device__ __forceinline__ void load_frag(e16x8 (&f)[4], const e16* row, bool ok, int hl) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = ok ? ld8(row + 16 * s + 8 * hl) : zero8();
}

// Zero a fragment whose row takes no part (a mask-0 token may hold any
// values); applied when the block is used, so that the load itself need not
// wait for the mask byte.
__device__ __forceinline__ void keep_frag(e16x8 (&f)[4], bool ok) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = ok ? f[s] : zero8();
}

__device__ __forceinline__ void stage_frag(BwdShared& sh, int which, int c, int hl, const e16x8 (&f)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) *reinterpret_cast<e16x8*>(&sh.st[which][c][16 * s + 8 * hl]) = f[s];
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Column operand of k-step t for head dims 32 half .. + 31: lane (c, hl)
// gets staged rows 16 t + 8 (j / 4) + 4 hl + j % 4 (j = 0..7) at column
// 32 half + c -- the rows a 32x32 result holds in its registers 8 t .. + 7.
// Two ds_read_b64_tr_b16: within each group of 16 lanes, lane 4 e + q points
// at row base + e, columns 16 (group & 1) + 4 q .. + 3, and lane i receives
// column 16 (group & 1) + i of the four rows.
__device__ __forceinline__ e16x8 col_frag(const BwdShared& sh, int which, int t, int lane, int half) {
  const int g = lane >> 4, i = lane & 15;
  const int row = 16 * t + 4 * (g >> 1) + (i >> 2);
  const int col = 32 * half + 16 * (g & 1) + 4 * (i & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)&sh.st[which][row][col]);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)&sh.st[which][row + 8][col]);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(e16x8, v);
}

__device__ __forceinline__ bool in_win(int qt, int kt, int w, int causal) {
  const int d = qt - kt;
  return causal ? (d >= 0 && d <= w) : (d >= -w && d <= w);
}

// Query-owning wave: 32 query rows (lane c's row at qpos, residue index qt,
// type qty), nblk key blocks described by keyof(j, slot) -> (pos, t, slot code),
// membership member(qty, qt, kty, kt).  Returns dq^T in acc: lane (c, hl)
// holds head dims 32 half + acc_row(r, hl) of query c in acc[half][r].
// geom(j) is a wave-uniform claim that every (query, key) pair of block j
// lies in the relation when both are of the right type: then, if every key
// and query slot is of that type, the block needs no per-element test.
template <class KeyOf, class Member, class Geom>
__device__ void q_owner(const BwdParams& p, BwdShared& sh, size_t rs, const e16* qb, const e16* dob,
                        const e16* kb, const e16* vb, int qpos, int qt, int qty, float lse2, float dd,
                        int nblk, KeyOf keyof, Member member, Geom geom, int want_q, int want_k,
                        f32x16 (&acc)[2]) {
  const bool rows_ok = __all(qty == want_q);
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  e16x8 qf[4], df[4];
  load_frag(qf, qb + (size_t)(qty ? qpos : 0) * rs, qty != 0, hl);
  load_frag(df, dob + (size_t)(qty ? qpos : 0) * rs, qty != 0, hl);
  acc[0] = zero16();
  acc[1] = zero16();
  int kpos = -1, kt = 0, kcode = 0;
  e16x8 kf[4], vf[4];
  if (nblk > 0) {
    keyof(0, c, kpos, kt, kcode);
    load_frag(kf, kb + (size_t)(kpos >= 0 ? kpos : 0) * rs, kpos >= 0, hl);
    load_frag(vf, vb + (size_t)(kpos >= 0 ? kpos : 0) * rs, kpos >= 0, hl);
  }
  for (int j = 0; j < nblk; ++j) {
    const int kty = slot_type(kpos, kcode, p.use_globals);
    keep_frag(kf, kty != 0);
    keep_frag(vf, kty != 0);
    if (hl == 0) sh.info[c] = make_int4(kpos, kt, kty, 0);
    stage_frag(sh, 0, c, hl, kf);
    __syncthreads();
    // the next block's rows fly during this block's products: their loads
    // depend on positions only, not on the mask bytes loaded beside them
    int npos = -1, nt = 0, ncode = 0;
    if (j + 1 < nblk) keyof(j + 1, c, npos, nt, ncode);
    e16x8 nkf[4], nvf[4];
    load_frag(nkf, kb + (size_t)(npos >= 0 ? npos : 0) * rs, npos >= 0, hl);
    load_frag(nvf, vb + (size_t)(npos >= 0 ? npos : 0) * rs, npos >= 0, hl);
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      S = mma(kf[s], qf[s], S);
      dP = mma(vf[s], df[s], dP);
    }
    e16x8 ds8[2];
    if (rows_ok && geom(j) && __all(want_k < 0 ? kty != 0 : kty == want_k)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(p.c * S[r] - lse2);
        ds8[r >> 3][r & 7] = (e16)(pr * (dP[r] - dd));
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int4 ki = sh.info[acc_row(r, hl)];
        const bool ok = member(qty, qt, ki.z, ki.y);
        const float pr = ok ? __builtin_amdgcn_exp2f(p.c * S[r] - lse2) : 0.f;
        ds8[r >> 3][r & 7] = (e16)(ok ? pr * (dP[r] - dd) : 0.f);
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[half] = mma(col_frag(sh, 0, t, lane, half), ds8[t], acc[half]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = nkf[s];
      vf[s] = nvf[s];
    }
    kpos = npos;
    kt = nt;
    kcode = ncode;
  }
}

// Key-owning wave: 32 keys (lane c's key at kpos, residue index kt, type
// kty), nblk query blocks described by rowof(j, slot) -> (pos, t, slot code).
// Returns dk^T-free results: acc_k[half][r], acc_v[half][r] hold head dim
// 32 half + c of own key acc_row(r, hl).
template <class RowOf, class Member, class Geom>
__device__ void kv_owner(const BwdParams& p, BwdShared& sh, size_t rs, const e16* kb, const e16* vb,
                         const e16* qb, const e16* dob, const float* lse_bh, const float* d_bh, int kpos,
                         int kt, int kty, int nblk, RowOf rowof, Member member, Geom geom, int want_q,
                         int want_k, f32x16 (&acc_k)[2], f32x16 (&acc_v)[2]) {
  const bool keys_ok = __all(want_k < 0 ? kty != 0 : kty == want_k);
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  e16x8 kf[4], vf[4];
  load_frag(kf, kb + (size_t)(kty ? kpos : 0) * rs, kty != 0, hl);
  load_frag(vf, vb + (size_t)(kty ? kpos : 0) * rs, kty != 0, hl);
  acc_k[0] = acc_k[1] = acc_v[0] = acc_v[1] = zero16();
  int qpos = -1, qt = 0, qcode = 0;
  float ql = 0.f, qd = 0.f;
  e16x8 qf[4], df[4];
  auto fetch = [&](int j, int& pos, int& tt, int& code, float& l2, float& dd, e16x8 (&a)[4], e16x8 (&b)[4]) {
    pos = -1;
    tt = 0;
    code = 0;
    if (j < nblk) rowof(j, c, pos, tt, code);
    // loads depend on the position only; the mask type applies at use
    l2 = pos >= 0 ? lse_bh[pos] : 0.f;
    dd = pos >= 0 ? d_bh[pos] : 0.f;
    load_frag(a, qb + (size_t)(pos >= 0 ? pos : 0) * rs, pos >= 0, hl);
    load_frag(b, dob + (size_t)(pos >= 0 ? pos : 0) * rs, pos >= 0, hl);
  };
  if (nblk > 0) fetch(0, qpos, qt, qcode, ql, qd, qf, df);
  for (int j = 0; j < nblk; ++j) {
    const int qty = slot_type(qpos, qcode, p.use_globals);
    keep_frag(qf, qty != 0);
    keep_frag(df, qty != 0);
    if (hl == 0) {
      sh.info[c] = make_int4(qpos, qt, qty, 0);
      sh.stat[c] = qty ? make_float2(ql * kLog2e, qd) : make_float2(0.f, 0.f);
    }
    stage_frag(sh, 0, c, hl, qf);
    stage_frag(sh, 1, c, hl, df);
    __syncthreads();
    int npos, nt, ncode;
    float nl, nd;
    e16x8 nqf[4], ndf[4];
    fetch(j + 1, npos, nt, ncode, nl, nd, nqf, ndf);
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      S = mma(qf[s], kf[s], S);
      dP = mma(df[s], vf[s], dP);
    }
    e16x8 p8[2], ds8[2];
    if (keys_ok && geom(j) && __all(qty == want_q)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float2 st = sh.stat[acc_row(r, hl)];
        const float pr = __builtin_amdgcn_exp2f(p.c * S[r] - st.x);
        p8[r >> 3][r & 7] = (e16)pr;
        ds8[r >> 3][r & 7] = (e16)(pr * (dP[r] - st.y));
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, hl);
        const int4 qi = sh.info[row];
        const float2 st = sh.stat[row];
        const bool ok = member(qi.z, qi.y, kty, kt);
        const float pr = ok ? __builtin_amdgcn_exp2f(p.c * S[r] - st.x) : 0.f;
        p8[r >> 3][r & 7] = (e16)pr;
        ds8[r >> 3][r & 7] = (e16)(ok ? pr * (dP[r] - st.y) : 0.f);
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc_v[half] = mma(p8[t], col_frag(sh, 1, t, lane, half), acc_v[half]);
        acc_k[half] = mma(ds8[t], col_frag(sh, 0, t, lane, half), acc_k[half]);
      }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[s] = nqf[s];
      df[s] = ndf[s];
    }
    qpos = npos;
    qt = nt;
    qcode = ncode;
    ql = nl;
    qd = nd;
  }
}

// Residue tile of a batch row's role-Q / role-KV work: head, residue class,
// first residue index and class length.
struct ResTile {
  int h, r, t0, len, d;
};

__device__ __forceinline__ ResTile decode_res(const BwdParams& p, int idx) {
  ResTile t;
  int h = 0;
  while (h + 1 < p.H && p.tile0[h + 1] <= idx) ++h;
  const int d = p.dil[h];
  const int local = idx - p.tile0[h];
  t.h = h;
  t.d = d;
  t.r = local / p.rtiles[h];
  t.t0 = (local % p.rtiles[h]) * 32;
  t.len = t.r < p.n ? (p.n - t.r + d - 1) / d : 0;
  return t;
}

__device__ __forceinline__ void store_f4(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}

__device__ void bwd_body(const BwdParams& p) {
  __shared__ BwdShared sh;
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const int n = p.n;
  const size_t rs = (size_t)p.H * 64;
  // Workgroups go to the 8 XCDs round-robin (id % 8).  Remap so that groups
  // of kXcdGroup consecutive units run on one XCD, the groups dealt to the
  // XCDs in turn: neighbouring tiles share most of their window rows, which
  // then stay in that XCD's L2 instead of being fetched from HBM by every
  // XCD, and every XCD still gets an even share of each role.  A bijection
  // on [0, 8 * kXcdGroup * full); the remainder keeps its index.
  int bid = blockIdx.x;
  {
    const int span = kXcds * kXcdGroup;
    if (bid < (int)(gridDim.x / span) * span) {
      const int x = bid % kXcds, s = bid / kXcds;
      bid = ((s / kXcdGroup) * kXcds + x) * kXcdGroup + s % kXcdGroup;
    }
  }
  const e16* Q = reinterpret_cast<const e16*>(p.q);
  const e16* K = reinterpret_cast<const e16*>(p.k);
  const e16* V = reinterpret_cast<const e16*>(p.v);
  const e16* QG = reinterpret_cast<const e16*>(p.qg);
  const e16* KG = reinterpret_cast<const e16*>(p.kg);
  const e16* VG = reinterpret_cast<const e16*>(p.vg);
  const e16* DO = reinterpret_cast<const e16*>(p.dout);
  const int w = p.w, causal = p.causal, ug = p.use_globals;

  if (bid < 2 * p.n_res) {
    const bool own_q = bid < p.n_res;
    if (!own_q) bid -= p.n_res;
    const int b = bid / p.tiles_per_b;
    const ResTile rt = decode_res(p, bid - b * p.tiles_per_b);
    if (rt.t0 >= rt.len) return;  // a class shorter than the longest owns no rows here
    const size_t boff = (size_t)b * n * rs + (size_t)rt.h * 64;
    const int8_t* mb = p.mask + (size_t)b * n;
    const float* lse_bh = p.lse + ((size_t)b * p.H + rt.h) * n;
    const float* d_bh = p.Dsum + ((size_t)b * p.H + rt.h) * n;
    const int nG = ug ? p.gcount[b] : 0;
    const int32_t* gl = p.glist + (size_t)b * p.gstride;
    // this lane's own slot: query (role Q) or key (role KV) t0 + c of the class
    const int myt = rt.t0 + c;
    const int mypos = myt < rt.len ? rt.r + rt.d * myt : -1;
    const int myty = mypos >= 0 ? eff_mask(mb[mypos], ug) : 0;
    auto res_slot = [&](int t, int& pos, int& tt, int& code) {
      const bool in = t >= 0 && t < rt.len;
      const int sp = in ? rt.r + rt.d * t : 0;
      code = (uint8_t)mb[sp];
      pos = in ? sp : -1;
      tt = t;
    };
    if (own_q) {
      // window keys of the tile's rows, clipped to the class
      const int base = max(rt.t0 - w, 0);
      const int last = min(rt.t0 + 31 + (causal ? 0 : w), rt.len - 1);
      const int nwin = (last - base + 32) / 32;
      const int ngb = (nG + 31) / 32;
      auto keyof = [&](int j, int slot, int& pos, int& tt, int& code) {
        if (j < nwin) {
          res_slot(base + 32 * j + slot, pos, tt, code);
        } else {
          const int g = 32 * (j - nwin) + slot;
          pos = g < nG ? gl[g] : -1;
          const int rel = pos - rt.r;
          tt = (pos >= rt.r && rel % rt.d == 0) ? rel / rt.d : kSentinel;
          // type 6 marks a global-column slot (window slots carry the mask
          // byte's type, 1 or 2)
          code = 256 + 6;
        }
      };
      // window slots: any valid key in W(i); global-column slots (type 6):
      // global keys not already in W(i)
      auto member = [&](int qty, int qt, int kty, int kt) {
        if (qty != 1 || kty == 0) return false;
        return kty == 6 ? !in_win(qt, kt, w, causal) : in_win(qt, kt, w, causal);
      };
      const float lse2 = myty ? lse_bh[mypos] * kLog2e : 0.f;
      const float dd = myty ? d_bh[mypos] : 0.f;
      f32x16 acc[2];
      // a window block is full when its 32 keys lie in every window of the
      // tile's 32 rows: first key >= t0 + 31 - w, last key <= t0 (+ w)
      auto geom = [&](int j) {
        const int k0 = base + 32 * j;
        return j < nwin && k0 >= rt.t0 + 31 - w && k0 + 31 <= rt.t0 + (causal ? 0 : w);
      };
      q_owner(p, sh, rs, Q + boff, DO + boff, K + boff, V + boff, mypos, myt, myty, lse2, dd, nwin + ngb, keyof,
              member, geom, 1, -1, acc);
      if (mypos >= 0) {
        float* dst = p.dq + boff + (size_t)mypos * rs;
        const float sc = myty == 1 ? p.scale : 0.f;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = sc * acc[half][4 * g + e];
            store_f4(dst + 32 * half + 8 * g + 4 * hl, v4);
          }
      }
    } else {
      // rows whose windows hold the tile's keys, clipped to the class
      const int base = causal ? rt.t0 : max(rt.t0 - w, 0);
      const int last = min(rt.t0 + 31 + w, rt.len - 1);
      const int nq = (last - base + 32) / 32;
      auto rowof = [&](int j, int slot, int& pos, int& tt, int& code) { res_slot(base + 32 * j + slot, pos, tt, code); };
      auto member = [&](int qty, int qt, int kty, int kt) { return qty == 1 && kty == 1 && in_win(qt, kt, w, causal); };
      if (hl == 0) sh.opos[c] = (myty == 2) ? -1 : mypos;
      f32x16 ak[2], av[2];
      // a query block is full when its 32 rows' windows all hold the tile's
      // 32 keys: first row >= t0 + 31 - (causal ? 0 : w), last row <= t0 + w
      auto geom = [&](int j) {
        const int r0 = base + 32 * j;
        return r0 >= rt.t0 + 31 - (causal ? 0 : w) && r0 + 31 <= rt.t0 + w;
      };
      kv_owner(p, sh, rs, K + boff, V + boff, Q + boff, DO + boff, lse_bh, d_bh, mypos, myt, myty, nq, rowof,
               member, geom, 1, 1, ak, av);
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = sh.opos[acc_row(r, hl)];
        if (pos < 0) continue;
        float* dk = p.dk + boff + (size_t)pos * rs;
        float* dv = p.dv + boff + (size_t)pos * rs;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          dk[32 * half + c] = p.scale * ak[half][r];
          dv[32 * half + c] = av[half][r];
        }
      }
    }
    return;
  }
  bid -= 2 * p.n_res;

  // global roles: GKV (key blocks of every (b, h)), then GQ and GK
  if (bid < p.n_gkv) {
    const int kblocks = (n + 31) / 32;
    const int bh = bid / kblocks;
    const int kb0 = (bid - bh * kblocks) * 32;
    const int b = bh / p.H, h = bh - b * p.H;
    const size_t boff = (size_t)b * n * rs + (size_t)h * 64;
    const int8_t* mb = p.mask + (size_t)b * n;
    const int nG = p.gcount[b];
    const int32_t* gl = p.glist + (size_t)b * p.gstride;
    const int mypos = kb0 + c < n ? kb0 + c : -1;
    const int myty = mypos >= 0 ? eff_mask(mb[mypos], 1) : 0;
    auto rowof = [&](int j, int slot, int& pos, int& tt, int& code) {
      const int g = 32 * j + slot;
      pos = g < nG ? gl[g] : -1;
      tt = 0;
      code = 256 + 2;
    };
    auto member = [](int qty, int, int kty, int) { return qty == 2 && kty != 0; };
    if (hl == 0) sh.opos[c] = mypos;
    f32x16 ak[2], av[2];
    kv_owner(p, sh, rs, KG + boff, VG + boff, QG + boff, DO + boff, p.lse + (size_t)bh * n, p.Dsum + (size_t)bh * n,
             mypos, 0, myty, (nG + 31) / 32, rowof, member, [](int) { return true; }, 2, -1, ak, av);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pos = sh.opos[acc_row(r, hl)];
      if (pos < 0) continue;
      float* dk = p.dkg + boff + (size_t)pos * rs;
      float* dv = p.dvg + boff + (size_t)pos * rs;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        dk[32 * half + c] = p.scale * ak[half][r];
        dv[32 * half + c] = av[half][r];
      }
    }
    return;
  }
  bid -= p.n_gkv;

  // GQ and GK: (b, h, block of 32 global slots, 512-token chunk)
  const bool gq = bid < p.n_gq;
  if (!gq) bid -= p.n_gq;
  const int per_bh = p.gslots * p.chunks;
  const int bh = bid / per_bh;
  const int rem = bid - bh * per_bh;
  const int sb = rem / p.chunks;
  const int ch = rem - sb * p.chunks;
  const int b = bh / p.H, h = bh - b * p.H;
  const int nG = p.gcount[b];
  if (32 * sb >= nG) return;
  const size_t boff = (size_t)b * n * rs + (size_t)h * 64;
  const int8_t* mb = p.mask + (size_t)b * n;
  const int32_t* gl = p.glist + (size_t)b * p.gstride;
  const int c0 = ch * kBwdChunk;
  const int nblk = (min(kBwdChunk, n - c0) + 31) / 32;
  const int g = 32 * sb + c;
  const int gpos = g < nG ? gl[g] : -1;
  const int gty = g < nG ? 2 : 0;
  auto tok = [&](int j, int slot, int& pos, int& tt, int& code) {
    const int t = c0 + 32 * j + slot;
    pos = t < n ? t : -1;
    tt = 0;
    code = (uint8_t)mb[t < n ? t : 0];
  };
  const float* lse_bh = p.lse + (size_t)bh * n;
  const float* d_bh = p.Dsum + (size_t)bh * n;
  if (gq) {
    auto member = [](int qty, int, int kty, int) { return qty == 2 && kty != 0; };
    const float lse2 = gty ? lse_bh[gpos] * kLog2e : 0.f;
    const float dd = gty ? d_bh[gpos] : 0.f;
    f32x16 acc[2];
    q_owner(p, sh, rs, QG + boff, DO + boff, KG + boff, VG + boff, gpos, 0, gty, lse2, dd, nblk, tok, member,
            [](int) { return true; }, 2, -1, acc);
    if (gpos >= 0) {
      float* dst = p.dqg + boff + (size_t)gpos * rs;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          unsafeAtomicAdd(dst + 32 * half + acc_row(r, hl), p.scale * acc[half][r]);
    }
  } else {
    auto member = [](int qty, int, int kty, int) { return qty == 1 && kty == 2; };
    if (hl == 0) sh.opos[c] = gpos;
    f32x16 ak[2], av[2];
    kv_owner(p, sh, rs, K + boff, V + boff, Q + boff, DO + boff, lse_bh, d_bh, gpos, 0, gty, nblk, tok, member,
             [](int) { return true; }, 1, 2, ak, av);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pos = sh.opos[acc_row(r, hl)];
      if (pos < 0) continue;
      float* dk = p.dk + boff + (size_t)pos * rs;
      float* dv = p.dv + boff + (size_t)pos * rs;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        unsafeAtomicAdd(dk + 32 * half + c, p.scale * ak[half][r]);
        unsafeAtomicAdd(dv + 32 * half + c, av[half][r]);
      }
    }
  }
}

// Global list of batch row b, ascending, by one workgroup of 256 threads:
// each thread tests 16 mask bytes, a workgroup-wide prefix sum places its
// hits.  At most max_global entries are kept (more sets the status bit).
__device__ void glist_body(const BwdParams& p, int b) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int8_t* mb = p.mask + (size_t)b * p.n;
  int32_t* gl = p.glist + (size_t)b * p.gstride;
  int total = 0;
  for (int base = 0; base < p.n; base += 256 * 16) {
    const int i0 = base + 16 * tid;
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (i0 + k < p.n && mb[i0 + k] == 2) bits |= 1u << k;
    const int cnt = __popc(bits);
    int x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int off = total + x - cnt;
    for (int u = 0; u < wv; ++u) off += wsum[u];
    while (bits) {
      const int k = __ffs(bits) - 1;
      bits &= bits - 1;
      if (off < p.max_global) gl[off] = i0 + k;
      ++off;
    }
    total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) {
    p.gcount[b] = min(total, p.max_global);
    if (total > p.max_global) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
  }
}

// Preparation launch: with global work, workgroups 0 .. B-1 build the global
// lists; the rest take one row (b, i, h) per 16 lanes: D = <dout, out>; dq_g
// zeroed; dk, dv of global tokens zeroed (global-key work adds to them);
// dk_g, dv_g zeroed when no global work runs.
__device__ void prep_body(const BwdParams& p) {
  const int nlist = p.use_globals ? p.B : 0;
  if ((int)blockIdx.x < nlist) {
    glist_body(p, blockIdx.x);
    return;
  }
  const size_t rows = (size_t)p.B * p.n * p.H;
  const size_t row = (size_t)(blockIdx.x - nlist) * (blockDim.x / 16) + (threadIdx.x >> 4);
  if (row >= rows) return;
  const int q4 = threadIdx.x & 15;
  const size_t bi = row / p.H;
  const int h = (int)(row - bi * p.H);
  const int b = (int)(bi / p.n);
  const int i = (int)(bi - (size_t)b * p.n);
  const size_t off = row * 64 + 4 * q4;
  const e16* o = reinterpret_cast<const e16*>(p.out) + off;
  const e16* d = reinterpret_cast<const e16*>(p.dout) + off;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += (float)o[e] * (float)d[e];
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
  if (q4 == 0) p.Dsum[((size_t)b * p.H + h) * p.n + i] = s;
  const float z[4] = {0.f, 0.f, 0.f, 0.f};
  store_f4(p.dqg + off, z);
  if (p.use_globals) {
    if (eff_mask(p.mask[bi], 1) == 2) {
      store_f4(p.dk + off, z);
      store_f4(p.dv + off, z);
    }
  } else {
    store_f4(p.dkg + off, z);
    store_f4(p.dvg + off, z);
  }
}

#if LF_HALF_F16
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void lf_attn_bwd_f16(const BwdParams p) { bwd_body(p); }
__global__ __launch_bounds__(256) void lf_attn_bwd_prep_f16(const BwdParams p) { prep_body(p); }
#else
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void lf_attn_bwd_bf16(const BwdParams p) { bwd_body(p); }
__global__ __launch_bounds__(256) void lf_attn_bwd_prep_bf16(const BwdParams p) { prep_body(p); }
#endif

}  // namespace

#if LF_HALF_F16
int launch_backward_f16(const BwdParams& bp, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t rows = (size_t)bp.B * bp.n * bp.H;
  const unsigned nlist = bp.use_globals ? (unsigned)bp.B : 0u;
  hipLaunchKernelGGL(lf_attn_bwd_prep_f16, dim3(nlist + (unsigned)((rows + 15) / 16)), dim3(256), 0, s, bp);
  hipLaunchKernelGGL(lf_attn_bwd_f16, dim3(2 * bp.n_res + bp.n_gkv + bp.n_gq + bp.n_gk), dim3(64), 0, s, bp);
  return (int)hipGetLastError();
}
#else
int launch_backward(const BwdParams& bp, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (bp.dtype == LF_F16) return launch_backward_f16(bp, stream);
  const size_t rows = (size_t)bp.B * bp.n * bp.H;
  const unsigned nlist = bp.use_globals ? (unsigned)bp.B : 0u;
  hipLaunchKernelGGL(lf_attn_bwd_prep_bf16, dim3(nlist + (unsigned)((rows + 15) / 16)), dim3(256), 0, s, bp);
  hipLaunchKernelGGL(lf_attn_bwd_bf16, dim3(2 * bp.n_res + bp.n_gkv + bp.n_gq + bp.n_gk), dim3(64), 0, s, bp);
  return (int)hipGetLastError();
}
#endif

}  // namespace lf
