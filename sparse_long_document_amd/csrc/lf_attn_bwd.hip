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

__device__ __forceinline__ void stage_frag(BwdShared& sh, int which, int c, int hl, const e16x8 (&f)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) *reinterpret_cast<e16x8*>(&sh.st[which][c][16 * s + 8 * hl]) = f[s];
}

// Column operand of k-step t: staged rows 16 t + 8 (j / 4) + 4 hl + j % 4 at
// column col -- the rows a 32x32 result holds in its registers 8 t .. 8 t + 7.
__device__ __forceinline__ e16x8 col_frag(const BwdShared& sh, int which, int t, int hl, int col) {
  e16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = sh.st[which][16 * t + 8 * (j >> 2) + 4 * hl + (j & 3)][col];
  return a;
}

__device__ __forceinline__ bool in_win(int qt, int kt, int w, int causal) {
  const int d = qt - kt;
  return causal ? (d >= 0 && d <= w) : (d >= -w && d <= w);
}

// Query-owning wave: 32 query rows (lane c's row at qpos, residue index qt,
// type qty), nblk key blocks described by keyof(j, slot) -> (pos, t, ty),
// membership member(qty, qt, kty, kt).  Returns dq^T in acc: lane (c, hl)
// holds head dims 32 half + acc_row(r, hl) of query c in acc[half][r].
template <class KeyOf, class Member>
__device__ void q_owner(const BwdParams& p, BwdShared& sh, size_t rs, const e16* qb, const e16* dob,
                        const e16* kb, const e16* vb, int qpos, int qt, int qty, float lse2, float dd,
                        int nblk, KeyOf keyof, Member member, f32x16 (&acc)[2]) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  e16x8 qf[4], df[4];
  load_frag(qf, qb + (size_t)(qty ? qpos : 0) * rs, qty != 0, hl);
  load_frag(df, dob + (size_t)(qty ? qpos : 0) * rs, qty != 0, hl);
  acc[0] = zero16();
  acc[1] = zero16();
  for (int j = 0; j < nblk; ++j) {
    int kpos, kt, kty;
    keyof(j, c, kpos, kt, kty);
    if (hl == 0) sh.info[c] = make_int4(kpos, kt, kty, 0);
    e16x8 kf[4], vf[4];
    load_frag(kf, kb + (size_t)(kty ? kpos : 0) * rs, kty != 0, hl);
    load_frag(vf, vb + (size_t)(kty ? kpos : 0) * rs, kty != 0, hl);
    stage_frag(sh, 0, c, hl, kf);
    __syncthreads();
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      S = mma(kf[s], qf[s], S);
      dP = mma(vf[s], df[s], dP);
    }
    e16x8 ds8[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int4 ki = sh.info[acc_row(r, hl)];
      const bool ok = member(qty, qt, ki.z, ki.y);
      const float pr = ok ? __builtin_amdgcn_exp2f(p.c * S[r] - lse2) : 0.f;
      ds8[r >> 3][r & 7] = (e16)(ok ? pr * (dP[r] - dd) : 0.f);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[half] = mma(col_frag(sh, 0, t, hl, 32 * half + c), ds8[t], acc[half]);
    __syncthreads();
  }
}

// Key-owning wave: 32 keys (lane c's key at kpos, residue index kt, type
// kty), nblk query blocks described by rowof(j, slot) -> (pos, t, ty).
// Returns dk^T-free results: acc_k[half][r], acc_v[half][r] hold head dim
// 32 half + c of own key acc_row(r, hl).
template <class RowOf, class Member>
__device__ void kv_owner(const BwdParams& p, BwdShared& sh, size_t rs, const e16* kb, const e16* vb,
                         const e16* qb, const e16* dob, const float* lse_bh, const float* d_bh, int kpos,
                         int kt, int kty, int nblk, RowOf rowof, Member member, f32x16 (&acc_k)[2],
                         f32x16 (&acc_v)[2]) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  e16x8 kf[4], vf[4];
  load_frag(kf, kb + (size_t)(kty ? kpos : 0) * rs, kty != 0, hl);
  load_frag(vf, vb + (size_t)(kty ? kpos : 0) * rs, kty != 0, hl);
  acc_k[0] = acc_k[1] = acc_v[0] = acc_v[1] = zero16();
  for (int j = 0; j < nblk; ++j) {
    int qpos, qt, qty;
    rowof(j, c, qpos, qt, qty);
    if (hl == 0) {
      sh.info[c] = make_int4(qpos, qt, qty, 0);
      sh.stat[c] = qty ? make_float2(lse_bh[qpos] * kLog2e, d_bh[qpos]) : make_float2(0.f, 0.f);
    }
    e16x8 qf[4], df[4];
    load_frag(qf, qb + (size_t)(qty ? qpos : 0) * rs, qty != 0, hl);
    load_frag(df, dob + (size_t)(qty ? qpos : 0) * rs, qty != 0, hl);
    stage_frag(sh, 0, c, hl, qf);
    stage_frag(sh, 1, c, hl, df);
    __syncthreads();
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      S = mma(qf[s], kf[s], S);
      dP = mma(df[s], vf[s], dP);
    }
    e16x8 p8[2], ds8[2];
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
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc_v[half] = mma(p8[t], col_frag(sh, 1, t, hl, 32 * half + c), acc_v[half]);
        acc_k[half] = mma(ds8[t], col_frag(sh, 0, t, hl, 32 * half + c), acc_k[half]);
      }
    __syncthreads();
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
  int bid = blockIdx.x;
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
    auto res_slot = [&](int t, int& pos, int& tt, int& ty) {
      const bool in = t >= 0 && t < rt.len;
      pos = in ? rt.r + rt.d * t : -1;
      tt = t;
      ty = in ? eff_mask(mb[pos], ug) : 0;
    };
    if (own_q) {
      // window keys of the tile's rows, clipped to the class
      const int base = max(rt.t0 - w, 0);
      const int last = min(rt.t0 + 31 + (causal ? 0 : w), rt.len - 1);
      const int nwin = (last - base + 32) / 32;
      const int ngb = (nG + 31) / 32;
      auto keyof = [&](int j, int slot, int& pos, int& tt, int& ty) {
        if (j < nwin) {
          res_slot(base + 32 * j + slot, pos, tt, ty);
        } else {
          const int g = 32 * (j - nwin) + slot;
          pos = g < nG ? gl[g] : -1;
          ty = g < nG ? 2 : 0;
          const int rel = pos - rt.r;
          tt = (pos >= rt.r && rel % rt.d == 0) ? rel / rt.d : kSentinel;
          // marks the slot as a global-column slot: window keys carry their
          // own residue index, which always lies within the class
          ty = ty ? 6 : 0;
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
      q_owner(p, sh, rs, Q + boff, DO + boff, K + boff, V + boff, mypos, myt, myty, lse2, dd, nwin + ngb, keyof,
              member, acc);
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
      auto rowof = [&](int j, int slot, int& pos, int& tt, int& ty) { res_slot(base + 32 * j + slot, pos, tt, ty); };
      auto member = [&](int qty, int qt, int kty, int kt) { return qty == 1 && kty == 1 && in_win(qt, kt, w, causal); };
      if (hl == 0) sh.opos[c] = (myty == 2) ? -1 : mypos;
      f32x16 ak[2], av[2];
      kv_owner(p, sh, rs, K + boff, V + boff, Q + boff, DO + boff, lse_bh, d_bh, mypos, myt, myty, nq, rowof,
               member, ak, av);
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
    auto rowof = [&](int j, int slot, int& pos, int& tt, int& ty) {
      const int g = 32 * j + slot;
      pos = g < nG ? gl[g] : -1;
      tt = 0;
      ty = g < nG ? 2 : 0;
    };
    auto member = [](int qty, int, int kty, int) { return qty == 2 && kty != 0; };
    if (hl == 0) sh.opos[c] = mypos;
    f32x16 ak[2], av[2];
    kv_owner(p, sh, rs, KG + boff, VG + boff, QG + boff, DO + boff, p.lse + (size_t)bh * n, p.Dsum + (size_t)bh * n,
             mypos, 0, myty, (nG + 31) / 32, rowof, member, ak, av);
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
  auto tok = [&](int j, int slot, int& pos, int& tt, int& ty) {
    const int t = c0 + 32 * j + slot;
    pos = t < n ? t : -1;
    tt = 0;
    ty = t < n ? eff_mask(mb[t], 1) : 0;
  };
  const float* lse_bh = p.lse + (size_t)bh * n;
  const float* d_bh = p.Dsum + (size_t)bh * n;
  if (gq) {
    auto member = [](int qty, int, int kty, int) { return qty == 2 && kty != 0; };
    const float lse2 = gty ? lse_bh[gpos] * kLog2e : 0.f;
    const float dd = gty ? d_bh[gpos] : 0.f;
    f32x16 acc[2];
    q_owner(p, sh, rs, QG + boff, DO + boff, KG + boff, VG + boff, gpos, 0, gty, lse2, dd, nblk, tok, member, acc);
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
    kv_owner(p, sh, rs, K + boff, V + boff, Q + boff, DO + boff, lse_bh, d_bh, gpos, 0, gty, nblk, tok, member, ak,
             av);
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

// Preparation, one row (b, i, h) per 16 lanes: D = <dout, out>; dq_g zeroed;
// dk, dv of global tokens zeroed (global-key work adds to them); dk_g, dv_g
// zeroed when no global work runs.
__device__ void prep_body(const BwdParams& p) {
  const size_t rows = (size_t)p.B * p.n * p.H;
  const size_t row = (size_t)blockIdx.x * (blockDim.x / 16) + (threadIdx.x >> 4);
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

#if !LF_HALF_F16
// Global list of each batch row, ascending: one workgroup of 256 threads per
// batch row; at most max_global entries kept (more sets the status bit).
__global__ __launch_bounds__(256) void lf_attn_bwd_glist(const BwdParams p) {
  __shared__ int wsum[4];
  __shared__ int total;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int8_t* mb = p.mask + (size_t)b * p.n;
  int32_t* gl = p.glist + (size_t)b * p.gstride;
  if (tid == 0) total = 0;
  __syncthreads();
  for (int base = 0; base < p.n; base += 256) {
    const int i = base + tid;
    const bool g = i < p.n && mb[i] == 2;
    const uint64_t bal = __ballot(g);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int x = 0; x < wv; ++x) off += wsum[x];
    const int idx = off + before;
    if (g && idx < p.max_global) gl[idx] = i;
    __syncthreads();
    if (tid == 0) total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) {
    p.gcount[b] = min(total, p.max_global);
    if (total > p.max_global) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
  }
}
#endif

#if LF_HALF_F16
__global__ __launch_bounds__(64) void lf_attn_bwd_f16(const BwdParams p) { bwd_body(p); }
__global__ __launch_bounds__(256) void lf_attn_bwd_prep_f16(const BwdParams p) { prep_body(p); }
#else
__global__ __launch_bounds__(64) void lf_attn_bwd_bf16(const BwdParams p) { bwd_body(p); }
__global__ __launch_bounds__(256) void lf_attn_bwd_prep_bf16(const BwdParams p) { prep_body(p); }
#endif

}  // namespace

#if LF_HALF_F16
int launch_backward_f16(const BwdParams& bp, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t rows = (size_t)bp.B * bp.n * bp.H;
  hipLaunchKernelGGL(lf_attn_bwd_prep_f16, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, bp);
  hipLaunchKernelGGL(lf_attn_bwd_f16, dim3(2 * bp.n_res + bp.n_gkv + bp.n_gq + bp.n_gk), dim3(64), 0, s, bp);
  return (int)hipGetLastError();
}
#else
int launch_backward(const BwdParams& bp, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (bp.use_globals) hipLaunchKernelGGL(lf_attn_bwd_glist, dim3(bp.B), dim3(256), 0, s, bp);
  if (bp.dtype == LF_F16) {
    const int e = (int)hipGetLastError();
    return e ? e : launch_backward_f16(bp, stream);
  }
  const size_t rows = (size_t)bp.B * bp.n * bp.H;
  hipLaunchKernelGGL(lf_attn_bwd_prep_bf16, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, bp);
  hipLaunchKernelGGL(lf_attn_bwd_bf16, dim3(2 * bp.n_res + bp.n_gkv + bp.n_gq + bp.n_gk), dim3(64), 0, s, bp);
  return (int)hipGetLastError();
}
#endif

}  // namespace lf
