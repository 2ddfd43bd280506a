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
// Two launches:
//   * preparation: the global token list of each batch row, -D_i and
//     -lse_i / scale per row, and zeroed rows for the gradients that the
//     global-token work adds to;
//   * gradient launch: 4-wave band workgroups over tiles of 128 consecutive
//     rows of one residue class of one head (a dilated window is a plain
//     window over its residue class: segmentfault summary, "Dilated sliding
//     window").  A dq workgroup owns 128 query rows (wave w: 32 of them) and
//     streams the key blocks of its window span and then the batch row's
//     global tokens through LDS; a dk/dv workgroup owns 128 key rows and
//     streams the query blocks whose windows reach them, with their
//     statistics.  Each staged block is read by all four waves; every
//     gradient row has one owner, and S and dP are formed once per (block,
//     wave) in each of the two roles.  After the band workgroups, in the
//     same grid, the global-token work (only with global tokens) runs as
//     single-wave units, four per workgroup, adding the local rows' dk, dv of
//     global tokens and the global rows' dq_g (fp32 atomics onto rows the
//     preparation zeroed), and writing dk_g, dv_g:
//       GKV: one wave per 32 tokens; walks the global rows; writes dk_g, dv_g.
//       GQ:  one wave per 32 global rows and 128 keys; adds to dq_g.
//       GK:  one wave per 32 global tokens and 128 rows; adds to dk, dv.
// Block products are 32x32x16 MFMA chains; the transposed operands come from
// staged rows through ds_read_b64_tr_b16.  The gradient launch runs three
// waves per SIMD (at most 168 VGPRs), so that a CU holds three band
// workgroups: both band roles read a staged block one tensor at a time, the
// dk/dv role keeps its K and V fragments in LDS rather than in registers,
// the staged blocks go through two LDS stages (block i + 1 loads while
// block i is used), and the global-token units load each block when they
// use it.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "lf_attn_bwd_internal.h"

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
  e16 st[2][32][kLdsRow];                 // rows staged for the column-wise operand
  __attribute__((aligned(16))) float sx[32];  // streamed query rows: -lse in base 2 (key-owning units)
  __attribute__((aligned(16))) float sy[32];  // ... and -D
  int opos[32];                           // positions of the wave's own 32 keys
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

// The global-token units below run one per wave: the rows a wave stages in
// LDS are read back only by lanes of the same wave, whose LDS operations
// complete in order; the wave waits for its own LDS operations and the
// compiler moves no memory access across this point.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

// A row fragment read from a row that exists (the caller clamps the
// position), without a branch, so that the compiler's count of loads in
// flight stays exact; rows that take no part are zeroed with keep_frag.
__device__ __forceinline__ void load_frag_any(e16x8 (&f)[4], const e16* row, int hl) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = ld8(row + 16 * s + 8 * hl);
}

// Membership of a slot type: want < 0 takes every type but 0, otherwise
// exactly type want.
__device__ __forceinline__ bool takes(int ty, int want) { return want < 0 ? ty != 0 : ty == want; }

// Query-owning wave of the global units: 32 query rows (lane c's row at
// qpos, type qty; its -lse in base 2 and -D in lse2, dd), nblk key blocks
// described by keyof(j, slot) -> (pos, slot code).  A (query, key) pair
// takes part when the query's type is want_q and the key's type is taken
// by want_k.  Returns dq^T in acc: lane (c, hl) holds head dims 32 half +
// acc_row(r, hl) of query c in acc[half][r].  The next block's rows load
// while the current one is used.
template <class KeyOf>
__device__ void q_owner(const BwdParams& p, BwdShared& sh, size_t rs, const e16* qb, const e16* dob,
                        const e16* kb, const e16* vb, int qpos, int qty, float lse2, float dd, int nblk,
                        KeyOf keyof, int want_q, int want_k, f32x16 (&acc)[2]) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const bool qin = qty == want_q;
  e16x8 qf[4], df[4];
  load_frag_any(qf, qb + (size_t)(qty ? qpos : 0) * rs, hl);
  load_frag_any(df, dob + (size_t)(qty ? qpos : 0) * rs, hl);
  keep_frag(qf, qty != 0);
  keep_frag(df, qty != 0);
  acc[0] = zero16();
  acc[1] = zero16();
  int npos = -1, ncode = 0;
  e16x8 nkf[4], nvf[4];
  auto fetch = [&](int j) {
    keyof(j, c, npos, ncode);
    const size_t at = (size_t)(npos >= 0 ? npos : 0) * rs;
    load_frag_any(nkf, kb + at, hl);
    load_frag_any(nvf, vb + at, hl);
  };
  if (nblk > 0) fetch(0);
  for (int j = 0; j < nblk; ++j) {
    const int kpos = npos, kcode = ncode;
    e16x8 kf[4], vf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = nkf[s];
      vf[s] = nvf[s];
    }
    if (j + 1 < nblk) fetch(j + 1);
    const int kty = slot_type(kpos, kcode, p.use_globals);
    keep_frag(kf, kty != 0);
    keep_frag(vf, kty != 0);
    // keys taking part, by key row (lanes c and c + 32 hold key c)
    const uint32_t kbits = (uint32_t)__ballot(takes(kty, want_k));
    stage_frag(sh, 0, c, hl, kf);
    wave_lds_sync();
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      S = mma(kf[s], qf[s], S);
      dP = mma(vf[s], df[s], dP);
    }
    e16x8 ds8[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = qin && ((kbits >> acc_row(r, hl)) & 1u);
      const float pr = __builtin_amdgcn_exp2f(p.c * S[r] - lse2);
      ds8[r >> 3][r & 7] = (e16)(ok ? pr * (dP[r] - dd) : 0.f);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[half] = mma(col_frag(sh, 0, t, lane, half), ds8[t], acc[half]);
    wave_lds_sync();
  }
}

// Key-owning wave of the global units: 32 keys (lane c's key at kpos, type
// kty), nblk query blocks described by rowof(j, slot) -> (pos, slot code),
// the rows' -lse / scale and -D in lse_bh, d_bh.  A pair takes part when the
// query row's type is want_q and the key's type is taken by want_k.
// Returns acc_k[half][r], acc_v[half][r]: head dim 32 half + c of own key
// acc_row(r, hl).  The next block's rows load while the current one is used.
template <class RowOf>
__device__ void kv_owner(const BwdParams& p, BwdShared& sh, size_t rs, const e16* kb, const e16* vb,
                         const e16* qb, const e16* dob, const float* lse_bh, const float* d_bh, int kpos, int kty,
                         int nblk, RowOf rowof, int want_q, int want_k, f32x16 (&acc_k)[2], f32x16 (&acc_v)[2]) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const bool kin = takes(kty, want_k);
  e16x8 kf[4], vf[4];
  load_frag_any(kf, kb + (size_t)(kty ? kpos : 0) * rs, hl);
  load_frag_any(vf, vb + (size_t)(kty ? kpos : 0) * rs, hl);
  keep_frag(kf, kty != 0);
  keep_frag(vf, kty != 0);
  acc_k[0] = acc_k[1] = acc_v[0] = acc_v[1] = zero16();
  int npos = -1, ncode = 0;
  float nl = 0.f, nd = 0.f;
  e16x8 nqf[4], ndf[4];
  auto fetch = [&](int j) {
    rowof(j, c, npos, ncode);
    const int at = npos >= 0 ? npos : 0;
    nl = -p.c * lse_bh[at];  // lse in base 2
    nd = -d_bh[at];
    load_frag_any(nqf, qb + (size_t)at * rs, hl);
    load_frag_any(ndf, dob + (size_t)at * rs, hl);
  };
  if (nblk > 0) fetch(0);
  for (int j = 0; j < nblk; ++j) {
    const int qpos = npos, qcode = ncode;
    const float ql = nl, qd = nd;
    e16x8 qf[4], df[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[s] = nqf[s];
      df[s] = ndf[s];
    }
    if (j + 1 < nblk) fetch(j + 1);
    const int qty = slot_type(qpos, qcode, p.use_globals);
    const bool qin = qty == want_q;
    keep_frag(qf, qty != 0);
    keep_frag(df, qty != 0);
    // rows taking part, by row (lanes c and c + 32 hold row c); their
    // statistics go through LDS, four consecutive rows per read below
    const uint32_t qbits = (uint32_t)__ballot(qin);
    if (hl == 0) {
      sh.sx[c] = qin ? ql : 0.f;
      sh.sy[c] = qin ? qd : 0.f;
    }
    stage_frag(sh, 0, c, hl, qf);
    stage_frag(sh, 1, c, hl, df);
    wave_lds_sync();
    // the row products from the fragments in registers; the staged rows
    // serve the transposed reads below
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      S = mma(qf[s], kf[s], S);
      dP = mma(df[s], vf[s], dP);
    }
    // accumulator elements 4 g .. 4 g + 3 hold rows 8 g + 4 hl .. + 3
    f32x4 sx4[4], sy4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sx4[g] = *reinterpret_cast<const f32x4*>(&sh.sx[8 * g + 4 * hl]);
      sy4[g] = *reinterpret_cast<const f32x4*>(&sh.sy[8 * g + 4 * hl]);
    }
    e16x8 p8[2], ds8[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = kin && ((qbits >> acc_row(r, hl)) & 1u);
      const float pr = __builtin_amdgcn_exp2f(p.c * S[r] - sx4[r >> 2][r & 3]);
      p8[r >> 3][r & 7] = (e16)(ok ? pr : 0.f);
      ds8[r >> 3][r & 7] = (e16)(ok ? pr * (dP[r] - sy4[r >> 2][r & 3]) : 0.f);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc_v[half] = mma(p8[t], col_frag(sh, 1, t, lane, half), acc_v[half]);
        acc_k[half] = mma(ds8[t], col_frag(sh, 0, t, lane, half), acc_k[half]);
      }
    wave_lds_sync();
  }
}

__device__ __forceinline__ void store_f4(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}

// Work on the global tokens, in a launch of its own (global roles):
//   GKV: one wave per 32 tokens of one (b, h); walks the global rows as
//        queries and writes dk_g, dv_g of its tokens;
//   GQ:  a workgroup per (b, h, block of 32 global slots, group of four
//        kBwdChunk-token chunks), wave w taking chunk 4 g + w: dq_g of the
//        global rows;
//   GK:  the same grouping with local rows as queries: dk, dv of the
//        global tokens as keys of local rows.
// GQ and GK add into rows the preparation zeroed; the four waves of a
// workgroup sum their partials through LDS first, so that a group of four
// chunks costs one set of atomic adds.

// GKV unit `bid`, run by one wave with its own staging area sh.
__device__ void bwd_gkv_unit(const BwdParams& p, BwdShared& sh, int bid) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const int n = p.n;
  const size_t rs = (size_t)p.H * 64;
  const e16* QG = reinterpret_cast<const e16*>(p.qg);
  const e16* KG = reinterpret_cast<const e16*>(p.kg);
  const e16* VG = reinterpret_cast<const e16*>(p.vg);
  const e16* DO = reinterpret_cast<const e16*>(p.dout);

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
  auto rowof = [&](int j, int slot, int& pos, int& code) {
    const int g = 32 * j + slot;
    const int e = gl[min(g, p.gstride - 1)];  // in the list whatever the count; taken below it only
    pos = g < nG ? e : -1;
    code = 256 + 2;
  };
  if (hl == 0) sh.opos[c] = mypos;
  f32x16 ak[2], av[2];
  // global rows (type 2) against every token that is not padding
  kv_owner(p, sh, rs, KG + boff, VG + boff, QG + boff, DO + boff, p.lneg + (size_t)bh * n, p.dneg + (size_t)bh * n,
           mypos, myty, (nG + 31) / 32, rowof, 2, -1, ak, av);
  wave_lds_sync();
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
}

// Sums the 32 accumulator values per lane of the four waves of a workgroup
// (same lane layout in every wave) through LDS and passes each sum once to
// add(half, r, value): wave w takes r = 4 w .. 4 w + 3 of both halves.  A
// wave's partial goes to its own staging rows, which it no longer reads;
// every wave of the workgroup calls this (it holds two barriers).
template <class Add>
__device__ __forceinline__ void group_add(BwdShared (&unit)[4], int wv, int lane, const f32x16 (&acc)[2], Add add) {
  static_assert(sizeof(unit[0].st) >= 32 * 64 * sizeof(float), "a partial fits the staging rows");
  float* mine = reinterpret_cast<float*>(&unit[wv].st[0][0][0]);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int r = 0; r < 16; ++r) mine[(16 * half + r) * 64 + lane] = acc[half][r];
  __syncthreads();
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * wv + rr;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += reinterpret_cast<const float*>(&unit[w].st[0][0][0])[(16 * half + r) * 64 + lane];
      add(half, r, v);
    }
  __syncthreads();  // the partials are read before the staging rows are written again
}

// GQ (gq) or GK work of workgroup `grp` of its role; wave wv, with its own
// staging area unit[wv].
__device__ void bwd_gqk_group(const BwdParams& p, BwdShared (&unit)[4], int wv, int grp, bool gq) {
  BwdShared& sh = unit[wv];
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const int n = p.n;
  const size_t rs = (size_t)p.H * 64;
  const e16* Q = reinterpret_cast<const e16*>(p.q);
  const e16* K = reinterpret_cast<const e16*>(p.k);
  const e16* V = reinterpret_cast<const e16*>(p.v);
  const e16* QG = reinterpret_cast<const e16*>(p.qg);
  const e16* KG = reinterpret_cast<const e16*>(p.kg);
  const e16* VG = reinterpret_cast<const e16*>(p.vg);
  const e16* DO = reinterpret_cast<const e16*>(p.dout);

  // (b, h, block of 32 global slots, group of four chunks); this wave's chunk
  const int cg = (p.chunks + 3) / 4;
  const int per_bh = p.gslots * cg;
  const int bh = grp / per_bh;
  const int rem = grp - bh * per_bh;
  const int sb = rem / cg;
  const int ch = 4 * (rem - sb * cg) + wv;
  const int b = bh / p.H, h = bh - b * p.H;
  const int nG = p.gcount[b];
  if (32 * sb >= nG) return;  // the same for every wave of the workgroup
  const size_t boff = (size_t)b * n * rs + (size_t)h * 64;
  const int8_t* mb = p.mask + (size_t)b * n;
  const int32_t* gl = p.glist + (size_t)b * p.gstride;
  const int c0 = ch * kBwdChunk;
  const int nblk = ch < p.chunks ? (min(kBwdChunk, n - c0) + 31) / 32 : 0;
  const int g = 32 * sb + c;
  const int ge = gl[min(g, p.gstride - 1)];  // in the list whatever the count; taken below it only
  const int gpos = g < nG ? ge : -1;
  const int gty = g < nG ? 2 : 0;
  auto tok = [&](int j, int slot, int& pos, int& code) {
    const int t = c0 + 32 * j + slot;
    pos = t < n ? t : -1;
    code = (uint8_t)mb[t < n ? t : 0];
  };
  const float* lse_bh = p.lneg + (size_t)bh * n;  // -lse / scale
  const float* d_bh = p.dneg + (size_t)bh * n;     // -D
  if (gq) {
    const float lse2 = gty ? -p.c * lse_bh[gpos] : 0.f;
    const float dd = gty ? -d_bh[gpos] : 0.f;
    f32x16 acc[2];
    // global rows (type 2) against the chunk's tokens that are not padding
    q_owner(p, sh, rs, QG + boff, DO + boff, KG + boff, VG + boff, gpos, gty, lse2, dd, nblk, tok, 2, -1, acc);
    float* dst = p.dqg + boff + (size_t)(gpos >= 0 ? gpos : 0) * rs;
    group_add(unit, wv, lane, acc, [&](int half, int r, float v) {
      if (gpos >= 0) unsafeAtomicAdd(dst + 32 * half + acc_row(r, hl), p.scale * v);
    });
  } else {
    if (hl == 0) sh.opos[c] = gpos;
    f32x16 ak[2], av[2];
    // the chunk's local rows (type 1) against the global tokens as keys (type 2)
    kv_owner(p, sh, rs, K + boff, V + boff, Q + boff, DO + boff, lse_bh, d_bh, gpos, gty, nblk, tok, 1, 2, ak, av);
    wave_lds_sync();
    group_add(unit, wv, lane, ak, [&](int half, int r, float v) {
      const int pos = sh.opos[acc_row(r, hl)];
      if (pos >= 0) unsafeAtomicAdd(p.dk + boff + (size_t)pos * rs + 32 * half + c, p.scale * v);
    });
    group_add(unit, wv, lane, av, [&](int half, int r, float v) {
      const int pos = sh.opos[acc_row(r, hl)];
      if (pos >= 0) unsafeAtomicAdd(p.dv + boff + (size_t)pos * rs + 32 * half + c, v);
    });
  }
}


// ===========================================================================
// Band kernel
// ===========================================================================
#define LDS_AS __attribute__((address_space(3)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRowB = 128;                   // staged row: 64 head dims of 16 bits
constexpr int kBlkB = 32 * kRowB;            // one 32-row block of one tensor
constexpr int kStatB = 256;                  // dk/dv role: -lse / scale then -D of the block's 32 rows
constexpr int kStageB = 2 * kBlkB + kStatB;  // two tensors and the row statistics
constexpr int kBandStages = 2;               // block i + 1 flies while block i is used

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(LDS_AS const void*)p; }

constexpr int kBandTab = 64;                 // blocks whose row validity is tabulated up front

struct BandShared {
  __attribute__((aligned(16))) unsigned char ring[kBandStages * kStageB];
  uint32_t tab[kBandTab];     // row-validity bits of blocks i0 .. i0 + kBandTab - 1 (entry i % kBandTab)
  union {
    int32_t gpos[LF_MAX_GLOBAL];  // dq role: the batch row's global positions
    // dk/dv role: each wave's K and V fragments, [wave][fragment s][lane]
    // 16 bytes each
    struct {
      __attribute__((aligned(16))) unsigned char kfr[4 * 4 * 64 * 16];
      __attribute__((aligned(16))) unsigned char vfr[4 * 4 * 64 * 16];
    };
  };
};

// A 32-bit LDS word read in an asm block that waits for its own read (see
// the fragment reads below).
__device__ __forceinline__ uint32_t lds_word(const void* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// The validity table for blocks i0 .. i0 + kBandTab - 1 (below nblk): bit
// row of tab[i % kBandTab] is ok(i, row, mask byte of the row).  Each wave
// takes blocks i0 + 2 wv + 8 k and the next (lanes 0-31 and 32-63).  The
// loads are waited for here, and a workgroup barrier ends it.
template <class Pos, class Ok>
__device__ __forceinline__ void tab_fill(BandShared& sh, const int8_t* mb, int i0, int nblk, int wv, int lane,
                                         Pos pos, Ok ok) {
  const int end = min(nblk, i0 + kBandTab);
  for (int a = i0 + 2 * wv; a < end; a += 8) {
    const int i = a + (lane >> 5), row = lane & 31;
    const bool v = i < end && ok(i, row, (int)mb[pos(i < end ? i : a, row)]);
    const unsigned long long bits = __ballot(v);
    if (lane == 0) {
      sh.tab[a % kBandTab] = (uint32_t)bits;
      if (a + 1 < end) sh.tab[(a + 1) % kBandTab] = (uint32_t)(bits >> 32);
    }
  }
  __syncthreads();
}

// 16-byte chunk c of staged row r sits at chunk c ^ bswz(r).  With 128-byte
// rows two rows share a 256-byte bank span; the swizzle is a bit reversal of
// (r / 2) mod 8.  Row reads (16 consecutive rows at one chunk) then hit 16
// distinct 16-byte slots, and the transposed reads of a half-wave (rows
// 4a .. 4a + 3, one 64-byte column group) 4 distinct 64-byte quarters.
__device__ __forceinline__ int bswz(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | (x >> 2);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }


// This wave's share (load t = wave of each tensor: rows 8 t .. 8 t + 7) of
// the direct-to-LDS loads of one 32-row block of two tensors x0, x1 into a
// stage: lane l fetches chunk (l % 8) ^ bswz(row) of row 8 t + l / 8 (token
// position pos(row), always a valid row), landing at byte 1024 t + 16 l.
template <class Pos>
__device__ __forceinline__ void issue_pair(const e16* x0, const e16* x1, size_t rs, Pos pos, unsigned char* stage,
                                           int wv, int lane) {
  const int row = 8 * wv + (lane >> 3);
  const size_t off = (size_t)pos(row) * rs + 8 * ((lane & 7) ^ bswz(row));
  __builtin_amdgcn_global_load_lds(x0 + off, (LDS_AS void*)(stage + 1024 * wv), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(x1 + off, (LDS_AS void*)(stage + kBlkB + 1024 * wv), 16, 0, 0);
}

// Per-lane LDS addresses of the fragment reads of a block at the ring's
// start (a stage is kStageB further; the second tensor kBlkB).
//   ro[s]: row operand, lane (row = lane % 32, hl = lane / 32) reads head
//          dims 16 s + 8 hl .. + 7 of its row;
//   co[db][half]: transposed operand, ds_read_b64_tr_b16: in each group g of
//          16 lanes, lane 4 e + q addresses row 4 (g / 2) + e + 8 half,
//          head dims 32 db + 16 (g % 2) + 4 q .. + 3; lane i of the group
//          receives head dim 32 db + 16 (g % 2) + i of those four rows.  The
//          rows 16 further (k-step 1) share the swizzle: + 2048 bytes.
//   Together lane l gets head dim 32 db + l % 32 of rows 16 ks + {4 hl ..
//   4 hl + 3, 8 + 4 hl .. 8 + 4 hl + 3}, the row order of a 32x32 result's
//   registers 8 ks .. 8 ks + 7.
struct BandAddr {
  uint32_t ro[4];
  uint32_t co[2][2];
};

__device__ __forceinline__ BandAddr band_addr(const unsigned char* ring, int lane) {
  BandAddr a;
  const uint32_t base = lds_addr(ring);
  const int row = lane & 31, hl = lane >> 5;
  const int sw = bswz(row);
#pragma unroll
  for (int s = 0; s < 4; ++s) a.ro[s] = base + (uint32_t)(row * kRowB + (((2 * s + hl) ^ sw) << 4));
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r = 8 * half + 4 * (g >> 1) + (i >> 2);
      const int byte = 64 * db + 32 * (g & 1) + 8 * (i & 3);
      a.co[db][half] = base + (uint32_t)(r * kRowB + ((((byte >> 4) ^ bswz(r)) << 4) | (byte & 15)));
    }
  return a;
}

__device__ __forceinline__ e16x8 as8(u32x4 x) { return __builtin_bit_cast(e16x8, x); }
__device__ __forceinline__ e16x8 join8(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(e16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// The reads of one staged block, one tensor per asm block (so that few
// registers are live at once), each asm block waiting for its own reads:
// the compiler cannot tell them from the direct-to-LDS loads still in
// flight into the other stage and would otherwise wait for those first.
// so is the stage's byte offset in the ring, added to the fragment
// addresses computed once (BandAddr).
//   read_rows4<kT>: the rows of tensor kT (0 or 1 of the stage).
template <int kT>
__device__ __forceinline__ void read_rows4(e16x8 (&f)[4], const BandAddr& a, uint32_t so) {
  u32x4 q[4];
  const uint32_t r0 = a.ro[0] + so, r1 = a.ro[1] + so, r2 = a.ro[2] + so, r3 = a.ro[3] + so;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n"
      "ds_read_b128 %1, %5 offset:%8\n"
      "ds_read_b128 %2, %6 offset:%8\n"
      "ds_read_b128 %3, %7 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3])
      : "v"(r0), "v"(r1), "v"(r2), "v"(r3), "i"(kT * kBlkB)
      : "memory");
#pragma unroll
  for (int s = 0; s < 4; ++s) f[s] = as8(q[s]);
}

//   read_rows_stats<kT> (dk/dv role): the rows of tensor kT (0: Q, 1: dO),
//   their row statistics (this lane's 16 rows 8 g + 4 hl .. + 3: float4 g of
//   -lse / scale for Q, of -D for dO, at sa) and the wave's K (kT = 0) or V
//   (kT = 1) fragments from LDS at fb (fragment s at fb + 1024 s).
template <int kT>
__device__ __forceinline__ void read_rows_stats(e16x8 (&f)[4], f32x4 (&st)[4], e16x8 (&bf)[4], const BandAddr& a,
                                                uint32_t sa, uint32_t fb, uint32_t so) {
  u32x4 q[4], v[4];
  const uint32_t r0 = a.ro[0] + so, r1 = a.ro[1] + so, r2 = a.ro[2] + so, r3 = a.ro[3] + so, s0 = sa + so;
  asm volatile(
      "ds_read_b128 %0, %12 offset:%18\n"
      "ds_read_b128 %1, %13 offset:%18\n"
      "ds_read_b128 %2, %14 offset:%18\n"
      "ds_read_b128 %3, %15 offset:%18\n"
      "ds_read_b128 %4, %16 offset:%19\n"
      "ds_read_b128 %5, %16 offset:%20\n"
      "ds_read_b128 %6, %16 offset:%21\n"
      "ds_read_b128 %7, %16 offset:%22\n"
      "ds_read_b128 %8, %17\n"
      "ds_read_b128 %9, %17 offset:1024\n"
      "ds_read_b128 %10, %17 offset:2048\n"
      "ds_read_b128 %11, %17 offset:3072\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(st[0]), "=&v"(st[1]), "=&v"(st[2]), "=&v"(st[3]),
        "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(r0), "v"(r1), "v"(r2), "v"(r3), "v"(s0), "v"(fb), "i"(kT * kBlkB), "i"(128 * kT),
        "i"(128 * kT + 32), "i"(128 * kT + 64), "i"(128 * kT + 96)
      : "memory");
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f[s] = as8(q[s]);
    bf[s] = as8(v[s]);
  }
}

//   read_cols<kT>: tensor kT transposed (ds_read_b64_tr_b16): t8[db][ks]
//   holds head dim 32 db + lane % 32 of the block's rows 16 ks + {4 hl ..
//   4 hl + 3, 8 + 4 hl .. 8 + 4 hl + 3}.
template <int kT>
__device__ __forceinline__ void read_cols(e16x8 (&t8)[2][2], const BandAddr& a, uint32_t so) {
  u32x2 t[8];  // [db][ks][half]
  const uint32_t c00 = a.co[0][0] + so, c01 = a.co[0][1] + so, c10 = a.co[1][0] + so, c11 = a.co[1][1] + so;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n"
      "ds_read_b64_tr_b16 %1, %9 offset:%12\n"
      "ds_read_b64_tr_b16 %2, %8 offset:%13\n"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n"
      "ds_read_b64_tr_b16 %5, %11 offset:%12\n"
      "ds_read_b64_tr_b16 %6, %10 offset:%13\n"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
      : "v"(c00), "v"(c01), "v"(c10), "v"(c11), "i"(kT * kBlkB), "i"(kT * kBlkB + 2048)
      : "memory");
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) t8[db][ks] = join8(t[4 * db + 2 * ks], t[4 * db + 2 * ks + 1]);
}

// Zero the entries of a transposed operand whose row is clear in vm (a row
// outside every pair of the block may hold non-finite values; its products
// must be exact zeros).
__device__ __forceinline__ void zero_cols(e16x8 (&t)[2][2], uint32_t vm, int hl) {
  const uint32_t m = vm >> (4 * hl);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 keep;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      // elements 2 dw, 2 dw + 1; element e is row 16 ks + 8 (e / 4) + e % 4 (+ 4 hl)
      const int r0 = 16 * ks + 8 * ((2 * dw) >> 2) + ((2 * dw) & 3);
      keep[dw] = (((m >> r0) & 1u) ? 0x0000ffffu : 0u) | (((m >> (r0 + 1)) & 1u) ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) t[db][ks] = __builtin_bit_cast(e16x8, __builtin_bit_cast(u32x4, t[db][ks]) & keep);
  }
}

// Bits lo .. hi of a word (empty when lo > hi); lo, hi clipped to [0, 31].
__device__ __forceinline__ uint32_t bit_range(int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, 31);
  return lo > hi ? 0u : ((0xffffffffu >> (31 - hi)) & (0xffffffffu << lo));
}

// Band tile: batch row b, head h (dilation d), residue class r (len rows),
// rows t0 .. t0 + 127 of the class.
struct BandTile {
  int b, h, d, r, t0, len;
};

__device__ __forceinline__ BandTile decode_band(const BwdParams& p, int tile) {
  BandTile t;
  t.b = tile / p.bt_per_b;
  const int id0 = tile - t.b * p.bt_per_b;
  int h = 0;
  while (h + 1 < p.H && p.btile0[h + 1] <= id0) ++h;
  const int d = p.dil[h];
  const int id = id0 - p.btile0[h];
  const int qn = p.n / d, rm = p.n % d;
  const int T1 = (qn + kBwdBandRows) / kBwdBandRows, T0 = (qn + kBwdBandRows - 1) / kBwdBandRows;
  if (id < rm * T1) {
    t.r = id / T1;
    t.t0 = (id - t.r * T1) * kBwdBandRows;
    t.len = qn + 1;
  } else {
    const int id2 = id - rm * T1;
    t.r = rm + id2 / T0;
    t.t0 = (id2 - (t.r - rm) * T0) * kBwdBandRows;
    t.len = qn;
  }
  t.h = h;
  t.d = d;
  return t;
}

// The block loop shared by both roles: blocks i < nblk, block i staged in
// stage i % 2.  Every wave runs every step (one barrier each): it waits for
// its own loads of block i (the only ones in flight), and after the barrier
// (all of block i is in LDS, every wave is done with block i - 1) issues
// the direct-to-LDS loads of block i + 1 into block i - 1's stage (issue(i,
// stage): its share of the block), which land during
// step i.  prologue() makes the role's own loads; refill(i0)
// fills the validity table for blocks i0 .. i0 + kBandTab - 1 (every wave,
// at a barrier).  step(i, stage) uses block i.  gate(), after the first
// refill, decides for the whole workgroup whether the loop runs at all
// (false: the loads in flight are waited for and the loop is skipped), so
// that the loads the decision needs fly with all the others.  Returns
// gate()'s answer.
template <class Issue, class Prologue, class Refill, class Gate, class Step>
__device__ __forceinline__ bool band_loop(int nblk, int pre, Issue issue, Prologue prologue, Refill refill,
                                          Gate gate, Step step) {
  // the first block's loads (if it needs no table: pre > 0) fly while the
  // prologue's own loads and the table's mask bytes load
  const int early = min(min(pre, nblk), 1);
  for (int i = 0; i < early; ++i) issue(i, i);
  prologue();
  refill(0);
  if (!gate()) {
    wait_vmem_all();  // no direct-to-LDS load may outlive the workgroup
    return false;
  }
  for (int i = early; i < min(nblk, 1); ++i) issue(i, i);
  wait_vmem_all();  // so that no wait for the prologue's loads lands inside the loop
  int stage = 0;
  for (int i = 0; i < nblk; ++i) {
    wait_vmem_all();  // block i's loads (the only ones in flight)
    block_barrier();
    // every wave is past step i - 1: the table may take the next blocks,
    // and the stage of block i - 1 the loads of block i + 1
    if (i > 0 && i % kBandTab == 0) refill(i);
    if (i + 1 < nblk) issue(i + 1, stage ^ 1);
    step(i, stage);
    stage ^= 1;
  }
  wait_vmem_all();
  return true;
}

// dq workgroup.  Wave wv owns query rows t0 + 32 wv + lane % 32 (Q and dO
// as B operands, its base-2 lse and D in registers); the key blocks are the
// window span kbase + 32 (jlo + i) + row (residue indices), then the global
// tokens G[32 (i - nwin) + row] (scored by local rows whose window does not
// hold them).  Per block: S^T = K Q^T, dP^T = V dO^T (lane: one query, 16
// keys), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
__device__ void band_dq(const BwdParams& p, BandShared& sh, const BandTile& bt, int wv) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const int n = p.n, w = p.w, d = bt.d;
  const int w_hi = p.causal ? 0 : w;
  const int ug = p.use_globals;
  const size_t rs = (size_t)p.H * 64;
  const size_t boff = (size_t)bt.b * n * rs + (size_t)bt.h * 64;
  const e16* Q = reinterpret_cast<const e16*>(p.q) + boff;
  const e16* K = reinterpret_cast<const e16*>(p.k) + boff;
  const e16* V = reinterpret_cast<const e16*>(p.v) + boff;
  const e16* DO = reinterpret_cast<const e16*>(p.dout) + boff;
  const int8_t* mb = p.mask + (size_t)bt.b * n;
  const size_t bh = (size_t)bt.b * p.H + bt.h;

  const int tq = bt.t0 + 32 * wv + c;
  const bool qin = tq < bt.len;
  const int qpos = bt.r + d * (qin ? tq : bt.len - 1);
  // the row's mask byte, statistics and the batch row's global count load
  // together (qpos is a valid row in every case); the validity test waits
  // for the block loop's first loads as well
  const int8_t mq = mb[qpos];
  const float lneg_q = p.lneg[bh * n + qpos], dneg_q = p.dneg[bh * n + qpos];
  const int nG = ug ? p.gcount[bt.b] : 0;
  int qty = 0;
  bool qloc = false;
  float lse2 = 0.f, dd = 0.f;  // lse in base 2, and D
  e16x8 qf[4], df[4];

  const int kbase = bt.t0 - w;
  const int S = (kBwdBandRows - 1 + w + w_hi) / 32 + 1;
  const int jlo = kbase >= 0 ? 0 : (-kbase) / 32;
  const int jhi = min(S, (bt.len - kbase + 31) / 32);
  const int nwin = max(jhi - jlo, 0);
  const int32_t* gl = p.glist + (size_t)bt.b * p.gstride;
  const int nblk = nwin + (nG + 31) / 32;
  // token position of key row `row` of block i (a valid row in every case)
  // the global list in LDS (read in asm: no vector-memory instruction in
  // the block loop but its direct-to-LDS loads)
  auto kpos = [&](int i, int row) -> int {
    if (i < nwin) {
      const int kk = kbase + 32 * (jlo + i) + row;
      return bt.r + d * (kk < 0 ? 0 : (kk >= bt.len ? bt.len - 1 : kk));
    }
    const int gi = 32 * (i - nwin) + row;
    return (int)lds_word(&sh.gpos[gi < nG ? gi : nG - 1]);
  };
  const BandAddr ad = band_addr(sh.ring, lane);
  const int q0w = bt.t0 + 32 * wv;  // the wave's first query row
  // window key rows that exist and are valid (mask 1 or 2)
  auto key_ok = [&](int i, int row, int m) {
    const int kk = kbase + 32 * (jlo + i) + row;
    return kk >= 0 && kk < bt.len && eff_mask((int8_t)m, ug) != 0;
  };
  // the first refill also puts the global list in LDS: its loads fly with
  // the table's, its stores follow the table's barrier and get their own
  static_assert(LF_MAX_GLOBAL <= 4 * 256, "four list entries per thread");
  auto refill = [&](int i0) {
    int gv[4] = {0, 0, 0, 0};
    if (i0 == 0)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((int)threadIdx.x + 256 * k < nG) gv[k] = gl[threadIdx.x + 256 * k];
    if (i0 < nwin) tab_fill(sh, mb, i0, nwin, wv, lane, kpos, key_ok);
    if (i0 == 0 && nG > 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((int)threadIdx.x + 256 * k < nG) sh.gpos[threadIdx.x + 256 * k] = gv[k];
      __syncthreads();
    } else if (i0 >= nwin) {
      __syncthreads();
    }
  };
  // every wave takes every block; a tile with no local row only writes zeros
  auto gate = [&]() {
    qty = qin ? eff_mask(mq, ug) : 0;
    qloc = qty == 1;
    lse2 = qloc ? -p.c * lneg_q : 0.f;
    dd = qloc ? -dneg_q : 0.f;
    return __syncthreads_or(qloc) != 0;
  };
  f32x16 acc[2] = {zero16(), zero16()};
  auto issue = [&](int i, int stg) {
    issue_pair(K, V, rs, [&](int row) { return kpos(i, row); }, sh.ring + stg * kStageB, wv, lane);
  };
  auto step = [&](int i, int stage) {
    uint32_t kval;
    int k0 = 0;
    if (i < nwin) {
      k0 = kbase + 32 * (jlo + i);
      // no key of the block in the window of any of the wave's queries
      if (k0 > q0w + 31 + w_hi || k0 + 31 < q0w - w) return;
      kval = __builtin_amdgcn_readfirstlane(lds_word(&sh.tab[i % kBandTab]));
    } else {
      kval = (uint32_t)__ballot(32 * (i - nwin) + c < nG);
    }
    if (kval == 0u) return;
    // one tensor at a time (few registers live at once): S^T from the K
    // rows, dP^T from the V rows, then K^T for dQ^T
    const uint32_t so = (uint32_t)(stage * kStageB);
    f32x16 sc = zero16(), dp = zero16();
    {
      e16x8 rf[4];
      read_rows4<0>(rf, ad, so);
#pragma unroll
      for (int s = 0; s < 4; ++s) sc = mma(rf[s], qf[s], sc);
      read_rows4<1>(rf, ad, so);
#pragma unroll
      for (int s = 0; s < 4; ++s) dp = mma(rf[s], df[s], dp);
    }
    bool fast = false;
    uint32_t okb = 0;  // bit k: (this lane's query, key row k) is a scored pair
    if (i < nwin) {
      fast = kval == 0xffffffffu && k0 >= q0w + 31 - w && k0 + 31 <= q0w + w_hi && __all(qloc);
      if (!fast) okb = qloc ? (kval & bit_range(tq - w - k0, tq + w_hi - k0)) : 0u;
    } else if (__any(qloc)) {
      // global keys score where they are not already in the window:
      // in W(i) when |i - g| <= w d and d divides i - g
      const int gp = kpos(i, c);
      const int wd = w * d;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = acc_row(r, hl);
        const int g = __shfl(gp, kr);
        const int dg = qpos - g;
        const bool in_w = dg >= -wd && dg <= wd && dg % d == 0;
        okb |= (!in_w ? 1u : 0u) << kr;
      }
      okb = qloc ? (okb & kval) : 0u;
    }
    e16x8 ds8[2];
    if (fast) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(p.c, sc[r], -lse2));
        ds8[r >> 3][r & 7] = (e16)(pr * (dp[r] - dd));
      }
    } else {
      const uint32_t okh = okb >> (4 * hl);  // row acc_row(r, hl) is bit acc_row(r, 0)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = (okh >> acc_row(r, 0)) & 1u;
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(p.c, sc[r], -lse2));
        ds8[r >> 3][r & 7] = (e16)(ok ? pr * (dp[r] - dd) : 0.f);
      }
    }
    e16x8 kt[2][2];
    read_cols<0>(kt, ad, so);  // K^T
    if (!fast && kval != 0xffffffffu) zero_cols(kt, kval, hl);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc[db] = mma(kt[db][ks], ds8[ks], acc[db]);
  };
  auto prologue = [&]() {
    load_frag(qf, Q + (size_t)qpos * rs, true, hl);
    load_frag(df, DO + (size_t)qpos * rs, true, hl);
  };
  band_loop(nblk, nwin, issue, prologue, refill, gate, step);
  if (qin) {
    float* dst = p.dq + boff + (size_t)qpos * rs;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = qloc ? sc * acc[db][4 * g + e] : 0.f;
        store_f4(dst + 32 * db + 8 * g + 4 * hl, v4);
      }
  }
}

// dk/dv workgroup.  Wave wv owns key rows t0 + 32 wv + lane % 32 (K and V
// as B operands, kept in LDS and read with each block); the query blocks
// are the rows qbase + 32 (jlo + j) + row
// whose windows reach the tile's keys, staged with their -lse / scale and
// -D.  Per block: S = Q K^T, dP = dO V^T (lane: one key, 16 queries), P and
// dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.  Keys with mask 2 are
// left to the global-token work (which adds every local row's terms to
// them); keys with mask 0 get zeros.
__device__ void band_dkv(const BwdParams& p, BandShared& sh, const BandTile& bt, int wv) {
  const int lane = threadIdx.x & 63, c = lane & 31, hl = lane >> 5;
  const int n = p.n, w = p.w, d = bt.d;
  const int w_hi = p.causal ? 0 : w;
  const int ug = p.use_globals;
  const size_t rs = (size_t)p.H * 64;
  const size_t boff = (size_t)bt.b * n * rs + (size_t)bt.h * 64;
  const e16* Q = reinterpret_cast<const e16*>(p.q) + boff;
  const e16* K = reinterpret_cast<const e16*>(p.k) + boff;
  const e16* V = reinterpret_cast<const e16*>(p.v) + boff;
  const e16* DO = reinterpret_cast<const e16*>(p.dout) + boff;
  const int8_t* mb = p.mask + (size_t)bt.b * n;
  const size_t bh = (size_t)bt.b * p.H + bt.h;
  const float* lse_bh = p.lneg + bh * n;  // -lse / scale
  const float* d_bh = p.dneg + bh * n;     // -D

  const int tk = bt.t0 + 32 * wv + c;
  const bool kin = tk < bt.len;
  const int kp = bt.r + d * (kin ? tk : bt.len - 1);
  // the key's mask byte loads with the block loop's first loads (kp is a
  // valid row in every case)
  const int8_t mk = mb[kp];
  int kty = 0;
  bool kok = false, all_keys = false;
  f32x16 ak[2], av[2];  // zeroed at the gate, after the prologue's registers are free
  auto write_out = [&]() {
    if (!kin || kty == 2) return;
    float* dk = p.dk + boff + (size_t)kp * rs;
    float* dv = p.dv + boff + (size_t)kp * rs;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float k4[4], v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = kok ? p.scale * ak[db][4 * g + e] : 0.f;
          v4[e] = kok ? av[db][4 * g + e] : 0.f;
        }
        store_f4(dk + 32 * db + 8 * g + 4 * hl, k4);
        store_f4(dv + 32 * db + 8 * g + 4 * hl, v4);
      }
  };
  e16x8 kf[4], vf[4];

  // rows whose windows reach the tile's keys: tq in [tk - w_hi, tk + w]
  const int qbase = bt.t0 - w_hi;
  const int S = (kBwdBandRows - 1 + w + w_hi) / 32 + 1;
  const int jlo = qbase >= 0 ? 0 : (-qbase) / 32;
  const int jhi = min(S, (bt.len - qbase + 31) / 32);
  const int nq = max(jhi - jlo, 0);
  auto qrow0 = [&](int j) -> int { return qbase + 32 * (jlo + j); };
  auto qpos = [&](int j, int row) -> int {
    const int t = qrow0(j) + row;
    return bt.r + d * (t < 0 ? 0 : (t >= bt.len ? bt.len - 1 : t));
  };
  const BandAddr ad = band_addr(sh.ring, lane);
  const uint32_t sa = lds_addr(sh.ring + 2 * kBlkB) + 16u * (uint32_t)hl;
  const uint32_t vb = lds_addr(sh.vfr) + 4096u * (uint32_t)wv + 16u * (uint32_t)lane;
  const uint32_t kb = lds_addr(sh.kfr) + 4096u * (uint32_t)wv + 16u * (uint32_t)lane;
  const int k0w = bt.t0 + 32 * wv;  // the wave's first key row
  // query rows that exist and are local (mask 1)
  auto row_ok = [&](int j, int row, int m) {
    const int t = qrow0(j) + row;
    return t >= 0 && t < bt.len && eff_mask((int8_t)m, ug) == 1;
  };
  auto refill = [&](int j0) { tab_fill(sh, mb, j0, nq, wv, lane, qpos, row_ok); };
  // stage: Q rows, dO rows, then the 32 rows' lse (lanes 0-31) and D
  // (lanes 32-63); every wave loads the statistics (the same bytes), so that
  // every wave issues the same number of loads
  auto issue = [&](int j, int stg) {
    unsigned char* stage = sh.ring + stg * kStageB;
    issue_pair(Q, DO, rs, [&](int row) { return qpos(j, row); }, stage, wv, lane);
    const float* src = ((lane >> 5) ? d_bh : lse_bh) + qpos(j, c);
    __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(stage + 2 * kBlkB), 4, 0, 0);
  };
  auto step = [&](int j, int stage) {
    const int t0q = qrow0(j);
    // no row of the block has a key of the wave in its window
    if (t0q > k0w + 31 + w || t0q + 31 < k0w - w_hi) return;
    const uint32_t qval = __builtin_amdgcn_readfirstlane(lds_word(&sh.tab[j % kBandTab]));
    if (qval == 0u) return;
    // (query row q, this lane's key) in the window: tk - w_hi <= t0q + q <= tk + w
    const bool fast = all_keys && qval == 0xffffffffu && t0q + 31 - k0w <= w && k0w + 31 - t0q <= w_hi;
    // One tensor at a time, so that few registers are live at once: S from
    // the Q rows, dP from the dO rows (V from LDS), P and dS, then
    // dV^T += dO^T P and dK^T += Q^T dS from the transposed rows.
    auto body = [&](uint32_t so) {
      e16x8 rf[4];
      f32x4 st4[4];
      // S + (-lse / scale) and dP + (-D): the row statistics enter as the
      // accumulators' starting values (element r of a lane is row 8 (r / 4)
      // + 4 hl + r % 4, float4 r / 4 of the staged values)
      // P first (bf16, 8 registers), so that S is dead before dP is formed;
      // dS = P dP takes the rounded P
      e16x8 p8[2], ds8[2];
      {
        f32x16 sc;
        e16x8 kf[4];
        read_rows_stats<0>(rf, st4, kf, ad, sa, kb, so);
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = st4[r >> 2][r & 3];
#pragma unroll
        for (int s = 0; s < 4; ++s) sc = mma(rf[s], kf[s], sc);
        __builtin_amdgcn_sched_barrier(0);
        if (fast) {
#pragma unroll
          for (int r = 0; r < 16; ++r) p8[r >> 3][r & 7] = (e16)__builtin_amdgcn_exp2f(p.c * sc[r]);
        } else {
          // bits of this lane's rows: row acc_row(r, hl) is bit acc_row(r, 0) of okh
          const uint32_t okh = (kok ? (qval & bit_range(tk - w_hi - t0q, tk + w - t0q)) : 0u) >> (4 * hl);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = (okh >> acc_row(r, 0)) & 1u;
            p8[r >> 3][r & 7] = (e16)(ok ? __builtin_amdgcn_exp2f(p.c * sc[r]) : 0.f);
          }
        }
      }
      {
        f32x16 dp;
        e16x8 vf[4];
        read_rows_stats<1>(rf, st4, vf, ad, sa, vb, so);
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = st4[r >> 2][r & 3];
#pragma unroll
        for (int s = 0; s < 4; ++s) dp = mma(rf[s], vf[s], dp);
#pragma unroll
        for (int r = 0; r < 16; ++r) ds8[r >> 3][r & 7] = (e16)((float)p8[r >> 3][r & 7] * dp[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool zc = !fast && qval != 0xffffffffu;
      e16x8 t8[2][2];
      read_cols<1>(t8, ad, so);  // dO^T
      if (zc) zero_cols(t8, qval, hl);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) av[db] = mma(t8[db][ks], p8[ks], av[db]);
      __builtin_amdgcn_sched_barrier(0);
      read_cols<0>(t8, ad, so);  // Q^T
      if (zc) zero_cols(t8, qval, hl);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) ak[db] = mma(t8[db][ks], ds8[ks], ak[db]);
    };
    body((uint32_t)(stage * kStageB));
  };
  auto prologue = [&]() {
    load_frag(kf, K + (size_t)kp * rs, true, hl);
    load_frag(vf, V + (size_t)kp * rs, true, hl);
  };
  // a tile with no key of mask 1 only writes zeros
  auto gate = [&]() {
    kty = kin ? eff_mask(mk, ug) : 0;
    kok = kty == 1;
    all_keys = __all(kok);
    const bool go = __syncthreads_or(kok) != 0;
    // the wave's V fragments to LDS (read back each step, by this wave only)
    if (go)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<e16x8*>(sh.kfr + 4096 * wv + 1024 * s + 16 * lane) = kf[s];
        *reinterpret_cast<e16x8*>(sh.vfr + 4096 * wv + 1024 * s + 16 * lane) = vf[s];
      }
    ak[0] = ak[1] = av[0] = av[1] = zero16();
    return go;
  };
  band_loop(nq, nq, issue, prologue, refill, gate, step);
  write_out();
}

// Units of the band launch: unit x runs on XCD x % 8; each XCD is dealt a
// contiguous range of units (neighbouring tiles share their window rows,
// which then stay in that XCD's L2), and a tile's dq and dk/dv units are
// neighbours.
__device__ void bwd_band_body(const BwdParams& p) {
  __shared__ BandShared sh;
  const int N = 2 * p.n_bt;
  const int x = blockIdx.x;
  const int per = N / 8, rem = N % 8;
  const int xcd = x % 8, y = x / 8;
  const int m = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + y;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BandTile bt = decode_band(p, m >> 1);
  if (bt.t0 >= bt.len) return;  // every wave of the workgroup returns here
  if (m & 1)
    band_dkv(p, sh, bt, wv);
  else
    band_dq(p, sh, bt, wv);
}

// The global-token launch: four units per workgroup, one per wave.
__device__ void bwd_glob_body(const BwdParams& p) {
  __shared__ BwdShared unit[4];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = blockIdx.x;
  // the GQ and GK workgroups first (each walks four chunks), the shorter
  // GKV units after them, in the slots the first ones leave
  const int per = p.B * p.H * p.gslots * ((p.chunks + 3) / 4);
  if (x < 2 * per) {
    bwd_gqk_group(p, unit, wv, x < per ? x : x - per, x < per);
    return;
  }
  const int u = 4 * (x - 2 * per) + wv;  // GKV: four units per workgroup
  if (u < p.n_gkv) bwd_gkv_unit(p, unit[wv], u);
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
  if (q4 == 0) {
    const size_t at = ((size_t)b * p.H + h) * p.n + i;
    p.dneg[at] = -s;
    const float l = p.lse[at];
    p.lneg[at] = __builtin_isfinite(l) ? -l / p.scale : 0.f;  // -inf: a row with no keys
  }
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void lf_attn_bwd_f16(const BwdParams p) {
  bwd_band_body(p);
}
__global__ __launch_bounds__(256) void lf_attn_bwd_prep_f16(const BwdParams p) { prep_body(p); }
// No wave-count bound: the units' loops keep their fragments, accumulators
// and block descriptions in registers (bounded to the band kernel's budget
// they spill, and every reload waits on memory inside the loop).
__global__ __launch_bounds__(256) void lf_attn_bwd_glob_f16(const BwdParams p) { bwd_glob_body(p); }
#else
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void lf_attn_bwd_bf16(const BwdParams p) {
  bwd_band_body(p);
}
__global__ __launch_bounds__(256) void lf_attn_bwd_prep_bf16(const BwdParams p) { prep_body(p); }
// No wave-count bound: the units' loops keep their fragments, accumulators
// and block descriptions in registers (bounded to the band kernel's budget
// they spill, and every reload waits on memory inside the loop).
__global__ __launch_bounds__(256) void lf_attn_bwd_glob_bf16(const BwdParams p) { bwd_glob_body(p); }
#endif

}  // namespace

#if LF_HALF_F16
#define LF_BWD_SUFFIX(x) x##_f16
#else
#define LF_BWD_SUFFIX(x) x##_bf16
#endif
namespace {
void LF_BWD_SUFFIX(band_launch)(const BwdParams& bp, void* stream) {
  hipLaunchKernelGGL(LF_BWD_SUFFIX(lf_attn_bwd), dim3(2 * bp.n_bt), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     bp);
}
void LF_BWD_SUFFIX(glob_launch)(const BwdParams& bp, void* stream) {
  const unsigned nglob = (unsigned)bwd_glob_workgroups(bp.n_gkv, bp.B, bp.H, bp.gslots, bp.chunks);
  hipLaunchKernelGGL(LF_BWD_SUFFIX(lf_attn_bwd_glob), dim3(nglob), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     bp);
}
}  // namespace

#if LF_HALF_F16
int launch_backward_f16(const BwdParams& bp, void* stream) {
#else
int launch_backward(const BwdParams& bp, void* stream) {
  if (bp.dtype == LF_F16) return launch_backward_f16(bp, stream);
#endif
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t rows = (size_t)bp.B * bp.n * bp.H;
  const unsigned nlist = bp.use_globals ? (unsigned)bp.B : 0u;
  hipLaunchKernelGGL(LF_BWD_SUFFIX(lf_attn_bwd_prep), dim3(nlist + (unsigned)((rows + 15) / 16)), dim3(256), 0, s, bp);
  if (bwd_glob_workgroups(bp.n_gkv, bp.B, bp.H, bp.gslots, bp.chunks) == 0) {
    LF_BWD_SUFFIX(band_launch)(bp, stream);
    return (int)hipGetLastError();
  }
  return launch_backward_pair(bp, stream, LF_BWD_SUFFIX(band_launch), LF_BWD_SUFFIX(glob_launch));
}
#undef LF_BWD_SUFFIX

#if !LF_HALF_F16
// The library's second stream per device for the backward's global-token
// launch (default priority, not synchronising with the null stream) and its
// fork and join events, created once, outside graph capture.
namespace {
constexpr int kAuxDevices = 64;
struct BwdAux {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};
BwdAux g_aux[kAuxDevices];

bool make_aux(BwdAux& a) {
  if (hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) != hipSuccess) a.s = nullptr;
  if (a.s && hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess) a.fork = nullptr;
  if (a.s && a.fork && hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess) a.join = nullptr;
  if (a.s && a.fork && a.join) return true;
  if (a.fork) (void)hipEventDestroy(a.fork);
  if (a.s) (void)hipStreamDestroy(a.s);
  a.s = nullptr;
  a.fork = a.join = nullptr;
  a.failed = true;
  (void)hipGetLastError();  // the failure is handled: both launches go on the caller's stream
  return false;
}
}  // namespace

int launch_backward_pair(const BwdParams& bp, void* stream, BwdLaunch band, BwdLaunch glob) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kAuxDevices) {
    BwdAux& a = g_aux[dev];
    std::lock_guard<std::mutex> lock(a.mu);
    if (!a.s && !a.failed) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) make_aux(a);
    }
    // the fork point is after the work already on s (the preparation);
    // the band launch is enqueued first, so that its workgroups take the
    // CUs first and the global-token workgroups fill the slots they free
    if (a.s && hipEventRecord(a.fork, s) == hipSuccess) {
      band(bp, stream);
      if (hipStreamWaitEvent(a.s, a.fork, 0) != hipSuccess) {
        glob(bp, stream);
        return (int)hipGetLastError();
      }
      glob(bp, a.s);
      // without the join the caller's stream would not wait for the
      // global-token launch: report it
      hipError_t e = hipEventRecord(a.join, a.s);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, a.join, 0);
      if (e != hipSuccess) return (int)e;
      return (int)hipGetLastError();
    }
  }
  band(bp, stream);
  glob(bp, stream);
  return (int)hipGetLastError();
}
#endif

}  // namespace lf
