// Longformer combined sliding-window + global attention forward for gfx950.
//
// One launch computes every output row:
//   * band workgroups own a tile of kTileQ consecutive query rows of one
//     (batch row b, head h, residue class r of the head's dilation d).  A
//     dilated window over positions {r, r+d, r+2d, ...} is a plain window
//     over that subsequence, so each residue class is handled as an
//     undilated sequence with row stride d*H*D (segmentfault Longformer
//     summary, "Dilated sliding window": the dilated window keeps the cost
//     of the plain one).  They write local rows (mask 1) and zero rows
//     (mask 0);
//   * global-row workgroups own one split of kGlobalChunk keys of one
//     (b, h) for every global token of b: each global token attends to all
//     tokens with the global projections (segmentfault summary, "Global
//     attention" and "Linear projections for global attention").  Each
//     split leaves a partial (max, sum, unnormalised output) in the
//     workspace; the last split to arrive merges them and writes the rows.
//
// Inner block (both kinds): 32 keys x 64 queries per wave.
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 key rows, B = 32 query
//   columns, K-dim = head dim).  In the 32x32 accumulator a lane owns one
//   column (a query) and 16 of its 32 keys; the other 16 sit in lane ^ 32.
//   So the softmax row max and row sum are in-lane plus one lane swap.
//   The accumulator, rounded to bf16, is directly the B operand of
//   O^T = V^T P^T (A = 32 head-dim rows of V^T read from LDS, B = P^T), with
//   the key order of P^T as the accumulator holds it and V^T read in the
//   same order.  Only V goes through LDS, transposed on the way in.
//   Softmax is online in base 2 (scale*log2e folded into one FMA), fp32,
//   with a lazy rescale: the running reference max only moves when a block
//   max exceeds it by more than 2^8, which leaves the result exact while
//   skipping most accumulator rescales.
//
// The key range of a band tile (kTileQ + 2w keys) is split over the 4 waves
// of the workgroup block by block; their partial results are merged
// through LDS at the end.  Global columns of local rows (the symmetric half
// of global attention) are extra gathered key blocks, masked so that a
// global key already inside the row's window is not counted twice
// (ultralytics glossary worked example: the window and the global
// row/column are OR-ed into one boolean pattern).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lf_attn_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// LDS staging of one 32-key V block, per wave.
//   bf16: V^T [64 head dims][kVtStride keys] (transposed)
//   f32:  V   [32 keys][kVStrideF32 dims]
constexpr int kVtStride = 40;      // bf16 elements per V^T row (32 + pad)
constexpr int kVStrideF32 = 68;    // floats per V row (64 + pad)
constexpr int kStageBytesBf16 = kHeadDim * kVtStride * 2;
constexpr int kStageBytesF32 = kBlockK * kVStrideF32 * 4;
constexpr int kStageBytes = kStageBytesF32 > kStageBytesBf16 ? kStageBytesF32 : kStageBytesBf16;
// Merge of partial outputs: 2 slots of 64 lanes x 64 floats.
constexpr int kMergeSlotFloats = 64 * 64;
constexpr int kMergeBytes = 2 * kMergeSlotFloats * 4;
constexpr int kBufBytes = (kWaves * kStageBytes > kMergeBytes) ? kWaves * kStageBytes : kMergeBytes;

template <bool B16>
using elem_t = typename std::conditional<B16, __bf16, float>::type;

// Per-lane operand fragment of 64 head dims of one row (query or key) for
// the QK^T contraction; the head dims a lane holds depend on lane / 32.
template <bool B16>
struct Frag;
template <>
struct Frag<true> {
  bf16x8 x[4];  // dims 16s + 8*(lane/32) + [0, 8)
};
template <>
struct Frag<false> {
  float x[32];  // dims 32*(lane/32) + [0, 32)
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void load_frag(Frag<true>& f, const __bf16* row, int hh) {
  const bf16x8* p = reinterpret_cast<const bf16x8*>(row);
#pragma unroll
  for (int s = 0; s < 4; ++s) f.x[s] = p[2 * s + hh];
}

__device__ __forceinline__ void load_frag(Frag<false>& f, const float* row, int hh) {
  const f32x4* p = reinterpret_cast<const f32x4*>(row + 32 * hh);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 t = p[i];
    f.x[4 * i + 0] = t[0];
    f.x[4 * i + 1] = t[1];
    f.x[4 * i + 2] = t[2];
    f.x[4 * i + 3] = t[3];
  }
}

// acc (32 keys x 32 queries) += K Q^T over the 64 head dims.
__device__ __forceinline__ void qk(f32x16& acc, const Frag<true>& kf, const Frag<true>& qf) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.x[s], qf.x[s], acc, 0, 0, 0);
}

__device__ __forceinline__ void qk(f32x16& acc, const Frag<false>& kf, const Frag<false>& qf) {
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x[i], qf.x[i], acc, 0, 0, 0);
}

// Accumulator element r of a lane holds key row kr(r) of the block.
__device__ __forceinline__ int acc_key(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Stage the V rows of one 32-key block into this wave's LDS area.  Keys
// whose bit is clear in keymask are stored as zeros, so that keys outside a
// row's key set contribute exactly nothing even if their stored values are
// not finite.  key_pos is this lane's key row position (row lane % 32).
__device__ __forceinline__ void stage_v(unsigned char* lds, const __bf16* vbase, size_t rstride,
                                        int key_pos, uint32_t keymask) {
  const int lane = lane_id();
  const int kg = lane & 7;   // keys 4kg .. 4kg+3
  const int dg = lane >> 3;  // dims 8dg .. 8dg+7
  u32x4 rows[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kr = 4 * kg + e;
    const int pos = __shfl(key_pos, kr);
    rows[e] = *reinterpret_cast<const u32x4*>(vbase + (size_t)pos * rstride + 8 * dg);
    if (!((keymask >> kr) & 1u)) rows[e] = u32x4{0u, 0u, 0u, 0u};
  }
  __bf16* vt = reinterpret_cast<__bf16*>(lds);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // dword i of a row holds dims 2i (low half) and 2i+1 (high half)
    u32x2 lo, hi;
    lo[0] = (rows[0][i] & 0xffffu) | (rows[1][i] << 16);
    lo[1] = (rows[2][i] & 0xffffu) | (rows[3][i] << 16);
    hi[0] = (rows[0][i] >> 16) | (rows[1][i] & 0xffff0000u);
    hi[1] = (rows[2][i] >> 16) | (rows[3][i] & 0xffff0000u);
    const int d = 8 * dg + 2 * i;
    *reinterpret_cast<u32x2*>(vt + d * kVtStride + 4 * kg) = lo;
    *reinterpret_cast<u32x2*>(vt + (d + 1) * kVtStride + 4 * kg) = hi;
  }
}

__device__ __forceinline__ void stage_v(unsigned char* lds, const float* vbase, size_t rstride,
                                        int key_pos, uint32_t keymask) {
  const int lane = lane_id();
  const int kr = lane >> 1;
  const int half = lane & 1;
  const int pos = __shfl(key_pos, kr);
  const bool keep = (keymask >> kr) & 1u;
  const f32x4* src = reinterpret_cast<const f32x4*>(vbase + (size_t)pos * rstride + 32 * half);
  float* dst = reinterpret_cast<float*>(lds) + kr * kVStrideF32 + 32 * half;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 t = src[i];
    if (!keep) t = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dst + 4 * i) = t;
  }
}

// Probabilities of one block in the operand form of the PV product.
template <bool B16>
struct PFrag;
template <>
struct PFrag<true> {
  bf16x8 x[2];  // PV k-step ks holds accumulator elements 8ks .. 8ks+7
};
template <>
struct PFrag<false> {
  float x[16];
};

__device__ __forceinline__ void to_pfrag(PFrag<true>& pf, const f32x16& p) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf.x[ks][e] = (__bf16)p[8 * ks + e];
}

__device__ __forceinline__ void to_pfrag(PFrag<false>& pf, const f32x16& p) {
#pragma unroll
  for (int r = 0; r < 16; ++r) pf.x[r] = p[r];
}

// O^T (64 dims x 32 queries, as two 32x32 accumulators) += V^T P^T.
__device__ __forceinline__ void pv(f32x16 (&o)[2], const PFrag<true>& pf, const unsigned char* lds, int lane) {
  const __bf16* vt = reinterpret_cast<const __bf16*>(lds);
  const int hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const __bf16* row = vt + (32 * db + (lane & 31)) * kVtStride;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(row + 16 * ks + 4 * hh);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(row + 16 * ks + 8 + 4 * hh);
      const u32x4 a = u32x4{a0[0], a0[1], a1[0], a1[1]};
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf.x[ks], o[db], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void pv(f32x16 (&o)[2], const PFrag<false>& pf, const unsigned char* lds, int lane) {
  const float* vs = reinterpret_cast<const float*>(lds);
  const int hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float a = vs[acc_key(r, hh) * kVStrideF32 + 32 * db + (lane & 31)];
      o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf.x[r], o[db], 0, 0, 0);
    }
  }
}

// Running state of one wave: 64 query columns as two 32-column halves.
struct WaveState {
  f32x16 o[2][2];   // [query half nb][dim half db]
  float m[2];       // reference max (log2 domain) of the lane's query
  float l[2];       // partial row sum of this lane (16 of the 32 keys per block)
  int cnt[2];       // partial count of scored keys of this lane
};

__device__ __forceinline__ void state_init(WaveState& st) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.m[nb] = kNegInf;
    st.l[nb] = 0.f;
    st.cnt[nb] = 0;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nb][db][r] = 0.f;
  }
}

// One 32-key block against the wave's 64 queries.  keep(nb, r) decides,
// for edge blocks, whether accumulator element r of query half nb is in
// the row's key set; on interior blocks every element is.
template <bool B16, class Keep>
__device__ __forceinline__ void attend_block(WaveState& st, const Frag<B16> (&qf)[2], const elem_t<B16>* kbase,
                                             const elem_t<B16>* vbase, size_t rstride, int key_pos,
                                             uint32_t keymask, bool edge, Keep keep, unsigned char* lds,
                                             float c) {
  const int lane = lane_id();
  const int hh = lane >> 5;
  Frag<B16> kf;
  load_frag(kf, kbase + (size_t)key_pos * rstride, hh);
  stage_v(lds, vbase, rstride, key_pos, keymask);

  f32x16 s[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[nb][r] = 0.f;
    qk(s[nb], kf, qf[nb]);
  }

  if (edge) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      int kept = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = acc_key(r, hh);
        const bool ok = ((keymask >> kr) & 1u) && keep(nb, kr);
        kept += ok ? 1 : 0;
        if (!ok) s[nb][r] = kNegInf;
      }
      st.cnt[nb] += kept;
    }
  } else {
    st.cnt[0] += 16;
    st.cnt[1] += 16;
  }

  float mb[2];
  bool need = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float mx = s[nb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mb[nb] = mx * c;
    need |= mb[nb] > st.m[nb] + kRescaleSlack;
  }
  if (__any(need)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mn = fmaxf(st.m[nb], mb[nb]);
      const float alpha = (st.m[nb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m[nb] - mn);
      st.m[nb] = mn;
      st.l[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[nb][db][r] *= alpha;
    }
  }

  PFrag<B16> pf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float msub = (st.m[nb] == kNegInf) ? 0.f : st.m[nb];
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][r], c, -msub));
      s[nb][r] = pr;
      sum += pr;
    }
    st.l[nb] += sum;
    to_pfrag(pf[nb], s[nb]);
  }

  wave_sync();  // V block staged by all lanes of the wave
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) pv(st.o[nb], pf[nb], lds, lane);
  wave_sync();  // reads done before the next block overwrites the staging area
}

// Ordered list of positions j with mask_row[j] == 2 into G (LDS), at most
// cap entries; returns the total count.  Every thread of the workgroup
// calls it and gets the same result.
__device__ int scan_globals(const int8_t* __restrict__ mrow, int n, int* G, int cap, int* s_wave) {
  int total = 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  for (int base = 0; base < n; base += kThreads * 4) {
    const int p0 = base + tid * 4;
    unsigned bits = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pidx = p0 + e;
      if (pidx < n && mrow[pidx] == 2) bits |= 1u << e;
    }
    if (!__syncthreads_or(bits != 0)) continue;
    const int cnt = __popc(bits);
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wv] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int t = s_wave[i];
      before += (i < wv) ? t : 0;
      all += t;
    }
    int slot = total + before + x - cnt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((bits >> e) & 1u) {
        if (slot < cap) G[slot] = p0 + e;
        ++slot;
      }
    }
    total += all;
    __syncthreads();
  }
  return total;
}

struct Shared {
  int G[LF_MAX_GLOBAL];
  int wave_tmp[kWaves];
  int flag;
  float m[kWaves][kTileQ];
  float l[kWaves][kTileQ];
  int cnt[kWaves][kTileQ];
  __attribute__((aligned(16))) unsigned char buf[kBufBytes];
};

// Merge the partial results of the 4 waves into wave 0's registers.
__device__ void merge_waves(WaveState& st, Shared& sh) {
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.l[nb] += __shfl_xor(st.l[nb], 32);
    st.cnt[nb] += __shfl_xor(st.cnt[nb], 32);
    if (hh == 0) {
      sh.m[wv][32 * nb + lane] = st.m[nb];
      sh.l[wv][32 * nb + lane] = st.l[nb];
      sh.cnt[wv][32 * nb + lane] = st.cnt[nb];
    }
  }
  float* slots = reinterpret_cast<float*>(sh.buf);
  auto write_slot = [&](int slot) {
    f32x4* dst = reinterpret_cast<f32x4*>(slots + slot * kMergeSlotFloats);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 t = f32x4{st.o[nb][db][4 * g], st.o[nb][db][4 * g + 1], st.o[nb][db][4 * g + 2],
                                st.o[nb][db][4 * g + 3]};
          dst[((nb * 2 + db) * 4 + g) * 64 + lane] = t;
        }
  };
  auto absorb = [&](int slot, int other) {
    const f32x4* src = reinterpret_cast<const f32x4*>(slots + slot * kMergeSlotFloats);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int q = 32 * nb + (lane & 31);
      const float mo = sh.m[other][q];
      const float lo = sh.l[other][q];
      const int co = sh.cnt[other][q];
      const float mn = fmaxf(st.m[nb], mo);
      const float fs = (st.m[nb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m[nb] - mn);
      const float fo = (mo == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
      st.m[nb] = mn;
      st.l[nb] = st.l[nb] * fs + lo * fo;
      st.cnt[nb] += co;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 t = src[((nb * 2 + db) * 4 + g) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) st.o[nb][db][4 * g + i] = st.o[nb][db][4 * g + i] * fs + t[i] * fo;
        }
    }
  };
  __syncthreads();  // all waves done with their staging areas (aliased below)
  if (wv >= 2) write_slot(wv - 2);
  __syncthreads();
  if (wv < 2) absorb(wv, wv + 2);
  __syncthreads();
  if (wv == 1) {
    write_slot(0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      if (hh == 0) {
        sh.m[1][32 * nb + lane] = st.m[nb];
        sh.l[1][32 * nb + lane] = st.l[nb];
        sh.cnt[1][32 * nb + lane] = st.cnt[nb];
      }
  }
  __syncthreads();
  if (wv == 0) absorb(0, 1);
}

template <bool B16>
__device__ __forceinline__ void store4(elem_t<B16>* dst, const float* v);

template <>
__device__ __forceinline__ void store4<true>(__bf16* dst, const float* v) {
  bf16x4 t;
  t[0] = (__bf16)v[0];
  t[1] = (__bf16)v[1];
  t[2] = (__bf16)v[2];
  t[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(dst) = t;
}

template <>
__device__ __forceinline__ void store4<false>(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ int xcd_remap(int x, int N) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of tiles so neighbouring tiles (which share K/V
  // halos) share one L2.
  const int per = N / 8, rem = N % 8;
  const int xcd = x % 8, y = x / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + y;
}

// ---------------------------------------------------------------------------
// Band workgroup: one tile of kTileQ query rows of (b, h, residue r).
// ---------------------------------------------------------------------------
template <bool B16>
__device__ void band_tile(const KernelParams& p, int L, Shared& sh) {
  using T = elem_t<B16>;
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int b = L / p.tiles_per_b;
  const int rem = L - b * p.tiles_per_b;
  int h = 0;
  while (h + 1 < p.H && p.tile0[h + 1] <= rem) ++h;
  const int id = rem - p.tile0[h];
  const int dil = p.dil[h];
  const int n = p.n;
  const int qn = n / dil, rm = n % dil;
  const int T1 = (qn + 1 + kTileQ - 1) / kTileQ, T0 = (qn + kTileQ - 1) / kTileQ;
  int r, tt, n_r;
  if (id < rm * T1) {
    r = id / T1;
    tt = id - r * T1;
    n_r = qn + 1;
  } else {
    const int id2 = id - rm * T1;
    r = rm + id2 / T0;
    tt = id2 - (r - rm) * T0;
    n_r = qn;
  }
  const int t0 = tt * kTileQ;
  const int w = p.w;
  const bool causal = p.causal != 0;
  const int8_t* mrow = p.mask + (size_t)b * n;

  int nG = 0;
  if (p.use_globals) {
    nG = scan_globals(mrow, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
    if (nG > p.max_global) {
      if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
      nG = p.max_global;
    }
  }

  // Query rows of this lane: t = t0 + 32nb + lane%32 in the residue sequence.
  const size_t rstride_pos = (size_t)p.H * kHeadDim;  // elements between tokens
  const size_t rstride = rstride_pos * dil;           // between residue-sequence neighbours
  const size_t head_off = (size_t)b * n * rstride_pos + (size_t)h * kHeadDim + (size_t)r * rstride_pos;
  bool is_local[2], is_zero[2];
  int qpos[2];
  bool any_local = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int tq = t0 + 32 * nb + (lane & 31);
    const bool inq = tq < n_r;
    qpos[nb] = r + dil * (inq ? tq : n_r - 1);
    const int qm = inq ? mrow[qpos[nb]] : 0;
    bool loc, glo;
    if (p.use_globals) {
      loc = qm == 1;
      glo = qm == 2;
    } else {
      loc = qm == 1 || qm == 2;
      glo = false;
      if (qm == 2 && !causal && p.max_global == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
    }
    is_local[nb] = inq && loc;
    is_zero[nb] = inq && !loc && !glo;
    any_local |= is_local[nb];
  }
  any_local = __any(any_local);

  T* out = reinterpret_cast<T*>(p.out);
  const size_t out_head = (size_t)b * n * rstride_pos + (size_t)h * kHeadDim;

  if (!any_local) {
    if (wv == 0) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (!is_zero[nb]) continue;
        T* orow = out + out_head + (size_t)qpos[nb] * rstride_pos;
#pragma unroll
        for (int g = 0; g < 8; ++g) store4<B16>(orow + 8 * g + 4 * hh, z);
        if (p.row_nnz && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qpos[nb]] = 0;
      }
    }
    return;
  }

  const T* q = reinterpret_cast<const T*>(p.q);
  const T* k = reinterpret_cast<const T*>(p.k);
  const T* v = reinterpret_cast<const T*>(p.v);
  Frag<B16> qf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) load_frag(qf[nb], q + (size_t)b * n * rstride_pos + (size_t)qpos[nb] * rstride_pos + (size_t)h * kHeadDim, hh);

  WaveState st;
  state_init(st);
  unsigned char* lds = sh.buf + wv * kStageBytes;

  // Window blocks: keys t0 - w + 32j of the residue sequence, clipped.
  const int kbase = t0 - w;
  const int t_last = min(t0 + kTileQ, n_r) - 1;
  const int kfirst = max(kbase, 0);
  const int klast = min(n_r - 1, causal ? t_last : t_last + w);
  const int jlo = (kfirst - kbase) / kBlockK;
  const int nblk = (klast - kbase) / kBlockK - jlo + 1;
  const int ngblk = (nG + kBlockK - 1) / kBlockK;
  const T* kh = k + head_off;
  const T* vh = v + head_off;
  const T* kfull = k + (size_t)b * n * rstride_pos + (size_t)h * kHeadDim;
  const T* vfull = v + (size_t)b * n * rstride_pos + (size_t)h * kHeadDim;
  const float c = p.c;

  for (int vb = wv; vb < nblk + ngblk; vb += kWaves) {
    if (vb < nblk) {
      const int kb = kbase + kBlockK * (jlo + vb);
      const int kk = kb + (lane & 31);
      const bool inr = kk >= 0 && kk < n_r;
      const int kkc = inr ? kk : (kk < 0 ? 0 : n_r - 1);
      const bool kval = inr && (mrow[r + dil * kkc] == 1 || mrow[r + dil * kkc] == 2);
      const uint32_t keymask = (uint32_t)__ballot(kval);
      bool interior = keymask == 0xffffffffu && (t0 + kTileQ - 1 - kb <= w);
      interior = interior && (causal ? (t0 >= kb + kBlockK - 1) : (kb + kBlockK - 1 - t0 <= w));
      auto keep = [&](int nb, int kr) {
        const int d = t0 + 32 * nb + (lane & 31) - (kb + kr);
        return causal ? (unsigned)d <= (unsigned)w : (unsigned)(d + w) <= (unsigned)(2 * w);
      };
      attend_block<B16>(st, qf, kh, vh, rstride, kkc, keymask, !interior, keep, lds, c);
    } else {
      const int gi = vb - nblk;
      const int gidx = kBlockK * gi + (lane & 31);
      const bool gval = gidx < nG;
      const int gpos = gval ? sh.G[gidx] : 0;
      const uint32_t keymask = (uint32_t)__ballot(gval);
      const int wd = w * dil;
      auto keep = [&](int nb, int kr) {
        // global key g is a column of this local row unless g is in W(i)
        const int g = sh.G[kBlockK * gi + kr];
        const int dd = qpos[nb] - g;
        const bool in_w = (dd <= wd && dd >= -wd) && (dil == 1 || dd % dil == 0);
        return !in_w;
      };
      attend_block<B16>(st, qf, kfull, vfull, rstride_pos, gpos, keymask, true, keep, lds, c);
    }
  }

  merge_waves(st, sh);
  if (wv != 0) return;

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if (!is_local[nb] && !is_zero[nb]) continue;
    T* orow = out + out_head + (size_t)qpos[nb] * rstride_pos;
    const float inv = is_local[nb] ? 1.0f / st.l[nb] : 0.f;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = st.o[nb][db][4 * g + i] * inv;
        store4<B16>(orow + 32 * db + 8 * g + 4 * hh, t);
      }
    if (p.row_nnz && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qpos[nb]] = is_local[nb] ? st.cnt[nb] : 0;
  }
}

// ---------------------------------------------------------------------------
// Global-row workgroup: split c of (b, h); all global tokens of b.
// ---------------------------------------------------------------------------
template <bool B16>
__device__ void global_split(const KernelParams& p, int gid, Shared& sh) {
  using T = elem_t<B16>;
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.S;
  const int bh = gid / S;
  const int cidx = gid - bh * S;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int n = p.n;
  const int8_t* mrow = p.mask + (size_t)b * n;

  int nG = scan_globals(mrow, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
  if (nG > p.max_global) {
    if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
    nG = p.max_global;
  }
  if (nG == 0) return;

  const size_t rs = (size_t)p.H * kHeadDim;
  const size_t head = (size_t)b * n * rs + (size_t)h * kHeadDim;
  const T* qg = reinterpret_cast<const T*>(p.qg) + head;
  const T* kg = reinterpret_cast<const T*>(p.kg) + head;
  const T* vg = reinterpret_cast<const T*>(p.vg) + head;
  const int cbeg = cidx * kGlobalChunk;
  const int cend = min(n, cbeg + kGlobalChunk);
  const int nblk = (cend - cbeg + kBlockK - 1) / kBlockK;
  unsigned char* lds = sh.buf + wv * kStageBytes;
  const float c = p.c;
  float* part_bh = p.partials + (size_t)bh * p.max_global * S * kPartialStride;

  for (int g0 = 0; g0 < nG; g0 += kTileQ) {
    Frag<B16> qf[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int gi = g0 + 32 * nb + (lane & 31);
      const int pos = sh.G[gi < nG ? gi : nG - 1];
      load_frag(qf[nb], qg + (size_t)pos * rs, hh);
    }
    WaveState st;
    state_init(st);
    for (int j = wv; j < nblk; j += kWaves) {
      const int kk = cbeg + kBlockK * j + (lane & 31);
      const bool inr = kk < cend;
      const int kkc = inr ? kk : cend - 1;
      const bool kval = inr && (mrow[kkc] == 1 || mrow[kkc] == 2);
      const uint32_t keymask = (uint32_t)__ballot(kval);
      auto keep = [](int, int) { return true; };
      attend_block<B16>(st, qf, kg, vg, rs, kkc, keymask, keymask != 0xffffffffu, keep, lds, c);
    }
    merge_waves(st, sh);
    if (wv == 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int gi = g0 + 32 * nb + (lane & 31);
        if (gi >= nG) continue;
        float* rec = part_bh + ((size_t)gi * S + cidx) * kPartialStride;
        if (hh == 0) {
          rec[0] = st.m[nb];
          rec[1] = st.l[nb];
          rec[2] = __builtin_bit_cast(float, st.cnt[nb]);
        }
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(rec + 4 + 32 * db + 8 * g + 4 * hh) =
                f32x4{st.o[nb][db][4 * g], st.o[nb][db][4 * g + 1], st.o[nb][db][4 * g + 2],
                      st.o[nb][db][4 * g + 3]};
      }
    }
    __syncthreads();  // merge buffers are reused by the next group of globals
  }

  // Arrival: the last split of (b, h) merges all partials.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(p.tickets + bh, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = (t == S - 1);
  }
  __syncthreads();
  if (!sh.flag) return;
  __threadfence();

  T* out = reinterpret_cast<T*>(p.out) + head;
  const int d = threadIdx.x & 63;
  for (int gi = wv; gi < nG; gi += kWaves) {
    const float* recs = part_bh + (size_t)gi * S * kPartialStride;
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, __builtin_nontemporal_load(recs + s * kPartialStride));
    float Lsum = 0.f, acc = 0.f;
    int cnt = 0;
    for (int s = 0; s < S; ++s) {
      const float* rec = recs + s * kPartialStride;
      const float ms = __builtin_nontemporal_load(rec);
      const float f = (ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      Lsum += __builtin_nontemporal_load(rec + 1) * f;
      acc += __builtin_nontemporal_load(rec + 4 + d) * f;
      cnt += __builtin_bit_cast(int, __builtin_nontemporal_load(rec + 2));
    }
    const int pos = sh.G[gi];
    out[(size_t)pos * rs + d] = (T)(acc / Lsum);
    if (p.row_nnz && d == 0) p.row_nnz[(size_t)bh * n + pos] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(p.tickets + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool B16>
__global__ __launch_bounds__(kThreads) void lf_attn_fwd(const KernelParams p) {
  __shared__ Shared sh;
  const int bid = blockIdx.x;
  if (bid < p.n_glob_pad) {
    if (bid < p.n_glob) global_split<B16>(p, bid, sh);
    return;
  }
  band_tile<B16>(p, xcd_remap(bid - p.n_glob_pad, p.n_band), sh);
}

}  // namespace

int launch_forward(const KernelParams& kp, int dtype, void* stream) {
  const int grid = kp.n_glob_pad + kp.n_band;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == LF_BF16)
    hipLaunchKernelGGL(lf_attn_fwd<true>, dim3(grid), dim3(kThreads), 0, s, kp);
  else
    hipLaunchKernelGGL(lf_attn_fwd<false>, dim3(grid), dim3(kThreads), 0, s, kp);
  return (int)hipGetLastError();
}

}  // namespace lf
