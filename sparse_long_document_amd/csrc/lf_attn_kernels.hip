// Longformer combined sliding-window + global attention forward for gfx950.
//
// One launch computes every output row with two kinds of workgroups:
//   * global-row splits (dispatched first): split c of one (batch row b,
//     head h) scores every global token of b against keys
//     [512c, 512c + 512) with the global projections (each global token
//     attends to every token: segmentfault Longformer summary, "Global
//     attention" and "Linear projections for global attention").  Each
//     split leaves a partial (max, sum, unnormalised output) record in the
//     workspace; the last split of (b, h) to arrive merges them and writes
//     the global rows;
//   * band tiles: 64 consecutive query rows of one (b, h, residue class r
//     of the head's dilation d).  A dilated window over positions
//     {r, r+d, r+2d, ...} is a plain window over that subsequence, so each
//     residue class is an undilated sequence whose neighbours are d tokens
//     apart (segmentfault summary, "Dilated sliding window").  The tile's
//     keys are its window span (64 + 2w keys, or 64 + w when causal) plus
//     the row's global tokens as extra columns, masked so that a global key
//     already inside a row's window is not counted twice (ultralytics
//     glossary worked example: window and global row/column are OR-ed into
//     one pattern).  They write local rows (mask 1) and zero rows (mask 0).
//
// Inner block: 32 keys x 64 queries per wave, as two 32-query halves.
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 key rows, B = 32
//   query columns, K-dim = head dim), so a lane owns one query column and
//   16 of its 32 keys (the other 16 sit in lane ^ 32).  K and V rows travel
//   from HBM to LDS by direct-to-LDS buffer loads (no registers, no VALU),
//   K comes back as the A fragment and V as the V^T A operand of
//   O^T = V^T P^T through ds_read_b64_tr_b16; the accumulator rounded to
//   bf16 is directly the P^T operand.  Softmax is online in base 2 (score
//   scale * log2e folded into one FMA), fp32, with a lazy rescale: the
//   reference max only moves when a block max exceeds it by more than 2^8,
//   which keeps the result exact while skipping most accumulator rescales.
//
// A band tile's key blocks are dealt to its 4 waves round-robin; each wave
// streams its blocks through its own two-stage LDS area (the next block's
// loads fly while the current one is computed) and the four partial
// states are merged through LDS with one barrier.
//
// The fp32 instantiation computes in true fp32 (v_mfma_f32_32x32x2_f32, P
// kept in fp32).
#include <hip/hip_runtime.h>
#include <stdint.h>


#include <type_traits>

#include "lf_attn_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
// Initial reference max: finite and far below any score, so that
// exp2(x - m) needs no special case (it is 0 for x = -inf or x = kMInit
// against a real max, and the first scored block always moves m).
constexpr float kMInit = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// Per-wave LDS area: two stages, each holding one key block of K rows then
// one of V rows (32 rows of 64 head dims each), filled by direct-to-LDS
// loads while the other stage is consumed.
template <bool B16>
struct Lay {
  static constexpr int kElt = B16 ? 2 : 4;
  static constexpr int kRowBytes = kHeadDim * kElt;      // 128 | 256
  static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows covered by one wave-wide load
  static constexpr int kLoads = kBlockK / kRowsPerLoad;  // loads per block and tensor
  static constexpr int kBlockBytes = kBlockK * kRowBytes;
  static constexpr int kStageBytes = 2 * kBlockBytes;
  static constexpr int kWaveBytes = 2 * kStageBytes;
};

// Chunk swizzles (the LDS position of 16-byte chunk c of row `row` is
// c ^ swz(row)).  K: 16 consecutive rows at one chunk index land on
// distinct banks, for the K fragment reads.  V (bf16): the transposed reads
// of a half-wave land on distinct banks.  V (fp32) is read along rows.
template <bool B16>
__device__ __forceinline__ int kswz(int row) {
  return B16 ? ((row >> 1) & 7) : (row & 15);
}
template <bool B16>
__device__ __forceinline__ int vswz(int row) {
  return B16 ? (((row >> 1) & 1) << 2) : 0;
}

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

// The lane index computed where it is used: values derived from it in a
// rarely taken branch are then recomputed there instead of being hoisted
// out of the loop and kept live (or spilled) through every iteration.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until every vector-memory load this wave issued has completed
// (direct-to-LDS loads included); other counters are left alone.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N vector-memory instructions of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until every LDS (and scalar-memory) access of this wave has completed.
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

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

// Accumulator element r of a lane holds key row c_r + 4*(lane/32) of the
// block, c_r = 8*(r/4) + r%4.
__host__ __device__ constexpr int acc_c(int r) { return 8 * (r >> 2) + (r & 3); }

// ---------------------------------------------------------------------------
// One key block through LDS.
// ---------------------------------------------------------------------------

// Issue the direct-to-LDS loads of a block's K and V rows into `stage`.
// kpos(row) gives the token position of key row `row` (0..31) of the block,
// always a valid position (rows outside the key set are clamped here and
// masked later).  Lane l of load i fetches chunk (l % kChunks) ^ swz(row)
// of row kRowsPerLoad*i + l / kChunks; it lands at byte 1024i + 16l.
template <bool B16, class KPos>
__device__ __forceinline__ void issue_block(const elem_t<B16>* kb, const elem_t<B16>* vb, uint32_t rs, KPos kpos,
                                            unsigned char* stage, int lane) {
  using L = Lay<B16>;
  constexpr int kEltPerChunk = 16 / L::kElt;
#pragma unroll
  for (int i = 0; i < L::kLoads; ++i) {
    const int row = L::kRowsPerLoad * i + lane / L::kChunks;
    const int c = lane % L::kChunks;
    const uint32_t base = (uint32_t)kpos(row) * rs;
    __builtin_amdgcn_global_load_lds(kb + (base + (c ^ kswz<B16>(row)) * kEltPerChunk),
                                     (LDS_AS void*)(stage + 1024 * i), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + (base + (c ^ vswz<B16>(row)) * kEltPerChunk),
                                     (LDS_AS void*)(stage + L::kBlockBytes + 1024 * i), 16, 0, 0);
  }
}

// K operand fragment of key row lane % 32.
__device__ __forceinline__ void read_kfrag(Frag<true>& f, const unsigned char* kbuf, int lane) {
  const int row = lane & 31;
  const int hh = lane >> 5;
  const unsigned char* rp = kbuf + row * Lay<true>::kRowBytes;
  const int sw = kswz<true>(row);
#pragma unroll
  for (int s = 0; s < 4; ++s) f.x[s] = *reinterpret_cast<const bf16x8*>(rp + (((2 * s + hh) ^ sw) << 4));
}

__device__ __forceinline__ void read_kfrag(Frag<false>& f, const unsigned char* kbuf, int lane) {
  const int row = lane & 31;
  const int hh = lane >> 5;
  const unsigned char* rp = kbuf + row * Lay<false>::kRowBytes;
  const int sw = kswz<false>(row);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(rp + (((8 * hh + j) ^ sw) << 4));
    f.x[4 * j + 0] = t[0];
    f.x[4 * j + 1] = t[1];
    f.x[4 * j + 2] = t[2];
    f.x[4 * j + 3] = t[3];
  }
}

// Zero the V rows whose key bit is clear in keymask, so keys outside a
// row's key set contribute exactly nothing to P V even where their stored
// values are not finite.
template <bool B16>
__device__ __forceinline__ void zero_dead_v_rows(unsigned char* vbuf, uint32_t keymask, int lane) {
  using L = Lay<B16>;
  const int row = lane >> 1;
  if (!((keymask >> row) & 1u)) {
    u32x4* dst = reinterpret_cast<u32x4*>(vbuf + row * L::kRowBytes + (L::kRowBytes / 2) * (lane & 1));
#pragma unroll
    for (int j = 0; j < L::kChunks / 2; ++j) dst[j] = u32x4{0u, 0u, 0u, 0u};
  }
}

// V^T operand of the PV product for one block, in registers.
//   bf16: a[db][ks] covers head dims 32db + lane%32 and keys 16ks +
//         {4hh..4hh+3, 8+4hh..8+4hh+3} (hh = lane/32), the key order of the
//         P^T fragments;
//   fp32: a[db][r] is V[key c_r + 4hh][32db + lane%32].
template <bool B16>
struct VtFrag;
template <>
struct VtFrag<true> {
  bf16x8 a[2][2];
};
template <>
struct VtFrag<false> {
  float a[2][16];
};

// ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives element
// j%4 of the 8-byte chunk addressed by lane 4e + j/4, as its element e.
// Lane 4e+q of group g points at key row 16ks + 8half + 4(g/2) + e, head
// dims 32db + 16(g%2) + 4q .. +3, so lane j of the group gets head dim
// 32db + 16(g%2) + j for keys e = 0..3.
__device__ __forceinline__ void read_vt(VtFrag<true>& vt, const unsigned char* vbuf, int lane) {
  const int g = lane >> 4;
  const int row0 = 4 * (g >> 1) + ((lane & 15) >> 2);
  const int byte0 = 32 * (g & 1) + 8 * (lane & 3);
  const int sw = vswz<true>(row0);  // rows 16ks + 8half + row0 share bit 1 with row0
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int byte = 64 * db + byte0;
    const int off = row0 * 128 + (((byte >> 4) ^ sw) << 4) + (byte & 15);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vbuf + off + 2048 * ks));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(vbuf + off + 2048 * ks + 1024));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
      vt.a[db][ks] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
    }
  }
}

// The same reads in one asm block that waits for them before it ends.  The
// band loop uses it while the next block's direct-to-LDS loads (into the
// other stage) are in flight: the compiler cannot tell the transposed reads
// from those writes and would otherwise wait for every outstanding load
// first.  The caller has already waited for this stage's loads.
__device__ __forceinline__ void read_vt_now(VtFrag<true>& vt, const unsigned char* vbuf, int lane) {
  const int g = lane >> 4;
  const int row0 = 4 * (g >> 1) + ((lane & 15) >> 2);
  const int byte0 = 32 * (g & 1) + 8 * (lane & 3);
  const int sw = vswz<true>(row0);
  const uint32_t base = (uint32_t)(uintptr_t)(LDS_AS const void*)vbuf;
  uint32_t a[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int byte = 64 * db + byte0;
    a[db] = base + (uint32_t)(row0 * 128 + (((byte >> 4) ^ sw) << 4) + (byte & 15));
  }
  u32x2 r[8];  // [db][ks][lo, hi]: key rows 16ks + 8half at +2048ks + 1024half
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %8 offset:1024\n"
      "ds_read_b64_tr_b16 %2, %8 offset:2048\n"
      "ds_read_b64_tr_b16 %3, %8 offset:3072\n"
      "ds_read_b64_tr_b16 %4, %9\n"
      "ds_read_b64_tr_b16 %5, %9 offset:1024\n"
      "ds_read_b64_tr_b16 %6, %9 offset:2048\n"
      "ds_read_b64_tr_b16 %7, %9 offset:3072\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1])
      : "memory");
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x2 lo = r[4 * db + 2 * ks], hi = r[4 * db + 2 * ks + 1];
      vt.a[db][ks] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
}

__device__ __forceinline__ void read_vt(VtFrag<false>& vt, const unsigned char* vbuf, int lane) {
  const float* vs = reinterpret_cast<const float*>(vbuf);
  const int hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) vt.a[db][r] = vs[(acc_c(r) + 4 * hh) * kHeadDim + 32 * db + (lane & 31)];
}

__device__ __forceinline__ void read_vt_now(VtFrag<false>& vt, const unsigned char* vbuf, int lane) {
  read_vt(vt, vbuf, lane);
}

// Zero the V^T operand entries of keys whose bit is clear in keymask, so
// keys outside a row's key set contribute exactly nothing to P V even where
// their stored values are not finite.
__device__ __forceinline__ void zero_dead_keys(VtFrag<true>& vt, uint32_t keymask, int lane) {
  const uint32_t km = keymask >> (4 * (lane >> 5));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 keep;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // dword d holds items 2d, 2d+1; item e is key 16ks + 8(e/4) + e%4 (+4hh)
      const int k0 = 16 * ks + 8 * ((2 * d) >> 2) + ((2 * d) & 3);
      keep[d] = (((km >> k0) & 1u) ? 0x0000ffffu : 0u) | (((km >> (k0 + 1)) & 1u) ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
      vt.a[db][ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vt.a[db][ks]) & keep);
  }
}

__device__ __forceinline__ void zero_dead_keys(VtFrag<false>& vt, uint32_t keymask, int lane) {
  const uint32_t km = keymask >> (4 * (lane >> 5));
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (!((km >> acc_c(r)) & 1u)) {
      vt.a[0][r] = 0.f;
      vt.a[1][r] = 0.f;
    }
}

// -1 where bit `pos` of x is set, else 0 (one v_bfe_i32; written out so
// the compiler keeps it instead of a compare-and-select chain through VCC).
template <int pos>
__device__ __forceinline__ int bit_as_mask(uint32_t x) {
  int r;
  asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(r) : "v"(x), "i"(pos));
  return r;
}

// 1 where u > span, else 0: med3(u, span, span + 1) - span (span < 2^32 - 1).
__device__ __forceinline__ uint32_t above_span(uint32_t u, uint32_t span) {
  uint32_t m;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(m) : "v"(u), "s"(span), "v"(span + 1u));  // one scalar operand per VALU op
  return m - span;
}

// Zero this lane's K fragment when its key row (lane % 32) is clear in
// keymask, so that row's scores are exactly 0 before the mask is added.
__device__ __forceinline__ void zero_dead_krow(Frag<true>& kf, uint32_t keymask, int lane) {
  if (!((keymask >> (lane & 31)) & 1u)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) kf.x[s] = bf16x8{};
  }
}

__device__ __forceinline__ void zero_dead_krow(Frag<false>& kf, uint32_t keymask, int lane) {
  if (!((keymask >> (lane & 31)) & 1u)) {
#pragma unroll
    for (int j = 0; j < 32; ++j) kf.x[j] = 0.f;
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

// Running state of one wave: 64 query columns as two 32-column halves.
struct WaveState {
  f32x16 o[2][2];  // [query half nb][dim half db]
  float m[2];      // reference max (log2 domain) of the lane's query
  float l[2];      // partial row sum of this lane (16 of the 32 keys per block)
  int cnt[2];      // partial count of scored keys of this lane
};

__device__ __forceinline__ void state_init(WaveState& st) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.m[nb] = kMInit;
    st.l[nb] = 0.f;
    st.cnt[nb] = 0;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nb][db][r] = 0.f;
  }
}


// Scores of one block for query half nb -> masked, online-softmax
// probabilities, with that half's running state rescaled if its reference
// max moves.  On edge blocks valid() gives this lane's bitmask of elements
// in their row's key set (bit c_r for element r); on interior blocks every
// element is.
template <bool B16, class Valid>
__device__ __forceinline__ void softmax_half(WaveState& st, int nb, f32x16& s, PFrag<B16>& pf, bool edge,
                                             Valid valid, float c) {
  if (edge) {
    // keep the mask work inside the (uniform) branch
    __asm__ volatile("" ::: "memory");
    const uint32_t vm = valid();  // bit c_r set <=> element r is in its row's key set
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (vm & (1u << acc_c(r))) ? s[r] : kNegInf;
    st.cnt[nb] += __popc(vm & 0x0f0f0f0fu);
  } else {
    st.cnt[nb] += 16;
  }

  // Local max of this lane's 16 scores (a tree, to keep the chain short).
  // Lanes l and l^32 hold the same query's other 16 keys, but the exchange
  // is only needed when the reference max moves: the test "some score
  // exceeds the reference by more than the slack" is a wave-wide vote.
  float m4[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) m4[g] = fmaxf(fmaxf(s[4 * g], s[4 * g + 1]), fmaxf(s[4 * g + 2], s[4 * g + 3]));
  const float mloc = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * c;
  if (__any(mloc > st.m[nb] + kRescaleSlack)) {
    const float mn = fmaxf(st.m[nb], fmaxf(mloc, __shfl_xor(mloc, 32)));
    const float alpha = __builtin_amdgcn_exp2f(st.m[nb] - mn);
    st.m[nb] = mn;
    st.l[nb] *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nb][db][r] *= alpha;
  }

#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -st.m[nb]));
  float t8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t8[i] = s[2 * i] + s[2 * i + 1];
  const float sum = ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
  if constexpr (B16) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.x[ks][e] = (__bf16)s[8 * ks + e];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) pf.x[r] = s[r];
  }
  st.l[nb] += sum;
}

// O^T (64 dims x 32 queries of half nb) += V^T P^T.
__device__ __forceinline__ void pv(f32x16 (&o)[2], const PFrag<true>& pf, const VtFrag<true>& vt) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt.a[db][ks], pf.x[ks], o[db], 0, 0, 0);
}

__device__ __forceinline__ void pv(f32x16 (&o)[2], const PFrag<false>& pf, const VtFrag<false>& vt) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt.a[db][r], pf.x[r], o[db], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// A wave's stream of 32-key blocks first, first + 4, ... < end of one key
// source, staged through the wave's own two-stage LDS area.  A block's K
// and V^T fragments are read into registers before the direct-to-LDS loads
// of the wave's next block are issued into the other stage, so those loads
// are in flight while the current block is computed.
// Src provides:
//   kpos(i, row) -> int           token position of key row `row` (clamped)
//   locate(i, mb&, inr&)          mask byte / existence of key row lane%32
//   edge(i, keymask) -> bool      whether masking is needed
//   valid_bits(i, nb) -> uint32   this lane's rows c_r in the key sets (edge blocks)
//   dstep(), affine(i, p0&)       evenly spaced in-range blocks: positions p0 + dstep*row
// ---------------------------------------------------------------------------
template <bool B16, class Src>
struct BlockPipe {
  using T = elem_t<B16>;
  using L = Lay<B16>;
  const Src& src;
  const T* kb;
  const T* vb;
  uint32_t rs;
  unsigned char* lds;
  int lane;
  // Blocks whose 32 rows are in range and evenly spaced use a wave-uniform
  // base address plus per-lane byte offsets that do not change from block
  // to block.
  uint32_t off_k0, off_k1, off_v;
  int mb;    // mask byte of key row lane%32 of the last issued block
  bool inr;  // whether that row exists

  __device__ BlockPipe(const Src& s, const T* k, const T* v, uint32_t rs_, unsigned char* area)
      : src(s), kb(k), vb(v), rs(rs_), lds(area), lane(lane_id()), off_k0(0), off_k1(0), off_v(0), mb(0),
        inr(false) {
    if constexpr (B16) {
      const uint32_t row_off = (uint32_t)src.dstep() * (uint32_t)(lane >> 3) * rs;
      const int ck = (lane & 7) ^ (lane >> 4);  // kswz of rows 8i + lane/8, i even
      const int cv = (lane & 7) ^ (((lane >> 4) & 1) << 2);
      off_k0 = 2u * (row_off + 8u * (uint32_t)ck);
      off_k1 = 2u * (row_off + 8u * (uint32_t)(ck ^ 4));
      off_v = 2u * (row_off + 8u * (uint32_t)cv);
    }
  }

  __device__ void issue(int blk, int stage) {
    unsigned char* dst = lds + stage * L::kStageBytes;
    src.locate(blk, mb, inr);
    int p0;
    if (B16 && src.affine(blk, p0)) {
      const size_t step = (size_t)src.dstep() * L::kRowsPerLoad * rs * 2;
      const char* kbase = reinterpret_cast<const char*>(kb) + (size_t)p0 * rs * 2;
      const char* vbase = reinterpret_cast<const char*>(vb) + (size_t)p0 * rs * 2;
#pragma unroll
      for (int i = 0; i < L::kLoads; ++i) {
        __builtin_amdgcn_global_load_lds(kbase + i * step + ((i & 1) ? off_k1 : off_k0),
                                         (LDS_AS void*)(dst + 1024 * i), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + i * step + off_v, (LDS_AS void*)(dst + L::kBlockBytes + 1024 * i),
                                         16, 0, 0);
      }
    } else {
      issue_block<B16>(kb, vb, rs, [&](int row) { return src.kpos(blk, row); }, dst, lane);
    }
  }

  // Blocks first, first + 4, ... < end into st; `primed`: block `first` has
  // already been issued into stage 0.  halves: query halves holding rows.
  __device__ void run(WaveState& st, const Frag<B16> (&qf)[2], int first, int end, float c, int halves,
                      bool primed) {
    const int hh = lane >> 5;
    if (first < end && !primed) issue(first, 0);
    int it = 0;
    for (int blk = first; blk < end; blk += kWaves, ++it) {
      const unsigned char* cst = lds + (it & 1) * L::kStageBytes;
      const bool kval = inr && (mb == 1 || mb == 2);
      const uint32_t keymask = (uint32_t)__ballot(kval);
      wait_vmem_all();  // this block's rows have landed
      Frag<B16> kf;
      read_kfrag(kf, cst, lane);
      VtFrag<B16> vt;
      read_vt(vt, cst + L::kBlockBytes, lane);
      if (blk + kWaves < end) issue(blk + kWaves, (it + 1) & 1);
      if (keymask == 0u) continue;  // no key of the block is in any key set
      if (keymask != 0xffffffffu) zero_dead_keys(vt, keymask, lane);

      const bool edge = src.edge(blk, keymask);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (nb >= halves) break;  // query half without rows
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        qk(s, kf, qf[nb]);
        PFrag<B16> pf;
        softmax_half<B16>(st, nb, s, pf, edge,
                          [&]() { return src.valid_bits(blk, nb) & (keymask >> (4 * hh)); }, c);
        pv(st.o[nb], pf, vt);
      }
    }
  }
};


// Bitmask of the bytes equal to 2 among mrow[p0 .. p0+16) (clipped to n).
__device__ __forceinline__ uint32_t match16(const int8_t* __restrict__ mrow, int p0, int n) {
  uint32_t bits = 0;
  if (p0 + 16 <= n && ((reinterpret_cast<uintptr_t>(mrow + p0) & 15u) == 0)) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(mrow + p0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) bits |= (((x[j] >> (8 * e)) & 0xffu) == 2u ? 1u : 0u) << (4 * j + e);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (p0 + e < n && mrow[p0 + e] == 2) bits |= 1u << e;
  }
  return bits;
}

// Exclusive prefix sum over the wave of a per-lane count in [0, 31],
// from one ballot per bit (no lane exchange through LDS).
__device__ __forceinline__ int wave_prefix(int cnt) {
  int pre = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const unsigned long long m = __ballot((cnt >> i) & 1);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    pre += below << i;
  }
  return pre;
}

// Ordered list of positions j with mask_row[j] == 2 into G (LDS), at most
// cap entries; returns the total count.  Every thread of the workgroup
// calls it and gets the same result.  Each thread looks at 16 bytes of each
// 4 KB step; four steps are loaded together and ranked with one barrier.
__device__ int scan_globals(const int8_t* __restrict__ mrow, int n, int* G, int cap, int (*s_tot)[kWaves]) {
  constexpr int kStep = kThreads * 16;
  int total = 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  for (int base = 0; base < n; base += 4 * kStep) {
    uint32_t bits[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) bits[u] = match16(mrow, base + u * kStep + 16 * tid, n);
    if (!__syncthreads_or((bits[0] | bits[1] | bits[2] | bits[3]) != 0)) continue;
    int pre[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cnt = __popc(bits[u]);
      pre[u] = wave_prefix(cnt);
      if (lane == 63) s_tot[u][wv] = pre[u] + cnt;
    }
    __syncthreads();
    int off = total;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int slot = off + pre[u];
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const int t = s_tot[u][i];
        slot += (i < wv) ? t : 0;
        off += t;
      }
      uint32_t bm = bits[u];
      while (bm) {
        const int e = __builtin_ctz(bm);
        bm &= bm - 1;
        if (slot < cap) G[slot] = base + u * kStep + 16 * tid + e;
        ++slot;
      }
    }
    total = off;
    __syncthreads();  // s_tot is reused by the next steps
  }
  return __builtin_amdgcn_readfirstlane(total);  // the same in every lane
}

template <bool B16>
struct Shared {
  int G[LF_MAX_GLOBAL];
  int wave_tmp[4][kWaves];
  int flag;
  float m[kWaves][kWaveQ];
  float l[kWaves][kWaveQ];
  int cnt[kWaves][kWaveQ];
  uint32_t ktab[kWaves][32];  // band tiles: validity bits of each wave's window blocks
  __attribute__((aligned(16))) unsigned char buf[kWaves * Lay<B16>::kWaveBytes];
};

// The waves of a workgroup hold partial results for the same 64 query
// columns over disjoint key subsets.  Each wave parks its state in its own
// LDS area (all its loads have landed, and no other wave touches that
// area); after one barrier, each wave merges its share of the quadrants
// (query half nb, head-dim half db) of all partials and passes, per lane,
// the merged max M (log2 domain), row sum L, key count and the 16
// unnormalised outputs of head dims 32db + 8g + 4(lane/32) + i (in
// o[4g + i]) to emit(nb, db, M, L, cnt, o).
template <bool B16, class Emit>
__device__ void combine_waves(const WaveState& st, Shared<B16>& sh, Emit emit) {
  static_assert(Lay<B16>::kWaveBytes >= 64 * 64 * 4, "a wave's area holds its 64 x 64 fp32 partial");
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x4* mine = reinterpret_cast<f32x4*>(sh.buf + wv * Lay<B16>::kWaveBytes);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        mine[((nb * 2 + db) * 4 + g) * 64 + lane] = f32x4{st.o[nb][db][4 * g], st.o[nb][db][4 * g + 1],
                                                          st.o[nb][db][4 * g + 2], st.o[nb][db][4 * g + 3]};
    const float l = st.l[nb] + __shfl_xor(st.l[nb], 32);
    const int cnt = st.cnt[nb] + __shfl_xor(st.cnt[nb], 32);
    if (hh == 0) {
      sh.m[wv][32 * nb + lane] = st.m[nb];
      sh.l[wv][32 * nb + lane] = l;
      sh.cnt[wv][32 * nb + lane] = cnt;
    }
  }
  __syncthreads();
  // wave w takes quadrants w * kQuads .. (w + 1) * kQuads - 1 (index 2 nb + db)
  constexpr int kQuads = 4 / kWaves;
#pragma unroll
  for (int k = 0; k < kQuads; ++k) {
    const int quad = wv * kQuads + k;
    const int nb = quad >> 1, db = quad & 1;
    const int q = 32 * nb + (lane & 31);
    float mw[kWaves];
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = sh.m[w][q];
      M = fmaxf(M, mw[w]);
    }
    float Lsum = 0.f, o[16];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w] - M);
      Lsum = __builtin_fmaf(sh.l[w][q], f, Lsum);
      cnt += sh.cnt[w][q];
      const f32x4* part = reinterpret_cast<const f32x4*>(sh.buf + w * Lay<B16>::kWaveBytes);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 t = part[((nb * 2 + db) * 4 + g) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 * g + i] = __builtin_fmaf(t[i], f, o[4 * g + i]);
      }
    }
    emit(nb, db, M, Lsum, cnt, o);
  }
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

// Partial records of the global-row splits cross XCDs, whose L2 caches are
// not coherent with each other.  They are written with agent-scope atomic
// stores and read back with agent-scope atomic loads, both of which go to
// the device-wide coherence point; this avoids an agent-scope release
// fence, which would write back every dirty line of the XCD's L2.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int xcd_remap(int x, int N) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of tiles so neighbouring tiles (which share K/V
  // halos) share one L2.
  const int per = N / 8, rem = N % 8;
  const int xcd = x % 8, y = x / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + y;
}

// Output values of one quadrant of a row: head dims 32db + 8g + 4hh + i
// from o[4g + i], times inv (or zeros).
template <bool B16>
__device__ __forceinline__ void store_quadrant(elem_t<B16>* row, int db, int hh, const float* o, float inv,
                                               bool zero) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = zero ? 0.f : o[4 * g + i] * inv;
    store4<B16>(row + 32 * db + 8 * g + 4 * hh, t);
  }
}

// ---------------------------------------------------------------------------
// Key sources
// ---------------------------------------------------------------------------

// Blocks of one split of a global row: keys cbeg + 32 j + row.
struct ChunkSrc {
  const int8_t* mrow;
  int cbeg, cend, lane;
  __device__ int kpos(int j, int row) const {
    const int kk = cbeg + kBlockK * j + row;
    return kk < cend ? kk : cend - 1;
  }
  __device__ void locate(int j, int& mb, bool& inr) const {
    inr = cbeg + kBlockK * j + (lane & 31) < cend;
    mb = mrow[kpos(j, lane & 31)];
  }
  __device__ bool edge(int, uint32_t keymask) const { return keymask != 0xffffffffu; }
  __device__ int dstep() const { return 1; }
  __device__ bool affine(int j, int& p0) const {
    p0 = cbeg + kBlockK * j;
    return p0 + kBlockK - 1 < cend;
  }
  __device__ uint32_t valid_bits(int, int) const { return 0xffffffffu; }
};

// Blocks of a band tile: first the non-empty 32-key blocks of the tile's
// window span (residue-sequence keys kbase + 32 (jlo + i) + row, tokens
// r + dil * key), then the blocks of the row's global tokens G[32 (i - nwin) + row].
struct BandSrc {
  const int8_t* mrow;
  const int* G;
  int kbase, jlo, nwin;
  int n_r, r, dil, nG, lane;
  int t0, w, wd;
  bool causal;
  int w_hi;  // w, or 0 when causal
  // Query row of this lane in half nb (residue-sequence index, clamped to
  // the last row) and its token position; recomputed where needed rather
  // than held in registers through the block loop.
  __device__ int qrow(int nb) const {
    const int tq = t0 + 32 * nb + (lane & 31);
    return tq < n_r ? tq : n_r - 1;
  }
  __device__ int qpos(int nb) const { return r + dil * qrow(nb); }
  __device__ int key(int i, int row) const { return kbase + kBlockK * (jlo + i) + row; }
  __device__ int kpos(int i, int row) const {
    if (i < nwin) {
      const int kk = key(i, row);
      return r + dil * (kk < 0 ? 0 : (kk >= n_r ? n_r - 1 : kk));
    }
    const int gi = kBlockK * (i - nwin) + row;
    return G[gi < nG ? gi : nG - 1];
  }
  // whether key row `row` of block i exists (a window key in [0, n_r) or
  // one of the nG global keys)
  __device__ bool exists(int i, int row) const {
    if (i < nwin) {
      const int kk = key(i, row);
      return kk >= 0 && kk < n_r;
    }
    return kBlockK * (i - nwin) + row < nG;
  }
  __device__ int dstep() const { return dil; }
  __device__ bool affine(int i, int& p0) const {
    if (i >= nwin) return false;
    const int k0 = key(i, 0);
    p0 = r + dil * k0;
    return k0 >= 0 && k0 + kBlockK - 1 < n_r;
  }
  __device__ uint32_t valid_bits(int i, int nb) const {
    if (i < nwin) {
      const int sh32 = kBlockK * (jlo + i);
      // window rows c (block-relative, minus 4 (lane/32)) in [lo, hi] hold keys
      // in the query's window
      const int ln = lane_id_here();
      const int tq = t0 + 32 * nb + (ln & 31);
      const int a = tq - kbase - w - 4 * (ln >> 5), b = tq - kbase + w_hi - 4 * (ln >> 5);
      const int lo = max(a - sh32, 0);
      const int hi = min(b - sh32, 31);
      return lo > hi ? 0u : ((0xffffffffu >> (31 - hi)) & (0xffffffffu << lo));
    }
    // A global key g joins local row i unless g is already in W(i):
    // |i - g| <= w d and d divides i - g (no causal rows have global columns).
    // rows 8 g4 + 4 hh + [0, 4) of the block: one asm block that waits for
    // its reads (the compiler would otherwise wait for the key loads in
    // flight into the staging area first)
    const int ln = lane_id_here();
    const uint32_t ga = (uint32_t)(uintptr_t)(LDS_AS const void*)(G + kBlockK * (i - nwin) + 4 * (ln >> 5));
    u32x4 xs[4];
    asm volatile(
        "ds_read_b128 %0, %4\n"
        "ds_read_b128 %1, %4 offset:32\n"
        "ds_read_b128 %2, %4 offset:64\n"
        "ds_read_b128 %3, %4 offset:96\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(xs[0]), "=&v"(xs[1]), "=&v"(xs[2]), "=&v"(xs[3])
        : "v"(ga)
        : "memory");
    const uint32_t span = 2u * (uint32_t)wd;
    const int tq = t0 + 32 * nb + (ln & 31);
    const int qp = r + dil * (tq < n_r ? tq : n_r - 1);
    uint32_t vb = 0;
    if (dil == 1) {
      // bit = 1 when u = qp - g + wd exceeds span (g outside the window):
      // med3(u, span, span + 1) - span, without a compare through VCC
      const uint32_t qpw = (uint32_t)(qp + wd);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vb |= above_span(qpw - xs[g4][e], span) << (8 * g4 + e);
        }
      return vb;
    }
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x4 x = xs[g4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = qp - (int)x[e];
        bool in_w = (uint32_t)(dd + wd) <= span;
        if (dil != 1) in_w = in_w && (dd % dil == 0);
        vb |= in_w ? 0u : (1u << (8 * g4 + e));
      }
    }
    return vb;
  }
};

// ---------------------------------------------------------------------------
// Band tile block loop.
// ---------------------------------------------------------------------------

// Raw (untyped) buffer resource over `bytes` bytes at `base`; accesses past
// the end read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float max16(const f32x16& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
  const float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float d = fmaxf(fmaxf(s[6], s[7]), s[8]);
  const float e = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float f = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(a, b), d), fmaxf(fmaxf(e, f), s[15]));
}

// One query half of a block, after masking (masked scores are -inf):
// online softmax (same arithmetic as softmax_half); counts 16 scored keys
// per lane.
template <bool B16>
__device__ __forceinline__ void softmax_core(WaveState& st, int nb, f32x16& s, PFrag<B16>& pf, float c) {
  const float ml = max16(s) * c;
  if (__any(ml > st.m[nb] + kRescaleSlack)) {
    const float mn = fmaxf(st.m[nb], fmaxf(ml, __shfl_xor(ml, 32)));
    const float alpha = __builtin_amdgcn_exp2f(st.m[nb] - mn);
    st.m[nb] = mn;
    st.l[nb] *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nb][db][r] *= alpha;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -st.m[nb]));
  st.cnt[nb] += 16;
  if constexpr (B16) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.x[ks][e] = (__bf16)s[8 * ks + e];
    // row sum of the rounded probabilities that enter P V (two bf16 at a
    // time with fp32 accumulation), in two chains
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x2 p0 = {pf.x[0][2 * j], pf.x[0][2 * j + 1]};
      const bf16x2 p1 = {pf.x[1][2 * j], pf.x[1][2 * j + 1]};
      la = __builtin_amdgcn_fdot2_f32_bf16(p0, one, la, false);
      lb = __builtin_amdgcn_fdot2_f32_bf16(p1, one, lb, false);
    }
    st.l[nb] += la + lb;
  } else {
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t8[i] = s[2 * i] + s[2 * i + 1];
    st.l[nb] += ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
#pragma unroll
    for (int r = 0; r < 16; ++r) pf.x[r] = s[r];
  }
}

// A wave's blocks i = first, first + 4, ... < end of a band tile: window
// blocks (i < nwin) then global-column blocks, staged through the wave's
// two-stage LDS area.  Every (block, query half) pair is classified on the
// scalar unit as full (all 32 keys in every row's key set), partial (masked
// per element) or empty; only blocks with a full half on both sides skip
// the masking, and blocks empty on both sides are skipped.
template <bool B16>
struct BandLoop {
  using T = elem_t<B16>;
  using L = Lay<B16>;
  const BandSrc& src;
  const T* kb;
  const T* vb;
  uint32_t rs;
  unsigned char* lds;
  int lane;
  int t0, w, w_hi;
  // buffer resources and per-lane offsets of the evenly spaced (affine) fast path
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t vk0, vk1, vv;
  // key-validity bits of this wave's window blocks (entry k: block
  // first + kWaves k), filled in the prologue; null when the window has
  // more blocks than the table holds
  const uint32_t* ktab;
  // vector-memory instructions one issue() emits (K and V rows)
  static constexpr int kIssueLoads = 2 * L::kLoads;

  __device__ BandLoop(const BandSrc& s, const T* k, const T* v, uint32_t rs_, unsigned char* area, int n, int t0_,
                      int w_, int w_hi_)
      : src(s), kb(k), vb(v), rs(rs_), lds(area), lane(lane_id()), t0(t0_), w(w_), w_hi(w_hi_), ktab(nullptr) {
    const uint32_t bytes = (uint32_t)(((size_t)(n - 1) * rs + kHeadDim) * sizeof(T));
    rk = make_rsrc(k, bytes);
    rv = make_rsrc(v, bytes);
    const uint32_t row_off = (uint32_t)src.dil * (uint32_t)(lane >> 3) * rs;
    const int ck = (lane & 7) ^ (lane >> 4);  // kswz of rows 8t + lane/8, t even
    const int cv = (lane & 7) ^ (((lane >> 4) & 1) << 2);
    vk0 = 2u * (row_off + 8u * (uint32_t)ck);
    vk1 = 2u * (row_off + 8u * (uint32_t)(ck ^ 4));
    vv = 2u * (row_off + 8u * (uint32_t)cv);
  }

  // Loads of block i into stage st (exactly kIssueLoads vector-memory
  // instructions on every path, and nothing else: the loop's waits count
  // them).
  __device__ void issue(int i, int st) {
    unsigned char* dst = lds + st * L::kStageBytes;
    int p0;
    if (B16 && src.affine(i, p0)) {
      // scalar offsets: wave-uniform by construction; readfirstlane keeps
      // them in SGPRs even where register pressure moved a term to a VGPR
      const uint32_t so = (uint32_t)p0 * rs * 2u;
      const uint32_t step = (uint32_t)src.dil * (uint32_t)L::kRowsPerLoad * rs * 2u;
#pragma unroll
      for (int t = 0; t < L::kLoads; ++t) {
        const uint32_t sot = __builtin_amdgcn_readfirstlane(so + t * step);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS_AS void*)(dst + 1024 * t), 16, (t & 1) ? vk1 : vk0, sot,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS_AS void*)(dst + L::kBlockBytes + 1024 * t), 16, vv, sot,
                                                 0, 0);
      }
    } else {
      issue_block<B16>(kb, vb, rs, [&](int r) { return src.kpos(i, r); }, dst, lane);
    }
  }

  // Validity bits of window block i read from the mask now (rows in
  // [0, n_r) with mask 1 or 2).
  __device__ uint32_t window_keymask(int i) const {
    const int row = lane_id_here() & 31;
    const int m = src.exists(i, row) ? (int)src.mrow[src.kpos(i, row)] : 0;
    return (uint32_t)__ballot(m == 1 || m == 2);
  }

  // This wave's table of window-block validity bits (blocks first,
  // first + kWaves, ... < nwin): tab_load issues the mask-byte loads (two
  // blocks per load, lanes 32-63 take the second) and tab_commit, after the
  // caller has issued its first K/V loads, turns them into bits.  Windows
  // with more than 2 kTabPairs blocks per wave go without the table.
  static constexpr int kTabPairs = 12;
  int tabv[kTabPairs];
  int tab_cnt = 0;
  int first_ = 0;
  __device__ void tab_load(int first) {
    first_ = first;
    tab_cnt = first < src.nwin ? (src.nwin - first + kWaves - 1) / kWaves : 0;
    if (tab_cnt > 2 * kTabPairs) return;
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int p = 0; p < kTabPairs; ++p) {
      const int k = 2 * p + half;
      const int i = first + kWaves * k;
      const bool ok = k < tab_cnt && src.exists(i, row);
      tabv[p] = ok ? (int)src.mrow[src.kpos(i, row)] : 0;
    }
  }
  __device__ void tab_commit(uint32_t* tab) {
    if (tab_cnt > 2 * kTabPairs) return;  // ktab stays null, no block is taken as full
#pragma unroll
    for (int p = 0; p < kTabPairs; ++p) {
      if (2 * p >= tab_cnt) break;
      const unsigned long long bits = __ballot(tabv[p] == 1 || tabv[p] == 2);
      if (lane == 0) {
        tab[2 * p] = (uint32_t)bits;
        tab[2 * p + 1] = (uint32_t)(bits >> 32);
      }
      full_keys |= ((uint32_t)bits == 0xffffffffu ? 1u : 0u) << (2 * p);
      full_keys |= ((uint32_t)(bits >> 32) == 0xffffffffu ? 1u : 0u) << (2 * p + 1);
    }
    ktab = tab;
  }

  // Window blocks (list index) whose 32 keys exist and lie in the window of
  // every query of both halves: [fast_lo, fast_hi).  Among them, those whose
  // keys all carry mask 1 or 2 (bit k of full_keys for block first + kWaves k)
  // take fast_step.
  int fast_lo = 0, fast_hi = 0;
  uint32_t full_keys = 0;
  __device__ void set_fast_range() {
    // block j holds keys kbase + 32 j ..: 32 j - w >= 63 - w and 32 j - w + 31 <= w_hi
    int jl = (kTileQ - 1 + kBlockK - 1) / kBlockK;
    int jh = w + w_hi - (kBlockK - 1) >= 0 ? (w + w_hi - (kBlockK - 1)) / kBlockK + 1 : 0;  // exclusive
    // keys in [0, n_r): kbase + 32 j >= 0 and kbase + 32 j + 31 < n_r
    const int kb0 = src.kbase;
    jl = max(jl, kb0 >= 0 ? 0 : (-kb0 + kBlockK - 1) / kBlockK);
    jh = min(jh, src.n_r - kb0 - kBlockK >= 0 ? (src.n_r - kb0 - kBlockK) / kBlockK + 1 : 0);
    if (t0 + 32 >= src.n_r) jh = jl;  // the second half has no rows
    fast_lo = max(jl - src.jlo, 0);
    fast_hi = max(min(jh - src.jlo, src.nwin), fast_lo);
  }
  __device__ bool is_fast(int i) const {
    const int k = (i - first_) / kWaves;
    return i >= fast_lo && i < fast_hi && k < 32 && ((full_keys >> k) & 1u);
  }

  // A block known full for both halves: no classification, no masks.
  template <int kStage>
  __device__ __forceinline__ void fast_step(WaveState& st, const Frag<B16> (&qf)[2], int i, int end, float c) {
    const unsigned char* cst = lds + kStage * L::kStageBytes;
    if (i + kWaves < end)
      wait_vmem_but<kIssueLoads>();
    else
      wait_vmem_all();
    Frag<B16> kf;
    read_kfrag(kf, cst, lane);
    VtFrag<B16> vt;
    read_vt_now(vt, cst + L::kBlockBytes, lane);
    if (i + 2 * kWaves < end) {
      wait_lds_all();  // the fragment reads of this stage are done before it is refilled
      issue(i + 2 * kWaves, kStage);
    }
    f32x16 s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][r] = 0.f;
      qk(s[nb], kf, qf[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      PFrag<B16> pf;
      softmax_core<B16>(st, nb, s[nb], pf, c);
      pv(st.o[nb], pf, vt);
    }
  }

  // 0 = empty, 1 = partial, 2 = full for query half nb of window block i.
  __device__ int classify(int i, int nb, uint32_t keymask) const {
    const int k0 = src.key(i, 0);
    const int qlo = t0 + 32 * nb, qhi = qlo + 31;
    if (k0 > qhi + w_hi || k0 + kBlockK - 1 < qlo - w) return 0;
    if (qlo >= src.n_r) return 0;  // no rows in this half
    const bool full = keymask == 0xffffffffu && k0 >= qhi - w && k0 + kBlockK - 1 <= qlo + w_hi;
    return full ? 2 : 1;
  }

  // A general block (window edge, padded keys, global columns).
  __device__ __forceinline__ void step(WaveState& st, const Frag<B16> (&qf)[2], int i, int end, float c,
                                       int kStage) {
    const int hh = lane >> 5;
    const unsigned char* cst = lds + kStage * L::kStageBytes;
    // Block i landed in this stage; block i + kWaves (other stage) may still
    // be in flight: wait for all but its loads.
    uint32_t keymask;
    if (i >= src.nwin) {
      // global-column rows: key rows up to nG exist and are global (mask 2)
      const int left = src.nG - kBlockK * (i - src.nwin);
      keymask = left >= kBlockK ? 0xffffffffu : ((1u << left) - 1u);
    } else if (ktab) {
      keymask = ktab[(i - first_) / kWaves];
    } else {
      keymask = window_keymask(i);  // waits for every outstanding load: wide windows only
    }
    if (i + kWaves < end)
      wait_vmem_but<kIssueLoads>();
    else
      wait_vmem_all();
    Frag<B16> kf;
    read_kfrag(kf, cst, lane);
    VtFrag<B16> vt;
    read_vt_now(vt, cst + L::kBlockBytes, lane);
    if (i + 2 * kWaves < end) {
      wait_lds_all();  // the fragment reads of this stage are done before it is refilled
      issue(i + 2 * kWaves, kStage);
    }
    if (keymask == 0u) return;  // no key of the block is in any key set
    if (keymask != 0xffffffffu) {
      // rows of keys outside every key set contribute exactly nothing, even
      // where their stored values are not finite
      zero_dead_keys(vt, keymask, lane);
      zero_dead_krow(kf, keymask, lane);
    }

    const bool win = i < src.nwin;
    int cls[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) cls[nb] = win ? classify(i, nb, keymask) : (t0 + 32 * nb < src.n_r ? 1 : 0);
    if (cls[0] == 0 && cls[1] == 0) return;

    // The mask enters through the accumulators' starting values: 0 where
    // the key is scored, -inf where it is not, so the QK products come out
    // masked (-inf + finite = -inf) with no pass over the scores after them.
    f32x16 s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (cls[nb] == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] = 0.f;
      } else if (cls[nb] == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] = kNegInf;
        st.cnt[nb] -= 16;  // softmax_core adds 16
      } else {
        const uint32_t vmk = src.valid_bits(i, nb) & (keymask >> (4 * hh));  // bit c_r: element r scored
        const uint32_t inv = ~vmk;
        // all ones where element r is not scored, then the bits of -inf
#define LF_BIAS(r) s[nb][r] = __builtin_bit_cast(float, (uint32_t)bit_as_mask<acc_c(r)>(inv) & 0xff800000u)
        LF_BIAS(0); LF_BIAS(1); LF_BIAS(2); LF_BIAS(3); LF_BIAS(4); LF_BIAS(5); LF_BIAS(6); LF_BIAS(7);
        LF_BIAS(8); LF_BIAS(9); LF_BIAS(10); LF_BIAS(11); LF_BIAS(12); LF_BIAS(13); LF_BIAS(14); LF_BIAS(15);
#undef LF_BIAS
        st.cnt[nb] += __popc(vmk & 0x0f0f0f0fu) - 16;  // softmax_core adds 16
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) qk(s[nb], kf, qf[nb]);
    // half 0's softmax runs while half 1's QK products are in flight, and
    // half 0's PV products while half 1's softmax runs
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      PFrag<B16> pf;
      softmax_core<B16>(st, nb, s[nb], pf, c);
      pv(st.o[nb], pf, vt);
    }
  }

  // first: the wave's first block; blocks first and first + kWaves must
  // already be issued into stages 0 and 1 (those that exist).
  __device__ void run(WaveState& st, const Frag<B16> (&qf)[2], int first, int end, float c) {
    for (int i = first; i < end; i += 2 * kWaves) {
      if (is_fast(i))
        fast_step<0>(st, qf, i, end, c);
      else
        step(st, qf, i, end, c, 0);
      if (i + kWaves >= end) break;
      if (is_fast(i + kWaves))
        fast_step<1>(st, qf, i + kWaves, end, c);
      else
        step(st, qf, i + kWaves, end, c, 1);
    }
  }
};

// ---------------------------------------------------------------------------
// Band workgroup: one tile of kTileQ = 64 query rows t0 .. t0 + 63 of the
// residue sequence r of (b, h).  Its key blocks (window span, then the
// global columns) are dealt to the 4 waves round-robin; every wave scores
// all 64 queries against its own blocks, and the partials are merged
// through LDS at the end.  Writes local rows (mask 1) and zero rows (mask 0).
// ---------------------------------------------------------------------------
template <bool B16>
__device__ void band_tile(const KernelParams& p, int L, Shared<B16>& sh) {
  using T = elem_t<B16>;
  using Ly = Lay<B16>;
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int b = L / p.tiles_per_b;
  const int rem = L - b * p.tiles_per_b;
  // head: tile0 is non-decreasing; count entries <= rem, 8 loads per round
  int h = 0;
  for (int k0 = 1; k0 < p.H; k0 += 8) {
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) cnt += (k0 + k < p.H && p.tile0[k0 + k] <= rem) ? 1 : 0;
    h += cnt;
    if (cnt < 8) break;
  }
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
  const int w_hi = causal ? 0 : w;
  const int8_t* mrow = p.mask + (size_t)b * n;
  const uint32_t rs = (uint32_t)p.H * kHeadDim;  // elements between tokens
  const size_t head = (size_t)b * n * rs + (size_t)h * kHeadDim;
  const T* qh = reinterpret_cast<const T*>(p.q) + head;
  T* out = reinterpret_cast<T*>(p.out) + head;

  // Window span: residue-sequence keys kbase + 32 j + row, j < S; only
  // blocks jlo .. jhi - 1 hold keys in [0, n_r).
  const int kbase = t0 - w;
  const int S = (kTileQ - 1 + w + w_hi) / kBlockK + 1;
  const int jlo = kbase >= 0 ? 0 : (-kbase) / kBlockK;
  const int jhi = min(S, (n_r - kbase + kBlockK - 1) / kBlockK);

  BandSrc src;
  src.mrow = mrow;
  src.G = sh.G;
  src.kbase = kbase;
  src.jlo = jlo;
  src.nwin = jhi - jlo;
  src.n_r = n_r;
  src.r = r;
  src.dil = dil;
  src.nG = 0;
  src.lane = lane;
  src.t0 = t0;
  src.w = w;
  src.w_hi = w_hi;
  src.wd = w * dil;
  src.causal = causal;

  // Query rows of this lane: t = t0 + 32nb + lane%32, token r + dil*t.
  int qm[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) qm[nb] = t0 + 32 * nb + (lane & 31) < n_r ? mrow[src.qpos(nb)] : 0;
  Frag<B16> qf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) load_frag(qf[nb], qh + (size_t)src.qpos(nb) * rs, hh);
  unsigned char* area = sh.buf + wv * Ly::kWaveBytes;
  BandLoop<B16> loop(src, reinterpret_cast<const T*>(p.k) + head, reinterpret_cast<const T*>(p.v) + head, rs, area, n,
                     t0, w, w_hi);
  // validity bytes of the wave's window blocks, then its first two window
  // blocks: all of them fly during the scan
  loop.tab_load(wv);
  loop.set_fast_range();
  if (wv < src.nwin) loop.issue(wv, 0);
  if (wv + kWaves < src.nwin) loop.issue(wv + kWaves, 1);
  loop.tab_commit(sh.ktab[wv]);

  if (p.use_globals) {
    int nG = scan_globals(mrow, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
    if (nG > p.max_global) {
      if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
      nG = p.max_global;
    }
    src.nG = __builtin_amdgcn_readfirstlane(nG);  // uniform (the status write above diverges)
  }
  const int end = src.nwin + (src.nG + kBlockK - 1) / kBlockK;
  // first blocks that are global-column blocks go after the scan
  if (wv >= src.nwin && wv < end) loop.issue(wv, 0);
  if (wv + kWaves >= src.nwin && wv + kWaves < end) loop.issue(wv + kWaves, 1);

  bool is_local[2], is_zero[2];
  bool any_local = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int tq = t0 + 32 * nb + (lane & 31);
    const bool inq = tq < n_r;
    bool loc, glo;
    if (p.use_globals) {
      loc = qm[nb] == 1;
      glo = qm[nb] == 2;
    } else {
      loc = qm[nb] == 1 || qm[nb] == 2;
      glo = false;
      if (qm[nb] == 2 && !causal && p.max_global == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
    }
    is_local[nb] = inq && loc;
    is_zero[nb] = inq && !loc && !glo;
    any_local |= is_local[nb];
  }
  // every wave holds the same queries, so this test agrees across the workgroup
  if (!__any(any_local)) {
    wait_vmem_all();  // the primed loads land before the workgroup's LDS is released
    constexpr int kQuads = 4 / kWaves;
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
      const int quad = wv * kQuads + k;
      const int nb = quad >> 1, db = quad & 1;
      if (nb ? is_zero[1] : is_zero[0]) {
        const int qp = src.qpos(nb);
        store_quadrant<B16>(out + (size_t)qp * rs, db, hh, nullptr, 0.f, true);
        if (p.row_nnz && db == 0 && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qp] = 0;
      }
    }
    return;
  }

  WaveState st;
  state_init(st);
  loop.run(st, qf, wv, end, p.c);
  combine_waves<B16>(st, sh, [&](int nb, int db, float, float Lsum, int cnt, const float* o) {
    const bool loc = nb ? is_local[1] : is_local[0];
    const bool zer = nb ? is_zero[1] : is_zero[0];
    if (!loc && !zer) return;
    const int qp = src.qpos(nb);
    store_quadrant<B16>(out + (size_t)qp * rs, db, hh, o, loc ? 1.0f / Lsum : 0.f, !loc);
    if (p.row_nnz && db == 0 && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qp] = loc ? cnt : 0;
  });
}

// ---------------------------------------------------------------------------
// Global-row workgroup: split c of (b, h); all global tokens of b.
// ---------------------------------------------------------------------------
template <bool B16>
__device__ void global_split(const KernelParams& p, int gid, Shared<B16>& sh) {
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

  const uint32_t rs = (uint32_t)p.H * kHeadDim;
  const size_t head = (size_t)b * n * rs + (size_t)h * kHeadDim;
  const T* qg = reinterpret_cast<const T*>(p.qg) + head;
  ChunkSrc src;
  src.mrow = mrow;
  src.cbeg = cidx * kGlobalChunk;
  src.cend = min(n, src.cbeg + kGlobalChunk);
  src.lane = lane;
  const int nblk = (src.cend - src.cbeg + kBlockK - 1) / kBlockK;
  BlockPipe<B16, ChunkSrc> pipe(src, reinterpret_cast<const T*>(p.kg) + head,
                                reinterpret_cast<const T*>(p.vg) + head, rs,
                                sh.buf + wv * Lay<B16>::kWaveBytes);
  bool primed = wv < nblk;
  if (primed) pipe.issue(wv, 0);  // the split's keys do not depend on the scan

  int nG = scan_globals(mrow, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
  if (nG > p.max_global) {
    if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
    nG = p.max_global;
  }
  nG = __builtin_amdgcn_readfirstlane(nG);  // uniform (the status write above diverges)
  if (nG == 0) {
    wait_vmem_all();
    return;
  }
  const float c = p.c;
  float* part_bh = p.partials + (size_t)bh * p.max_global * S * kPartialStride;

  for (int g0 = 0; g0 < nG; g0 += kWaveQ) {
    Frag<B16> qf[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int gi = g0 + 32 * nb + (lane & 31);
      const int pos = sh.G[gi < nG ? gi : nG - 1];
      load_frag(qf[nb], qg + (size_t)pos * rs, hh);
    }
    WaveState st;
    state_init(st);
    pipe.run(st, qf, wv, nblk, c, nG - g0 > 32 ? 2 : 1, primed);
    primed = false;
    combine_waves<B16>(st, sh, [&](int nb, int db, float M, float Lsum, int cnt, const float* o) {
      const int gi = g0 + 32 * nb + (lane & 31);
      if (gi >= nG) return;
      float* rec = part_bh + ((size_t)gi * S + cidx) * kPartialStride;
      if (db == 0 && hh == 0) {
        st_agent(rec, M);
        st_agent(rec + 1, Lsum);
        st_agent(rec + 2, __builtin_bit_cast(float, cnt));
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) st_agent(rec + 4 + 32 * db + 8 * g + 4 * hh + e, o[4 * g + e]);
    });
    __syncthreads();  // LDS areas and merge arrays are reused by the next group of globals
  }

  // Arrival: the last split of (b, h) merges all partials.  Every thread's
  // record stores have completed (at the coherence point) before the
  // barrier that precedes the ticket increment.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmem_all();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(p.tickets + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = (t == S - 1);
  }
  __syncthreads();
  if (!sh.flag) return;

  T* out = reinterpret_cast<T*>(p.out) + head;
  const int d = threadIdx.x & 63;
  for (int gi = wv; gi < nG; gi += kWaves) {
    // online log-sum-exp merge of the S partials; loads issued 8 at a time
    const float* recs = part_bh + (size_t)gi * S * kPartialStride;
    float M = kNegInf, Lsum = 0.f, acc = 0.f;
    int cnt = 0;
    for (int s0 = 0; s0 < S; s0 += 8) {
      float ms[8], ls[8], os[8];
      int cs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* rec = recs + (size_t)min(s0 + j, S - 1) * kPartialStride;
        ms[j] = ld_agent(rec);
        ls[j] = ld_agent(rec + 1);
        cs[j] = __builtin_bit_cast(int, ld_agent(rec + 2));
        os[j] = ld_agent(rec + 4 + d);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (s0 + j >= S) break;
        const float mn = fmaxf(M, ms[j]);
        const float fa = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - mn);
        const float fb = (ms[j] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms[j] - mn);
        M = mn;
        Lsum = Lsum * fa + ls[j] * fb;
        acc = acc * fa + os[j] * fb;
        cnt += cs[j];
      }
    }
    const int pos = sh.G[gi];
    out[(size_t)pos * rs + d] = (T)(acc / Lsum);
    if (p.row_nnz && d == 0) p.row_nnz[(size_t)bh * n + pos] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(p.tickets + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool B16>
__device__ __forceinline__ void fwd_body(const KernelParams& p) {
  __shared__ Shared<B16> sh;
  const int bid = blockIdx.x;
  if (bid < p.n_glob) {
    global_split<B16>(p, bid, sh);  // first: their merge waits for the last split
    return;
  }
  band_tile<B16>(p, xcd_remap(bid - p.n_glob, p.n_band), sh);
}

// bf16: two waves per SIMD (two workgroups per CU).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void lf_attn_fwd_bf16(
    const KernelParams p) {
  fwd_body<true>(p);
}

// fp32: larger operand fragments; one wave per SIMD.
__global__ __launch_bounds__(kThreads) void lf_attn_fwd_f32(const KernelParams p) { fwd_body<false>(p); }

}  // namespace

int launch_forward(const KernelParams& kp, int dtype, void* stream) {
  const int grid = kp.n_band + kp.n_glob;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == LF_BF16)
    hipLaunchKernelGGL(lf_attn_fwd_bf16, dim3(grid), dim3(kThreads), 0, s, kp);
  else
    hipLaunchKernelGGL(lf_attn_fwd_f32, dim3(grid), dim3(kThreads), 0, s, kp);
  return (int)hipGetLastError();
}

}  // namespace lf
