// Longformer combined sliding-window + global attention forward for gfx950.
//
// One launch computes every output row:
//   * band workgroups own a tile of kTileQ consecutive query rows of one
//     (batch row b, head h, residue class r of the head's dilation d).  A
//     dilated window over positions {r, r+d, r+2d, ...} is a plain window
//     over that subsequence, so each residue class is handled as an
//     undilated sequence whose neighbours are d tokens apart (segmentfault
//     Longformer summary, "Dilated sliding window": the dilated window
//     keeps the cost of the plain one).  They write local rows (mask 1)
//     and zero rows (mask 0);
//   * global-row workgroups own one split of kGlobalChunk keys of one
//     (b, h) for every global token of b: each global token attends to all
//     tokens with the global projections (segmentfault summary, "Global
//     attention" and "Linear projections for global attention").  Each
//     split leaves a partial (max, sum, unnormalised output) in the
//     workspace; the last split to arrive merges them and writes the rows.
//
// Inner block (both kinds): 32 keys x 64 queries per wave.
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 key rows straight
//   from global memory into registers, B = 32 query columns, K-dim = head
//   dim).  In the 32x32 accumulator a lane owns one column (a query) and 16
//   of its 32 keys; the other 16 sit in lane ^ 32, so the softmax row max
//   is in-lane plus one lane exchange.  The accumulator, rounded to
//   bf16, is directly the B operand of O^T = V^T P^T.  V rows travel from
//   global memory to LDS with direct-to-LDS loads (no registers, no VALU)
//   and come back as the V^T A operand through ds_read_b64_tr_b16, whose
//   16-lane transpose hands each lane 4 keys of one head dim.  Softmax is
//   online in base 2 (scale*log2e folded into one FMA), fp32, with a lazy
//   rescale: the running reference max only moves when a block max exceeds
//   it by more than 2^8, which leaves the result exact while skipping most
//   accumulator rescales.
//   Each wave fetches its next block (K into registers, V into the other
//   half of its LDS double buffer) while it computes the current one.
//
// The key range of a band tile (kTileQ + 2w keys) is split over the 4 waves
// of the workgroup block by block; their partial results are merged
// through LDS at the end.  Global columns of local rows (the symmetric half
// of global attention) are extra gathered key blocks, masked so that a
// global key already inside the row's window is not counted twice
// (ultralytics glossary worked example: the window and the global
// row/column are OR-ed into one boolean pattern).
//
// The fp32 instantiation computes in true fp32 (v_mfma_f32_32x32x2_f32, P
// kept in fp32) with V staged through registers.
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
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// Merge of partial outputs: 2 slots of 64 lanes x 64 floats.
constexpr int kMergeSlotFloats = 64 * 64;
constexpr int kMergeBytes = 2 * kMergeSlotFloats * 4;

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
  static constexpr int kRingBytes = 8 * kStageBytes;  // shared ring of a band tile
  static constexpr int kBufBytes0 = kWaves * kWaveBytes > kMergeBytes ? kWaves * kWaveBytes : kMergeBytes;
  static constexpr int kBufBytes = kBufBytes0 > kRingBytes ? kBufBytes0 : kRingBytes;
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

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until every vector-memory load this wave issued has completed
// (direct-to-LDS loads included); other counters are left alone.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

__device__ __forceinline__ void read_vt(VtFrag<false>& vt, const unsigned char* vbuf, int lane) {
  const float* vs = reinterpret_cast<const float*>(vbuf);
  const int hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) vt.a[db][r] = vs[(acc_c(r) + 4 * hh) * kHeadDim + 32 * db + (lane & 31)];
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
    st.m[nb] = kNegInf;
    st.l[nb] = 0.f;
    st.cnt[nb] = 0;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nb][db][r] = 0.f;
  }
}

__device__ __forceinline__ float max_across_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
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

  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  const float mb = max_across_halves(mx) * c;
  if (__any(mb > st.m[nb] + kRescaleSlack)) {
    const float mn = fmaxf(st.m[nb], mb);
    const float alpha = (st.m[nb] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m[nb] - mn);
    st.m[nb] = mn;
    st.l[nb] *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nb][db][r] *= alpha;
  }

  const float msub = (st.m[nb] == kNegInf) ? 0.f : st.m[nb];
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -msub));
  float sum = 0.f;
  if constexpr (B16) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.x[ks][e] = (__bf16)s[8 * ks + e];
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += s[r];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pf.x[r] = s[r];
      sum += s[r];
    }
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
// A wave's pass over blocks first, first+4, ... < end of one key source.
// Src provides:
//   kpos(vb, row) -> int           token position of key row `row` (clamped)
//   locate(vb, mb&, inr&)          mask byte / existence of key row lane%32
//   edge(vb, keymask) -> bool      whether masking is needed
//   valid_bits(vb, nb) -> uint32   this lane's rows c_r in the key sets (edge blocks)
//   dstep(), affine(vb, p0&)       evenly spaced in-range blocks: positions p0 + dstep*row
// The loads of the wave's next block are in flight while the current one
// is computed: its K and V^T fragments are read from LDS into registers
// before the next block's direct-to-LDS loads are issued into the other
// stage.
// ---------------------------------------------------------------------------
template <bool B16, class Src>
__device__ __forceinline__ void run_blocks(WaveState& st, const Frag<B16> (&qf)[2], const Src& src,
                                           const elem_t<B16>* kb, const elem_t<B16>* vb, uint32_t rs, int first,
                                           int end, unsigned char* lds, float c) {
  using L = Lay<B16>;
  const int lane = lane_id();
  const int hh = lane >> 5;
  int mb = 0;
  bool inr = false;
  // Blocks whose 32 rows are in range and evenly spaced (token positions
  // p0 + dstep*row) use a wave-uniform base address plus per-lane byte
  // offsets that do not change from block to block.
  const int dstep = src.dstep();
  uint32_t off_k0 = 0, off_k1 = 0, off_v = 0;
  if constexpr (B16) {
    const uint32_t row_off = (uint32_t)dstep * (uint32_t)(lane >> 3) * rs;
    const int ck = (lane & 7) ^ (lane >> 4);  // kswz of rows 8i + lane/8, i even
    const int cv = (lane & 7) ^ (((lane >> 4) & 1) << 2);
    off_k0 = 2u * (row_off + 8u * (uint32_t)ck);
    off_k1 = 2u * (row_off + 8u * (uint32_t)(ck ^ 4));
    off_v = 2u * (row_off + 8u * (uint32_t)cv);
  }
  auto issue = [&](int blk, unsigned char* stage) {
    src.locate(blk, mb, inr);
    int p0;
    if (B16 && src.affine(blk, p0)) {
      const size_t step = (size_t)dstep * L::kRowsPerLoad * rs * 2;
      const char* kbase = reinterpret_cast<const char*>(kb) + (size_t)p0 * rs * 2;
      const char* vbase = reinterpret_cast<const char*>(vb) + (size_t)p0 * rs * 2;
#pragma unroll
      for (int i = 0; i < L::kLoads; ++i) {
        __builtin_amdgcn_global_load_lds(kbase + i * step + ((i & 1) ? off_k1 : off_k0),
                                         (LDS_AS void*)(stage + 1024 * i), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + i * step + off_v,
                                         (LDS_AS void*)(stage + L::kBlockBytes + 1024 * i), 16, 0, 0);
      }
    } else {
      issue_block<B16>(kb, vb, rs, [&](int row) { return src.kpos(blk, row); }, stage, lane);
    }
  };
  if (first < end) issue(first, lds);
  int it = 0;
  for (int blk = first; blk < end; blk += kWaves, ++it) {
    unsigned char* cst = lds + (it & 1) * L::kStageBytes;
    unsigned char* nst = lds + ((it + 1) & 1) * L::kStageBytes;
    const bool kval = inr && (mb == 1 || mb == 2);
    const uint32_t keymask = (uint32_t)__ballot(kval);
    wait_vmem_all();  // this block's rows have landed in cst
    if (keymask != 0xffffffffu) {
      zero_dead_v_rows<B16>(cst + L::kBlockBytes, keymask, lane);
      wave_sync();
    }
    Frag<B16> kf;
    read_kfrag(kf, cst, lane);
    VtFrag<B16> vt;
    read_vt(vt, cst + L::kBlockBytes, lane);
    if (blk + kWaves < end) issue(blk + kWaves, nst);

    const bool edge = src.edge(blk, keymask);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
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

// Ordered list of positions j with mask_row[j] == 2 into G (LDS), at most
// cap entries; returns the total count.  Every thread of the workgroup
// calls it and gets the same result.  Each thread looks at 16 bytes of a
// 4 KB step; four steps are loaded together.
__device__ int scan_globals(const int8_t* __restrict__ mrow, int n, int* G, int cap, int* s_wave) {
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
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!__syncthreads_or(bits[u] != 0)) continue;
      const int cnt = __popc(bits[u]);
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
      uint32_t b = bits[u];
      while (b) {
        const int e = __builtin_ctz(b);
        b &= b - 1;
        if (slot < cap) G[slot] = base + u * kStep + 16 * tid + e;
        ++slot;
      }
      total += all;
    }
  }
  return total;
}

// Band tiles keep the key-validity bits of their whole key span in LDS when
// it has at most this many 32-key blocks.
constexpr int kMaxSpanBlocks = 512;
constexpr int kRingSlots = 8;

template <bool B16>
struct Shared {
  int G[LF_MAX_GLOBAL];
  uint32_t kmask[kMaxSpanBlocks];
  int wave_tmp[kWaves];
  int flag;
  float m[kWaves][kWaveQ];
  float l[kWaves][kWaveQ];
  int cnt[kWaves][kWaveQ];
  __attribute__((aligned(16))) unsigned char buf[Lay<B16>::kBufBytes];
};

// Merge the partial results of the 4 waves into wave 0's registers.
template <bool B16>
__device__ void merge_waves(WaveState& st, Shared<B16>& sh) {
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
  __syncthreads();  // all waves done with their V buffers (aliased below)
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

// ---------------------------------------------------------------------------
// Band workgroup: one tile of kTileQ = 256 query rows of (b, h, residue r);
// wave w owns rows t0 + 64w .. t0 + 64w + 63 outright.
//
// The tile's key span is cut into 32-key blocks; wave w needs blocks
// 2w .. 2w + S - 1.  The waves walk their blocks in lockstep, staggered:
// at step s wave w computes block 2w + s, so the blocks in use at one step
// are s, s+2, s+4, s+6.  Blocks live in an 8-slot LDS ring shared by the
// workgroup (slot = block % 8); each block is fetched once per workgroup
// with direct-to-LDS loads, one part per wave, one step before its first
// use.  After the window blocks come the global-column blocks (the global
// keys of the batch row), which every wave computes at the same step.
// One barrier per step separates the ring's reuse from its reads.
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
  const int tw0 = t0 + kWaveQ * wv;  // this wave's first query row
  const int w = p.w;
  const bool causal = p.causal != 0;
  const int w_hi = causal ? 0 : w;
  const int8_t* mrow = p.mask + (size_t)b * n;
  const uint32_t rs = (uint32_t)p.H * kHeadDim;  // elements between tokens
  const size_t head = (size_t)b * n * rs + (size_t)h * kHeadDim;

  int nG = 0;
  if (p.use_globals) {
    nG = scan_globals(mrow, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
    if (nG > p.max_global) {
      if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
      nG = p.max_global;
    }
  }

  // Query rows of this lane: t = tw0 + 32nb + lane%32, token r + dil*t.
  bool is_local[2], is_zero[2];
  int qpos[2];
  bool any_local = false;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int tq = tw0 + 32 * nb + (lane & 31);
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
  const bool wave_active = __any(any_local);

  const T* qh = reinterpret_cast<const T*>(p.q) + head;
  const T* kh = reinterpret_cast<const T*>(p.k) + head;
  const T* vh = reinterpret_cast<const T*>(p.v) + head;
  T* out = reinterpret_cast<T*>(p.out) + head;

  if (!__syncthreads_or(wave_active)) {
    // nothing local in the tile: only zero rows to write
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (!is_zero[nb]) continue;
      T* orow = out + (size_t)qpos[nb] * rs;
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 8; ++g) store4<B16>(orow + 8 * g + 4 * hh, z);
      if (p.row_nnz && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qpos[nb]] = 0;
    }
    return;
  }

  Frag<B16> qf[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) load_frag(qf[nb], qh + (size_t)qpos[nb] * rs, hh);

  // Key span: keys kbase + 32*blk + row of the residue sequence.
  const int kbase = t0 - w;
  const int S = (kWaveQ - 1 + w + w_hi) / kBlockK + 1;  // blocks per wave
  const int nbt = 2 * (kWaves - 1) + S;                  // window blocks of the tile
  const int ngb = (nG + kBlockK - 1) / kBlockK;         // global-column blocks
  const int total = nbt + ngb;                           // blocks through the ring
  const bool mask_in_lds = nbt <= kMaxSpanBlocks;

  // Validity bits of window block blk: key in [0, n_r) with mask 1 or 2.
  auto window_keymask = [&](int blk) -> uint32_t {
    const int kk = kbase + kBlockK * blk + (lane & 31);
    const bool inr = kk >= 0 && kk < n_r;
    const int m = inr ? mrow[r + dil * kk] : 0;
    return (uint32_t)__ballot(m == 1 || m == 2);
  };
  if (mask_in_lds) {
    for (int blk = wv; blk < nbt; blk += kWaves) {
      const uint32_t km = window_keymask(blk);
      if (lane == 0) sh.kmask[blk] = km;
    }
  }

  // Direct-to-LDS loads of ring block idx (window block idx, or global
  // block idx - nbt): this wave fetches its parts of the K and V rows.
  unsigned char* ring = sh.buf;
  auto row_pos = [&](int idx, int row) -> int {
    if (idx < nbt) {
      const int kk = kbase + kBlockK * idx + row;
      return r + dil * (kk < 0 ? 0 : (kk >= n_r ? n_r - 1 : kk));
    }
    const int gi = kBlockK * (idx - nbt) + row;
    return sh.G[gi < nG ? gi : nG - 1];
  };
  auto block_empty = [&](int idx) {
    const int k0 = kbase + kBlockK * idx;
    return idx < nbt && (k0 + kBlockK - 1 < 0 || k0 >= n_r);
  };
  auto issue = [&](int idx) {
    if (block_empty(idx)) return;
    unsigned char* slot = ring + (idx % kRingSlots) * Ly::kStageBytes;
    constexpr int kEltPerChunk = 16 / Ly::kElt;
#pragma unroll
    for (int part = wv; part < Ly::kLoads; part += kWaves) {
      const int row = Ly::kRowsPerLoad * part + lane / Ly::kChunks;
      const int c = lane % Ly::kChunks;
      const uint32_t base = (uint32_t)row_pos(idx, row) * rs;
      __builtin_amdgcn_global_load_lds(kh + (base + (c ^ kswz<B16>(row)) * kEltPerChunk),
                                       (LDS_AS void*)(slot + 1024 * part), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vh + (base + (c ^ vswz<B16>(row)) * kEltPerChunk),
                                       (LDS_AS void*)(slot + Ly::kBlockBytes + 1024 * part), 16, 0, 0);
    }
  };
  for (int idx = 0; idx < kRingSlots && idx < total; ++idx) issue(idx);

  WaveState st;
  state_init(st);
  const float c = p.c;
  const int wd = w * dil;
  // window rows c in [A - 32 blk, B - 32 blk] hold keys in the query's window
  int A[2], B[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int tq = tw0 + 32 * nb + (lane & 31);
    A[nb] = tq - kbase - w - 4 * hh;
    B[nb] = tq - kbase + w_hi - 4 * hh;
  }

  const int steps = S + ngb;
  for (int s = 0; s < steps; ++s) {
    wait_vmem_all();   // this wave's parts of the blocks of step s have landed
    __syncthreads();   // ... and every other wave's; step s-1 is done everywhere
    if (s >= 1 && s + kRingSlots - 1 < total) issue(s + kRingSlots - 1);
    if (!wave_active) continue;

    const bool win = s < S;
    const int idx = win ? 2 * wv + s : nbt + (s - S);
    if (block_empty(idx)) continue;
    uint32_t keymask;
    if (win) {
      keymask = mask_in_lds ? sh.kmask[idx] : window_keymask(idx);
    } else {
      const int left = nG - kBlockK * (s - S);
      keymask = left >= kBlockK ? 0xffffffffu : ((1u << left) - 1u);
    }
    const unsigned char* slot = ring + (idx % kRingSlots) * Ly::kStageBytes;
    Frag<B16> kf;
    read_kfrag(kf, slot, lane);
    VtFrag<B16> vt;
    read_vt(vt, slot + Ly::kBlockBytes, lane);
    if (keymask != 0xffffffffu) zero_dead_keys(vt, keymask, lane);

    bool edge = true;
    const int kb = kbase + kBlockK * idx;
    if (win) {
      bool interior = keymask == 0xffffffffu && (tw0 + kWaveQ - 1 - kb <= w);
      interior = interior && (causal ? (tw0 >= kb + kBlockK - 1) : (kb + kBlockK - 1 - tw0 <= w));
      edge = !interior;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      f32x16 sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
      qk(sc, kf, qf[nb]);
      PFrag<B16> pf;
      softmax_half<B16>(st, nb, sc, pf, edge,
                        [&]() -> uint32_t {
                          uint32_t vb;
                          if (win) {
                            const int sh32 = kBlockK * idx;
                            const int lo = max(A[nb] - sh32, 0);
                            const int hi = min(B[nb] - sh32, 31);
                            vb = lo > hi ? 0u : ((0xffffffffu >> (31 - hi)) & (0xffffffffu << lo));
                          } else {
                            // a global key g joins local row i unless g is already in W(i)
                            vb = 0;
                            const int* gl = sh.G + kBlockK * (s - S) + 4 * hh;
#pragma unroll
                            for (int e = 0; e < 16; ++e) {
                              const int dd = qpos[nb] - gl[acc_c(e)];
                              const bool in_w = (dd <= wd && dd >= -wd) && (dil == 1 || dd % dil == 0);
                              vb |= in_w ? 0u : (1u << acc_c(e));
                            }
                          }
                          return vb & (keymask >> (4 * hh));
                        },
                        c);
      pv(st.o[nb], pf, vt);
    }
  }

  // a wave without local rows still writes its zero (padding) rows
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.l[nb] += __shfl_xor(st.l[nb], 32);
    st.cnt[nb] += __shfl_xor(st.cnt[nb], 32);
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if (!is_local[nb] && !is_zero[nb]) continue;
    T* orow = out + (size_t)qpos[nb] * rs;
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
  unsigned char* lds = sh.buf + wv * Lay<B16>::kWaveBytes;
  const float c = p.c;
  float* part_bh = p.partials + (size_t)bh * p.max_global * S * kPartialStride;

  ChunkSrc src;
  src.mrow = mrow;
  src.cbeg = cbeg;
  src.cend = cend;
  src.lane = lane;

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
    run_blocks<B16>(st, qf, src, kg, vg, rs, wv, nblk, lds, c);
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
__device__ __forceinline__ void fwd_body(const KernelParams& p) {
  __shared__ Shared<B16> sh;
  const int bid = blockIdx.x;
  if (bid < p.n_glob_pad) {
    if (bid < p.n_glob) global_split<B16>(p, bid, sh);
    return;
  }
  band_tile<B16>(p, xcd_remap(bid - p.n_glob_pad, p.n_band), sh);
}

// bf16: two waves per SIMD, so one wave's softmax overlaps the other's MFMAs.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void lf_attn_fwd_bf16(
    const KernelParams p) {
  fwd_body<true>(p);
}

// fp32: larger operand fragments; one wave per SIMD.
__global__ __launch_bounds__(kThreads) void lf_attn_fwd_f32(const KernelParams p) { fwd_body<false>(p); }

}  // namespace

int launch_forward(const KernelParams& kp, int dtype, void* stream) {
  const int grid = kp.n_glob_pad + kp.n_band;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == LF_BF16)
    hipLaunchKernelGGL(lf_attn_fwd_bf16, dim3(grid), dim3(kThreads), 0, s, kp);
  else
    hipLaunchKernelGGL(lf_attn_fwd_f32, dim3(grid), dim3(kThreads), 0, s, kp);
  return (int)hipGetLastError();
}

}  // namespace lf
