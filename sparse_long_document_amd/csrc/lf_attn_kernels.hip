// Longformer combined sliding-window + global attention forward for gfx950.
//
// One launch computes every output row with two kinds of workgroups:
//   * global-row splits (dispatched before the band tiles, or after them
//     when the whole launch is resident at once): split c of one (batch row b,
//     head h) scores every global token of b against keys
//     [1024c, 1024c + 1024) with the global projections (each global token
//     attends to every token: segmentfault Longformer summary, "Global
//     attention" and "Linear projections for global attention").  Each
//     split leaves a partial (max, sum, unnormalised output) record in the
//     workspace; the last split of (b, h) to arrive merges them and writes
//     the global rows.  With at most 32 global tokens per batch row the four
//     waves of a split share the keys instead of the queries ("solo");
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
// Workgroup: 4 waves.  Wave w takes query half qh = w & 1 (32 of the 64
// query rows) and key parity kp = w >> 1 (key blocks kp, kp + 2, ... of the
// tile's block list).  The two waves of a parity share that parity's ring
// of LDS stages: each issues half of a block's direct-to-LDS loads, waits
// for its own, and one workgroup barrier per step makes the whole block
// visible to both; the ring runs kStages - 1 blocks ahead.  At the end the
// two parities' partial states of each half are merged through LDS.
//
// Inner block: 32 keys x 32 queries per wave.
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
// The fp32 instantiation computes in true fp32 (v_mfma_f32_32x32x2_f32, P
// kept in fp32).
//
// Head dim: the source is compiled once per head dim D = LF_KD (32, 64 or
// 128; 64 when not defined) into its own namespace lf::d<D>.  The pages
// describe the layer with one head size (64 in the longformer-base shape)
// and the window and global pattern never look at the head dim, so D only
// sets the fragment counts, the stage sizes and the swizzles below.
#include <hip/hip_runtime.h>
#include <stdint.h>


#include <atomic>
#include <type_traits>

#include "lf_attn_internal.h"

#ifndef LF_KD
#define LF_KD 64
#endif
#define LF_CAT2(a, b) a##b
#define LF_CAT(a, b) LF_CAT2(a, b)

namespace lf {
namespace LF_CAT(d, LF_KD) {
namespace {

constexpr int kD = LF_KD;     // head dim of this instantiation
constexpr int kND = kD / 32;  // 32-dim blocks of O^T (kD x 32 queries) per wave
static_assert(kD == 32 || kD == 64 || kD == 128, "head dims 32, 64 and 128");
constexpr int kPartialStride = partial_stride(kD);

// The 16-bit element type of this translation unit: bf16, or f16 when the
// source is compiled with LF_HALF_F16 (which then yields the f16 kernel).
#if LF_HALF_F16
typedef _Float16 h16;
#else
typedef __bf16 h16;
#endif
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));

// 32x32x16 MFMA and two-term dot product on 16-bit operands with fp32
// accumulation, for the element type above.
__device__ __forceinline__ auto mfma16(h16x8 a, h16x8 b, __attribute__((ext_vector_type(16))) float c) {
#if LF_HALF_F16
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}
__device__ __forceinline__ float dot2h(h16x2 a, h16x2 b, float c) {
#if LF_HALF_F16
  return __builtin_amdgcn_fdot2(a, b, c, false);
#else
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
#endif
}
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

// Natural log-sum-exp of a row's scaled scores from its log2-domain
// reference max M and the row sum L = sum_j 2^(c s_j - M).
__device__ __forceinline__ float row_lse(float M, float L) {
  return (M + __builtin_amdgcn_logf(L)) * 0.69314718055994531f;
}

// LDS staging of key blocks.  A stage holds one block's K rows then its V
// rows (32 rows of kD head dims each); each key parity owns a ring of
// kStages stages, filled by direct-to-LDS loads while older stages are
// consumed.
template <bool B16>
struct Lay {
  static constexpr int kElt = B16 ? 2 : 4;
  static constexpr int kRowBytes = kD * kElt;            // 64 .. 512
  static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row
  // rows that share one 256-byte span of the LDS banks (1, 2 or 4)
  static constexpr int kRowsPerSpan = kRowBytes >= 256 ? 1 : 256 / kRowBytes;
  static_assert(kRowsPerSpan == 1 || kRowsPerSpan == 2 || kRowsPerSpan == 4, "row sizes 64 B and up");
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows covered by one wave-wide load
  static constexpr int kLoads = kBlockK / kRowsPerLoad;  // loads per block and tensor
  static constexpr int kHalfLoads = kLoads / 2;          // of those, issued by one wave of the pair
  static constexpr int kBlockBytes = kBlockK * kRowBytes;
  static constexpr int kStageBytes = 2 * kBlockBytes;
  static constexpr int kStages = 2;
  static constexpr int kRingBytes = kStages * kStageBytes;
};

// Chunk swizzles (the LDS position of 16-byte chunk c of row `row` is
// c ^ swz(row)).  With R rows per 256-byte bank span, row `row` starts at
// span offset (row % R) * rowbytes.  K: 16 consecutive rows at one chunk
// index land on distinct 16-byte slots of the span (R offsets times 16 / R
// swizzle values), for the K fragment reads.  V (16-bit): the transposed
// reads of a half-wave cover 4 consecutive rows (key rows 4a + e, e < 4) at
// one 64-byte column group, which land on distinct 64-byte quarters of the
// span (R offsets times 4 / R swizzle values of the group index).  V (fp32)
// is read along rows.
template <bool B16>
__device__ __forceinline__ int kswz(int row) {
  constexpr int R = Lay<B16>::kRowsPerSpan;
  constexpr int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  return (row >> lgR) & (16 / R - 1);
}
template <bool B16>
__device__ __forceinline__ int vswz(int row) {
  constexpr int R = Lay<B16>::kRowsPerSpan;
  constexpr int lgR = R == 4 ? 2 : (R == 2 ? 1 : 0);
  return B16 ? (((row >> lgR) & (4 / R - 1)) << 2) : 0;
}

template <bool B16>
using elem_t = typename std::conditional<B16, h16, float>::type;

// Per-lane operand fragment of the kD head dims of one row (query or key)
// for the QK^T contraction; the head dims a lane holds depend on lane / 32.
template <bool B16>
struct Frag;
template <>
struct Frag<true> {
  h16x8 x[kD / 16];  // dims 16s + 8*(lane/32) + [0, 8)
};
template <>
struct Frag<false> {
  float x[kD / 2];  // dims (kD/2)*(lane/32) + [0, kD/2)
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

// Workgroup execution barrier without the memory fences of
// __syncthreads(): the caller has already waited for the accesses that
// must be visible across it (the fences would also wait for the loads of
// later blocks still in flight).  The asm statement keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Barrier after which this wave's LDS writes are visible to the workgroup
// (vector-memory loads in flight are not waited for).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void load_frag(Frag<true>& f, const h16* row, int hh) {
  const h16x8* p = reinterpret_cast<const h16x8*>(row);
#pragma unroll
  for (int s = 0; s < kD / 16; ++s) f.x[s] = p[2 * s + hh];
}

__device__ __forceinline__ void load_frag(Frag<false>& f, const float* row, int hh) {
  const f32x4* p = reinterpret_cast<const f32x4*>(row + (kD / 2) * hh);
#pragma unroll
  for (int i = 0; i < kD / 8; ++i) {
    f32x4 t = p[i];
    f.x[4 * i + 0] = t[0];
    f.x[4 * i + 1] = t[1];
    f.x[4 * i + 2] = t[2];
    f.x[4 * i + 3] = t[3];
  }
}

// acc (32 keys x 32 queries) += K Q^T over the kD head dims.
__device__ __forceinline__ void qk(f32x16& acc, const Frag<true>& kf, const Frag<true>& qf) {
#pragma unroll
  for (int s = 0; s < kD / 16; ++s) acc = mfma16(kf.x[s], qf.x[s], acc);
}

__device__ __forceinline__ void qk(f32x16& acc, const Frag<false>& kf, const Frag<false>& qf) {
#pragma unroll
  for (int i = 0; i < kD / 2; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x[i], qf.x[i], acc, 0, 0, 0);
}

// Accumulator element r of a lane holds key row c_r + 4*(lane/32) of the
// block, c_r = 8*(r/4) + r%4.
__host__ __device__ constexpr int acc_c(int r) { return 8 * (r >> 2) + (r & 3); }

// ---------------------------------------------------------------------------
// One key block through LDS.
// ---------------------------------------------------------------------------

// Issue this wave's share of the direct-to-LDS loads of a block's K and V
// rows into `stage`: loads t = t0 .. t0 + kHalfLoads - 1 of each tensor.
// kpos(row) gives the token position of key row `row` (0..31) of the block,
// always a valid position (rows outside the key set are clamped here and
// masked later).  Lane l of load t fetches chunk (l % kChunks) ^ swz(row)
// of row kRowsPerLoad*t + l / kChunks; it lands at byte 1024t + 16l.
template <bool B16, int kN, class KPos>
__device__ __forceinline__ void issue_rows(const elem_t<B16>* kb, const elem_t<B16>* vb, uint32_t rs, KPos kpos,
                                           unsigned char* stage, int lane, int t0) {
  using L = Lay<B16>;
  constexpr int kEltPerChunk = 16 / L::kElt;
#pragma unroll
  for (int u = 0; u < kN; ++u) {
    const int t = t0 + u;
    const int row = L::kRowsPerLoad * t + lane / L::kChunks;
    const int c = lane % L::kChunks;
    const uint32_t base = (uint32_t)kpos(row) * rs;
    __builtin_amdgcn_global_load_lds(kb + (base + (c ^ kswz<B16>(row)) * kEltPerChunk),
                                     (LDS_AS void*)(stage + 1024 * t), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + (base + (c ^ vswz<B16>(row)) * kEltPerChunk),
                                     (LDS_AS void*)(stage + L::kBlockBytes + 1024 * t), 16, 0, 0);
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
  h16x8 a[kND][2];
};
template <>
struct VtFrag<false> {
  float a[kND][16];
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(LDS_AS const void*)p;
}

// Per-lane LDS addresses of the fragment reads of stage 0 of a ring (the
// other stage is kStageBytes further, an immediate offset).
//   K: key row lane % 32, 16-byte chunks 2s + lane/32 (s < kD/16), swizzled;
//   V: ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives
//   element j%4 of the 8-byte chunk addressed by lane 4e + j/4, as its
//   element e.  Lane 4e+q of group g points at key row 16ks + 8half +
//   4(g/2) + e, head dims 32db + 16(g%2) + 4q .. +3, so lane j of the group
//   gets head dim 32db + 16(g%2) + j for keys e = 0..3.
struct FragAddr {
  uint32_t k[kD / 16];
  uint32_t v[kND];
};

__device__ __forceinline__ FragAddr frag_addr(const unsigned char* ring, int lane) {
  using L = Lay<true>;
  FragAddr fa;
  const int row = lane & 31;
  const int hh = lane >> 5;
  const uint32_t kbase = lds_addr(ring) + (uint32_t)(row * L::kRowBytes);
  const int sw = kswz<true>(row);
#pragma unroll
  for (int s = 0; s < kD / 16; ++s) fa.k[s] = kbase + (uint32_t)(((2 * s + hh) ^ sw) << 4);
  const int g = lane >> 4;
  const int row0 = 4 * (g >> 1) + ((lane & 15) >> 2);
  const int byte0 = 32 * (g & 1) + 8 * (lane & 3);
  // vswz depends on the row mod 4 only, so rows 16ks + 8half + row0 share
  // row0's swizzle
  const int vsw = vswz<true>(row0);
  const uint32_t vbase = lds_addr(ring + L::kBlockBytes);
#pragma unroll
  for (int db = 0; db < kND; ++db) {
    const int byte = 64 * db + byte0;
    fa.v[db] = vbase + (uint32_t)(row0 * L::kRowBytes + (((byte >> 4) ^ vsw) << 4) + (byte & 15));
  }
  return fa;
}

// K fragment and V^T operand of the block in the stage kOff bytes into the
// ring, read in one asm block that waits for its reads before it ends.  The
// compiler cannot tell these reads from the direct-to-LDS loads still in
// flight into the other stage and would otherwise wait for all of them
// first; the caller has waited for this stage's loads (and the barrier
// after which the other wave's share is visible).  V rows 16ks + 8half sit
// kV8 (ks = 0, half = 1), 2 kV8 and 3 kV8 bytes past the first.
constexpr int kV8 = 8 * Lay<true>::kRowBytes;

// r[4db + 2ks + half] back into the V^T operand
__device__ __forceinline__ void assemble_vt(VtFrag<true>& vt, const u32x2* r) {
#pragma unroll
  for (int db = 0; db < kND; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x2 lo = r[4 * db + 2 * ks], hi = r[4 * db + 2 * ks + 1];
      vt.a[db][ks] = __builtin_bit_cast(h16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
}

#if LF_KD == 32
template <int kOff>
__device__ __forceinline__ void read_frags_at(Frag<true>& kf, VtFrag<true>& vt, const FragAddr& fa) {
  u32x4 k[2];
  u32x2 r[4];
  asm volatile(
      "ds_read_b128 %0, %6 offset:%9\n"
      "ds_read_b128 %1, %7 offset:%9\n"
      "ds_read_b64_tr_b16 %2, %8 offset:%9\n"
      "ds_read_b64_tr_b16 %3, %8 offset:%10\n"
      "ds_read_b64_tr_b16 %4, %8 offset:%11\n"
      "ds_read_b64_tr_b16 %5, %8 offset:%12\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(fa.k[0]), "v"(fa.k[1]), "v"(fa.v[0]), "i"(kOff), "i"(kOff + kV8), "i"(kOff + 2 * kV8),
        "i"(kOff + 3 * kV8)
      : "memory");
#pragma unroll
  for (int s = 0; s < 2; ++s) kf.x[s] = __builtin_bit_cast(h16x8, k[s]);
  assemble_vt(vt, r);
}
#elif LF_KD == 128
template <int kOff>
__device__ __forceinline__ void read_frags_at(Frag<true>& kf, VtFrag<true>& vt, const FragAddr& fa) {
  u32x4 k[8];
  u32x2 r[16];
  asm volatile(
      "ds_read_b128 %0, %24 offset:%36\n"
      "ds_read_b128 %1, %25 offset:%36\n"
      "ds_read_b128 %2, %26 offset:%36\n"
      "ds_read_b128 %3, %27 offset:%36\n"
      "ds_read_b128 %4, %28 offset:%36\n"
      "ds_read_b128 %5, %29 offset:%36\n"
      "ds_read_b128 %6, %30 offset:%36\n"
      "ds_read_b128 %7, %31 offset:%36\n"
      "ds_read_b64_tr_b16 %8, %32 offset:%36\n"
      "ds_read_b64_tr_b16 %9, %32 offset:%37\n"
      "ds_read_b64_tr_b16 %10, %32 offset:%38\n"
      "ds_read_b64_tr_b16 %11, %32 offset:%39\n"
      "ds_read_b64_tr_b16 %12, %33 offset:%36\n"
      "ds_read_b64_tr_b16 %13, %33 offset:%37\n"
      "ds_read_b64_tr_b16 %14, %33 offset:%38\n"
      "ds_read_b64_tr_b16 %15, %33 offset:%39\n"
      "ds_read_b64_tr_b16 %16, %34 offset:%36\n"
      "ds_read_b64_tr_b16 %17, %34 offset:%37\n"
      "ds_read_b64_tr_b16 %18, %34 offset:%38\n"
      "ds_read_b64_tr_b16 %19, %34 offset:%39\n"
      "ds_read_b64_tr_b16 %20, %35 offset:%36\n"
      "ds_read_b64_tr_b16 %21, %35 offset:%37\n"
      "ds_read_b64_tr_b16 %22, %35 offset:%38\n"
      "ds_read_b64_tr_b16 %23, %35 offset:%39\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]),
        "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
        "=&v"(r[15])
      : "v"(fa.k[0]), "v"(fa.k[1]), "v"(fa.k[2]), "v"(fa.k[3]), "v"(fa.k[4]), "v"(fa.k[5]), "v"(fa.k[6]),
        "v"(fa.k[7]), "v"(fa.v[0]), "v"(fa.v[1]), "v"(fa.v[2]), "v"(fa.v[3]), "i"(kOff), "i"(kOff + kV8),
        "i"(kOff + 2 * kV8), "i"(kOff + 3 * kV8)
      : "memory");
#pragma unroll
  for (int s = 0; s < 8; ++s) kf.x[s] = __builtin_bit_cast(h16x8, k[s]);
  assemble_vt(vt, r);
}
#else
template <int kOff>
__device__ __forceinline__ void read_frags_at(Frag<true>& kf, VtFrag<true>& vt, const FragAddr& fa) {
  u32x4 k[4];
  u32x2 r[8];  // [db][ks][lo, hi]: key rows 16ks + 8half at +2 kV8 ks + kV8 half
  asm volatile(
      "ds_read_b128 %0, %12 offset:%18\n"
      "ds_read_b128 %1, %13 offset:%18\n"
      "ds_read_b128 %2, %14 offset:%18\n"
      "ds_read_b128 %3, %15 offset:%18\n"
      "ds_read_b64_tr_b16 %4, %16 offset:%18\n"
      "ds_read_b64_tr_b16 %5, %16 offset:%19\n"
      "ds_read_b64_tr_b16 %6, %16 offset:%20\n"
      "ds_read_b64_tr_b16 %7, %16 offset:%21\n"
      "ds_read_b64_tr_b16 %8, %17 offset:%18\n"
      "ds_read_b64_tr_b16 %9, %17 offset:%19\n"
      "ds_read_b64_tr_b16 %10, %17 offset:%20\n"
      "ds_read_b64_tr_b16 %11, %17 offset:%21\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
        "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(fa.k[0]), "v"(fa.k[1]), "v"(fa.k[2]), "v"(fa.k[3]), "v"(fa.v[0]), "v"(fa.v[1]), "i"(kOff),
        "i"(kOff + kV8), "i"(kOff + 2 * kV8), "i"(kOff + 3 * kV8)
      : "memory");
#pragma unroll
  for (int s = 0; s < 4; ++s) kf.x[s] = __builtin_bit_cast(h16x8, k[s]);
  assemble_vt(vt, r);
}
#endif

__device__ __forceinline__ void read_frags(Frag<true>& kf, VtFrag<true>& vt, const FragAddr& fa,
                                           const unsigned char*, int stage) {
  static_assert(Lay<true>::kStages == 2, "two stages: offsets 0 and kStageBytes");
  if (stage == 0)
    read_frags_at<0>(kf, vt, fa);
  else
    read_frags_at<Lay<true>::kStageBytes>(kf, vt, fa);
}

// fp32: plain reads (the compiler may wait for every load in flight first;
// this instantiation is not tuned).
__device__ __forceinline__ void read_frags(Frag<false>& kf, VtFrag<false>& vt, const FragAddr&,
                                           const unsigned char* stage, int) {
  using L = Lay<false>;
  const int lane = lane_id();
  const int row = lane & 31;
  const int hh = lane >> 5;
  const unsigned char* rp = stage + row * L::kRowBytes;
  const int sw = kswz<false>(row);
#pragma unroll
  for (int j = 0; j < kD / 8; ++j) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(rp + ((((kD / 8) * hh + j) ^ sw) << 4));
    kf.x[4 * j + 0] = t[0];
    kf.x[4 * j + 1] = t[1];
    kf.x[4 * j + 2] = t[2];
    kf.x[4 * j + 3] = t[3];
  }
  const float* vs = reinterpret_cast<const float*>(stage + L::kBlockBytes);
#pragma unroll
  for (int db = 0; db < kND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) vt.a[db][r] = vs[(acc_c(r) + 4 * hh) * kD + 32 * db + (lane & 31)];
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
    for (int db = 0; db < kND; ++db)
      vt.a[db][ks] = __builtin_bit_cast(h16x8, __builtin_bit_cast(u32x4, vt.a[db][ks]) & keep);
  }
}

__device__ __forceinline__ void zero_dead_keys(VtFrag<false>& vt, uint32_t keymask, int lane) {
  const uint32_t km = keymask >> (4 * (lane >> 5));
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (!((km >> acc_c(r)) & 1u)) {
#pragma unroll
      for (int db = 0; db < kND; ++db) vt.a[db][r] = 0.f;
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
  const uint32_t sspan = __builtin_amdgcn_readfirstlane(span);  // uniform: the asm takes it from an SGPR
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(m) : "v"(u), "s"(sspan), "v"(span + 1u));  // one scalar operand per VALU op
  return m - span;
}

// Zero this lane's K fragment when its key row (lane % 32) is clear in
// keymask, so that row's scores are exactly 0 before the mask is added.
__device__ __forceinline__ void zero_dead_krow(Frag<true>& kf, uint32_t keymask, int lane) {
  if (!((keymask >> (lane & 31)) & 1u)) {
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) kf.x[s] = h16x8{};
  }
}

__device__ __forceinline__ void zero_dead_krow(Frag<false>& kf, uint32_t keymask, int lane) {
  if (!((keymask >> (lane & 31)) & 1u)) {
#pragma unroll
    for (int j = 0; j < kD / 2; ++j) kf.x[j] = 0.f;
  }
}

// Probabilities of one block in the operand form of the PV product.
template <bool B16>
struct PFrag;
template <>
struct PFrag<true> {
  h16x8 x[2];  // PV k-step ks holds accumulator elements 8ks .. 8ks+7
};
template <>
struct PFrag<false> {
  float x[16];
};

// Running state of one wave: 32 query columns.
struct HalfState {
  f32x16 o[kND];  // O^T of head dims 32db + ..., per 32-dim block db
  float m;      // reference max (log2 domain) of the lane's query
  float l;      // partial row sum of this lane (16 of the 32 keys per block)
  int cnt;      // partial count of scored keys of this lane, beyond 16 per full block
  int nfull;    // blocks whose 16 keys of every lane were all scored (uniform)
  float thr;    // (m + kRescaleSlack) / c: a raw score above it moves the reference
};

__device__ __forceinline__ void state_init(HalfState& st) {
  st.m = kMInit;
  st.l = 0.f;
  st.cnt = 0;
  st.nfull = 0;
  st.thr = kMInit;  // set by softmax_core before its first use
#pragma unroll
  for (int db = 0; db < kND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[db][r] = 0.f;
}

// O^T (kD dims x 32 queries) += V^T P^T.
__device__ __forceinline__ void pv(f32x16 (&o)[kND], const PFrag<true>& pf, const VtFrag<true>& vt) {
#pragma unroll
  for (int db = 0; db < kND; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      o[db] = mfma16(vt.a[db][ks], pf.x[ks], o[db]);
}

__device__ __forceinline__ void pv(f32x16 (&o)[kND], const PFrag<false>& pf, const VtFrag<false>& vt) {
#pragma unroll
  for (int db = 0; db < kND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt.a[db][r], pf.x[r], o[db], 0, 0, 0);
}


// Largest of the 16 scores of a lane.  Plain fmaxf: the compiler sees
// that it reads MFMA results and inserts the wait states such a read needs
// (it cannot see into inline asm).
__device__ __forceinline__ float max16(const f32x16& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
  const float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float d = fmaxf(fmaxf(s[6], s[7]), s[8]);
  const float e = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float f = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(a, b), d), fmaxf(fmaxf(e, f), s[15]));
}

// Scores of one block (masked scores are -inf) -> online-softmax
// probabilities, with the running state rescaled if its reference max
// moves.  Lanes l and l ^ 32 hold the same query's other 16 keys, but the
// exchange is only needed when the reference max moves: the test "some raw
// score exceeds thr = (m + slack) / c" is a wave-wide vote.  The row sum is
// that of the probabilities as they enter P V (rounded to the element
// type; one chain of two-term dot products).
template <bool B16>
__device__ __forceinline__ void softmax_core(HalfState& st, f32x16& s, PFrag<B16>& pf, float c) {
  const float mx = max16(s);
  if (__any(mx > st.thr)) {
    const float ml = mx * c;
    const float mn = fmaxf(st.m, fmaxf(ml, __shfl_xor(ml, 32)));
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.m = mn;
    st.thr = (mn + kRescaleSlack) / c;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < kND; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -st.m));
  if constexpr (B16) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.x[ks][e] = (h16)s[8 * ks + e];
    const h16x2 one = {(h16)1.0f, (h16)1.0f};
    float l = st.l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const h16x2 pj = {pf.x[j >> 2][2 * (j & 3)], pf.x[j >> 2][2 * (j & 3) + 1]};
      l = dot2h(pj, one, l);
    }
    st.l = l;
  } else {
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t8[i] = s[2 * i] + s[2 * i + 1];
    st.l += ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
#pragma unroll
    for (int r = 0; r < 16; ++r) pf.x[r] = s[r];
  }
}

// Raw (untyped) buffer resource over `bytes` bytes at `base`; accesses past
// the end read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Bit 7 of byte e of the result: byte e of x is 2.  After x ^ 0x02 the
// bytes that were 2 are the zero bytes; per byte, ((t & 0x7f) + 0x7f) | t
// has bit 7 set exactly when the byte is not zero (no carry leaves a byte).
__device__ __forceinline__ uint32_t twos_flags(uint32_t x) {
  const uint32_t t = x ^ 0x02020202u;
  return ~(((t & 0x7f7f7f7fu) + 0x7f7f7f7fu) | t) & 0x80808080u;
}

// Bits 7, 15, 23, 31 of f as bits 0 .. 3.
__device__ __forceinline__ uint32_t gather_flags(uint32_t f) {
  return ((f >> 7) & 1u) | ((f >> 14) & 2u) | ((f >> 21) & 4u) | ((f >> 28) & 8u);
}

// The mask bytes of one batch row, read through a buffer resource over the
// whole mask: reads past its end return zero, so no load needs a guard and
// none waits for another.  Rows whose 16-byte chunks are all aligned (n and
// the mask's address multiples of 16) are read 16 bytes per load, others a
// byte per load.
struct MaskRow {
  __amdgpu_buffer_rsrc_t rm;
  uint32_t row;  // byte offset of the row
  bool wide;
};

__device__ __forceinline__ MaskRow mask_row(const int8_t* mask, int B, int n, int b) {
  MaskRow m;
  m.rm = make_rsrc(mask, (uint32_t)B * (uint32_t)n);
  m.row = (uint32_t)b * (uint32_t)n;
  m.wide = (n & 15) == 0 && (reinterpret_cast<uintptr_t>(mask) & 15u) == 0;
  return m;
}

// Bytes p0 .. p0 + 15 of the row (any beyond the row are masked by the caller).
__device__ __forceinline__ u32x4 mask_chunk(const MaskRow& m, int p0) {
  const uint32_t off = m.row + (uint32_t)p0;
  if (m.wide) return __builtin_amdgcn_raw_buffer_load_b128(m.rm, off, 0, 0);
  u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e)
    x[e >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(m.rm, off + (uint32_t)e, 0, 0) << (8 * (e & 3));
  return x;
}

// Bits of the chunk at p0 that lie in the row [0, n).
__device__ __forceinline__ uint32_t chunk_in_row(int p0, int n) {
  const int k = n - p0;
  return k >= 16 ? 0xffffu : (k <= 0 ? 0u : (1u << k) - 1u);
}

// Bit e of the result: byte p0 + e of the row is 2 (p0 + e < n), for the
// 16 bytes x at p0.  Most chunks hold no global token: the bit gather only
// runs when some lane of the wave has one.
__device__ __forceinline__ uint32_t twos16(const u32x4& x, int p0, int n) {
  uint32_t f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = twos_flags(x[j]);
  const bool any = ((f[0] | f[1] | f[2] | f[3]) != 0u) && p0 < n;
  if (!__any(any)) return 0u;
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) bits |= gather_flags(f[j]) << (4 * j);
  return bits & chunk_in_row(p0, n);
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

// The scan's first round of mask loads (bytes [4096 u + 16 tid, +16) for
// u < 4), issued before anything else so that they do not queue behind the
// key and value loads.
constexpr int kScanStep = kThreads * 16;
struct ScanPre {
  u32x4 x[4];
  uint32_t bits[4];  // bytes equal to 2, formed by scan_ready
};
__device__ __forceinline__ void scan_preload(ScanPre& sp, const MaskRow& m, int n) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    sp.x[u] = u * kScanStep < n ? mask_chunk(m, u * kScanStep + 16 * tid) : u32x4{0u, 0u, 0u, 0u};
}

// Turns the preloaded chunks into bitmasks in straight-line code, where the
// compiler's count of loads in flight is exact (at the scan loop's entry it
// would wait for every load, the key loads included).
__device__ __forceinline__ void scan_ready(ScanPre& sp, int n) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) sp.bits[u] = u * kScanStep < n ? twos16(sp.x[u], u * kScanStep + 16 * tid, n) : 0u;
}

// Ordered list of positions j with mask_row[j] == 2 into G (LDS), at most
// cap entries; returns the total count.  Every thread of the workgroup
// calls it and gets the same result.  Each thread looks at 16 bytes of each
// 4 KB step; four steps are loaded together (the first four from sp) and
// ranked with one barrier.
__device__ __forceinline__ int scan_globals(const ScanPre& sp, const MaskRow& m, int n, int* G, int cap,
                                            int (*s_tot)[kWaves]) {
  int total = 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  for (int base = 0; base < n; base += 4 * kScanStep) {
    uint32_t bits[4];
    if (base == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) bits[u] = sp.bits[u];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p0 = base + u * kScanStep + 16 * tid;
        bits[u] = base + u * kScanStep < n ? twos16(mask_chunk(m, p0), p0, n) : 0u;
      }
    }
    // (barriers without fences: the key loads already in flight are not
    // waited for here)
    int pre[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cnt = __popc(bits[u]);
      pre[u] = __any(cnt != 0) ? wave_prefix(cnt) : 0;
      if (lane == 63) s_tot[u][wv] = pre[u] + cnt;
    }
    lds_barrier();
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
        if (slot < cap) G[slot] = base + u * kScanStep + 16 * tid + e;
        ++slot;
      }
    }
    total = off;
    lds_barrier();  // G is complete; s_tot is reused by the next steps
  }
  return __builtin_amdgcn_readfirstlane(total);  // the same in every lane
}

// A lane's O^T accumulators hold kND * 16 values; value j = 16 db + 4 g + i
// (o[db][4g + i]) is head dim 32 db + 8 g + 4 (lane / 32) + i.  The merge
// splits them in two halves of kHalfO values: key parity kp's wave emits
// j in [kHalfO kp, kHalfO (kp + 1)).
constexpr int kHalfO = 8 * kND;

__host__ __device__ constexpr int odim(int j, int hh) { return 32 * (j >> 4) + 8 * ((j >> 2) & 3) + 4 * hh + (j & 3); }
// Half `part` of the values covers head dims [kD/2 part, kD/2 (part + 1)):
// odim(kHalfO part + u, hh) = kD/2 part + odim(u, hh) for u < kHalfO.
static_assert(odim(kHalfO, 0) == kD / 2 && odim(kHalfO + 4, 1) == kD / 2 + odim(4, 1), "halves are contiguous");

__device__ __forceinline__ float oval(const HalfState& st, int j) { return st.o[j >> 4][j & 15]; }

// Partial state of one wave parked in LDS for the merge: the half of O^T
// that the partner wave emits, as [g][lane] f32x4, then per query
// (lane % 32) the reference max, the row sum and the key count.
constexpr int kParkOBytes = (kHalfO / 4) * 64 * 16;
constexpr int kParkBytes = kParkOBytes + 3 * 32 * 4;

template <bool B16>
struct Shared {
  static constexpr int kRings = 2 * Lay<B16>::kRingBytes;
  static constexpr int kBufBytes = kRings > kWaves * kParkBytes ? kRings : kWaves * kParkBytes;
  int G[LF_MAX_GLOBAL];
  int wave_tmp[4][kWaves];
  int flag;
  uint32_t ktab[kWaves][32];  // validity bits of each wave's table blocks
  __attribute__((aligned(16))) unsigned char buf[kBufBytes];  // the two rings; then the parked states
};

// The two waves of query half qh (key parities 0 and 1) hold partial
// results for the same 32 queries over disjoint key subsets; wave (qh, kp)
// emits half kp of the O^T values.  Every wave parks the half its partner
// emits with its (m, l, count) (after a barrier: the rings it overwrites
// are no longer read), and after a second barrier combines its own half
// with the partner's parked one.  It passes, per lane, the merged max M
// (log2 domain), row sum L, key count and the kHalfO unnormalised outputs
// (o[u] is value j = kHalfO kp + u, head dim odim(j, lane / 32)) to
// emit(kp, M, L, cnt, o).  Both waves of a row form M, L and the outputs
// with parity 0's terms first, so the row's two halves share one L.
template <bool B16, class Emit>
__device__ void merge_parities(const HalfState& st, Shared<B16>& sh, int qh, int kp, Emit emit) {
  const int lane = lane_id();
  const int hh = lane >> 5;
  __syncthreads();
  unsigned char* mine = sh.buf + (2 * kp + qh) * kParkBytes;
  f32x4* po = reinterpret_cast<f32x4*>(mine);
  float give[kHalfO];  // the partner's half: values [kHalfO (1 - kp), ...)
#pragma unroll
  for (int u = 0; u < kHalfO; ++u) give[u] = kp ? oval(st, u) : oval(st, kHalfO + u);
#pragma unroll
  for (int g = 0; g < kHalfO / 4; ++g)
    po[g * 64 + lane] = f32x4{give[4 * g], give[4 * g + 1], give[4 * g + 2], give[4 * g + 3]};
  const float l = st.l + __shfl_xor(st.l, 32);
  const int mycnt = st.cnt + 16 * st.nfull;
  const int cnt = mycnt + __shfl_xor(mycnt, 32);
  float* pm = reinterpret_cast<float*>(mine + kParkOBytes);
  if (hh == 0) {
    pm[lane] = st.m;
    pm[32 + lane] = l;
    reinterpret_cast<int*>(pm + 64)[lane] = cnt;
  }
  __syncthreads();
  const int q = lane & 31;
  const unsigned char* pp = sh.buf + (2 * (1 - kp) + qh) * kParkBytes;
  const float* mp = reinterpret_cast<const float*>(pp + kParkOBytes);
  const float m_p = mp[q], l_p = mp[32 + q];
  const int c = cnt + reinterpret_cast<const int*>(mp + 64)[q];
  // parity 0's terms are "a", parity 1's "b"
  const float ma = kp ? m_p : st.m, mb = kp ? st.m : m_p;
  const float la = kp ? l_p : l, lb = kp ? l : l_p;
  const float M = fmaxf(ma, mb);
  const float fa = __builtin_amdgcn_exp2f(ma - M);
  const float fb = __builtin_amdgcn_exp2f(mb - M);
  const float Lsum = la * fa + lb * fb;
  const float f_own = kp ? fb : fa, f_p = kp ? fa : fb;
  float own[kHalfO];
#pragma unroll
  for (int u = 0; u < kHalfO; ++u) own[u] = kp ? oval(st, kHalfO + u) : oval(st, u);
  const f32x4* op = reinterpret_cast<const f32x4*>(pp);
  float o[kHalfO];
#pragma unroll
  for (int g = 0; g < kHalfO / 4; ++g) {
    const f32x4 y = op[g * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float xo = own[4 * g + i];
      o[4 * g + i] = kp ? __builtin_fmaf(y[i], f_p, xo * f_own) : __builtin_fmaf(xo, f_own, y[i] * f_p);
    }
  }
  emit(kp, M, Lsum, c, o);
}

template <bool B16>
__device__ __forceinline__ void store4(elem_t<B16>* dst, const float* v);

template <>
__device__ __forceinline__ void store4<true>(h16* dst, const float* v) {
  h16x4 t;
  t[0] = (h16)v[0];
  t[1] = (h16)v[1];
  t[2] = (h16)v[2];
  t[3] = (h16)v[3];
  *reinterpret_cast<h16x4*>(dst) = t;
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
  // halos) share one L2.  x is the band index blockIdx.x - (0 or n_glob):
  // every x of one class x % 8 has one blockIdx.x % 8, so each class runs
  // on one XCD whatever the offset is (the class is a relabelling of the
  // XCD index), and the classes are dealt contiguous ranges of tiles.
  const int per = N / 8, rem = N % 8;
  const int xcd = x % 8, y = x / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + y;
}

// Output values of one quarter of a row (half `part` of the O^T values of
// lane half hh): head dims odim(kHalfO part + u, hh) from o[u], times inv
// (or zeros).
template <bool B16>
__device__ __forceinline__ void store_quadrant(elem_t<B16>* row, int part, int hh, const float* o, float inv,
                                               bool zero) {
  elem_t<B16>* dst = row + (kD / 2) * part + 4 * hh;
#pragma unroll
  for (int g = 0; g < kHalfO / 4; ++g) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = zero ? 0.f : o[4 * g + i] * inv;
    store4<B16>(dst + odim(4 * g, 0), t);
  }
}

// ---------------------------------------------------------------------------
// Key sources.  A source lists a wave's key blocks by index i: blocks
// i < nwin have their key validity in the wave's table, blocks i >= nwin are
// global-column blocks (band tiles only).  Each provides:
//   kpos(i, row), exists(i, row)  token position (clamped) / existence of key row `row`
//   dstep(), affine_range(lo&, hi&, base&)
//                                 blocks [lo, hi) are evenly spaced and in range: row r of
//                                 block i is token base + dstep (32 i + r)
//   classify(i, keymask)          0 empty, 1 masked per element, 2 full, for the wave's half
//   valid_bits(i)                 this lane's rows c_r in its query's key set (classify 1)
//   fast_range(lo&, hi&)          table blocks that are full wherever their keys are valid
// ---------------------------------------------------------------------------

// Blocks of one split of a global row: keys cbeg + 32 i + row.  A global
// row attends to every key with mask 1 or 2 (the table bits), so a block is
// full exactly when all 32 of its keys are valid.
struct ChunkSrc {
  const int8_t* mrow;
  int cbeg, cend, nwin;
  int nG;  // no global-column blocks
  __device__ int kpos(int i, int row) const {
    const int kk = cbeg + kBlockK * i + row;
    return kk < cend ? kk : cend - 1;
  }
  __device__ bool exists(int i, int row) const { return cbeg + kBlockK * i + row < cend; }
  __device__ int dstep() const { return 1; }
  // blocks [lo, hi) have all 32 rows in the chunk; block i starts at base + 32 i
  __device__ void affine_range(int& lo, int& hi, int& base) const {
    lo = 0;
    hi = (cend - cbeg) / kBlockK;
    base = cbeg;
  }
  __device__ int classify(int, uint32_t keymask) const { return keymask == 0xffffffffu ? 2 : 1; }
  __device__ uint32_t valid_bits(int) const { return 0xffffffffu; }
  __device__ void fast_range(int& lo, int& hi) const {
    lo = 0;
    hi = nwin;
  }
};

// Blocks of a band tile for query half qh (rows t0 + 32 qh + lane % 32 of
// the residue sequence): first the non-empty 32-key blocks of the tile's
// window span (residue-sequence keys kbase + 32 (jlo + i) + row, tokens
// r + dil * key), then the blocks of the row's global tokens
// G[32 (i - nwin) + row].
struct BandSrc {
  const int8_t* mrow;
  const int* G;
  int kbase, jlo, nwin;
  int n_r, r, dil, nG;
  int t0, qh, w, wd;
  int w_hi;  // w, or 0 when causal
  // Query row of this lane (residue-sequence index, clamped to the last
  // row) and its token position.
  __device__ int qrow() const {
    const int tq = t0 + 32 * qh + (lane_id() & 31);
    return tq < n_r ? tq : n_r - 1;
  }
  __device__ int qpos() const { return r + dil * qrow(); }
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
  // window blocks [lo, hi) have all 32 keys in [0, n_r); block i starts at
  // token base + 32 dil i
  __device__ void affine_range(int& lo, int& hi, int& base) const {
    const int k0 = kbase + kBlockK * jlo;  // key of row 0 of block 0
    lo = k0 >= 0 ? 0 : (-k0 + kBlockK - 1) / kBlockK;
    const int top = n_r - kBlockK - k0;  // block i fits when 32 i <= top
    hi = top < 0 ? 0 : min(nwin, top / kBlockK + 1);
    base = r + dil * k0;
  }
  __device__ int classify(int i, uint32_t keymask) const {
    if (i >= nwin) return 1;  // global columns: masked against each row's window
    const int k0 = key(i, 0);
    const int qlo = t0 + 32 * qh, qhi = qlo + 31;
    if (k0 > qhi + w_hi || k0 + kBlockK - 1 < qlo - w) return 0;
    const bool full = keymask == 0xffffffffu && k0 >= qhi - w && k0 + kBlockK - 1 <= qlo + w_hi;
    return full ? 2 : 1;
  }
  __device__ void fast_range(int& lo, int& hi) const {
    // span block j (keys kbase + 32 j ..) lies in the window of every query
    // of the half: 32 j >= 32 qh + 31 and 32 j + 31 <= 32 qh + w + w_hi
    int jl = qh + 1;
    const int top = 32 * qh + w + w_hi - (kBlockK - 1);
    int jh = top >= 0 ? top / kBlockK + 1 : 0;  // exclusive
    // and its keys are in [0, n_r)
    jl = max(jl, kbase >= 0 ? 0 : (-kbase + kBlockK - 1) / kBlockK);
    jh = min(jh, n_r - kbase - kBlockK >= 0 ? (n_r - kbase - kBlockK) / kBlockK + 1 : 0);
    lo = max(jl - jlo, 0);
    hi = max(min(jh - jlo, nwin), lo);
  }
  __device__ uint32_t valid_bits(int i) const {
    if (i < nwin) {
      const int sh32 = kBlockK * (jlo + i);
      // window rows c (block-relative, minus 4 (lane/32)) in [lo, hi] hold keys
      // in the query's window
      const int ln = lane_id_here();
      const int tq = t0 + 32 * qh + (ln & 31);
      const int a = tq - kbase - w - 4 * (ln >> 5), b = tq - kbase + w_hi - 4 * (ln >> 5);
      const int lo = max(a - sh32, 0);
      const int hi = min(b - sh32, 31);
      return lo > hi ? 0u : ((0xffffffffu >> (31 - hi)) & (0xffffffffu << lo));
    }
    // A global key g joins local row i unless g is already in W(i):
    // |i - g| <= w d and d divides i - g (no causal rows have global columns).
    // Rows 8 g4 + 4 hh + [0, 4) of the block, four at a time, each read in
    // an asm block that waits for it (the compiler would otherwise wait for
    // the key loads in flight into the staging area first).
    const int ln = lane_id_here();
    const uint32_t ga = lds_addr(G + kBlockK * (i - nwin) + 4 * (ln >> 5));
    const uint32_t span = 2u * (uint32_t)wd;
    const int tq = t0 + 32 * qh + (ln & 31);
    const int qp = r + dil * (tq < n_r ? tq : n_r - 1);
    uint32_t vb = 0;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x4 x;
      asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(ga), "i"(32 * g4) : "memory");
      if (dil == 1) {
        // bit = 1 when u = qp - g + wd exceeds span (g outside the window):
        // med3(u, span, span + 1) - span, without a compare through VCC
        const uint32_t qpw = (uint32_t)(qp + wd);
#pragma unroll
        for (int e = 0; e < 4; ++e) vb |= above_span(qpw - x[e], span) << (8 * g4 + e);
      } else {
        // the divisor passes through an empty asm so that the division's
        // setup is redone here instead of being hoisted out of the block loop
        // and held in a register through every block
        int d = __builtin_amdgcn_readfirstlane(dil);
        asm volatile("" : "+s"(d));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dd = qp - (int)x[e];
          const bool in_w = (uint32_t)(dd + wd) <= span && dd % d == 0;
          vb |= in_w ? 0u : (1u << (8 * g4 + e));
        }
      }
    }
    return vb;
  }
};

// ---------------------------------------------------------------------------
// Block loop of one wave: key blocks i = kp, kp + 2, ... < end of a source,
// step s handling block 2 s + kp from stage s % kStages of the parity's
// ring.  Every wave of the workgroup runs the same number of steps (one
// barrier each), whether or not it has a block or rows to score.
//
// Solo (a run-time choice, uniform): the wave owns its blocks i = kp,
// kp + 4, ... (kp is then the wave index) and one stage of its own, loads
// each block whole and needs no barrier (run_solo).
// ---------------------------------------------------------------------------
template <bool B16, class Src>
struct HalfLoop {
  using T = elem_t<B16>;
  using L = Lay<B16>;
  // vector-memory instructions one issue() emits (K and V rows) when the
  // wave shares the block with the other wave of its parity (twice that solo)
  static constexpr int kIssueLoads = 2 * L::kHalfLoads;
  static constexpr int kTabPairs = 12;
  const Src& src;
  const T* kb;
  const T* vb;
  uint32_t rs;
  unsigned char* ring;
  int lane, kp, qh;
  bool solo;
  int lg;  // log2 of the block index step between this wave's blocks (1, or 2 solo)
  // buffer resources and per-lane offsets of the evenly spaced (affine) path:
  // load t of a block takes K offset vk[t % kND] (the K swizzle of its rows
  // cycles with that period) and V offset vv
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t vk[kND], vv;
  // key-validity bits of this wave's table blocks (entry k: block
  // kp + (k << lg)), filled in the prologue; null when the source has more
  // table blocks than the table holds
  const uint32_t* ktab;
  int tabv[kTabPairs];
  int tab_cnt;
  uint32_t full_keys;  // bit k: every key of table entry k's block is valid
  int fast_lo, fast_hi;
  uint32_t fast_steps;  // bit s: the wave's block of step s is full for its half
  // evenly spaced blocks [aff_lo, aff_hi): block i's rows start at byte
  // so_base + i so_blk of each tensor
  int aff_lo, aff_hi, so_base, so_blk;
  FragAddr fa;  // this lane's fragment read addresses in stage 0 (bf16)

  __device__ HalfLoop(const Src& s, const T* k, const T* v, uint32_t rs_, unsigned char* ring_, int n, int kp_,
                      int qh_, bool solo_ = false)
      : src(s), kb(k), vb(v), rs(rs_), ring(ring_), lane(lane_id()), kp(kp_), qh(qh_), solo(solo_), lg(solo_ ? 2 : 1),
        ktab(nullptr), tab_cnt(0), full_keys(0), fast_lo(0), fast_hi(0), fast_steps(0) {
    const uint32_t bytes = (uint32_t)(((size_t)(n - 1) * rs + kD) * sizeof(T));
    rk = make_rsrc(k, bytes);
    rv = make_rsrc(v, bytes);
    // 16-bit rows: lane l of load t takes chunk c = l % kChunks of row
    // kRowsPerLoad t + l / kChunks.  With R rows per bank span, the row's
    // span index is 4 t + x, x = (l / kChunks) / R < 4, so its K swizzle is
    // ((4 t) mod kChunks) ^ x: 4 (t % kND) ^ x; its V swizzle does not
    // depend on t.
    constexpr uint32_t C = L::kChunks, R = L::kRowsPerSpan;
    const uint32_t ul = (uint32_t)lane;
    const uint32_t row_off = (uint32_t)src.dstep() * (ul / C) * rs;
    const uint32_t x = (ul / C) / R;
    const uint32_t ck = (ul % C) ^ x;
    const uint32_t cv = (ul % C) ^ ((x & (kND - 1)) << 2);
#pragma unroll
    for (int vi = 0; vi < kND; ++vi) vk[vi] = 2u * (row_off + 8u * (ck ^ (4u * vi)));
    vv = 2u * (row_off + 8u * cv);
    if constexpr (B16) fa = frag_addr(ring, lane);
    src.fast_range(fast_lo, fast_hi);
    int base;
    src.affine_range(aff_lo, aff_hi, base);
    so_base = base * (int)(2u * rs);
    so_blk = kBlockK * src.dstep() * (int)(2u * rs);
  }

  // This wave's loads of block i into stage st (exactly kIssueLoads
  // vector-memory instructions on every path, and nothing else: the loop's
  // waits count them).
  __device__ void issue(int i, int st) {
    unsigned char* dst = ring + st * L::kStageBytes;
    if (B16 && i >= aff_lo && i < aff_hi) {
      // scalar offsets: wave-uniform by construction; readfirstlane keeps
      // them in SGPRs even where register pressure moved a term to a VGPR
      const uint32_t so = (uint32_t)(so_base + i * so_blk);
      const uint32_t step = (uint32_t)src.dstep() * (uint32_t)L::kRowsPerLoad * rs * 2u;
#pragma unroll
      for (int u = 0; u < 2 * L::kHalfLoads; ++u) {
        if (u >= L::kHalfLoads && !solo) break;
        const int t = (solo ? 0 : qh * L::kHalfLoads) + u;
        const uint32_t sot = __builtin_amdgcn_readfirstlane(so + t * step);
        // t % kND = u % kND: the first load qh kHalfLoads of a wave's share is
        // a multiple of kND (kHalfLoads = kND for 16-bit rows)
        static_assert(!B16 || L::kHalfLoads % kND == 0, "K offset of load t is vk[u % kND]");
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS_AS void*)(dst + 1024 * t), 16, vk[u % kND], sot, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS_AS void*)(dst + L::kBlockBytes + 1024 * t), 16, vv, sot,
                                                 0, 0);
      }
    } else {
      // lane-derived terms recomputed here (a rare path) rather than hoisted
      // out of the block loop and held in registers
      if (solo)
        issue_rows<B16, 2 * L::kHalfLoads>(kb, vb, rs, [&](int r) { return src.kpos(i, r); }, dst, lane_id_here(), 0);
      else
        issue_rows<B16, L::kHalfLoads>(kb, vb, rs, [&](int r) { return src.kpos(i, r); }, dst, lane_id_here(),
                                       qh * L::kHalfLoads);
    }
  }

  // Validity bits of table block i read from the mask now (rows that exist
  // with mask 1 or 2).
  __device__ uint32_t table_keymask(int i) const {
    const int row = lane_id_here() & 31;
    const int m = src.exists(i, row) ? (int)src.mrow[src.kpos(i, row)] : 0;
    return (uint32_t)__ballot(m == 1 || m == 2);
  }

  // The table: tab_load issues the mask-byte loads (two blocks per load,
  // lanes 32-63 take the second) and tab_commit, after the caller has
  // issued its first K/V loads, turns them into bits.  Sources with more
  // than 2 kTabPairs table blocks per wave go without the table.
  __device__ void tab_load() {
    tab_cnt = kp < src.nwin ? (src.nwin - kp + (1 << lg) - 1) >> lg : 0;
    if (tab_cnt > 2 * kTabPairs) return;
    const int row = lane & 31, half = lane >> 5;
#pragma unroll
    for (int p = 0; p < kTabPairs; ++p) {
      if (2 * p >= tab_cnt) break;
      const int k = 2 * p + half;
      const int i = kp + (k << lg);
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
    // steps k whose block kp + (k << lg) lies in [fast_lo, fast_hi)
    const int k_lo = max(fast_lo - kp + (1 << lg) - 1, 0) >> lg;
    const int k_hi = max(fast_hi - kp + (1 << lg) - 1, 0) >> lg;
    const uint32_t below_hi = k_hi >= 32 ? 0xffffffffu : ((1u << k_hi) - 1u);
    const uint32_t below_lo = k_lo >= 32 ? 0xffffffffu : ((1u << k_lo) - 1u);
    fast_steps = full_keys & below_hi & ~below_lo;
  }

  // Block i, staged in stage `stage` (landed and visible).
  __device__ __forceinline__ void step(HalfState& st, const Frag<B16>& qf, int i, int stage, float c, bool fast) {
    const unsigned char* cst = ring + stage * L::kStageBytes;
    Frag<B16> kf;
    VtFrag<B16> vt;
    f32x16 s;
    if (fast) {
      // every key of the block is scored for every query of the half
      read_frags(kf, vt, fa, cst, stage);
      const f32x16 zero = {};
      s = zero;
      qk(s, kf, qf);
      st.nfull += 1;
    } else {
      uint32_t keymask;
      if (i >= src.nwin) {
        // global-column rows: key rows up to nG exist and are global (mask 2)
        const int left = src.nG - kBlockK * (i - src.nwin);
        keymask = left >= kBlockK ? 0xffffffffu : ((1u << left) - 1u);
      } else if (ktab) {
        keymask = ktab[(i - kp) >> lg];
      } else {
        keymask = table_keymask(i);  // waits for every outstanding load: wide windows only
      }
      if (keymask == 0u) return;  // no key of the block is in any key set
      const int cls = src.classify(i, keymask);
      if (cls == 0) return;
      read_frags(kf, vt, fa, cst, stage);
      const int ln = lane_id_here();
      if (keymask != 0xffffffffu) {
        // rows of keys outside every key set contribute exactly nothing, even
        // where their stored values are not finite
        zero_dead_keys(vt, keymask, ln);
        zero_dead_krow(kf, keymask, ln);
      }
      // The mask enters through the accumulators' starting values: 0 where
      // the key is scored, -inf where it is not, so the QK products come
      // out masked (-inf + finite = -inf) with no pass over the scores.
      if (cls == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        st.nfull += 1;
      } else {
        const uint32_t vmk = src.valid_bits(i) & (keymask >> (4 * (ln >> 5)));  // bit c_r: element r scored
        const uint32_t inv = ~vmk;
        // all ones where element r is not scored, then the bits of -inf
#define LF_BIAS(r) s[r] = __builtin_bit_cast(float, (uint32_t)bit_as_mask<acc_c(r)>(inv) & 0xff800000u)
        LF_BIAS(0); LF_BIAS(1); LF_BIAS(2); LF_BIAS(3); LF_BIAS(4); LF_BIAS(5); LF_BIAS(6); LF_BIAS(7);
        LF_BIAS(8); LF_BIAS(9); LF_BIAS(10); LF_BIAS(11); LF_BIAS(12); LF_BIAS(13); LF_BIAS(14); LF_BIAS(15);
#undef LF_BIAS
        st.cnt += __popc(vmk & 0x0f0f0f0fu);
      }
      qk(s, kf, qf);
    }
    PFrag<B16> pf;
    softmax_core<B16>(st, s, pf, c);
    pv(st.o, pf, vt);
  }

  // Issues, before the loop, the blocks of steps 0 .. kStages - 2 for which
  // pred(i) holds (in step order; the caller splits them around the global
  // scan, window blocks first).
  template <class Pred>
  __device__ void prime(int end, Pred pred) {
#pragma unroll
    for (int s = 0; s < L::kStages - 1; ++s) {
      const int i = (s << lg) + kp;
      if (i < end && pred(i)) issue(i, s);
    }
  }

  // Step s over block i = 2 s + kp (skipped when i >= end), in `stage`.
  __device__ __forceinline__ void one_step(HalfState& st, const Frag<B16>& qf, int s, int& stage, int end, float c,
                                           bool active) {
    const int i = 2 * s + kp;
    // this wave's share of block i has landed (the next block's may still fly)
    if (L::kStages > 2 && i + 2 < end)
      wait_vmem_but<kIssueLoads>();
    else
      wait_vmem_all();
    // ... and the other wave's share too; both waves are done reading the
    // stage of step s - 1, which the next issue refills
    block_barrier();
    const int nxt = i + 2 * (L::kStages - 1);
    if (nxt < end) issue(nxt, stage == 0 ? L::kStages - 1 : stage - 1);
    if (active && i < end) step(st, qf, i, stage, c, s < 32 && ((fast_steps >> s) & 1u));
    stage = stage == L::kStages - 1 ? 0 : stage + 1;
  }

  // Steps over blocks 2 s + kp < end; the blocks of steps 0 .. kStages - 2
  // are already issued.  `active`: the wave has rows to score (otherwise it
  // only keeps its share of the loads and the barriers going).
  __device__ void run(HalfState& st, const Frag<B16>& qf, int end, float c, bool active) {
    const int nsteps = (end + 1) >> 1;
    int stage = 0;
    for (int s = 0; s < nsteps; ++s) one_step(st, qf, s, stage, end, c, active);
  }

  // The same with after_first run in every wave once the first step is done
  // (outside the loop, so that what it uses is not held through it); it may
  // raise end, and the blocks it adds must have indices of at least
  // kp + 2 kStages, so that later steps issue them.
  template <class Hook>
  __device__ void run(HalfState& st, const Frag<B16>& qf, int end, float c, bool active, Hook after_first) {
    int stage = 0;
    one_step(st, qf, 0, stage, end, c, active);
    after_first(end);
    const int nsteps = (end + 1) >> 1;
    for (int s = 1; s < nsteps; ++s) one_step(st, qf, s, stage, end, c, active);
  }

  // Solo: this wave's blocks kp, kp + 4, ... < end through its one stage;
  // its first block is already issued.  A block's fragments are read (and
  // the reads waited for) inside step(), so the next block can be issued
  // into the same stage right after it.
  __device__ void run_solo(HalfState& st, const Frag<B16>& qf, int end, float c, bool active) {
    for (int s = 0; kp + 4 * s < end; ++s) {
      const int i = kp + 4 * s;
      wait_vmem_all();
      if (active) step(st, qf, i, 0, c, s < 32 && ((fast_steps >> s) & 1u));
      if (i + 4 < end) issue(i + 4, 0);
    }
  }
};

// ---------------------------------------------------------------------------
// Global columns of local rows when a batch row holds at most kVecGlobals
// global tokens.  Instead of a key block of their own (one more barrier
// step for every wave of the tile, for a handful of keys), the parity-0
// wave of each query half scores them after the block loop with dot
// products on the vector unit.  Their K and V rows are staged in LDS by one
// direct-to-LDS load as soon as the global list is known (after the scan),
// in the unused tail of the list: kVecBytes per query half, the K rows then
// the V rows, 2 kD bytes each.  Head dims up to 64 only (the rows of both
// halves must fit in the list's tail); larger ones take the key blocks.
// ---------------------------------------------------------------------------
constexpr int kVecGlobals = 4;
constexpr int kVecRowBytes = 2 * kD;
constexpr int kVecBytes = 2 * kVecGlobals * kVecRowBytes;
constexpr int kVecChunks = kVecRowBytes / 16;  // 16-byte chunks per row
constexpr bool kVecOk = 16 * 4 + 2 * kVecBytes <= LF_MAX_GLOBAL * 4 && kVecBytes <= 64 * 16;

__device__ __forceinline__ unsigned char* vec_rows(int* G, int qh) {
  return reinterpret_cast<unsigned char*>(G + 16) + kVecBytes * qh;
}

// Lane l < kVecBytes / 16 fetches 16-byte chunk l % kVecChunks of the K (l <
// kVecBytes / 32) or V row of global token (l / kVecChunks) % 4 (clamped to
// the last one); it lands at byte 16 l.
__device__ __forceinline__ void issue_vec_rows(const h16* kb, const h16* vb, uint32_t rs, const int* G, int nG,
                                               unsigned char* dst) {
  const int l = lane_id_here();
  if (l >= kVecBytes / 16) return;
  const int key = min((l / kVecChunks) & 3, nG - 1);
  const h16* src = ((l >= kVecBytes / 32) ? vb : kb) + (size_t)G[key] * rs + 8 * (l % kVecChunks);
  __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)dst, 16, 0, 0);
}

// Folds the global tokens G[0 .. nG) into the running state of this lane's
// query as extra keys, skipping those already in its window (they were
// scored as window keys): the same online softmax as a block step, with the
// probability rounded to bf16 as in P V.  Lanes l and l ^ 32 hold the two
// halves of the query's head dims, and each adds its half of the products.
__device__ void vec_global_columns(HalfState& st, const Frag<true>& qf, const BandSrc& src, const unsigned char* rows,
                                   float c) {
  const int lane = lane_id_here();
  const int hh = lane >> 5;
  const int tq = src.t0 + 32 * src.qh + (lane & 31);
  const int qp = src.r + src.dil * (tq < src.n_r ? tq : src.n_r - 1);
  const uint32_t span = 2u * (uint32_t)src.wd;
  for (int gi = 0; gi < src.nG; ++gi) {
    const int g = src.G[gi];
    const unsigned char* kr = rows + kVecRowBytes * gi;
    const unsigned char* vr = rows + kVecBytes / 2 + kVecRowBytes * gi;
    // q . k over this lane's kD / 2 head dims (16 s + 8 hh + [0, 8))
    float acc = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < kD / 16; ++s4) {
      const h16x8 kk = *reinterpret_cast<const h16x8*>(kr + 32 * s4 + 16 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h16x2 a = {qf.x[s4][2 * j], qf.x[s4][2 * j + 1]};
        const h16x2 bb = {kk[2 * j], kk[2 * j + 1]};
        acc = dot2h(a, bb, acc);
      }
    }
    const float sc = (acc + __shfl_xor(acc, 32)) * c;
    const int d = qp - g;
    const bool take = !((uint32_t)(d + src.wd) <= span && d % src.dil == 0);
    if (__any(take && sc > st.m + kRescaleSlack)) {
      const float mn = fmaxf(st.m, take ? sc : kNegInf);
      const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
      st.m = mn;
      st.thr = (mn + kRescaleSlack) / c;
      st.l *= alpha;
#pragma unroll
      for (int db = 0; db < kND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    }
    const float pr = take ? (float)(h16)__builtin_amdgcn_exp2f(sc - st.m) : 0.f;
    if (hh == 0) {
      st.l += pr;
      st.cnt += take ? 1 : 0;
    }
    // O^T element r of dim block db: head dim 32 db + 8 (r / 4) + 4 hh + r % 4
#pragma unroll
    for (int db = 0; db < kND; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const h16x4 vv = *reinterpret_cast<const h16x4*>(vr + 2 * (32 * db + 8 * g4 + 4 * hh));
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[db][4 * g4 + i] = __builtin_fmaf(pr, (float)vv[i], st.o[db][4 * g4 + i]);
      }
  }
}

// ---------------------------------------------------------------------------
// Band workgroup: one tile of kTileQ = 64 query rows t0 .. t0 + 63 of the
// residue sequence r of (b, h).  Its key blocks (window span, then the
// global columns) alternate between the two key parities; each wave scores
// its query half against its parity's blocks, and the two partials of each
// half are merged at the end.  Writes local rows (mask 1) and zero rows
// (mask 0).
// ---------------------------------------------------------------------------
template <bool B16>
__device__ void band_tile(const KernelParams& p, int L, Shared<B16>& sh) {
  using T = elem_t<B16>;
  using Ly = Lay<B16>;
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qh = wv & 1, kp = wv >> 1;

  const int b = L / p.tiles_per_b;
  const int rem = L - b * p.tiles_per_b;
  int h, id, dil;
  if (p.uni_dil > 0 && p.tiles_per_head > 0) {
    // every head has the same dilation and tile count: no table lookups
    h = rem / p.tiles_per_head;
    id = rem - h * p.tiles_per_head;
    dil = p.uni_dil;
  } else {
    // head: tile0 is non-decreasing; count entries <= rem, 8 loads per round
    h = 0;
    for (int k0 = 1; k0 < p.H; k0 += 8) {
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) cnt += (k0 + k < p.H && p.tile0[k0 + k] <= rem) ? 1 : 0;
      h += cnt;
      if (cnt < 8) break;
    }
    id = rem - p.tile0[h];
    dil = p.dil[h];
  }
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
  const uint32_t rs = (uint32_t)p.H * kD;  // elements between tokens
  const size_t head = (size_t)b * n * rs + (size_t)h * kD;
  const T* qbase = reinterpret_cast<const T*>(p.q) + head;
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
  src.t0 = t0;
  src.qh = qh;
  src.w = w;
  src.w_hi = w_hi;
  src.wd = w * dil;

  ScanPre sp;
  const MaskRow mr = mask_row(p.mask, p.B, n, b);
  if (p.use_globals) scan_preload(sp, mr, n);
  // Mask bytes of both halves' query rows (every wave sees the whole tile,
  // so the early-exit test below agrees across the workgroup).
  int qm[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int tq = t0 + 32 * nb + (lane & 31);
    qm[nb] = tq < n_r ? mrow[r + dil * tq] : 0;
  }
  Frag<B16> qf;
  load_frag(qf, qbase + (size_t)src.qpos() * rs, hh);
  HalfLoop<B16, BandSrc> loop(src, reinterpret_cast<const T*>(p.k) + head, reinterpret_cast<const T*>(p.v) + head,
                              rs, sh.buf + kp * Ly::kRingBytes, n, kp, qh);
  // validity bytes of the wave's window blocks, then its first window
  // blocks: all of them fly during the scan
  loop.tab_load();
  const int nwin = src.nwin;
  loop.prime(nwin, [](int) { return true; });

  bool is_local[2], is_zero[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const bool inq = t0 + 32 * nb + (lane & 31) < n_r;
    bool loc, glo;
    if (p.use_globals) {
      loc = qm[nb] == 1;
      glo = qm[nb] == 2;
    } else {
      loc = qm[nb] == 1 || qm[nb] == 2;
      glo = false;
      if (nb == qh && kp == 0 && qm[nb] == 2 && !causal && p.max_global == 0)
        atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
    }
    is_local[nb] = inq && loc;
    is_zero[nb] = inq && !loc && !glo;
  }
  const bool my_local = qh ? is_local[1] : is_local[0];
  const bool my_zero = qh ? is_zero[1] : is_zero[0];
  // a tile with no local row (padding, or only global rows) writes its
  // zero rows and stops here, before the table and the global scan
  if (!__any(is_local[0] || is_local[1])) {
    wait_vmem_all();  // the primed loads land before the workgroup's LDS is released
    if (my_zero) {
      const int qp = src.qpos();
      store_quadrant<B16>(out + (size_t)qp * rs, kp, hh, nullptr, 0.f, true);
      if (p.row_nnz && kp == 0 && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qp] = 0;
      if (p.lse && kp == 0 && hh == 0) p.lse[((size_t)b * p.H + h) * n + qp] = kNegInf;
    }
    return;
  }

  loop.tab_commit(sh.ktab[wv]);

  const bool active = __any(my_local);
  unsigned char* vrows = vec_rows(sh.G, qh);
  bool vec_g = false;
  // The global list: the scan, then the global-column work it implies.  A
  // few global tokens go to the vector unit after the loop (their K and V
  // rows are staged now), more of them into key blocks of their own after
  // the window blocks.  Returns the block count.
  auto globals = [&]() -> int {
    int nG = scan_globals(sp, mr, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
    if (nG > p.max_global) {
      if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
      nG = p.max_global;
    }
    src.nG = __builtin_amdgcn_readfirstlane(nG);  // uniform (the status write above diverges)
    vec_g = B16 && kVecOk && src.nG > 0 && src.nG <= kVecGlobals;
    if constexpr (B16 && kVecOk) {
      if (vec_g && kp == 0 && active)
        issue_vec_rows(reinterpret_cast<const h16*>(p.k) + head, reinterpret_cast<const h16*>(p.v) + head, rs,
                       sh.G, src.nG, vrows);
    }
    return nwin + (vec_g ? 0 : (src.nG + kBlockK - 1) / kBlockK);
  };
  // With enough window blocks the scan runs after the first block step (its
  // mask bytes have landed by then, and the next blocks' loads fly during
  // it): no global-column block is due before the third step.
  const bool late_scan = p.use_globals && nwin >= 2 * Ly::kStages;
  if (p.use_globals) scan_ready(sp, n);
  int end = nwin;
  if (p.use_globals && !late_scan) {
    end = globals();
    // first blocks that are global-column blocks go after the scan
    loop.prime(end, [&](int i) { return i >= nwin; });
  }

  HalfState st;
  state_init(st);
  __builtin_amdgcn_s_setprio(0);
  if (late_scan) {
    loop.run(st, qf, end, p.c, active, [&](int& e) {
      __builtin_amdgcn_s_setprio(2);
      e = globals();
      __builtin_amdgcn_s_setprio(0);
    });
  } else {
    loop.run(st, qf, end, p.c, active);
  }
  __builtin_amdgcn_s_setprio(2);
  if constexpr (B16 && kVecOk) {
    if (vec_g && kp == 0 && active) vec_global_columns(st, qf, src, vrows, p.c);
  }
  merge_parities<B16>(st, sh, qh, kp, [&](int db, float M, float Lsum, int cnt, const float* o) {
    if (!my_local && !my_zero) return;
    const int qp = src.qpos();
    store_quadrant<B16>(out + (size_t)qp * rs, db, hh, o, my_local ? 1.0f / Lsum : 0.f, !my_local);
    if (p.row_nnz && db == 0 && hh == 0) p.row_nnz[((size_t)b * p.H + h) * n + qp] = my_local ? cnt : 0;
    if (p.lse && db == 0 && hh == 0)
      p.lse[((size_t)b * p.H + h) * n + qp] = my_local ? row_lse(M, Lsum) : kNegInf;
  });
}

// Partial record of one (global token, split): merged max, row sum, key
// count, then the unnormalised outputs in head-dim order; this lane writes
// head dims odim(kHalfO part + u, hh) from o[u].
__device__ __forceinline__ void write_record(float* rec, int part, int hh, float M, float Lsum, int cnt,
                                             const float* o) {
  if (part == 0 && hh == 0) {
    st_agent(rec, M);
    st_agent(rec + 1, Lsum);
    st_agent(rec + 2, __builtin_bit_cast(float, cnt));
  }
  float* dst = rec + 4 + (kD / 2) * part + 4 * hh;
#pragma unroll
  for (int g = 0; g < kHalfO / 4; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) st_agent(dst + odim(4 * g, 0) + e, o[4 * g + e]);
}

// Second merge round of a solo split (below): waves (0, kp) and (1, kp)
// hold merged results of head-dim half kp for the same query slots over
// disjoint key sets.  Wave (1, kp) parks its (M, L, count, outputs) past
// the first round's parked states; after a barrier wave (0, kp) combines,
// its own terms first, and passes the result to emit(M, L, cnt, o).
constexpr int kRound2Off = kWaves * kParkBytes;

template <bool B16, class Emit>
__device__ void merge_halves(Shared<B16>& sh, int qh, int kp, float M, float L, int cnt, const float* o, Emit emit) {
  static_assert(kRound2Off + 2 * kParkBytes <= Shared<B16>::kBufBytes, "second-round park fits the buffer");
  const int lane = lane_id();
  const int q = lane & 31;
  unsigned char* r2 = sh.buf + kRound2Off + kp * kParkBytes;
  f32x4* po = reinterpret_cast<f32x4*>(r2);
  float* pm = reinterpret_cast<float*>(r2 + kParkOBytes);
  if (qh == 1) {
#pragma unroll
    for (int g = 0; g < kHalfO / 4; ++g)
      po[g * 64 + lane] = f32x4{o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]};
    if ((lane >> 5) == 0) {
      pm[lane] = M;
      pm[32 + lane] = L;
      reinterpret_cast<int*>(pm + 64)[lane] = cnt;
    }
  }
  __syncthreads();
  if (qh == 1) return;
  const float mb = pm[q], lb = pm[32 + q];
  const int c = cnt + reinterpret_cast<const int*>(pm + 64)[q];
  const float Mm = fmaxf(M, mb);
  const float fa = __builtin_amdgcn_exp2f(M - Mm);
  const float fb = __builtin_amdgcn_exp2f(mb - Mm);
  const float Lm = L * fa + lb * fb;
  float om[kHalfO];
#pragma unroll
  for (int g = 0; g < kHalfO / 4; ++g) {
    const f32x4 y = po[g * 64 + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) om[4 * g + e] = __builtin_fmaf(o[4 * g + e], fa, y[e] * fb);
  }
  emit(Mm, Lm, c, om);
}

// ---------------------------------------------------------------------------
// Global-row workgroup: split c of (b, h); all global tokens of b, 64 at a
// time (two query halves).  When a batch row holds at most 32 global tokens
// (one query half) the split runs solo: all four waves score the same 32
// query slots, each over its own quarter of the split's blocks (blocks w,
// w + 4, ...) in an 8 KB stage of its own.  The split's work then spreads
// over the four SIMDs instead of two, and its loop needs no barrier; the
// four partials are merged in two rounds (key parities, then the halves).
// ---------------------------------------------------------------------------
template <bool B16>
__device__ void global_split(const KernelParams& p, int gid, Shared<B16>& sh) {
  using T = elem_t<B16>;
  using Ly = Lay<B16>;
  const int lane = lane_id();
  const int hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qh = wv & 1, kp = wv >> 1;
  const int S = p.S;
  const int bh = gid / S;
  const int cidx = gid - bh * S;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int n = p.n;
  const int8_t* mrow = p.mask + (size_t)b * n;

  const uint32_t rs = (uint32_t)p.H * kD;
  const size_t head = (size_t)b * n * rs + (size_t)h * kD;
  const T* qg = reinterpret_cast<const T*>(p.qg) + head;
  ChunkSrc src;
  src.mrow = mrow;
  src.cbeg = cidx * p.chunk;
  src.cend = min(n, src.cbeg + p.chunk);
  src.nwin = (src.cend - src.cbeg + kBlockK - 1) / kBlockK;
  src.nG = 0;
  const int nblk = src.nwin;
  const float c = p.c;
  float* part_bh = p.partials + (size_t)bh * p.max_global * S * kPartialStride;
  ScanPre sp;
  const MaskRow mr = mask_row(p.mask, p.B, n, b);
  // solo split: one query half of slots, four owners of blocks
  const bool solo = B16 && p.max_global <= 32;
  HalfLoop<B16, ChunkSrc> loop(src, reinterpret_cast<const T*>(p.kg) + head,
                               reinterpret_cast<const T*>(p.vg) + head, rs,
                               solo ? sh.buf + wv * Ly::kStageBytes : sh.buf + kp * Ly::kRingBytes, n, solo ? wv : kp,
                               qh, solo);
  scan_preload(sp, mr, n);
  loop.tab_load();
  loop.prime(nblk, [](int) { return true; });  // the split's keys do not depend on the scan
  loop.tab_commit(sh.ktab[wv]);

  scan_ready(sp, n);
  int nG = scan_globals(sp, mr, n, sh.G, LF_MAX_GLOBAL, sh.wave_tmp);
  if (nG > p.max_global) {
    if (threadIdx.x == 0) atomicOr(p.status, LF_DEV_TOO_MANY_GLOBALS);
    nG = p.max_global;
  }
  nG = __builtin_amdgcn_readfirstlane(nG);  // uniform (the status write above diverges)
  if (nG == 0) {
    wait_vmem_all();
    return;
  }

  if (solo) {
    const int gi = lane & 31;
    Frag<B16> qf;
    load_frag(qf, qg + (size_t)sh.G[gi < nG ? gi : nG - 1] * rs, hh);
    HalfState st;
    state_init(st);
    __builtin_amdgcn_s_setprio(0);
    loop.run_solo(st, qf, nblk, c, true);
    __builtin_amdgcn_s_setprio(2);
    float M1 = 0.f, L1 = 0.f, o1[kHalfO];
    int c1 = 0;
    merge_parities<B16>(st, sh, qh, kp, [&](int, float M, float Lsum, int cnt, const float* o) {
      M1 = M;
      L1 = Lsum;
      c1 = cnt;
#pragma unroll
      for (int r = 0; r < kHalfO; ++r) o1[r] = o[r];
    });
    merge_halves<B16>(sh, qh, kp, M1, L1, c1, o1, [&](float M, float Lsum, int cnt, const float* o) {
      if (gi < nG) write_record(part_bh + ((size_t)gi * S + cidx) * kPartialStride, kp, hh, M, Lsum, cnt, o);
    });
  } else {
    for (int g0 = 0; g0 < nG; g0 += kTileQ) {
      if (g0 > 0) loop.prime(nblk, [](int) { return true; });  // after the previous group's last barrier
      const int gi = g0 + 32 * qh + (lane & 31);
      Frag<B16> qf;
      load_frag(qf, qg + (size_t)sh.G[gi < nG ? gi : nG - 1] * rs, hh);
      HalfState st;
      state_init(st);
      __builtin_amdgcn_s_setprio(0);
      loop.run(st, qf, nblk, c, g0 + 32 * qh < nG);
      __builtin_amdgcn_s_setprio(2);
      merge_parities<B16>(st, sh, qh, kp, [&](int db, float M, float Lsum, int cnt, const float* o) {
        if (gi < nG) write_record(part_bh + ((size_t)gi * S + cidx) * kPartialStride, db, hh, M, Lsum, cnt, o);
      });
      __syncthreads();  // the parked states are read before the rings are refilled
    }
  }

  // Arrival: the last split of (b, h) merges all partials.  Every thread's
  // record stores have completed (at the coherence point) before the
  // barrier that precedes the ticket increment.  The hardware guarantee
  // this rests on: an agent-scope store is written through the XCD's L2 to
  // the device coherence point, and the vector-memory counter counts a
  // store down only when the memory system acknowledges it there; so after
  // each thread's vmcnt(0) and the barrier, every record of this split is
  // visible to agent-scope loads from any XCD before the relaxed ticket
  // increment is issued.  The last arriver's agent-scope loads read the
  // coherence point, not a stale L2 line.  (A release/acquire fence pair
  // would give the same order, at the cost of writing back the whole L2.)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmem_all();
  __syncthreads();
  if (wv == 0 && lane_id_here() == 0) {
    const int t = __hip_atomic_fetch_add(p.tickets + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = (t == S - 1);
  }
  __syncthreads();
  if (!sh.flag) return;

  // Merge: a group of kD / 4 lanes per global token, each lane four head
  // dims; every split's record of the token is loaded before any is used
  // (the agent-scope loads go to the coherence point, so the merge is bound
  // by how many of them are in flight).
  T* out = reinterpret_cast<T*>(p.out) + head;
  const uint32_t tid = 64u * (uint32_t)wv + (uint32_t)lane_id_here();
  constexpr uint32_t kLanesPerTok = kD / 4;
  const int q4 = (int)(tid % kLanesPerTok);
  for (int gj = (int)(tid / kLanesPerTok); gj < nG; gj += kThreads / kLanesPerTok) {
    // online log-sum-exp merge of the S partials, 8 at a time
    const float* recs = part_bh + (size_t)gj * S * kPartialStride;
    float M = kNegInf, Lsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int cnt = 0;
    for (int s0 = 0; s0 < S; s0 += 8) {
      float ms[8], ls[8], os[8][4];
      int cs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* rec = recs + (size_t)min(s0 + j, S - 1) * kPartialStride;
        ms[j] = ld_agent(rec);
        ls[j] = ld_agent(rec + 1);
        cs[j] = __builtin_bit_cast(int, ld_agent(rec + 2));
#pragma unroll
        for (int e = 0; e < 4; ++e) os[j][e] = ld_agent(rec + 4 + 4 * q4 + e);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (s0 + j >= S) break;
        const float mn = fmaxf(M, ms[j]);
        const float fa = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - mn);
        const float fb = (ms[j] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms[j] - mn);
        M = mn;
        Lsum = Lsum * fa + ls[j] * fb;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = acc[e] * fa + os[j][e] * fb;
        cnt += cs[j];
      }
    }
    const int pos = sh.G[gj];
    const float inv = 1.0f / Lsum;
    float v4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v4[e] = acc[e] * inv;
    store4<B16>(out + (size_t)pos * rs + 4 * q4, v4);
    if (p.row_nnz && q4 == 0) p.row_nnz[(size_t)bh * n + pos] = cnt;
    if (p.lse && q4 == 0) p.lse[(size_t)bh * n + pos] = row_lse(M, Lsum);
  }
  __syncthreads();
  if (wv == 0 && lane_id_here() == 0) __hip_atomic_store(p.tickets + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool B16>
__device__ __forceinline__ void fwd_body(const KernelParams& p) {
  __shared__ Shared<B16> sh;
  const int bid = blockIdx.x;
  // Prologues and epilogues are chains of dependent loads, scans and
  // barriers; they run at a raised wave priority so that a workgroup that
  // starts next to others already in their block loops gets through them
  // quickly.  The block loops run at normal priority.
  __builtin_amdgcn_s_setprio(2);
  // Order of the two kinds in the grid: when the whole launch is resident
  // at once (the host then chose the short split chunk) the splits come
  // last, so that their loads queue behind the band tiles' first blocks;
  // otherwise first, so that their merge is not left to the last round.
  const bool splits_last = p.chunk == kGlobalChunkShort;
  const int first_band = splits_last ? 0 : p.n_glob;
  if (bid < first_band || bid >= first_band + p.n_band) {
    global_split<B16>(p, bid - (splits_last ? p.n_band : 0), sh);
    return;
  }
  band_tile<B16>(p, xcd_remap(bid - first_band, p.n_band), sh);
}

// Waves per SIMD: four workgroups (16 waves) per CU at head dims up to 64
// (at most 128 VGPRs, under 40 KB of LDS at D = 64); two at D = 128, whose
// rings take 64 KB of LDS and whose fragments and accumulators twice the
// registers.
#if LF_KD == 128
#define LF_WAVES_PER_EU 2
#else
#define LF_WAVES_PER_EU 4
#endif

#if LF_HALF_F16
// f16: the 16-bit kernel built for f16 elements.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(LF_WAVES_PER_EU))) void lf_attn_fwd_f16(
    const KernelParams p) {
  fwd_body<true>(p);
}
#else
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(LF_WAVES_PER_EU))) void lf_attn_fwd_bf16(
    const KernelParams p) {
  fwd_body<true>(p);
}

// fp32: larger operand fragments and stages.
__global__ __launch_bounds__(kThreads) void lf_attn_fwd_f32(const KernelParams p) { fwd_body<false>(p); }
#endif

}  // namespace

// Workgroups of one kernel that the current device holds at once (cached
// per device; devices past the 32nd are asked every time), or 0.
static int64_t resident_of(const void* kernel, std::atomic<int64_t>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 32) {
    const int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, 0) != hipSuccess) return 0;
  const int64_t r = (int64_t)cus * per;
  if (dev < 32) cache[dev].store(r, std::memory_order_relaxed);  // concurrent first calls store the same value
  return r;
}

#if LF_HALF_F16
int64_t resident_f16() {
  static std::atomic<int64_t> cache[32];
  return resident_of(reinterpret_cast<const void*>(lf_attn_fwd_f16), cache);
}

int launch_f16(const KernelParams& kp, void* stream) {
  hipLaunchKernelGGL(lf_attn_fwd_f16, dim3(kp.n_band + kp.n_glob), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), kp);
  return (int)hipGetLastError();
}
#else
int64_t resident(int dtype) {
  static std::atomic<int64_t> cache_bf16[32], cache_f32[32];
  return dtype == LF_BF16 ? resident_of(reinterpret_cast<const void*>(lf_attn_fwd_bf16), cache_bf16)
                          : resident_of(reinterpret_cast<const void*>(lf_attn_fwd_f32), cache_f32);
}

int launch(const KernelParams& kp, int dtype, void* stream) {
  const int grid = kp.n_band + kp.n_glob;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == LF_BF16)
    hipLaunchKernelGGL(lf_attn_fwd_bf16, dim3(grid), dim3(kThreads), 0, s, kp);
  else
    hipLaunchKernelGGL(lf_attn_fwd_f32, dim3(grid), dim3(kThreads), 0, s, kp);
  return (int)hipGetLastError();
}
#endif

}  // namespace LF_CAT(d, LF_KD)

#if !LF_HALF_F16 && LF_KD == 64
// The forward of head dim D and element type dtype (the units of each head
// dim are declared in lf_attn_internal.h).
int launch_forward(const KernelParams& kp, int dtype, int D, void* stream) {
  switch (D) {
    case 32: return dtype == LF_F16 ? d32::launch_f16(kp, stream) : d32::launch(kp, dtype, stream);
    case 64: return dtype == LF_F16 ? d64::launch_f16(kp, stream) : d64::launch(kp, dtype, stream);
    case 128: return dtype == LF_F16 ? d128::launch_f16(kp, stream) : d128::launch(kp, dtype, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

int64_t resident_workgroups(int dtype, int D) {
  switch (D) {
    case 32: return dtype == LF_F16 ? d32::resident_f16() : d32::resident(dtype);
    case 64: return dtype == LF_F16 ? d64::resident_f16() : d64::resident(dtype);
    case 128: return dtype == LF_F16 ? d128::resident_f16() : d128::resident(dtype);
    default: return 0;
  }
}
#endif

}  // namespace lf
