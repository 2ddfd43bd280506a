// Input projections of the Longformer attention layer on gfx950: the
// sliding-window projections Q_s, K_s, V_s and the separate global ones
// Q_g, K_g, V_g (segmentfault Longformer summary, "Linear projections for
// global attention") as one stacked linear map of the hidden states,
//   y[p][m][c] = sum_k x[m][k] w[p*C + c][k] + bias[p*C + c],
// with w in the [out features, in features] layout.  Each y[p], viewed as
// [B, n, H, D] with C = H * D, is one input of the attention kernels.
//
// One launch, one dense MFMA GEMM over the stacked output features
// n = p*C + c: D[n][m] = sum_k w[n][k] x[m][k].  Both operands are
// contiguous along the reduction, the operand layout of the 32x32x16 MFMA
// for its A (a row of w) and B (a row of x) inputs.
//
// Tiles of BM tokens x BN features, one per workgroup, in one of four
// configurations chosen per launch (the one whose busiest CU has the least
// work, tiles weighted by the bytes they stage per MFMA): 128 x 128 and
// 128 x 192 with four waves (two workgroups per CU), 256 x 288 with eight
// waves of 32 x 288 and 256 x 256 with eight waves of 128 x 64 (one
// workgroup per CU).  Each wave holds its share of
// the tile as 32 x 32 fp32 accumulators.  The reduction runs in steps of 64
// (one 128-byte line of every row) through two LDS stages: each step's
// rows are loaded into registers a step ahead (16 bytes per lane, whole
// lines per wave) and written to the LDS stage of the next step once the
// current one has been multiplied, so that every load has a full step to
// land.  Consecutive tiles on one XCD form blocks of 8 token tiles by the
// feature tiles, so that the tiles resident on one L2 share x and w rows.
//
// Projections flagged as needed at global tokens only (the global query
// projection, whose rows other than the global tokens' the attention never
// reads) are written as zero at the other tokens, and a tile of such
// features with no global token skips its reduction.
//
// The epilogue adds the bias in fp32, rounds to the element type (nearest
// even), regroups each lane's values with its partner 32 lanes away so
// that every lane holds eight consecutive features of one token, and
// writes them as 16-byte stores.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "lf_proj_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowB = 128;  // staged bytes of a row per reduction step (64 elements)

// Layout of one LDS stage: the x rows of the tile (BM x 128 B), then its w
// rows (BN x 128 B).  Every row holds eight 16-byte chunks; chunk c of row
// r sits at slot c ^ swz(r), swz(r) = (r / 2) mod 8.  Two rows share one
// 256-byte bank span, so the 16 rows that a quarter-wave reads at one chunk
// index (rows r0 .. r0 + 15, r0 a multiple of 16) land on 16 distinct
// 16-byte slots: conflict-free fragment reads.
//
// A tile of BM tokens x BN features is computed by WM x WN waves, wave
// (wm, wn) owning BM/WM tokens x BN/WN features: MT x NT MFMA tiles of
// 32 x 32.
template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int MT = BM / WM / 32, NT = BN / WN / 32;
  static_assert(MT * 32 * WM == BM && NT * 32 * WN == BN, "whole MFMA tiles per wave");
  static constexpr int kABytes = BM * kRowB;
  static constexpr int kStageBytes = kABytes + BN * kRowB;
  static constexpr int kALoads = BM / 8;  // 1 KB wave loads (8 rows) per step: x rows
  static constexpr int kBLoads = BN / 8;  // ... w rows
  // loads per wave (the last ones only by the first waves when the count
  // does not divide)
  static constexpr int kALoadsW = (kALoads + kWaves - 1) / kWaves;
  static constexpr int kBLoadsW = (kBLoads + kWaves - 1) / kWaves;
  // workgroups per CU (two stages of LDS each, 160 KB per CU)
  static constexpr int kPerCU = 163840 / (2 * kStageBytes) >= 2 ? 2 : 1;
};
// 128 x 192 and 128 x 128 for launches with few tiles (two workgroups per
// CU); 256 x 288 (eight waves of 32 x 288, one workgroup per CU) for large
// ones: 40 % fewer bytes staged per MFMA than 128 x 192.  256 x 256 with
// eight waves of 128 x 64 reads a third fewer fragment bytes from LDS per
// MFMA than 256 x 288 (six 1 KB reads per eight MFMAs against ten per
// nine); the chooser takes it where it needs no more rounds of tiles than
// 256 x 288 (feature counts that are multiples of 256).
using TileS = Tile<128, 128, 2, 2>;
using TileM = Tile<128, 192, 2, 2>;
using TileL = Tile<256, 288, 8, 1>;
using TileX = Tile<256, 256, 2, 4>;

template <class T>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (__is_same(T, _Float16)) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
}

// Buffer resource over `bytes` bytes of `base`: loads at offsets beyond it
// return 0, which pads the tiles past the last token and the last feature.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup barrier after this wave's LDS writes have completed; loads in
// flight are not waited for (no memory fences: the asm keeps memory
// accesses on their side).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Tile t of the launch for workgroup `bid`.  Workgroups are dealt to the 8
// XCDs in turn; each XCD is given a contiguous range of tile indices, and
// an index runs over groups of 8 token tiles, the token tile fastest, so
// that the tiles resident on one XCD at a time cover a block of about 8
// token tiles by 8 feature tiles.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& mt, int& nt) {
  const int ntiles = tiles_m * tiles_n;
  const int per = ntiles / 8, rem = ntiles % 8;
  const int xcd = bid % 8, y = bid / 8;
  const int t = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + y;
  constexpr int kGroup = 8;
  const int g = t / (kGroup * tiles_n), r = t - g * (kGroup * tiles_n);
  const int gm = min(kGroup, tiles_m - g * kGroup);
  mt = g * kGroup + r % gm;
  nt = r / gm;
}

template <class T, class Ly>
__device__ void proj_body(const ProjParams& p) {
  constexpr int BM = Ly::BM, BN = Ly::BN, MT = Ly::MT, NT = Ly::NT;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * Ly::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % Ly::WM, wn = wv / Ly::WM;
  const int M = p.M, C = p.C, N = p.N;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, tiles_m, tiles_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const uint32_t rowb = (uint32_t)C * 2u;
  const int steps = C / 64;

  // Projections needed at global tokens only: a tile whose features all
  // belong to such projections and whose tokens hold no global one only
  // writes zeros.
  bool skip = false;
  if (p.global_only) {
    const int plo = n0 / C, phi = (min(n0 + BN, N) - 1) / C;
    bool all = true;
    for (int q = plo; q <= phi; ++q) all = all && ((p.global_only >> q) & 1u);
    if (all) {
      // every wave scans all of the tile's tokens itself: no barrier
      bool any = false;
      for (int r = lane; r < BM; r += 64) any = any || (m0 + r < M && p.mask[m0 + r] == 2);
      skip = !__any(any);
    }
  }

  // Loads: wave wv stages x rows [8 j, 8 j + 8) for j = wv + kWaves u <
  // BM / 8 and the same w rows below BN.  Lane l of load j takes chunk
  // l % 8 of tile row 8 j + l / 8 (one 16-byte load; a wave covers eight
  // whole 128-byte lines) and writes it to slot (l % 8) ^ swz(row),
  // swz(row) = (4 j + l / 16) mod 8 = 4 (j mod 2) + l / 16.  Row offsets go
  // into the per-lane offset, where the buffer's bound check sees them.
  // The loads of step s + 2 are issued at the end of step s, after the
  // registers have been written to the LDS stage of step s + 1, so each
  // load has a whole step to land.
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, (uint32_t)M * rowb);
  const __amdgpu_buffer_rsrc_t rw = rsrc(p.w, (uint32_t)N * rowb);
  uint32_t offa[Ly::kALoadsW], offb[Ly::kBLoadsW], lda[Ly::kALoadsW], ldb[Ly::kBLoadsW];
#pragma unroll
  for (int u = 0; u < Ly::kALoadsW; ++u) {
    const int j = wv + Ly::kWaves * u;
    offa[u] = (uint32_t)(m0 + 8 * j + (lane >> 3)) * rowb + 16u * (uint32_t)(lane & 7);
    lda[u] = (uint32_t)((8 * j + (lane >> 3)) * kRowB + 16 * ((lane & 7) ^ (((j & 1) << 2) | (lane >> 4))));
  }
#pragma unroll
  for (int u = 0; u < Ly::kBLoadsW; ++u) {
    const int j = wv + Ly::kWaves * u;
    offb[u] = (uint32_t)(n0 + 8 * j + (lane >> 3)) * rowb + 16u * (uint32_t)(lane & 7);
    ldb[u] = (uint32_t)(Ly::kABytes + (8 * j + (lane >> 3)) * kRowB +
                        16 * ((lane & 7) ^ (((j & 1) << 2) | (lane >> 4))));
  }
  u32x4 ra[Ly::kALoadsW], rb[Ly::kBLoadsW];
  auto load = [&](int step) {
    const int so = step * kRowB;
#pragma unroll
    for (int u = 0; u < Ly::kALoadsW; ++u)
      if (wv + Ly::kWaves * u < Ly::kALoads) ra[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)offa[u], so, 0);
#pragma unroll
    for (int u = 0; u < Ly::kBLoadsW; ++u)
      if (wv + Ly::kWaves * u < Ly::kBLoads) rb[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)offb[u], so, 0);
  };
  auto store = [&](int stage) {
    unsigned char* st = smem + stage * Ly::kStageBytes;
#pragma unroll
    for (int u = 0; u < Ly::kALoadsW; ++u)
      if (wv + Ly::kWaves * u < Ly::kALoads) *reinterpret_cast<u32x4*>(st + lda[u]) = ra[u];
#pragma unroll
    for (int u = 0; u < Ly::kBLoadsW; ++u)
      if (wv + Ly::kWaves * u < Ly::kBLoads) *reinterpret_cast<u32x4*>(st + ldb[u]) = rb[u];
  };

  // Fragment reads: lane l reads row l % 32 of each MFMA tile at chunk
  // 2 ks + l / 32, in slot chunk ^ ((l / 2) % 8) (the tiles' first rows are
  // multiples of 16, so the swizzle is the lane's); tiles are 4096 bytes
  // apart.
  const int r32 = lane & 31, hl = lane >> 5, sw = (lane >> 1) & 7;
  const int rowa = (wm * (BM / Ly::WM) + r32) * kRowB;
  const int rowbb = Ly::kABytes + (wn * (BN / Ly::WN) + r32) * kRowB;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // the tile's bias, loaded during the last step and staged in LDS for the
  // epilogue (threads t < BN / 4 take features n0 + 4 t .. + 3)
  float4 bias4 = {0.f, 0.f, 0.f, 0.f};
  const bool bias_lane = p.bias && tid < BN / 4 && n0 + 4 * tid < N;

  if (!skip) {
  load(0);
  store(0);
  if (steps > 1) load(1);
  lds_barrier();
  for (int s = 0; s < steps; ++s) {
    if (s == steps - 1 && bias_lane) bias4 = *reinterpret_cast<const float4*>(p.bias + n0 + 4 * tid);
    const unsigned char* st = smem + (s & 1) * Ly::kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cb = 16 * ((2 * ks + hl) ^ sw);
      u32x4 fa[MT], fb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *reinterpret_cast<const u32x4*>(st + rowa + 4096 * i + cb);
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[j] = *reinterpret_cast<const u32x4*>(st + rowbb + 4096 * j + cb);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mma<T>(fb[j], fa[i], acc[i][j]);
    }
    if (s + 1 < steps) {
      // the other stage was last read in step s - 1, before the barrier
      // that ended it
      store((s + 1) & 1);
      if (s + 2 < steps) load(s + 2);
    }
    // the stage of step s + 1 is written and visible; every wave is done
    // reading the stage of step s (the bias staging below reuses it)
    lds_barrier();
  }
  }
  float* bias_lds = reinterpret_cast<float*>(smem + (steps & 1) * Ly::kStageBytes);
  if (!skip) {
    if (bias_lane) *reinterpret_cast<float4*>(bias_lds + 4 * tid) = bias4;
    lds_barrier();
  }

  // Epilogue.  Lane (c, h) = (l % 32, l / 32) of tile (i, j) holds token
  // m0 + wm BM/WM + 32 i + c and features f0 + 8 g + 4 h + e in acc[4 g + e]
  // (f0 = n0 + wn BN/WN + 32 j).  After rounding, each pair of registers
  // (g, g + 1), g even, is swapped across the two lane halves (the upper
  // half of the first with the lower half of the second), which leaves lane
  // (c, h) with features f0 + 16 (g / 2) + 8 h + [0, 8): one 16-byte store.
  T* out = reinterpret_cast<T*>(p.out);
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int f0 = n0 + wn * (BN / Ly::WN) + 32 * j;
    if (f0 >= N) continue;  // N is a multiple of 64: a 32-feature tile is all in or all out
    float4 bv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bv[g] = p.bias && !skip ? *reinterpret_cast<const float4*>(bias_lds + (f0 - n0) + 8 * g + 4 * h)
                              : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      uint32_t pk[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float b0 = e ? bv[g].z : bv[g].x, b1 = e ? bv[g].w : bv[g].y;
          const T lo = (T)(acc[i][j][4 * g + 2 * e] + b0);
          const T hi = (T)(acc[i][j][4 * g + 2 * e + 1] + b1);
          pk[g][e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
#pragma unroll
      for (int g = 0; g < 4; g += 2)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(pk[g][e], pk[g + 1][e], false, false);
          pk[g][e] = r[0];
          pk[g + 1][e] = r[1];
        }
      const int m = m0 + wm * (BM / Ly::WM) + 32 * i + c;
      if (m < M) {
        const bool global_row = p.global_only && p.mask[m] == 2;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int f = f0 + 16 * q + 8 * h;
          const int proj = f / C, col = f - proj * C;
          const bool zero = skip || (((p.global_only >> proj) & 1u) && !global_row);
          *reinterpret_cast<u32x4*>(out + ((size_t)proj * M + m) * C + col) =
              zero ? u32x4{0u, 0u, 0u, 0u} : u32x4{pk[2 * q][0], pk[2 * q][1], pk[2 * q + 1][0], pk[2 * q + 1][1]};
        }
      }
    }
  }
}

#define LF_PROJ_KERNELS(NAME, TL)                                                                              \
  __global__ __launch_bounds__(TL::kThreads) __attribute__((amdgpu_waves_per_eu(2))) void NAME##_bf16(       \
      const ProjParams p) {                                                                                    \
    proj_body<__bf16, TL>(p);                                                                                  \
  }                                                                                                            \
  __global__ __launch_bounds__(TL::kThreads) __attribute__((amdgpu_waves_per_eu(2))) void NAME##_f16(        \
      const ProjParams p) {                                                                                    \
    proj_body<_Float16, TL>(p);                                                                                \
  }
LF_PROJ_KERNELS(lf_proj_s, TileS)
LF_PROJ_KERNELS(lf_proj_m, TileM)
LF_PROJ_KERNELS(lf_proj_l, TileL)
LF_PROJ_KERNELS(lf_proj_x, TileX)
#undef LF_PROJ_KERNELS

template <class Ly>
long long tiles_of(int M, int N) {
  return (long long)((M + Ly::BM - 1) / Ly::BM) * ((N + Ly::BN - 1) / Ly::BN);
}

// Relative cost of a launch: the tiles are spread evenly over the CUs,
// so the busiest CU runs ceil(tiles / CUs) of them (sharing the CU with a
// second workgroup does not change its throughput), each weighted by the
// bytes it stages per MFMA (tiles whose operands take longer to stage run
// slower).
template <class Ly>
double cost_of(int M, int N, int cus) {
  const long long per_cu = (tiles_of<Ly>(M, N) + cus - 1) / cus;
  const double stage = (double)(Ly::BM + Ly::BN) / ((double)Ly::BM * Ly::BN);  // bytes per MAC, relative
  return (double)per_cu * Ly::BM * Ly::BN * (1.0 + 96.0 * stage);
}

}  // namespace

int proj_tile_config(int M, int N, int cus) {
  const double cs = cost_of<TileS>(M, N, cus), cm = cost_of<TileM>(M, N, cus), cl = cost_of<TileL>(M, N, cus);
  const double cx = cost_of<TileX>(M, N, cus);
  if (cx < cl && cx <= cm && cx <= cs) return 3;
  if (cl <= cm && cl <= cs) return 2;
  return cm <= cs ? 1 : 0;
}

int launch_project(const ProjParams& pp, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  const bool f16 = pp.dtype == LF_F16;
  switch (proj_tile_config(pp.M, pp.N, cus)) {
    case 0:
      hipLaunchKernelGGL(f16 ? lf_proj_s_f16 : lf_proj_s_bf16, dim3((unsigned)tiles_of<TileS>(pp.M, pp.N)),
                         dim3(TileS::kThreads), 0, s, pp);
      break;
    case 1:
      hipLaunchKernelGGL(f16 ? lf_proj_m_f16 : lf_proj_m_bf16, dim3((unsigned)tiles_of<TileM>(pp.M, pp.N)),
                         dim3(TileM::kThreads), 0, s, pp);
      break;
    case 3:
      hipLaunchKernelGGL(f16 ? lf_proj_x_f16 : lf_proj_x_bf16, dim3((unsigned)tiles_of<TileX>(pp.M, pp.N)),
                         dim3(TileX::kThreads), 0, s, pp);
      break;
    default:
      hipLaunchKernelGGL(f16 ? lf_proj_l_f16 : lf_proj_l_bf16, dim3((unsigned)tiles_of<TileL>(pp.M, pp.N)),
                         dim3(TileL::kThreads), 0, s, pp);
      break;
  }
  return (int)hipGetLastError();
}

}  // namespace lf
