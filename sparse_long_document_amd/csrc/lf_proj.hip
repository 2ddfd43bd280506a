// Input projections of the Longformer attention layer on gfx950: the
// sliding-window projections Q_s, K_s, V_s and the separate global ones
// Q_g, K_g, V_g (segmentfault Longformer summary, "Linear projections for
// global attention") as one stacked linear map of the hidden states,
//   y[p][m][c] = sum_k x[m][k] w[p*C + c][k] + bias[p*C + c],
// with w in the [out features, in features] layout.  Each y[p], viewed as
// [B, n, H, D] with C = H * D, is one input of the attention kernels.
//
// One launch, one dense MFMA GEMM: C_out[M, P*C] = x[M, C] w^T.  Both
// operands are contiguous along the reduction, which is the operand layout
// of the 32x32x16 MFMA for both A (a row of x) and B (a row of w), so LDS
// holds them as they are in HBM.  A workgroup of four waves computes a
// 128 x 128 tile, each wave 64 x 64 (2 x 2 MFMA tiles); the reduction runs
// in steps of 32 through two LDS buffers, the next step's tiles loaded into
// registers while the current one is multiplied.  fp32 accumulation; the
// bias is added in fp32 before rounding to the element type.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "lf_proj_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kRow = kBK + 8;  // LDS row: 32 reduction elements + 16 B of padding

template <class T>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (sizeof(T) == 2 && __is_same(T, _Float16)) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
}

template <class T>
struct ProjShared {
  T a[2][kBM][kRow];
  T b[2][kBN][kRow];
};

// Thread t stages chunks (t & 1) * 2 + {0, 1} (16 B each) of tile row t >> 1.
__device__ __forceinline__ void load_tile(u32x4 (&r)[2], const unsigned char* base, size_t row_bytes, int row,
                                          int rows, int k0, int tid) {
  const int rr = tid >> 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = (tid & 1) * 2 + u;
    const bool ok = row + rr < rows;
    r[u] = ok ? *reinterpret_cast<const u32x4*>(base + (size_t)(row + rr) * row_bytes + (size_t)k0 * 2 + ch * 16)
              : u32x4{0u, 0u, 0u, 0u};
  }
}

template <class T>
__device__ __forceinline__ void store_tile(T (*dst)[kRow], const u32x4 (&r)[2], int tid) {
  const int rr = tid >> 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = (tid & 1) * 2 + u;
    *reinterpret_cast<u32x4*>(&dst[rr][ch * 8]) = r[u];
  }
}

template <class T>
__device__ void proj_body(const ProjParams& p) {
  __shared__ ProjShared<T> sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, c = lane & 31, hl = lane >> 5;
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
  const int M = p.M, C = p.C, N = p.N;
  const size_t row_bytes = (size_t)C * 2;
  const unsigned char* xa = reinterpret_cast<const unsigned char*>(p.x);
  const unsigned char* wb = reinterpret_cast<const unsigned char*>(p.w);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[2], rb[2];
  load_tile(ra, xa, row_bytes, m0, M, 0, tid);
  load_tile(rb, wb, row_bytes, n0, N, 0, tid);
  store_tile<T>(sh.a[0], ra, tid);
  store_tile<T>(sh.b[0], rb, tid);
  __syncthreads();
  const int steps = C / kBK;
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) {
      load_tile(ra, xa, row_bytes, m0, M, (s + 1) * kBK, tid);
      load_tile(rb, wb, row_bytes, n0, N, (s + 1) * kBK, tid);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(&sh.a[buf][wm * 64 + 32 * i + c][16 * ks + 8 * hl]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(&sh.b[buf][wn * 64 + 32 * j + c][16 * ks + 8 * hl]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma<T>(fa[i], fb[j], acc[i][j]);
    }
    if (s + 1 < steps) {
      store_tile<T>(sh.a[buf ^ 1], ra, tid);
      store_tile<T>(sh.b[buf ^ 1], rb, tid);
    }
    __syncthreads();
  }

  // lane (c, hl) of tile (i, j) holds column c and rows 8 g + 4 hl + e
  T* out = reinterpret_cast<T*>(p.out);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + c;
    if (n >= N) continue;
    const int proj = n / C, col = n - proj * C;
    const float bias = p.bias ? p.bias[n] : 0.f;
    T* dst = out + (size_t)proj * M * C + col;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (m < M) dst[(size_t)m * C] = (T)(acc[i][j][r] + bias);
      }
  }
}

__global__ __launch_bounds__(256) void lf_proj_bf16(const ProjParams p) { proj_body<__bf16>(p); }
__global__ __launch_bounds__(256) void lf_proj_f16(const ProjParams p) { proj_body<_Float16>(p); }

}  // namespace

int launch_project(const ProjParams& pp, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((pp.M + kBM - 1) / kBM), (unsigned)((pp.N + kBN - 1) / kBN));
  if (pp.dtype == LF_F16)
    hipLaunchKernelGGL(lf_proj_f16, grid, dim3(256), 0, s, pp);
  else
    hipLaunchKernelGGL(lf_proj_bf16, grid, dim3(256), 0, s, pp);
  return (int)hipGetLastError();
}

}  // namespace lf
