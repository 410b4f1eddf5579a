// Per-column sums of squares (the imatrix statistic) on gfx950.
//
//   acc[j] += sum_t X[t][j]^2      for j < d, in float32
//
// The imatrix method keeps a float32 per-column sum of squares of the layer
// inputs rather than a Gram matrix (NVIDIA Model-Optimizer PR 3002 page,
// "What does this PR do?": a sum of squares per column is not a GEMM, so
// matrix cores do not apply).  It is a single streaming read of X.
//
// Pass 1: workgroup (c, s) takes one column group (64 lanes x 16 bytes:
// 512 bf16 or 256 float32 features) over one run of rows, rows s*R ..
// s*R + R - 1; its four waves each take a quarter of the run.  Each thread
// squares and sums its 8 (or 4) columns over its rows in float32 registers,
// with the next rows' loads in flight (nontemporal: each byte is read once;
// 44 us instead of 47 per 32,768 x 4,096 bf16 batch on MI355X); the four
// waves' sums meet in LDS and are added in wave order, and the workgroup
// writes one partial row, part[s][cols].  Pass 2 adds the splits' partials
// to acc in a fixed order (four waves over quarters of the splits, then
// their sums in wave order), so results do not depend on scheduling.
// Element-aligned inputs take a one-column-per-lane pass 1.

#include <algorithm>

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kImxWaves = 4;
// Pass-1 workgroups aimed at per batch (two per CU), when the rows allow.
constexpr int kImxTargetWgs = 512;

// The four waves' per-column sums (PER consecutive columns per lane, lane l
// at columns l*PER ..) added in wave order and written as the workgroup's
// partial row: part_row[col0 + j] for j < 64*PER, col0 + j < d.
template <int PER>
__device__ __forceinline__ void imx_combine(const float (&s)[PER], float* part_row, int col0, int d) {
  __shared__ float red[kImxWaves][64 * PER];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < PER; ++k) red[wave][lane * PER + k] = s[k];
  __syncthreads();
  for (int j = threadIdx.x; j < 64 * PER; j += 64 * kImxWaves) {
    const int col = col0 + j;
    if (col < d) part_row[col] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
  }
}

// This wave's rows: the wave-th quarter of the workgroup's run [r0, r1).
__device__ __forceinline__ void imx_rows(int64_t n, int64_t rows_per, int64_t& a, int64_t& b) {
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = min(n, r0 + rows_per);
  const int64_t q = (rows_per + kImxWaves - 1) / kImxWaves;
  a = min(r1, r0 + (threadIdx.x >> 6) * q);
  b = min(r1, a + q);
}

// bf16, 16-byte aligned rows: lane handles 8 consecutive columns
__global__ void __launch_bounds__(256) imx_part_bf16_vec(const char* X, int64_t ld_bytes, int64_t n, int d,
                                                          int64_t rows_per, float* part) {
  const int col0 = blockIdx.x * 512;
  const int c8 = col0 + (threadIdx.x & 63) * 8;  // this lane's first column
  int64_t a, b;
  imx_rows(n, rows_per, a, b);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c8 < d) {
    const char* p = X + a * ld_bytes + (int64_t)c8 * 2;
#pragma unroll 16
    for (int64_t r = a; r < b; ++r, p += ld_bytes) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = __uint_as_float(v[k] << 16), hi = __uint_as_float(v[k] & 0xffff0000u);
        s[2 * k] += lo * lo;
        s[2 * k + 1] += hi * hi;
      }
    }
  }
  imx_combine<8>(s, part + (int64_t)blockIdx.y * d, col0, d);
}

// float32, 16-byte aligned rows: lane handles 4 consecutive columns
__global__ void __launch_bounds__(256) imx_part_f32_vec(const char* X, int64_t ld_bytes, int64_t n, int d,
                                                         int64_t rows_per, float* part) {
  const int col0 = blockIdx.x * 256;
  const int c4 = col0 + (threadIdx.x & 63) * 4;
  int64_t a, b;
  imx_rows(n, rows_per, a, b);
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  if (c4 < d) {
    const char* p = X + a * ld_bytes + (int64_t)c4 * 4;
#pragma unroll 16
    for (int64_t r = a; r < b; ++r, p += ld_bytes) {
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#pragma unroll
      for (int k = 0; k < 4; ++k) s[k] += v[k] * v[k];
    }
  }
  imx_combine<4>(s, part + (int64_t)blockIdx.y * d, col0, d);
}

// any alignment: one column per lane
template <typename E>
__global__ void __launch_bounds__(256) imx_part_elem(const E* X, int64_t ld, int64_t n, int d, int64_t rows_per,
                                                     float* part) {
  const int col0 = blockIdx.x * 64;
  const int c = col0 + (threadIdx.x & 63);
  int64_t a, b;
  imx_rows(n, rows_per, a, b);
  float s[1] = {0.f};
  if (c < d) {
    for (int64_t r = a; r < b; ++r) {
      float x;
      if constexpr (sizeof(E) == 2) x = __uint_as_float((uint32_t)X[r * ld + c] << 16);
      else x = X[r * ld + c];
      s[0] += x * x;
    }
  }
  imx_combine<1>(s, part + (int64_t)blockIdx.y * d, col0, d);
}

// acc[j] += the splits' partials of column j: wave w sums its quarter of the
// splits in order, then the quarters are added in wave order.
__global__ void __launch_bounds__(256) imx_reduce(const float* part, int splits, int d, float* acc) {
  __shared__ float red[kImxWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int q = (splits + kImxWaves - 1) / kImxWaves;
  const int k0 = min(splits, wave * q), k1 = min(splits, k0 + q);
  float s = 0.f;
  if (j < d) {
#pragma unroll 16
    for (int k = k0; k < k1; ++k) s += part[(int64_t)k * d + j];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && j < d) acc[j] += ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

}  // namespace

hipError_t launch_imatrix(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* part,
                          int max_splits, float* acc, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int per_lane = vec ? (in_dtype == kInBF16 ? 8 : 4) : 1;
  const int colgroups = (d + 64 * per_lane - 1) / (64 * per_lane);
  // enough workgroups to fill the chip (about kImxTargetWgs), at least 64
  // rows each (16 per wave)
  int64_t splits = (kImxTargetWgs + colgroups - 1) / colgroups;
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, n / 64));
  splits = std::min<int64_t>(splits, max_splits);
  const int64_t rows_per = (n + splits - 1) / splits;
  splits = (n + rows_per - 1) / rows_per;
  const dim3 grid((unsigned)colgroups, (unsigned)splits);
  if (vec && in_dtype == kInBF16)
    hipLaunchKernelGGL(imx_part_bf16_vec, grid, dim3(256), 0, stream, static_cast<const char*>(X), ld * 2, n, d,
                       rows_per, part);
  else if (vec)
    hipLaunchKernelGGL(imx_part_f32_vec, grid, dim3(256), 0, stream, static_cast<const char*>(X), ld * 4, n, d,
                       rows_per, part);
  else if (in_dtype == kInBF16)
    hipLaunchKernelGGL(imx_part_elem<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(X), ld, n,
                       d, rows_per, part);
  else
    hipLaunchKernelGGL(imx_part_elem<float>, grid, dim3(256), 0, stream, static_cast<const float*>(X), ld, n, d,
                       rows_per, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(imx_reduce, dim3((unsigned)((d + 63) / 64)), dim3(256), 0, stream, part, (int)splits, d, acc);
  return hipGetLastError();
}

}  // namespace hess
