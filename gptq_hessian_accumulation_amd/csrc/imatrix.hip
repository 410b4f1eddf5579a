// Per-column sums of squares (the imatrix statistic) on gfx950.
//
//   acc[j] += sum_t X[t][j]^2      for j < d, in float32
//
// The imatrix method keeps a float32 per-column sum of squares of the layer
// inputs rather than a Gram matrix (NVIDIA Model-Optimizer PR 3002 page,
// "What does this PR do?": a sum of squares per column is not a GEMM, so
// matrix cores do not apply).  It is a single streaming read of X.
//
// Pass 1: workgroup (c, s) takes 256 threads x 16 bytes of one run of rows:
// columns c*CW .. c*CW + CW - 1 (CW = 2048 bf16 or 1024 float32 features),
// rows s*R .. s*R + R - 1.  Each thread squares and sums its 8 (or 4)
// columns over the rows in float32 registers, with the next row's load in
// flight, and writes its partial sums to part[s][cols].  Two more passes add
// the splits' partials to acc in a fixed order (results do not depend on
// scheduling).  Element-aligned inputs take a one-column-per-thread pass 1.

#include <algorithm>

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

// bf16, 16-byte aligned rows: thread handles 8 consecutive columns
__global__ void __launch_bounds__(256) imx_part_bf16_vec(const char* X, int64_t ld_bytes, int64_t n, int d,
                                                          int64_t rows_per, float* part) {
  const int c8 = (blockIdx.x * 256 + threadIdx.x) * 8;  // first column
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = min(n, r0 + rows_per);
  if (c8 >= d) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const char* p = X + r0 * ld_bytes + (int64_t)c8 * 2;
#pragma unroll 16
  for (int64_t r = r0; r < r1; ++r, p += ld_bytes) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = __uint_as_float(v[k] << 16), b = __uint_as_float(v[k] & 0xffff0000u);
      s[2 * k] += a * a;
      s[2 * k + 1] += b * b;
    }
  }
  float* o = part + (int64_t)blockIdx.y * d + c8;
  *reinterpret_cast<float4*>(o) = float4{s[0], s[1], s[2], s[3]};
  *reinterpret_cast<float4*>(o + 4) = float4{s[4], s[5], s[6], s[7]};
}

// float32, 16-byte aligned rows: thread handles 4 consecutive columns
__global__ void __launch_bounds__(256) imx_part_f32_vec(const char* X, int64_t ld_bytes, int64_t n, int d,
                                                         int64_t rows_per, float* part) {
  const int c4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = min(n, r0 + rows_per);
  if (c4 >= d) return;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  const char* p = X + r0 * ld_bytes + (int64_t)c4 * 4;
#pragma unroll 16
  for (int64_t r = r0; r < r1; ++r, p += ld_bytes) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    s[0] += v.x * v.x;
    s[1] += v.y * v.y;
    s[2] += v.z * v.z;
    s[3] += v.w * v.w;
  }
  *reinterpret_cast<float4*>(part + (int64_t)blockIdx.y * d + c4) = float4{s[0], s[1], s[2], s[3]};
}

// any alignment: one column per thread
template <typename E>
__global__ void __launch_bounds__(256) imx_part_elem(const E* X, int64_t ld, int64_t n, int d, int64_t rows_per,
                                                     float* part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = min(n, r0 + rows_per);
  if (c >= d) return;
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) {
    float x;
    if constexpr (sizeof(E) == 2) x = __uint_as_float((uint32_t)X[r * ld + c] << 16);
    else x = X[r * ld + c];
    s += x * x;
  }
  part[(int64_t)blockIdx.y * d + c] = s;
}

// Split partials are added in two levels, in a fixed order: first runs of
// 32 splits (part2[c][j] = part[32c][j] + ... + part[32c+31][j]), then the
// runs (acc[j] += part2[0][j] + ... ).
constexpr int kRun = 32;

__global__ void __launch_bounds__(256) imx_reduce_runs(const float* part, int splits, int d, float* part2) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  const int k0 = blockIdx.y * kRun, k1 = min(splits, k0 + kRun);
  float s = 0.f;
#pragma unroll 8
  for (int k = k0; k < k1; ++k) s += part[(int64_t)k * d + j];
  part2[(int64_t)blockIdx.y * d + j] = s;
}

__global__ void __launch_bounds__(256) imx_reduce_final(const float* part2, int runs, int d, float* acc) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  float s = 0.f;
  for (int c = 0; c < runs; ++c) s += part2[(int64_t)c * d + j];
  acc[j] += s;
}

}  // namespace

hipError_t launch_imatrix(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* part,
                          int max_splits, float* acc, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int per_thread = vec ? (in_dtype == kInBF16 ? 8 : 4) : 1;
  const int colgroups = (d + 256 * per_thread - 1) / (256 * per_thread);
  // enough workgroups to fill the chip (about 512), at least 16 rows each
  int64_t splits = (512 + colgroups - 1) / colgroups;
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, n / 16));
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
  const int runs = (int)((splits + kRun - 1) / kRun);
  float* part2 = part + (int64_t)max_splits * d;
  hipLaunchKernelGGL(imx_reduce_runs, dim3((unsigned)((d + 255) / 256), (unsigned)runs), dim3(256), 0, stream, part,
                     (int)splits, d, part2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(imx_reduce_final, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, stream, part2, runs, d, acc);
  return hipGetLastError();
}

}  // namespace hess
