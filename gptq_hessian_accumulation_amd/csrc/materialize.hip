// Materialize the Hessian from the Gram sum on gfx950.
//
//   H = neutralize(S * 2/N) + damp * I,   damp = damp_percent * mean(diag)
//
// The final scale by 2 / total tokens (GPTQModel PR 2979, What Changed:
// materialize_hessian scales the merged sum by 2 / total_samples), then the
// quantization pass's steps on the GPTQModel wiki "QQQ" (Concepts > Quadratic
// error compensation): step 2 neutralizes dead input columns, step 3 adds
// damp_percent * mean(diag(H)) to the diagonal.  A dead column is one whose
// Gram diagonal is exactly zero; its row and column are zero already and its
// diagonal becomes 1, so neutralization precedes the mean.
//
// Two kernels:
//  1. one workgroup reads the d diagonal entries, writes the dead mask and
//     reduces the (neutralized) diagonal in float64 in a fixed order; the
//     damping is that mean times damp_percent, rounded once to float32;
//  2. a tiled pass over the upper-triangle 64 x 64 tiles of S: each tile is
//     staged through LDS and written both to H's tile (I, J) and, transposed,
//     to tile (J, I), so both halves of every symmetric pair come from the
//     same S element with the same operations (H is bitwise symmetric) and
//     all global accesses are coalesced.  Only S's upper triangle is read,
//     so H may alias S (in-place materialize).

#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kDiagThreads = 1024;

__global__ void __launch_bounds__(kDiagThreads) diag_kernel(const float* S, int64_t lds, int d, float scale,
                                                            float damp_percent, int neutralize, uint8_t* dead,
                                                            float* damp_dev) {
  __shared__ double part[kDiagThreads / 64];
  double sum = 0.0;
  for (int j = threadIdx.x; j < d; j += kDiagThreads) {
    const float s = S[(int64_t)j * lds + j];
    const bool dj = neutralize && (s == 0.0f);
    dead[j] = dj ? 1 : 0;
    const float h = dj ? 1.0f : s * scale;
    sum += (double)h;
  }
  // fixed-order reduction: wave shuffles, then wave partials in order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_down(sum, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < kDiagThreads / 64; ++w) tot += part[w];
    damp_dev[0] = (float)((double)damp_percent * (tot / (double)d));
  }
}

constexpr int kT = 64;  // tile edge

__device__ __forceinline__ float hval(float s, float scale, bool di, bool dj, bool on_diag, float damp) {
  if (on_diag) return (di ? 1.0f : s * scale) + damp;
  return (di || dj) ? 0.0f : s * scale;
}

__global__ void __launch_bounds__(256) mirror_kernel(const float* S, int64_t lds, int d, float scale,
                                                     const uint8_t* dead, const float* damp_dev, float* H,
                                                     int nt) {
  __shared__ float tile[kT][kT + 1];
  // blockIdx.x -> (I, J), I <= J, row-major over the upper triangle
  int I = 0, rem = blockIdx.x;
  while (rem >= nt - I) {
    rem -= nt - I;
    ++I;
  }
  const int J = I + rem;
  const int r0 = I * kT, c0 = J * kT;
  const float damp = damp_dev[0];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4

  // stage the S tile (rows r0.., cols c0..); for the diagonal tile only the
  // upper part (c >= r) is meaningful and the lower part is taken mirrored
  for (int r = ty; r < kT; r += 4) {
    const int gi = r0 + r, gj = c0 + tx;
    float v = 0.0f;
    if (gi < d && gj < d && (I != J || tx >= r)) v = S[(int64_t)gi * lds + gj];
    tile[r][tx] = v;
  }
  __syncthreads();

  // tile (I, J): H[r0 + r][c0 + c]
  for (int r = ty; r < kT; r += 4) {
    const int gi = r0 + r, gj = c0 + tx;
    if (gi >= d || gj >= d) continue;
    const float s = (I == J && tx < r) ? tile[tx][r] : tile[r][tx];
    H[(int64_t)gi * lds + gj] = hval(s, scale, dead[gi] != 0, dead[gj] != 0, gi == gj, damp);
  }
  if (I == J) return;
  // tile (J, I): H[c0 + c][r0 + r] = value of S[r0 + r][c0 + c]
  for (int c = ty; c < kT; c += 4) {
    const int gi = c0 + c, gj = r0 + tx;
    if (gi >= d || gj >= d) continue;
    const float s = tile[tx][c];
    H[(int64_t)gi * lds + gj] = hval(s, scale, dead[gi] != 0, dead[gj] != 0, false, damp);
  }
}

}  // namespace

hipError_t launch_materialize(const float* S, int64_t lds, int d, float scale, float damp_percent, int neutralize,
                              float* H, uint8_t* dead, float* damp_dev, double* /*sum_scratch*/,
                              hipStream_t stream) {
  hipLaunchKernelGGL(diag_kernel, dim3(1), dim3(kDiagThreads), 0, stream, S, lds, d, scale, damp_percent,
                     neutralize, dead, damp_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = (d + kT - 1) / kT;
  const int tiles = nt * (nt + 1) / 2;
  hipLaunchKernelGGL(mirror_kernel, dim3(tiles), dim3(256), 0, stream, S, lds, d, scale, dead, damp_dev, H, nt);
  return hipGetLastError();
}

}  // namespace hess
