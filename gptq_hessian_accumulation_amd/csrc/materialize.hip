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
// One kernel when H does not alias S (and rows are 16-byte aligned): every
// workgroup of the tiled pass reads its tile's dead flags from S's diagonal,
// the diagonal tiles also take step 1's reduction (same order), and the first
// one writes the dead mask and the damping.  Otherwise two kernels:
//  1. one workgroup reads the d diagonal entries, writes the dead mask and
//     reduces the (neutralized) diagonal in float64 in a fixed order; the
//     damping is that mean times damp_percent, rounded once to float32;
//  2. a tiled pass over the upper-triangle 64 x 64 tiles of S: each tile is
//     staged through LDS and written both to H's tile (I, J) and, transposed,
//     to tile (J, I), so both halves of every symmetric pair come from the
//     same S element with the same operations (H is bitwise symmetric) and
//     all global accesses are coalesced (16-byte accesses when d % 4 == 0).
//     Only S's upper triangle is read, so H may alias S (in-place materialize).

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kDiagThreads = 256;       // the damping's sum order (and the tiled pass's workgroup)

// damp_percent * mean of the (neutralized) scaled diagonal, in float64 in a
// fixed order for NT threads: thread t sums entries t, t + NT, ..., then wave
// shuffles, then the NT / 64 wave partials in order.  Every caller with the
// same NT gets the same bits.  part: NT / 64 doubles of LDS.  The result is
// valid in every thread after the call.
template <int NT>
__device__ __forceinline__ float diag_damp(const float* S, int64_t lds, int d, float scale, float damp_percent,
                                           int neutralize, double* part) {
  double sum = 0.0;
  auto term = [&](float s) { return (double)((neutralize && s == 0.0f) ? 1.0f : s * scale); };
  int j = threadIdx.x;
  // eight strided diagonal loads in flight at a time; the additions keep
  // the order j = t, t + NT, t + 2 NT, ...
  for (; j + 7 * NT < d; j += 8 * NT) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = S[(int64_t)(j + k * NT) * lds + j + k * NT];
#pragma unroll
    for (int k = 0; k < 8; ++k) sum += term(v[k]);
  }
  for (; j < d; j += NT) sum += term(S[(int64_t)j * lds + j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_down(sum, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < NT / 64; ++w) tot += part[w];
  return (float)((double)damp_percent * (tot / (double)d));
}

// The two-launch path (in place, or rows not 16-byte aligned) runs this with
// NT = kDiagThreads, the order the one-launch path's diagonal tiles use.
template <int NT>
__global__ void __launch_bounds__(NT) diag_kernel(const float* S, int64_t lds, int d, float scale,
                                                  float damp_percent, int neutralize, uint8_t* dead, float* damp_dev) {
  __shared__ double part[NT / 64];
  for (int j = threadIdx.x; j < d; j += NT) dead[j] = (neutralize && S[(int64_t)j * lds + j] == 0.0f) ? 1 : 0;
  const float damp = diag_damp<NT>(S, lds, d, scale, damp_percent, neutralize, part);
  if (threadIdx.x == 0) damp_dev[0] = damp;
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

// The same pass with 16-byte accesses, for d % 4 == 0 (every S and H row
// 16-byte aligned): thread t moves columns 4 (t % 16) .. +3 of tile rows
// t / 16 + 16 k (k < 4), so 16 lanes cover one 256-byte tile row; the tile's
// row and column dead flags are read once into LDS.  H is written with
// nontemporal stores (nothing here reads it back; on MI355X they took the
// pass from 14.7 to 10.5 us at width 2,560 and from 23.5 to 20.8 us at 4,096).
// FUSED: H does not alias S, so S's diagonal stays intact throughout: each
// workgroup takes its tile's dead flags from S itself, only the diagonal
// tiles (the ones that add the damping) take the damping's fixed-order sum
// over the diagonal (the same bits as diag_kernel), and workgroup 0 (tile
// (0, 0)) writes the dead mask and the damping out, so materialize is one
// launch.
template <bool FUSED>
__device__ __forceinline__ void mirror_vec_body(const float* S, int64_t lds, int d, float scale, float damp_percent,
                                                int neutralize, uint8_t* dead, float* damp_dev, float* H) {
  __shared__ float tile[kT][kT + 1];
  __shared__ uint8_t dR[kT], dC[kT];
  __shared__ double part[kDiagThreads / 64];
  // blockIdx.x -> (I, J), I <= J: blockIdx.x = J (J + 1) / 2 + I
  const int b = blockIdx.x;
  int J = (int)((sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
  while (J * (J + 1) / 2 > b) --J;
  while ((J + 1) * (J + 2) / 2 <= b) ++J;
  const int I = b - J * (J + 1) / 2;
  const int r0 = I * kT, c0 = J * kT;
  const int t = threadIdx.x, cq = 4 * (t & 15), rr = t >> 4;
  float damp;
  if constexpr (FUSED) {
    auto is_dead = [&](int j) { return neutralize && S[(int64_t)j * lds + j] == 0.0f; };
    if (t < kT) dR[t] = r0 + t < d ? is_dead(r0 + t) : 0;
    else if (t < 2 * kT) dC[t - kT] = c0 + t - kT < d ? is_dead(c0 + t - kT) : 0;
    damp = I == J ? diag_damp<kDiagThreads>(S, lds, d, scale, damp_percent, neutralize, part) : 0.0f;
    if (b == 0) {
      for (int j = t; j < d; j += 256) dead[j] = is_dead(j) ? 1 : 0;
      if (t == 0) damp_dev[0] = damp;
    }
  } else {
    damp = damp_dev[0];
    if (t < kT) dR[t] = r0 + t < d ? dead[r0 + t] : 0;
    else if (t < 2 * kT) dC[t - kT] = c0 + t - kT < d ? dead[c0 + t - kT] : 0;
  }
  // stage the S tile (rows r0.., cols c0..); of the diagonal tile only the
  // upper part (c >= r) is read
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = rr + 16 * k, gi = r0 + r, gj = c0 + cq;
    float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
    if (gi < d && gj < d && (I != J || cq + 3 >= r)) v = *reinterpret_cast<const float4*>(S + (int64_t)gi * lds + gj);
    tile[r][cq] = v.x;
    tile[r][cq + 1] = v.y;
    tile[r][cq + 2] = v.z;
    tile[r][cq + 3] = v.w;
  }
  __syncthreads();
  // tile (I, J): H[r0 + r][c0 + c]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = rr + 16 * k, gi = r0 + r, gj = c0 + cq;
    if (gi >= d || gj >= d) continue;
    const bool di = dR[r] != 0;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = cq + q;
      const float sv = (I == J && c < r) ? tile[c][r] : tile[r][c];
      o[q] = hval(sv, scale, di, dC[c] != 0, gi == gj + q, damp);
    }
    __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(H + (int64_t)gi * lds + gj));
  }
  if (I == J) return;
  // tile (J, I): H[c0 + c][r0 + r] = value of S[r0 + r][c0 + c]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = rr + 16 * k, gi = c0 + c, gj = r0 + cq;
    if (gi >= d || gj >= d) continue;
    const bool di = dC[c] != 0;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = hval(tile[cq + q][c], scale, di, dR[cq + q] != 0, false, damp);
    __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(H + (int64_t)gi * lds + gj));
  }
}

template <bool FUSED>
__global__ void __launch_bounds__(256) mirror_kernel_vec(const float* S, int64_t lds, int d, float scale,
                                                         float damp_percent, int neutralize, uint8_t* dead,
                                                         float* damp_dev, float* H, int nt) {
  mirror_vec_body<FUSED>(S, lds, d, scale, damp_percent, neutralize, dead, damp_dev, H);
}

__device__ __forceinline__ void mirror_body(const float* S, int64_t lds, int d, float scale, const uint8_t* dead,
                                            const float* damp_dev, float* H) {
  mirror_vec_body<false>(S, lds, d, scale, 0.0f, 0, const_cast<uint8_t*>(dead), const_cast<float*>(damp_dev), H);
}

// Many Hessians of one width in two launches (MatGroupParams): one workgroup
// per Hessian writes its dead mask and damping with diag_kernel's order
// (the single path's order, so the bits are the same), then the
// tiles of every Hessian go through mirror_kernel_vec<false>'s body with
// blockIdx.y selecting the Hessian.
template <int NT>
__global__ void __launch_bounds__(NT) diag_grouped(MatGroupParams P) {
  const MatGroup& g = P.g[blockIdx.x];
  __shared__ double part[NT / 64];
  for (int j = threadIdx.x; j < P.d; j += NT)
    g.dead[j] = (P.neutralize && g.S[(int64_t)j * P.lds + j] == 0.0f) ? 1 : 0;
  const float damp = diag_damp<NT>(g.S, P.lds, P.d, g.scale, P.damp_percent, P.neutralize, part);
  if (threadIdx.x == 0) g.damp[0] = damp;
}

__global__ void __launch_bounds__(256) mirror_grouped(MatGroupParams P, int nt) {
  const MatGroup& g = P.g[blockIdx.y];
  mirror_body(g.S, P.lds, P.d, g.scale, g.dead, g.damp, g.H);
}

// Zero the part of S that holds the sum: row i from column 256 * (i / 256)
// on, which covers every upper-triangle tile of every SYRK tile size (their
// diagonal tiles included) and about half the bytes of the whole matrix.
__global__ void __launch_bounds__(256) zero_upper_kernel(float* S, int64_t lds, int d, int vec) {
  const int i = blockIdx.x;
  const int c0 = (i / 256) * 256;
  float* row = S + (int64_t)i * lds;
  if (vec) {
    for (int c = c0 + 4 * (int)threadIdx.x; c < d; c += 4 * 256)
      *reinterpret_cast<float4*>(row + c) = float4{0.0f, 0.0f, 0.0f, 0.0f};
  } else {
    for (int c = c0 + (int)threadIdx.x; c < d; c += 256) row[c] = 0.0f;
  }
}

// zero_upper_kernel for many Hessians of one width: blockIdx.y is the Hessian.
__global__ void __launch_bounds__(256) zero_upper_grouped(ZeroGroupParams P) {
  const int i = blockIdx.x;
  const int c0 = (i / 256) * 256;
  float* row = P.S[blockIdx.y] + (int64_t)i * P.lds;
  if (P.vec) {
    for (int c = c0 + 4 * (int)threadIdx.x; c < P.d; c += 4 * 256)
      *reinterpret_cast<float4*>(row + c) = float4{0.0f, 0.0f, 0.0f, 0.0f};
  } else {
    for (int c = c0 + (int)threadIdx.x; c < P.d; c += 256) row[c] = 0.0f;
  }
}

}  // namespace

hipError_t launch_zero_upper(float* S, int64_t lds, int d, hipStream_t stream) {
  if (d <= 0) return hipSuccess;
  const int vec = d % 4 == 0 && lds % 4 == 0 && (reinterpret_cast<uintptr_t>(S) & 15u) == 0;
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)d), dim3(256), 0, stream, S, lds, d, vec);
  return hipGetLastError();
}

hipError_t launch_materialize(const float* S, int64_t lds, int d, float scale, float damp_percent, int neutralize,
                              float* H, uint8_t* dead, float* damp_dev, double* /*sum_scratch*/,
                              hipStream_t stream) {
  const int nt = (d + kT - 1) / kT;
  const int tiles = nt * (nt + 1) / 2;
  const bool vec = d % 4 == 0 && lds % 4 == 0 && (reinterpret_cast<uintptr_t>(S) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(H) & 15u) == 0;
  if (vec && H != S) {
    hipLaunchKernelGGL(mirror_kernel_vec<true>, dim3(tiles), dim3(256), 0, stream, S, lds, d, scale, damp_percent,
                       neutralize, dead, damp_dev, H, nt);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(diag_kernel<kDiagThreads>, dim3(1), dim3(kDiagThreads), 0, stream, S, lds, d, scale,
                     damp_percent, neutralize, dead, damp_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (vec)
    hipLaunchKernelGGL(mirror_kernel_vec<false>, dim3(tiles), dim3(256), 0, stream, S, lds, d, scale, damp_percent,
                       neutralize, dead, damp_dev, H, nt);
  else
    hipLaunchKernelGGL(mirror_kernel, dim3(tiles), dim3(256), 0, stream, S, lds, d, scale, dead, damp_dev, H, nt);
  return hipGetLastError();
}

hipError_t launch_zero_upper_grouped(float* const* S, int n, int64_t lds, int d, hipStream_t stream) {
  if (d <= 0 || n <= 0) return hipSuccess;
  if (n > kMatMaxGroups) return hipErrorInvalidValue;
  ZeroGroupParams P;
  for (int e = 0; e < n; ++e) P.S[e] = S[e];
  P.lds = lds;
  P.d = d;
  P.vec = d % 4 == 0 && lds % 4 == 0;
  for (int e = 0; e < n; ++e) P.vec = P.vec && (reinterpret_cast<uintptr_t>(S[e]) & 15u) == 0;
  hipLaunchKernelGGL(zero_upper_grouped, dim3((unsigned)d, (unsigned)n), dim3(256), 0, stream, P);
  return hipGetLastError();
}

bool materialize_grouped_ok(const MatGroupParams& P) {
  if (P.d % 4 != 0 || P.lds % 4 != 0) return false;
  for (int e = 0; e < P.ngroups; ++e)
    if ((reinterpret_cast<uintptr_t>(P.g[e].S) & 15u) || (reinterpret_cast<uintptr_t>(P.g[e].H) & 15u)) return false;
  return true;
}

hipError_t launch_materialize_grouped(const MatGroupParams& P, hipStream_t stream) {
  if (P.ngroups <= 0) return hipSuccess;
  if (P.ngroups > kMatMaxGroups || !materialize_grouped_ok(P)) return hipErrorInvalidValue;
  const int nt = (P.d + kT - 1) / kT;
  const int tiles = nt * (nt + 1) / 2;
  hipLaunchKernelGGL(diag_grouped<kDiagThreads>, dim3(P.ngroups), dim3(kDiagThreads), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mirror_grouped, dim3(tiles, P.ngroups), dim3(256), 0, stream, P, nt);
  return hipGetLastError();
}

}  // namespace hess
