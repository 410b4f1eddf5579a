// Error-propagating 4-bit quantization of a weight matrix with the upper
// Cholesky factor U of the inverse damped Hessian (the quantization pass's
// step 5: GPTQModel wiki "QQQ", Concepts > Quadratic error compensation).
//
// Column i of W (rows = outputs) is quantized with its row's (or group's)
// symmetric 4-bit quantizer, its error is divided by U[i][i], and
// W[:, j] -= err U[i][j] for the columns j > i not yet quantized.  The pages
// process 128-column blocks: inside a block the propagation is applied column
// by column; the block's errors then reach the columns to its right in one
// product, W[:, right] -= Err U[block, right].  Blocking only reorders the
// float64 additions.
//
// Quantizer (wiki "QQQ", Whole-row and grouped weight quantization): step
// s = 2 max|w| / 15 over the row (group_size -1) or over a group of
// contiguous columns, taken from the weights as they are when the group is
// reached; code q = clip(rint(w / s) + 8, 0, 15); value s (q - 8).  A group
// that is all zero takes max|w| = 1.
//
// Arithmetic.  float64 working weights (W widened exactly, dead columns
// zeroed), U widened exactly; the code and error decisions use the same
// float64 divisions as a plain column-by-column implementation, so the codes
// match it except at rounding ties closer than the float64 reordering of the
// updates.  Outputs: dequantized weights and step sizes rounded to float32,
// codes as bytes, the loss sum_i sum_r (err_ri)^2 / nsamples in float64.
//
// Kernels per 128-column block: q_rows (one wave per weight row: the serial
// walk through the block's columns, lanes holding two columns each) and
// q_gemm (64 x 64 tiles of W right of the block, float64 matrix cores, the
// block's errors as A and U's rows as B).

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kQB = 128;  // columns per block
constexpr int kQT = 64;   // product tile edge

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double quant_step(double amax) { return 2.0 * (amax == 0.0 ? 1.0 : amax) / 15.0; }

// Wd (rowsP x ldd) = W widened, dead columns and padding zero; Err = 0.
__global__ void __launch_bounds__(256) q_load(const float* __restrict__ W, int64_t ldw, int N, int K,
                                              const uint8_t* __restrict__ dead, double* __restrict__ Wd, int ldd,
                                              double* __restrict__ Err) {
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < ldd; c += 256) {
    double v = 0.0;
    if (r < N && c < K && !(dead && dead[c])) v = (double)W[(int64_t)r * ldw + c];
    Wd[(int64_t)r * ldd + c] = v;
  }
  for (int c = threadIdx.x; c < kQB; c += 256) Err[(int64_t)r * kQB + c] = 0.0;
}

// Whole-row steps (group_size -1): one wave per row.
__global__ void __launch_bounds__(256) q_rowscale(const double* __restrict__ Wd, int ldd, int N, int K,
                                                  double* __restrict__ step, float* __restrict__ scales) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= N) return;
  double m = 0.0;
  for (int c = lane; c < K; c += 64) m = fmax(m, fabs(Wd[(int64_t)r * ldd + c]));
  m = wave_max(m);
  if (lane == 0) {
    const double s = quant_step(m);
    step[r] = s;
    scales[r] = (float)s;
  }
}

// The serial walk through block [i1, i1 + nb) for one row per wave.  Lane l
// holds the row's columns i1 + l and i1 + 64 + l.  group: 0 = whole row
// (steps in step[]), else the group size (a divisor of 128).
__global__ void __launch_bounds__(256) q_rows(double* __restrict__ Wd, int ldd, int N, int K, int i1,
                                              const float* __restrict__ U, int64_t ldu, int group,
                                              const double* __restrict__ step, float* __restrict__ scales,
                                              int ngroups, double* __restrict__ Err, float* __restrict__ Q,
                                              int64_t ldq, uint8_t* __restrict__ codes, int64_t ldc,
                                              double* __restrict__ lossp, int nblk) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= N) return;
  const int nb = min(kQB, K - i1);
  const int c0 = lane, c1 = lane + 64;
  double* wrow = Wd + (int64_t)r * ldd + i1;
  double w0 = c0 < nb ? wrow[c0] : 0.0;
  double w1 = c1 < nb ? wrow[c1] : 0.0;
  double s = group ? 0.0 : step[r];
  double q0 = 0.0, q1 = 0.0, d0 = 0.0, d1 = 0.0, e0 = 0.0, e1 = 0.0;
  double loss = 0.0;
  for (int i = 0; i < nb; ++i) {
    if (group && i % group == 0) {
      // the group's step from its current weights
      double m = fmax((c0 >= i && c0 < i + group && c0 < nb) ? fabs(w0) : 0.0,
                      (c1 >= i && c1 < i + group && c1 < nb) ? fabs(w1) : 0.0);
      m = wave_max(m);
      s = quant_step(m);
      if (lane == 0) scales[(int64_t)r * ngroups + (i1 + i) / group] = (float)s;
    }
    const int o = i & 63;
    const double w = readlane_f64(i < 64 ? w0 : w1, o);
    const double q = fmin(fmax(rint(w / s) + 8.0, 0.0), 15.0);
    const double dq = s * (q - 8.0);
    const double uii = (double)U[(int64_t)(i1 + i) * ldu + i1 + i];
    const double err = (w - dq) / uii;
    loss = fma(err, err, loss);
    const float* urow = U + (int64_t)(i1 + i) * ldu + i1;
    if (c0 > i && c0 < nb) w0 = fma(-err, (double)urow[c0], w0);
    if (c1 > i && c1 < nb) w1 = fma(-err, (double)urow[c1], w1);
    const bool mine0 = i < 64 && lane == o, mine1 = i >= 64 && lane == o;
    q0 = mine0 ? q : q0;
    d0 = mine0 ? dq : d0;
    e0 = mine0 ? err : e0;
    q1 = mine1 ? q : q1;
    d1 = mine1 ? dq : d1;
    e1 = mine1 ? err : e1;
  }
  if (c0 < nb) {
    Q[(int64_t)r * ldq + i1 + c0] = (float)d0;
    codes[(int64_t)r * ldc + i1 + c0] = (uint8_t)q0;
  }
  if (c1 < nb) {
    Q[(int64_t)r * ldq + i1 + c1] = (float)d1;
    codes[(int64_t)r * ldc + i1 + c1] = (uint8_t)q1;
  }
  Err[(int64_t)r * kQB + c0] = c0 < nb ? e0 : 0.0;
  Err[(int64_t)r * kQB + c1] = c1 < nb ? e1 : 0.0;
  if (lane == 0) lossp[(int64_t)r * nblk + i1 / kQB] = loss;
}

// Wd[:, i2 + 64 tc .. ] -= Err (rowsP x 128) U[i1 .. i1 + 128, i2 + ..]: one
// 64 x 64 tile per workgroup (rows 64 tr, columns i2 + 64 tc); wave w computes
// rows 32 (w >> 1) .. +31 and columns 32 (w & 1) .. +31 as 2 x 2 blocks of
// 16 x 16 (v_mfma_f64_16x16x4_f64: lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; register j of lane l holds D[l/16 + 4 j][l%16]).
__global__ void __launch_bounds__(256) q_gemm(double* __restrict__ Wd, int ldd, int K, int i1, int i2, int ntc,
                                              const float* __restrict__ U, int64_t ldu,
                                              const double* __restrict__ Err) {
  const int tr = blockIdx.x / ntc, tc = blockIdx.x - tr * ntc;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int row0 = kQT * tr + 32 * (w >> 1);
  const int col0 = i2 + kQT * tc + 32 * (w & 1);
  f64x4 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[rb][cb][j] = Wd[(int64_t)(row0 + 16 * rb + lk + 4 * j) * ldd + col0 + 16 * cb + li];
  const int kmax = min(kQB, K - i1);
#pragma unroll 4
  for (int kk = 0; kk < kQB; kk += 4) {
    double a[2], b[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) a[rb] = -Err[(int64_t)(row0 + 16 * rb + li) * kQB + kk + lk];
    const int ur = kk + lk;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int col = col0 + 16 * cb + li;
      b[cb] = (ur < kmax && col < K) ? (double)U[(int64_t)(i1 + ur) * ldu + col] : 0.0;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) Wd[(int64_t)(row0 + 16 * rb + lk + 4 * j) * ldd + col0 + 16 * cb + li] = acc[rb][cb][j];
}

// loss = sum of the per-row, per-block partials in a fixed order / nsamples.
__global__ void __launch_bounds__(256) q_loss(const double* __restrict__ lossp, int64_t n, double inv_n,
                                              double* __restrict__ loss) {
  __shared__ double part[4];
  double v = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) v += lossp[i];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) *loss = ((part[0] + part[1]) + (part[2] + part[3])) * inv_n;
}

}  // namespace

int64_t quant_rows_padded(int64_t n) { return (n + kQT - 1) / kQT * kQT; }
int64_t quant_cols_padded(int64_t k) { return (k + kQB - 1) / kQB * kQB; }

int64_t quant_workspace_doubles(int64_t n, int64_t k) {
  const int64_t rp = quant_rows_padded(n), ldd = quant_cols_padded(k);
  return rp * ldd + rp * kQB + n + n * (ldd / kQB);
}

hipError_t launch_gptq_quantize(const QuantParams& P, hipStream_t s) {
  const int N = P.rows, K = P.cols;
  const int rp = (int)quant_rows_padded(N), ldd = (int)quant_cols_padded(K);
  const int nblk = ldd / kQB;
  double* Wd = P.work;
  double* Err = Wd + (int64_t)rp * ldd;
  double* step = Err + (int64_t)rp * kQB;
  double* lossp = step + N;
  const int group = (P.group <= 0 || P.group >= K) ? 0 : P.group;
  const int ngroups = group ? (K + group - 1) / group : 1;
  hipLaunchKernelGGL(q_load, dim3(rp), dim3(256), 0, s, P.W, P.ldw, N, K, P.dead, Wd, ldd, Err);
  if (!group) hipLaunchKernelGGL(q_rowscale, dim3((N + 3) / 4), dim3(256), 0, s, Wd, ldd, N, K, step, P.scales);
  for (int b = 0; b < nblk; ++b) {
    const int i1 = b * kQB, i2 = i1 + kQB;
    hipLaunchKernelGGL(q_rows, dim3((N + 3) / 4), dim3(256), 0, s, Wd, ldd, N, K, i1, P.U, P.ldu, group, step,
                       P.scales, ngroups, Err, P.Q, P.ldq, P.codes, P.ldc, lossp, nblk);
    if (i2 < K) {
      const int ntc = (ldd - i2 + kQT - 1) / kQT;
      const int64_t tiles = (int64_t)(rp / kQT) * ntc;
      hipLaunchKernelGGL(q_gemm, dim3((unsigned)tiles), dim3(256), 0, s, Wd, ldd, K, i1, i2, ntc, P.U, P.ldu, Err);
    }
  }
  if (P.loss)
    hipLaunchKernelGGL(q_loss, dim3(1), dim3(256), 0, s, lossp, (int64_t)N * nblk, 1.0 / (double)P.nsamples, P.loss);
  return hipGetLastError();
}

}  // namespace hess
