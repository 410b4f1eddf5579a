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
// zeroed), U widened exactly; the code and error take reciprocals of the
// step and of U's diagonal, an ulp or so from the quotients, like the
// float64 reordering of the updates: a code can differ from a plain
// column-by-column implementation only at a rounding tie, where both codes
// are correct.  Outputs: dequantized weights and step sizes rounded to float32,
// codes as bytes, the loss sum_i sum_r (err_ri)^2 / nsamples in float64.
//
// Kernels per 128-column block: q_rows (16 lanes per weight row: the serial
// walk through the block's columns, lanes holding eight columns each) and
// q_gemm_lds (128 x 128 tiles of W right of the block, float64 matrix cores,
// the block's errors as A and U's rows as B, both staged through LDS).

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kQB = 128;  // columns per block
constexpr int kQT = 128;  // row padding: the product's tile edge

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

// The serial walk through block [i1, i1 + nb): 16 rows per workgroup, 4 per
// wave, 16 lanes per row; lane j of a row holds columns i1 + j + 16 k
// (k < 8).  The block's slice of U is staged in LDS with only its strict
// upper part kept (zeros on and below the diagonal) and the reciprocals of its
// diagonal beside it, so every update is unconditional and a column's
// register keeps, after its own step, exactly the value it was quantized
// from.  Every lane of a row also carries the value of the column being
// quantized (wn) and of the next one as of the previous step (wn2): step i
// takes the code and error of wn, applies err_i to all held columns and to
// wn2 (the same fused multiply-add the owner applies, so the copies equal the
// owner's register bit for bit), and fetches column i + 2 from its owner by a
// lane shuffle that is not needed until the next step's error is known, so
// the shuffle latency stays off the serial chain.  Code q = clip(rint(w / s),
// -8, 7) + 8 with w / s taken as w times the reciprocal step; error
// (w - s (q - 8)) / U[i][i] taken as w d - (s d)(q - 8) with d the reciprocal
// diagonal: within an ulp or so of the quotients, which can change a code only
// at a rounding tie.  The codes, values and errors are taken again from the
// kept values after the walk, with the same arithmetic, and written out then.
// group: 0 = whole row (steps in step[]), else the group size (a divisor of
// 128, so a power of two); a group's step comes from its columns' values when
// it is reached.
constexpr int kRowsPerWg = 16;
constexpr int kUbLd = kQB + 4;  // LDS row stride of the staged slice (floats)

__device__ __forceinline__ double shfl16_max(double v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double shfl16_sum(double v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// signed code in [-8, 7] and the scaled error of one weight
__device__ __forceinline__ double q_code(double w, double inv_s) { return fmin(fmax(rint(w * inv_s), -8.0), 7.0); }
__device__ __forceinline__ double q_err(double w, double q, double d, double sd) { return fma(-sd, q, w * d); }

// GC: the group size when known at compile time (0 = whole rows), or -1 to
// take it from group_rt; FULL: the block has all 128 columns.
template <int GC, bool FULL>
__global__ void __launch_bounds__(256) q_rows(double* __restrict__ Wd, int ldd, int N, int K, int i1,
                                              const float* __restrict__ U, int64_t ldu, int group_rt,
                                              const double* __restrict__ step, float* __restrict__ scales,
                                              int ngroups, double* __restrict__ Err, int lde, float* __restrict__ Q,
                                              int64_t ldq, uint8_t* __restrict__ codes, int64_t ldc,
                                              double* __restrict__ lossp, int nblk) {
  __shared__ float Ub[kQB * kUbLd];
  __shared__ double invd[kQB];
  const int group = GC >= 0 ? GC : group_rt;
  const int nb = FULL ? kQB : min(kQB, K - i1);
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int slot = (threadIdx.x >> 6) * 4 + (lane >> 4);  // row slot in the workgroup
  const int r = blockIdx.x * kRowsPerWg + slot;
  const bool live = r < N;
  const int base = lane & 48;
  // this lane's row entries and step are requested first, so that their
  // latency overlaps the staging of the factor slice below
  double wr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = j + 16 * k;
    wr[k] = (live && c < nb) ? Wd[(int64_t)r * ldd + i1 + c] : 0.0;
  }
  double s = (!group && live) ? step[r] : 1.0;
  {
    // all of a thread's loads in flight before its first store: thread t takes
    // column t % 128 of rows t / 128 + 2 q (q < 64)
    const int cc = threadIdx.x & (kQB - 1), r0 = threadIdx.x >> 7;
    float v[kQB / 2];
#pragma unroll
    for (int q = 0; q < kQB / 2; ++q) {
      const int rr = r0 + 2 * q;
      v[q] = (cc > rr && cc < nb) ? U[(int64_t)(i1 + rr) * ldu + i1 + cc] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kQB / 2; ++q) Ub[(r0 + 2 * q) * kUbLd + cc] = v[q];
  }
  if (threadIdx.x < kQB)
    invd[threadIdx.x] = threadIdx.x < nb ? 1.0 / (double)U[(int64_t)(i1 + threadIdx.x) * ldu + i1 + threadIdx.x] : 0.0;
  __syncthreads();
  double inv_s = 1.0 / s;
  double sk[8];  // the step of each held column's group
#pragma unroll
  for (int k = 0; k < 8; ++k) sk[k] = s;
  double wn = __shfl(wr[0], base | 0);   // column 0
  double wn2 = __shfl(wr[0], base | 1);  // column 1
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = 16 * m + u;
      if (i >= nb) continue;
      if (group && (i & (group - 1)) == 0) {
        // the group's step from its columns' current values
        double a = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = j + 16 * k;
          a = fmax(a, (c >= i && c < i + group && c < nb) ? fabs(wr[k]) : 0.0);
        }
        a = shfl16_max(a);
        s = quant_step(a);
        inv_s = 1.0 / s;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = j + 16 * k;
          sk[k] = (c >= i && c < i + group) ? s : sk[k];
        }
        if (j == 0 && live) scales[(int64_t)r * ngroups + (i1 + i) / group] = (float)s;
      }
      const double d = invd[i];
      const double err = q_err(wn, q_code(wn, inv_s), d, s * d);
      const float* urow = Ub + i * kUbLd;
      const double wnext = fma(-err, (double)urow[i + 1 < kQB ? i + 1 : i], wn2);
#pragma unroll
      for (int k = m; k < 8; ++k) wr[k] = fma(-err, (double)urow[j + 16 * k], wr[k]);
      if (i + 2 < kQB) wn2 = __shfl(wr[(i + 2) >> 4], base | ((i + 2) & 15));
      wn = wnext;
    }
  }
  // codes, values and errors from the kept values, as in the walk
  double loss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = j + 16 * k;
    double e = 0.0;
    if (c < nb) {
      const double sc = sk[k], w = wr[k], d = invd[c];
      const double q = q_code(w, 1.0 / sc);
      e = q_err(w, q, d, sc * d);
      loss = fma(e, e, loss);
      if (live) {
        Q[(int64_t)r * ldq + i1 + c] = (float)(sc * q);
        codes[(int64_t)r * ldc + i1 + c] = (uint8_t)(q + 8.0);
      }
    }
    if (live) Err[(int64_t)r * lde + c] = e;
  }
  loss = shfl16_sum(loss);
  if (j == 0 && live) lossp[(int64_t)r * nblk + i1 / kQB] = loss;
}

// Wd[rows, c_begin + ...] -= E (rows x 128) U[u0 .. u0 + 128, c_begin + ...]
// with operands staged through LDS: one 128 x 128 tile of W per workgroup,
// four waves of 64 x 64 (4 x 4 blocks of 16 x 16 on the float64 matrix
// instruction, accumulators held for the whole k range).  k runs in chunks of
// 16, double-buffered: the next chunk's global loads are issued before the
// current chunk's products, and stored to the other LDS buffer after them.
// E's chunk is 128 rows x 16 k (row-major, padded); U's is 16 rows x 128
// columns, widened from float32 as it is stored.  Rows of U at or past K, and
// columns past K, read as zero.
constexpr int kGT = 128;          // tile edge
constexpr int kGK = 16;           // k per chunk
constexpr int kEL = kGK + 2;      // LDS row stride of the E chunk (doubles)
constexpr int kUL = kGT + 2;      // LDS row stride of the U chunk (doubles)

__global__ void __launch_bounds__(256) q_gemm_lds(double* __restrict__ Wd, int ldd, int c_begin, int ntc,
                                                  const double* __restrict__ E, const float* __restrict__ U,
                                                  int64_t ldu, int u0, int K) {
  __shared__ __attribute__((aligned(16))) double Es[2][kGT * kEL];
  __shared__ __attribute__((aligned(16))) double Us[2][kGK * kUL];
  const int tr = blockIdx.x / ntc, tc = blockIdx.x - tr * ntc;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int R0 = kGT * tr, C0 = c_begin + kGT * tc;
  const int wr = 64 * (w >> 1), wc = 64 * (w & 1);
  // global -> register loads of one chunk: E rows t / 2 (two threads per row, 8 k each),
  // U rows t / 16 (16 threads per row, 8 columns each)
  const int er = t >> 1, ek = (t & 1) * 8;
  const int ur = t >> 4, uc = (t & 15) * 8;
  f64x4 ev[2];          // 8 doubles of E
  float uv[8];
  auto load = [&](int kc) {
    const double* src = E + (int64_t)(R0 + er) * kQB + kc + ek;
#pragma unroll
    for (int q = 0; q < 2; ++q) ev[q] = *reinterpret_cast<const f64x4*>(src + 4 * q);
    const int urow = u0 + kc + ur;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = C0 + uc + q;
      uv[q] = (urow < K && col < K) ? U[(int64_t)urow * ldu + col] : 0.0f;
    }
  };
  auto store = [&](int buf) {
    double* e = Es[buf] + er * kEL + ek;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int z = 0; z < 4; ++z) e[4 * q + z] = ev[q][z];
    double* u = Us[buf] + ur * kUL + uc;
#pragma unroll
    for (int q = 0; q < 8; ++q) u[q] = (double)uv[q];
  };
  f64x4 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[rb][cb][j] = Wd[(int64_t)(R0 + wr + 16 * rb + lk + 4 * j) * ldd + C0 + wc + 16 * cb + li];
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < kQB; kc += kGK) {
    const int buf = (kc / kGK) & 1;
    const bool more = kc + kGK < kQB;
    if (more) load(kc + kGK);
    const double* Eb = Es[buf];
    const double* Ubf = Us[buf];
#pragma unroll
    for (int kk = 0; kk < kGK; kk += 4) {
      double a[4], b[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[rb] = -Eb[(wr + 16 * rb + li) * kEL + kk + lk];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) b[cb] = Ubf[(kk + lk) * kUL + wc + 16 * cb + li];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Wd[(int64_t)(R0 + wr + 16 * rb + lk + 4 * j) * ldd + C0 + wc + 16 * cb + li] = acc[rb][cb][j];
}

// loss = sum of the per-row, per-block partials in a fixed order / nsamples.
__global__ void __launch_bounds__(1024) q_loss(const double* __restrict__ lossp, int64_t n, double inv_n,
                                               double* __restrict__ loss) {
  __shared__ double part[16];
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t i = threadIdx.x;
  for (; i + 3 * 1024 < n; i += 4 * 1024) {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] += lossp[i + u * 1024];
  }
  for (; i < n; i += 1024) v[0] += lossp[i];
  double t = wave_sum((v[0] + v[1]) + (v[2] + v[3]));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0;
    for (int w = 0; w < 16; ++w) a += part[w];
    *loss = a * inv_n;
  }
}

}  // namespace

int64_t quant_rows_padded(int64_t n) { return (n + kQT - 1) / kQT * kQT; }
int64_t quant_cols_padded(int64_t k) { return (k + kQB - 1) / kQB * kQB; }

int64_t quant_workspace_doubles(int64_t n, int64_t k) {
  const int64_t rp = quant_rows_padded(n), ldd = quant_cols_padded(k);
  return rp * ldd + rp * kQB + n + n * (ldd / kQB);
}

// After each 128-column block's walk, its errors reach every column to its
// right through one product (k = 128, 128 x 128 tiles staged through LDS).
hipError_t launch_gptq_quantize(const QuantParams& P, hipStream_t s) {
  const int N = P.rows, K = P.cols;
  const int rp = (int)quant_rows_padded(N), ldd = (int)quant_cols_padded(K);
  const int nblk = ldd / kQB;
  double* Wd = P.work;
  double* E = Wd + (int64_t)rp * ldd;
  double* step = E + (int64_t)rp * kQB;
  double* lossp = step + N;
  const int group = (P.group <= 0 || P.group >= K) ? 0 : P.group;
  const int ngroups = group ? (K + group - 1) / group : 1;
  hipLaunchKernelGGL(q_load, dim3(rp), dim3(256), 0, s, P.W, P.ldw, N, K, P.dead, Wd, ldd, E);
  if (!group) hipLaunchKernelGGL(q_rowscale, dim3((N + 3) / 4), dim3(256), 0, s, Wd, ldd, N, K, step, P.scales);
  for (int i1 = 0; i1 < K; i1 += kQB) {
    const int i2 = i1 + kQB;
    const bool full = i2 <= K;
    auto rows_kernel = [&]() -> void (*)(double*, int, int, int, int, const float*, int64_t, int, const double*,
                                         float*, int, double*, int, float*, int64_t, uint8_t*, int64_t, double*,
                                         int) {
      if (!full) return q_rows<-1, false>;
      switch (group) {
        case 0: return q_rows<0, true>;
        case 32: return q_rows<32, true>;
        case 64: return q_rows<64, true>;
        case 128: return q_rows<128, true>;
        default: return q_rows<-1, true>;
      }
    };
    hipLaunchKernelGGL(rows_kernel(), dim3((N + kRowsPerWg - 1) / kRowsPerWg), dim3(256), 0, s, Wd, ldd, N, K, i1,
                       P.U, P.ldu, group, step, P.scales, ngroups, E, kQB, P.Q, P.ldq, P.codes, P.ldc, lossp, nblk);
    if (i2 < K) {
      const int ntc = (ldd - i2) / kGT;
      hipLaunchKernelGGL(q_gemm_lds, dim3((unsigned)((rp / kGT) * ntc)), dim3(256), 0, s, Wd, ldd, i2, ntc, E, P.U,
                         P.ldu, i1, K);
    }
  }
  if (P.loss)
    hipLaunchKernelGGL(q_loss, dim3(1), dim3(1024), 0, s, lossp, (int64_t)N * nblk, 1.0 / (double)P.nsamples, P.loss);
  return hipGetLastError();
}

}  // namespace hess
