// Upper Cholesky factor of the inverse damped Hessian (the quantization
// pass's step 4: GPTQModel wiki "QQQ", Concepts > Quadratic error
// compensation): U upper triangular with a positive diagonal, U^T U = H^-1.
//
// Route.  Let J reverse the index order and R R^T = J H J be the lower
// Cholesky factorization of the reversed matrix.  Then H = (J R J)(J R J)^T
// with J R J upper triangular, so U = (J R J)^-1 = J R^-1 J: U is the
// reversed inverse of R.  The factorization and the inversion take
// d^3 / 3 multiply-adds each, 2 d^3 / 3 flops in all counted as 2 per
// multiply-add -- half of the three-call route (factor H, invert through the
// factor, factor the inverse) that a dense library would take.
//
// Arithmetic.  float64 throughout (H is widened exactly; U is rounded to
// float32 once at the end), on the float64 matrix cores
// (v_mfma_f64_16x16x4_f64) for the tile products.
//
// Blocking.  64 x 64 tiles of the reversed matrix A (float64, d rounded up to
// a multiple of 64 and padded with the identity) and of X, which receives
// R^-1; P holds the current block column of L transposed, tile by tile.  For
// each block column k:
//   diag    one workgroup factors A_kk = L_kk L_kk^T and inverts L_kk in LDS
//           (four 16-column panels, each factored by one wave without
//           barriers, then blocked updates and a blocked inverse on the
//           matrix cores), writing L_kk into A_kk and L_kk^-1 into X_kk
//           (for k > 0 inside the previous update launch: its first
//           workgroup updates A_kk and factors it while the others update
//           the rest);
//   panel   P_i <- (A_ik L_kk^-T)^T below the diagonal (a product with the
//           inverse, so it runs on the matrix cores; the transposed copy is
//           what the update reads) and, for the inverse, X_kj <- L_kk^-1 X_kj
//           left of it (block forward substitution);
//   update  A_ij -= A_ik A_jk^T for k < j <= i (the trailing Schur
//           complement) and X_ij -= A_ik X_kj for i > k, j <= k (the
//           right-looking update of the forward substitution).
// A final pass writes U[i][j] = float(X[d-1-i][d-1-j]) for j >= i.
//
// Failure.  A pivot that is not positive (or is NaN) marks H as not positive
// definite: the largest H column index whose pivot failed, plus one, is
// stored in *info (atomic max; factorization order runs from H's last column
// to its first), and the pivot is replaced by NaN so that the rest of the
// result is NaN.  Every kernel still runs to completion.

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kCB = 64;        // tile edge
constexpr int kLdsLd = 66;     // LDS row stride in doubles (528 bytes: 16-byte aligned rows, spread banks)

// v_mfma_f64_16x16x4_f64 (checked on the hardware by an in-bounds lane-layout
// test): lane l supplies A[l%16][l/16] and B[l/16][l%16]; register r of lane
// l holds D[l/16 + 4 r][l%16].
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, const f64x4& c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// A (rows x 64) tile of a dp-strided float64 matrix into LDS (stride kLdsLd):
// each of the 256 threads moves 16 doubles of one row as 8 16-byte pieces.
__device__ __forceinline__ void tile_to_lds(const double* __restrict__ src, int64_t dp, double* lds) {
  const int t = threadIdx.x;
  const int r = t >> 2, c0 = (t & 3) * 16;
  const f64x2* s = reinterpret_cast<const f64x2*>(src + (int64_t)r * dp + c0);
  f64x2 v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = s[q];
#pragma unroll
  for (int q = 0; q < 8; ++q) *reinterpret_cast<f64x2*>(lds + r * kLdsLd + c0 + 2 * q) = v[q];
}

// C (64 x 64 tile, row stride dp) -= A B with the fragments read straight
// from memory, no LDS: A is given transposed (At[k][row], 64 x 64, the panel
// copy written by chol_panel) and B row-major with row stride ldb (B[k][col]),
// so that each fragment load is 16 consecutive doubles of one row.  Wave w
// computes rows 32 (w >> 1) .. +31 and columns 32 (w & 1) .. +31; the waves
// never wait for one another.
// 512 threads: wave w computes rows 16 (w >> 1) .. +15 and columns
// 32 (w & 1) .. +31.  The result goes back to Cg, or to Out (row stride ldo)
// when given.
__device__ __forceinline__ void tile_update_direct(const double* __restrict__ At, const double* __restrict__ B,
                                                   int64_t ldb, double* __restrict__ Cg, int64_t dp,
                                                   double* Out = nullptr, int ldo = 0) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = 16 * (w >> 1), c0 = 32 * (w & 1);
  const int li = lane & 15, lk = lane >> 4;
  f64x4 acc[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[cb][r] = Cg[(int64_t)(r0 + lk + 4 * r) * dp + c0 + 16 * cb + li];
#pragma unroll
  for (int kk = 0; kk < kCB; kk += 4) {
    const double a = -At[(kk + lk) * kCB + r0 + li];
    double b[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) b[cb] = B[(int64_t)(kk + lk) * ldb + c0 + 16 * cb + li];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[cb] = mfma_f64(a, b[cb], acc[cb]);
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (Out) Out[(r0 + lk + 4 * r) * ldo + c0 + 16 * cb + li] = acc[cb][r];
      else Cg[(int64_t)(r0 + lk + 4 * r) * dp + c0 + 16 * cb + li] = acc[cb][r];
    }
}

__device__ __forceinline__ double* tile_at(double* M, int64_t dp, int I, int J) {
  return M + (int64_t)I * kCB * dp + (int64_t)J * kCB;
}

// A = reversed H (lower triangle and diagonal from H's upper triangle, zeros
// above), identity padding; X = 0; *info = 0.  One workgroup row of 256
// threads per A row.
__global__ void __launch_bounds__(256) chol_load(const float* __restrict__ H, int64_t ldh, int d, int dp,
                                                 double* __restrict__ A, double* __restrict__ X, int* info) {
  const int i = blockIdx.x;
  if (i == 0 && threadIdx.x == 0 && info) *info = 0;
  for (int j = threadIdx.x; j < dp; j += 256) {
    double v = 0.0;
    if (i < d && j < d) {
      if (j <= i) v = (double)H[(int64_t)(d - 1 - i) * ldh + (d - 1 - j)];
    } else if (i == j) {
      v = 1.0;
    }
    A[(int64_t)i * dp + j] = v;
    X[(int64_t)i * dp + j] = 0.0;
  }
}

constexpr int kTPR = 8;  // workgroup of the diagonal and update kernels: kCB * kTPR threads

// Square root and reciprocal square root of a pivot: the hardware estimate of
// 1 / sqrt(p) refined by one Newton step y <- y + y (1 - p y^2) / 2 (the
// estimate's relative error squared, far below the float32 rounding of the
// result), and l = p y.  A pivot that is not positive becomes NaN.  Every
// thread evaluates it on its own candidate, without a branch, so that the
// chain overlaps the thread's other updates; only the owner publishes it.
__device__ __forceinline__ void pivot_root(double p, double& l, double& y) {
  p = p > 0.0 ? p : __builtin_nan("");
  y = __builtin_amdgcn_rsq(p);
  y = fma(0.5 * y, fma(-p * y, y, 1.0), y);
  l = p * y;
}

__device__ __forceinline__ void report_pivot(double p, int col, int d, int* info) {
  if (!(p > 0.0) && info && col < d) atomicMax(info, d - col);
}

// Factor and invert the diagonal tile k, blocked: four panels of 16 columns.
// The tile T (lower triangle valid, float64, LDS, row stride kDL) is
// overwritten by L; Y = L^-1 is built in LDS.  For each panel:
//  * one wave factors the panel's 16 columns over all rows at or below it,
//    with no barrier: lane i holds row i's 16 entries of the panel (the
//    diagonal block filled symmetrically from its lower triangle); column
//    j's pivot and row (the pivot row's entries right of it, equal by
//    symmetry to the column's entries below the pivot) reach every lane by
//    readlane, and each lane applies T[i][c] -= (T[i][j] / p) T[j][c] to its
//    remaining panel entries (p the pivot, taken through its reciprocal
//    square root);
//  * the waves then subtract the panel's product L_p L_p^T from the lower
//    16 x 16 blocks right of it (float64 matrix cores).
// Y: each 16 x 16 diagonal block is inverted by one wave (row j of the
// block's inverse is final once scaled by 1 / L[j][j]; the rows below
// subtract L[i][j] times it), then each block column s of Y below the
// diagonal follows from Y_rs = -Y_rr (sum over s <= t < r of L_rt Y_ts),
// one wave per block column, top to bottom.
constexpr int kDL = kCB + 2;  // LDS row stride (doubles) of the diagonal step's tiles
constexpr int kPB = 16;       // panel width

struct DiagLdsB {
  double Y[kCB * kDL];
  double y[kCB];  // reciprocal of each column's diagonal entry of L
};

__device__ __forceinline__ double readlane_d(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// T (LDS, stride kDL, written by the caller, workgroup synchronized) ->
// L into A_kk and L^-1 into X_kk.  Needs at least 6 waves.
__device__ __forceinline__ void diag_blocked(double* T, double* __restrict__ A, double* __restrict__ X, int dp, int k,
                                             int d, int* info, DiagLdsB& S) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int s = 0; s < kCB / kPB; ++s) {
    const int c0 = kPB * s;
    if (w == 0) {
      const int i = lane;
      double P[kPB];
#pragma unroll
      for (int q = 0; q < kPB; ++q) {
        const int c = c0 + q;
        P[q] = c <= i ? T[i * kDL + c] : T[c * kDL + i];
      }
#pragma unroll
      for (int j = 0; j < kPB; ++j) {
        const int r = c0 + j;
        const double p = readlane_d(P[j], r);
        if (lane == 0) report_pivot(p, k * kCB + r, d, info);
        double l, y;
        pivot_root(p, l, y);
        const double lij = P[j] * y;
        const double f = lij * y;
#pragma unroll
        for (int q = j + 1; q < kPB; ++q) P[q] = fma(-f, readlane_d(P[q], r), P[q]);
        P[j] = i == r ? l : (i > r ? lij : 0.0);
        if (lane == 0) S.y[r] = y;
      }
      if (i >= c0) {
#pragma unroll
        for (int q = 0; q < kPB; ++q) T[i * kDL + c0 + q] = P[q];
      }
    }
    __syncthreads();
    // trailing lower blocks (bi, bk), bk <= bi, right of the panel: one per wave
    const int m = kCB / kPB - 1 - s;
    if (w < m * (m + 1) / 2) {
      int bi = 0, bk = w;
      while (bk > bi) {
        bk -= bi + 1;
        ++bi;
      }
      const int I0 = c0 + kPB * (1 + bi), K0 = c0 + kPB * (1 + bk);
      const int li = lane & 15, lk = lane >> 4;
      f64x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = T[(I0 + lk + 4 * r) * kDL + K0 + li];
#pragma unroll
      for (int q = 0; q < kPB; q += 4) {
        const double a = -T[(I0 + li) * kDL + c0 + q + lk];
        const double b = T[(K0 + li) * kDL + c0 + q + lk];
        acc = mfma_f64(a, b, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) T[(I0 + lk + 4 * r) * kDL + K0 + li] = acc[r];
    }
    __syncthreads();
  }
  // inverse of each diagonal block (wave s, lanes 0..15 = the block's rows)
  if (w < kCB / kPB) {
    const int c0 = kPB * w, i = lane & 15;
    double Lr[kPB], Yr[kPB];
#pragma unroll
    for (int q = 0; q < kPB; ++q) {
      Lr[q] = T[(c0 + i) * kDL + c0 + q];
      Yr[q] = q == i ? 1.0 : 0.0;
    }
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      const double yj = S.y[c0 + j];
      const double g = Lr[j] * yj;
#pragma unroll
      for (int q = 0; q <= j; ++q) {
        const double v = readlane_d(Yr[q], j);
        Yr[q] = i == j ? v * yj : fma(-g, v, Yr[q]);
      }
    }
    if (lane < kPB) {
#pragma unroll
      for (int q = 0; q < kPB; ++q) S.Y[(c0 + i) * kDL + c0 + q] = Yr[q];
    }
  }
  __syncthreads();
  // blocks below the diagonal, block column s = w (waves 0..2), rows top to bottom
  if (w < kCB / kPB - 1) {
    const int s0 = kPB * w;
    const int li = lane & 15, lk = lane >> 4;
    for (int rb = w + 1; rb < kCB / kPB; ++rb) {
      const int r0 = kPB * rb;
      f64x4 g = f64x4{0.0, 0.0, 0.0, 0.0};
      for (int tb = w; tb < rb; ++tb) {
        const int t0 = kPB * tb;
#pragma unroll
        for (int q = 0; q < kPB; q += 4) {
          const double a = T[(r0 + li) * kDL + t0 + q + lk];
          const double b = S.Y[(t0 + q + lk) * kDL + s0 + li];
          g = mfma_f64(a, b, g);
        }
      }
      // Y_rs = -Y_rr G: register q of g is G's rows 4 q + lane / 16, the
      // matrix instruction's B operand for k-step q
      f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = mfma_f64(-S.Y[(r0 + li) * kDL + r0 + 4 * q + lk], g[q], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) S.Y[(r0 + lk + 4 * r) * kDL + s0 + li] = acc[r];
    }
  }
  __syncthreads();
  double* Ag = tile_at(A, dp, k, k);
  double* Xg = tile_at(X, dp, k, k);
  for (int e = t; e < kCB * kCB; e += blockDim.x) {
    const int i = e / kCB, c = e % kCB;
    Ag[(int64_t)i * dp + c] = c <= i ? T[i * kDL + c] : 0.0;
    Xg[(int64_t)i * dp + c] = c <= i ? S.Y[i * kDL + c] : 0.0;
  }
}

__global__ void __launch_bounds__(kCB * kTPR) chol_diag(double* __restrict__ A, double* __restrict__ X, int dp, int k,
                                                        int d, int* info) {
  __shared__ double Tl[kCB * kDL];
  __shared__ DiagLdsB S;
  const double* src = tile_at(A, dp, k, k);
  for (int e = threadIdx.x; e < kCB * kCB; e += blockDim.x) Tl[(e / kCB) * kDL + e % kCB] = src[(int64_t)(e / kCB) * dp + e % kCB];
  __syncthreads();
  diag_blocked(Tl, A, X, dp, k, d, info, S);
}

// Panel of block column k, on four workgroups per tile below the diagonal
// and two per tile left of it, so that the float64 matrix cores of more CUs
// share each step of the serial chain:
//  * workgroups b < 4 m (m = nb - k - 1) take quadrant (b / 2 % 2, b % 2) of
//    A_ik L_kk^-T (i = k + 1 + b / 4): 32 rows of A_ik times 32 rows of
//    L_kk^-1, written transposed into P_i (P_i[c][r] = (A_ik L_kk^-T)[r][c]),
//    the copy the trailing update reads.  A_ik itself is read by nothing
//    later, so it is not rewritten, and the quadrants only read A_ik;
//  * the others take column half (b - 4 m) % 2 of X_kj <- L_kk^-1 X_kj
//    (j = (b - 4 m) / 2 < k), in place: each half reads only its own columns.
__global__ void __launch_bounds__(256) chol_panel(const double* __restrict__ A, double* __restrict__ X,
                                                  double* __restrict__ P, int dp, int k, int nb) {
  __shared__ __attribute__((aligned(16))) double Al[kCB * kLdsLd];
  __shared__ __attribute__((aligned(16))) double Bl[kCB * kLdsLd];
  const int m = nb - k - 1;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = lane & 15, lk = lane >> 4;
  if (b < 4 * m) {
    const int i = k + 1 + b / 4, rh = (b >> 1) & 1, ch = b & 1;
    // 32 rows of A_ik and 32 rows of L_kk^-1: thread t moves 8 doubles of row t / 8 of each
    {
      const int r = t >> 3, c = (t & 7) * 8;
      const double* sa = A + ((int64_t)i * kCB + 32 * rh + r) * dp + (int64_t)k * kCB + c;
      const double* sb = X + ((int64_t)k * kCB + 32 * ch + r) * dp + (int64_t)k * kCB + c;
      f64x2 va[4], vb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        va[q] = reinterpret_cast<const f64x2*>(sa)[q];
        vb[q] = reinterpret_cast<const f64x2*>(sb)[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<f64x2*>(Al + r * kLdsLd + c + 2 * q) = va[q];
        *reinterpret_cast<f64x2*>(Bl + r * kLdsLd + c + 2 * q) = vb[q];
      }
    }
    __syncthreads();
    // wave w: rows 16 (w >> 1) .. +15, columns 16 (w & 1) .. +15 of the quadrant
    const int r0 = 16 * (w >> 1), c0 = 16 * (w & 1);
    f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int kk = 0; kk < kCB; kk += 4)
      acc = mfma_f64(Al[(r0 + li) * kLdsLd + kk + lk], Bl[(c0 + li) * kLdsLd + kk + lk], acc);
    double* Pi = P + (int64_t)i * kCB * kCB;
#pragma unroll
    for (int r = 0; r < 4; ++r) Pi[(32 * ch + c0 + li) * kCB + 32 * rh + r0 + lk + 4 * r] = acc[r];
  } else {
    const int j = (b - 4 * m) >> 1, ch = (b - 4 * m) & 1;
    double* C = tile_at(X, dp, k, j) + 32 * ch;
    tile_to_lds(tile_at(X, dp, k, k), dp, Al);
    {
      // column half of X_kj: thread t moves 8 doubles of row t / 4
      const int r = t >> 2, c = (t & 3) * 8;
      const double* sc = C + (int64_t)r * dp + c;
      f64x2 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = reinterpret_cast<const f64x2*>(sc)[q];
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<f64x2*>(Bl + r * kLdsLd + c + 2 * q) = v[q];
    }
    __syncthreads();
    // wave w: rows 16 w .. +15, both 16-column blocks of the half
    f64x4 acc[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
#pragma unroll 4
    for (int kk = 0; kk < kCB; kk += 4) {
      const double a = Al[(16 * w + li) * kLdsLd + kk + lk];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[cb] = mfma_f64(a, Bl[(kk + lk) * kLdsLd + 16 * cb + li], acc[cb]);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) C[(int64_t)(16 * w + lk + 4 * r) * dp + 16 * cb + li] = acc[cb][r];
  }
}

// Trailing update after block column k.  Workgroups b < T1 = m (m + 1) / 2
// (m = nb - k - 1) take A_ij -= A_ik A_jk^T over the lower triangle of the
// trailing blocks (b = ii (ii + 1) / 2 + jj, i = k + 1 + ii, j = k + 1 + jj);
// the others take X_ij -= A_ik X_kj for i > k, j <= k.  A_ik comes from its
// transposed copy P_i, so A_jk^T = P_j is read row-major as well.
__global__ void __launch_bounds__(kCB * kTPR) chol_update(double* __restrict__ A, double* __restrict__ X,
                                                          const double* __restrict__ P, int dp, int k, int nb, int d,
                                                          int* info) {
  const int m = nb - k - 1;
  const int64_t T1 = (int64_t)m * (m + 1) / 2;
  const int64_t b = blockIdx.x;
  if (b == 0) {
    // tile (k+1, k+1): update it into LDS, then factor and invert it here
    // (the next block column's diagonal step), while the other workgroups
    // update the rest
    __shared__ double Tl[kCB * kDL];
    __shared__ DiagLdsB S;
    const int I = k + 1;
    tile_update_direct(P + (int64_t)I * kCB * kCB, P + (int64_t)I * kCB * kCB, kCB, tile_at(A, dp, I, I), dp, Tl,
                       kDL);
    __syncthreads();
    diag_blocked(Tl, A, X, dp, I, d, info, S);
  } else if (b < T1) {
    int ii = (int)((sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
    while ((int64_t)ii * (ii + 1) / 2 > b) --ii;
    while ((int64_t)(ii + 1) * (ii + 2) / 2 <= b) ++ii;
    const int jj = (int)(b - (int64_t)ii * (ii + 1) / 2);
    const int I = k + 1 + ii, J = k + 1 + jj;
    tile_update_direct(P + (int64_t)I * kCB * kCB, P + (int64_t)J * kCB * kCB, kCB, tile_at(A, dp, I, J), dp);
  } else {
    const int64_t r = b - T1;
    const int I = k + 1 + (int)(r / (k + 1)), J = (int)(r % (k + 1));
    tile_update_direct(P + (int64_t)I * kCB * kCB, tile_at(X, dp, k, J), dp, tile_at(X, dp, I, J), dp);
  }
}

// U[i][j] = float(X[d-1-i][d-1-j]) for j >= i, 0 below the diagonal.
__global__ void __launch_bounds__(256) chol_store(const double* __restrict__ X, int dp, int d, float* __restrict__ U,
                                                  int64_t ldu) {
  const int i = blockIdx.x;
  const double* row = X + (int64_t)(d - 1 - i) * dp;
  for (int j = threadIdx.x; j < d; j += 256) U[(int64_t)i * ldu + j] = j >= i ? (float)row[d - 1 - j] : 0.0f;
}

}  // namespace

int64_t chol_padded(int64_t d) { return (d + kCB - 1) / kCB * kCB; }

hipError_t launch_chol_inverse_upper(const float* H, int64_t ldh, int d, float* U, int64_t ldu, double* A, double* X,
                                     double* P, int* info, hipStream_t s) {
  const int dp = (int)chol_padded(d);
  const int nb = dp / kCB;
  hipLaunchKernelGGL(chol_load, dim3(dp), dim3(256), 0, s, H, ldh, d, dp, A, X, info);
  hipLaunchKernelGGL(chol_diag, dim3(1), dim3(kCB * kTPR), 0, s, A, X, dp, 0, d, info);
  for (int k = 0; k < nb; ++k) {
    // the update after block column k also factors diagonal tile k + 1
    const int m = nb - k - 1;
    if (m + k > 0) hipLaunchKernelGGL(chol_panel, dim3(4 * m + 2 * k), dim3(256), 0, s, A, X, P, dp, k, nb);
    const int64_t tiles = (int64_t)m * (m + 1) / 2 + (int64_t)m * (k + 1);
    // A trailing update of at most 5 rounds of one workgroup per CU reserves
    // 64 KiB of LDS more than it uses, so that no two of its workgroups share
    // a CU: workgroup 0's diagonal step, the serial chain, then has its CU's
    // float64 units to itself (measured on MI355X: d=2560 1.40 -> 1.31 ms,
    // d=4096 2.56 -> 2.51 ms; reserving it for every update made d=4096
    // slower, 2.72 ms, as its first, largest updates lose residency).
    const size_t excl = tiles <= 5 * 256 ? (size_t)64 << 10 : 0;
    if (tiles > 0)
      hipLaunchKernelGGL(chol_update, dim3((unsigned)tiles), dim3(kCB * kTPR), excl, s, A, X, P, dp, k, nb, d, info);
  }
  hipLaunchKernelGGL(chol_store, dim3(d), dim3(256), 0, s, X, dp, d, U, ldu);
  return hipGetLastError();
}

}  // namespace hess
