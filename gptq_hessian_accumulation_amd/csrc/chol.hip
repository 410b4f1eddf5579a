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
//           and registers, writing L_kk into A_kk and L_kk^-1 into X_kk
//           (for k > 0 inside the previous update launch: its first
//           workgroup updates A_kk and factors it while the others update
//           the rest);
//   panel   A_ik <- A_ik L_kk^-T below the diagonal (a product with the
//           inverse, so it runs on the matrix cores) and, for the inverse,
//           X_kj <- L_kk^-1 X_kj left of it (block forward substitution);
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

// C (64 x 64 tile at Cg, row stride dp) = init + sign * P, where P = A B^T
// (BT) or A B, with A and B 64 x 64 tiles in LDS.  init is C's old value
// (accumulate) or zero.  Wave w computes rows 32 (w >> 1) .. +31 and columns
// 32 (w & 1) .. +31 as 2 x 2 blocks of 16 x 16.
template <bool BT, bool ACCUM, bool NEG>
__device__ __forceinline__ void tile_product(const double* Al, const double* Bl, double* __restrict__ Cg, int64_t dp,
                                             double* __restrict__ Ct = nullptr) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = 32 * (w >> 1), c0 = 32 * (w & 1);
  const int li = lane & 15, lk = lane >> 4;
  f64x4 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[rb][cb][r] = ACCUM ? Cg[(int64_t)(r0 + 16 * rb + lk + 4 * r) * dp + c0 + 16 * cb + li] : 0.0;
    }
#pragma unroll 4
  for (int kk = 0; kk < kCB; kk += 4) {
    double a[2], b[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const double v = Al[(r0 + 16 * rb + li) * kLdsLd + kk + lk];
      a[rb] = NEG ? -v : v;
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      b[cb] = BT ? Bl[(c0 + 16 * cb + li) * kLdsLd + kk + lk] : Bl[(kk + lk) * kLdsLd + c0 + 16 * cb + li];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma_f64(a[rb], b[cb], acc[rb][cb]);
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Cg[(int64_t)(r0 + 16 * rb + lk + 4 * r) * dp + c0 + 16 * cb + li] = acc[rb][cb][r];
        if (Ct) Ct[(c0 + 16 * cb + li) * kCB + r0 + 16 * rb + lk + 4 * r] = acc[rb][cb][r];
      }
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

// Factor and invert the diagonal tile k.  512 threads: thread t owns row
// i = t / 8 and the columns cls + 8 m (cls = t % 8, m < 8) of Y (becoming
// L^-1, starting as the identity) and of T (the tile being factored).  Step
// j takes, from LDS, the column of T as it stands after steps 0 .. j-1
// (colv[r] = T[r][j] for r >= j, zero above), the row Y[j][.] (rowv; zero
// past j) and the pivot's square root l and reciprocal, all published by
// their owners during step j-1, so each step needs one barrier and issues all
// its LDS reads at once.  Column j of L (colv / l) is kept in LDS and written
// out with the tile at the end; the rank-one updates
// T[i][c] -= L[i][j] L[c][j] and Y[i][c] -= L[i][j] Y[j][c] / l are applied
// to every owned entry without tests: the zeros in colv and rowv leave the
// finished columns and the zero upper part of Y alone, and the entries of T
// above the diagonal or left of column j are never read again.  After every
// 8 steps the T registers shift down by one, dropping a finished column, so
// that the column of the next pivot always sits in a fixed register.  The
// owner of T[j+1][j+1] takes the next pivot's square root one step ahead of
// its use.
constexpr int kTPR = 8;               // threads per tile row (workgroup of kCB * kTPR)
constexpr int kPer = kCB / kTPR;      // owned columns per thread

struct DiagLds {
  double colv[2][2 * kCB];  // entries past kCB stay zero (reads for shifted-out registers)
  double rowv[2][kCB];
  double pv[2][2];
  double Lt[kCB * (kCB + 1)];  // the finished columns of L, written out at the end
};

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

// The tile to factor is read from src (row stride lds: global memory, or the
// LDS copy left by the fused update).  The caller synchronizes the workgroup
// after src is complete.
__device__ __forceinline__ void diag_body(const double* src, int64_t lds, double* __restrict__ A,
                                          double* __restrict__ X, int dp, int k, int d, int* info, DiagLds& S) {
  auto& colv = S.colv;
  auto& rowv = S.rowv;
  auto& pv = S.pv;
  const int t = threadIdx.x;
  const int i = t / kTPR, cls = t % kTPR;
  double* Ag = tile_at(A, dp, k, k);
  double* Xg = tile_at(X, dp, k, k);
  double T[kPer], Y[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int c = cls + kTPR * m;
    T[m] = src[(int64_t)i * lds + c];
    Y[m] = c == i ? 1.0 : 0.0;
  }
  if (t < 2 * kCB) {
    colv[0][kCB + (t & (kCB - 1))] = 0.0;
    colv[1][kCB + (t & (kCB - 1))] = 0.0;
  }
  // step 0's inputs: column 0, row 0 of Y, the first pivot
  if (cls == 0) colv[0][i] = T[0];
  if (i == 0) {
#pragma unroll
    for (int m = 0; m < kPer; ++m) rowv[0][cls + kTPR * m] = Y[m];
    if (cls == 0) {
      report_pivot(T[0], k * kCB, d, info);
      pivot_root(T[0], pv[0][0], pv[0][1]);
    }
  }
  __syncthreads();
  for (int jb = 0; jb < kCB; jb += kTPR) {
    const int cb = cls + jb;  // column held by T[0] in this block of steps
#pragma unroll
    for (int u = 0; u < kTPR; ++u) {
      const int j = jb + u;
      const int b = u & 1, nb = b ^ 1;
      // every read of the step at once: one LDS latency
      const double l = pv[b][0], inv = pv[b][1];
      const double ci = colv[b][i];
      double cv[kPer], rv[kPer];
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        cv[m] = colv[b][cb + kTPR * m];
        rv[m] = rowv[b][cls + kTPR * m];
      }
      const double lij = i > j ? ci * inv : 0.0;
      const double f = lij * inv;
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        T[m] = fma(-f, cv[m], T[m]);
        Y[m] = fma(-f, rv[m], Y[m]);
      }
      const double ys = i == j ? inv : 1.0;  // row j of L^-1
#pragma unroll
      for (int m = 0; m < kPer; ++m) Y[m] *= ys;
      if (cls == u && i >= j) S.Lt[i * (kCB + 1) + j] = i == j ? l : lij;  // column j of L
      const int c1 = j + 1;
      if (c1 < kCB) {
        // column c1 is T[0] of owner cls = u + 1, or T[1] of cls = 0 after the block's last step
        const bool owner = cls == (u + 1) % kTPR;
        const double next = (u + 1 < kTPR) ? T[0] : T[1];
        double nl, ny;
        pivot_root(next, nl, ny);
        if (owner) colv[nb][i] = i >= c1 ? next : 0.0;
        if (i == c1) {
#pragma unroll
          for (int m = 0; m < kPer; ++m) rowv[nb][cls + kTPR * m] = Y[m];
          if (owner) {
            report_pivot(next, k * kCB + c1, d, info);
            pv[nb][0] = nl;
            pv[nb][1] = ny;
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int m = 0; m + 1 < kPer; ++m) T[m] = T[m + 1];
    T[kPer - 1] = 0.0;
  }
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int c = cls + kTPR * m;
    Xg[(int64_t)i * dp + c] = Y[m];
    Ag[(int64_t)i * dp + c] = c <= i ? S.Lt[i * (kCB + 1) + c] : 0.0;
  }
}

__global__ void __launch_bounds__(kCB * kTPR) chol_diag(double* __restrict__ A, double* __restrict__ X, int dp, int k,
                                                        int d, int* info) {
  __shared__ DiagLds S;
  diag_body(tile_at(A, dp, k, k), dp, A, X, dp, k, d, info, S);
}

// Panel of block column k: workgroups b < m = nb - k - 1 take A_ib (i = k + 1
// + b) <- A_ib L_kk^-T, also written transposed to P_i (64 x 64, P_i[c][r] =
// A_ib[r][c]) for the update's fragment loads; the others take X_kj
// (j = b - m < k) <- L_kk^-1 X_kj.
__global__ void __launch_bounds__(256) chol_panel(double* __restrict__ A, double* __restrict__ X,
                                                  double* __restrict__ P, int dp, int k, int nb) {
  __shared__ __attribute__((aligned(16))) double Al[kCB * kLdsLd];
  __shared__ __attribute__((aligned(16))) double Bl[kCB * kLdsLd];
  const int m = nb - k - 1;
  const int b = blockIdx.x;
  if (b < m) {
    double* C = tile_at(A, dp, k + 1 + b, k);
    tile_to_lds(C, dp, Al);
    tile_to_lds(tile_at(X, dp, k, k), dp, Bl);
    __syncthreads();
    tile_product<true, false, false>(Al, Bl, C, dp, P + (int64_t)(k + 1 + b) * kCB * kCB);
  } else {
    double* C = tile_at(X, dp, k, b - m);
    tile_to_lds(tile_at(X, dp, k, k), dp, Al);
    tile_to_lds(C, dp, Bl);
    __syncthreads();
    tile_product<false, false, false>(Al, Bl, C, dp);
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
    __shared__ double Tl[kCB * kCB];
    __shared__ DiagLds S;
    const int I = k + 1;
    tile_update_direct(P + (int64_t)I * kCB * kCB, P + (int64_t)I * kCB * kCB, kCB, tile_at(A, dp, I, I), dp, Tl,
                       kCB);
    __syncthreads();
    diag_body(Tl, kCB, A, X, dp, I, d, info, S);
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
    if (m + k > 0) hipLaunchKernelGGL(chol_panel, dim3(m + k), dim3(256), 0, s, A, X, P, dp, k, nb);
    const int64_t tiles = (int64_t)m * (m + 1) / 2 + (int64_t)m * (k + 1);
    if (tiles > 0)
      hipLaunchKernelGGL(chol_update, dim3((unsigned)tiles), dim3(kCB * kTPR), 0, s, A, X, P, dp, k, nb, d, info);
  }
  hipLaunchKernelGGL(chol_store, dim3(d), dim3(256), 0, s, X, dp, d, U, ldu);
  return hipGetLastError();
}

}  // namespace hess
