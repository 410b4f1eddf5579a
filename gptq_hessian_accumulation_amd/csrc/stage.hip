// Row copy into a Hessian's staging buffer (the thin-batch path).
//
// A batch with fewer tokens than about d is not worth its own pass over the
// d x d sum (a 4 d^2-byte read-modify-write of the upper triangle): its rows
// are appended to a per-handle staging buffer instead (2 n d esize bytes of
// traffic) and the buffer is folded into S by one long SYRK when it fills or
// when the Hessian is materialized.  The sum of the per-batch Gram matrices
// is the Gram matrix of the concatenated rows, so only the float32 rounding
// order changes.
//
// The copy is a bandwidth kernel: 16-byte vector moves when rows allow it,
// element moves otherwise.
//
// bf16 handles whose flushes take the 256-tile kernel stage in that kernel's
// operand layout instead: 8-token blocks, each d 16-byte chunks holding 8
// consecutive tokens of one feature (the k-run of one matrix-core operand
// lane), with every batch padded by zero rows to a multiple of 8 tokens.
// Zero rows add nothing to the Gram sum.
//
// Activations of another type than the handle's staging type are converted
// by the copy: fp16 and bf16 widen exactly to float32, float32 and fp16 are
// rounded to the nearest bf16 (ties to even).  This is the staging dtype of
// GPTQModel PR 3052 ("Shared-input Hessian dedup", review finding P2) and
// Model-Optimizer's hessian_input_dtype (PR 3002 page, "What does this PR
// do?").

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Grid-stride 16-byte moves, for any size.
__global__ void __launch_bounds__(256) copy_rows_vec(const char* X, int64_t ld_bytes, char* dst, int64_t dld_bytes,
                                                     int64_t n, int64_t chunks_per_row) {
  const int64_t total = n * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / chunks_per_row, c = i - r * chunks_per_row;
    *reinterpret_cast<u32x4_t*>(dst + r * dld_bytes + c * 16) =
        *reinterpret_cast<const u32x4_t*>(X + r * ld_bytes + c * 16);
  }
}

// Staging-size copies (fewer than 2^31 chunks): one 16-byte chunk per
// thread with 32-bit index arithmetic; many small workgroups keep the most
// requests in flight for these few-megabyte copies.
__global__ void __launch_bounds__(256) copy_rows_vec32(const char* X, int64_t ld_bytes, char* dst, int64_t dld_bytes,
                                                       uint32_t total, uint32_t chunks_per_row) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= total) return;
  const uint32_t r = i / chunks_per_row, c = i - r * chunks_per_row;
  *reinterpret_cast<u32x4_t*>(dst + (int64_t)r * dld_bytes + c * 16u) =
      *reinterpret_cast<const u32x4_t*>(X + (int64_t)r * ld_bytes + c * 16u);
}

template <typename E>
__global__ void __launch_bounds__(256) copy_rows_elem(const E* X, int64_t ld, E* dst, int64_t dld, int64_t n,
                                                      int64_t d) {
  const int64_t total = n * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / d, c = i - r * d;
    dst[r * dld + c] = X[r * ld + c];
  }
}

// Element types of the rows a staging copy reads (the public dtype codes).
constexpr int kSrcBF16 = 0, kSrcF32 = 1, kSrcF16 = 2;

// Exact widening of one stored element to float32.
template <int SRC>
__device__ __forceinline__ float load_f32(const void* X, int64_t i) {
  if constexpr (SRC == kSrcF32) return static_cast<const float*>(X)[i];
  else if constexpr (SRC == kSrcF16) return (float)static_cast<const _Float16*>(X)[i];
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(X)[i]);
}

// Eight consecutive elements at p (16-byte aligned) as eight bf16 values in
// four dwords (element 2k in the low half of dword k), rounded to nearest even.
// Activations are read once, so the loads are non-temporal.
template <int SRC>
__device__ __forceinline__ u32x4 load8_bf16(const char* p) {
  if constexpr (SRC == kSrcBF16) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else if constexpr (SRC == kSrcF32) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 16));
    u32x4 o;
    o[0] = f32_to_bf16_bits(__uint_as_float(a[0])) | (f32_to_bf16_bits(__uint_as_float(a[1])) << 16);
    o[1] = f32_to_bf16_bits(__uint_as_float(a[2])) | (f32_to_bf16_bits(__uint_as_float(a[3])) << 16);
    o[2] = f32_to_bf16_bits(__uint_as_float(b[0])) | (f32_to_bf16_bits(__uint_as_float(b[1])) << 16);
    o[3] = f32_to_bf16_bits(__uint_as_float(b[2])) | (f32_to_bf16_bits(__uint_as_float(b[3])) << 16);
    return o;
  } else {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[k] & 0xFFFFu));
      const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[k] >> 16));
      o[k] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
    return o;
  }
}

// Transposed staging copy, 16-byte aligned rows: workgroup (g, F) moves
// tokens 8g..8g+7 (zeros past n) of features F .. F + kCQ * 256 - 1.  Its
// 256 threads read the 8 rows' pieces into LDS with 16-byte loads (all
// quarters' loads in flight at once), then thread t gathers each quarter's
// feature F + 256 k + t over the 8 tokens and writes them as one chunk, so
// that both the reads and the writes are contiguous across the workgroup.
// The staged rows are read back only by a later flush, long after the L2 has
// turned over, so they are written non-temporally (measured 1.5-2% faster
// per Hessian on the ragged d=2560 workload).
// Rows of fp16 or float32 are rounded to bf16 on the way.
constexpr int kCQ = 2;
template <int SRC>
__device__ __forceinline__ void t8_body(const char* X, int64_t ld_bytes, char* dst, int64_t n, int d, int nq) {
  constexpr int xes = SRC == kSrcF32 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t tile[kCQ][8][256];
  const int t = threadIdx.x;
  const int64_t g = blockIdx.x / nq;
  const int F = (int)(blockIdx.x - g * nq) * (kCQ * 256);
  {
    const int r = t >> 5, q = t & 31;
    const int64_t tok = 8 * g + r;
    u32x4 v[kCQ];
#pragma unroll
    for (int k = 0; k < kCQ; ++k) {
      const int f = F + k * 256 + 8 * q;
      v[k] = (tok < n && f < d) ? load8_bf16<SRC>(X + tok * ld_bytes + (int64_t)f * xes) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kCQ; ++k) *reinterpret_cast<u32x4*>(&tile[k][r][8 * q]) = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kCQ; ++k) {
    const int f = F + k * 256 + t;
    if (f < d) {
      u32x4 c;
#pragma unroll
      for (int p = 0; p < 4; ++p) c[p] = (uint32_t)tile[k][2 * p][t] | ((uint32_t)tile[k][2 * p + 1][t] << 16);
      __builtin_nontemporal_store(c, reinterpret_cast<u32x4*>(dst + (g * d + f) * 16));
    }
  }
}

__global__ void __launch_bounds__(256) copy_rows_t8(const char* X, int64_t ld_bytes, char* dst, int64_t n, int d,
                                                    int nq) {
  t8_body<kSrcBF16>(X, ld_bytes, dst, n, d, nq);
}

template <int SRC>
__global__ void __launch_bounds__(256) cast_rows_t8(const char* X, int64_t ld_bytes, char* dst, int64_t n, int d,
                                                    int nq) {
  t8_body<SRC>(X, ld_bytes, dst, n, d, nq);
}

// Transposed staging copy, any alignment: one element per thread.
__global__ void __launch_bounds__(256) copy_rows_t8_elem(const uint16_t* X, int64_t ld, uint16_t* dst, int64_t n,
                                                         int64_t d, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / d, f = i - t * d;
    dst[((t >> 3) * d + f) * 8 + (t & 7)] = t < n ? X[t * ld + f] : (uint16_t)0;
  }
}

template <int SRC>
__global__ void __launch_bounds__(256) cast_rows_t8_elem(const void* X, int64_t ld, uint16_t* dst, int64_t n,
                                                         int64_t d, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / d, f = i - t * d;
    dst[((t >> 3) * d + f) * 8 + (t & 7)] = t < n ? (uint16_t)f32_to_bf16_bits(load_f32<SRC>(X, t * ld + f)) : 0;
  }
}

// Row-major converting copy into a bf16 (DST = 0) or float32 (DST = 1)
// staging buffer.  vec: eight elements per thread (d % 8 == 0, rows and
// destination 16-byte aligned); otherwise one element per thread.
template <int SRC, int DST, bool VEC>
__global__ void __launch_bounds__(256) cast_rows(const void* X, int64_t ld, void* dst, int64_t dld, int64_t n,
                                                 int64_t d) {
  constexpr int xes = SRC == kSrcF32 ? 4 : 2;
  const int64_t per_row = VEC ? d / 8 : d;
  const int64_t total = n * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row, c = i - r * per_row;
    if constexpr (VEC) {
      if constexpr (DST == 0) {
        const char* p = static_cast<const char*>(X) + (r * ld + 8 * c) * xes;
        *reinterpret_cast<u32x4*>(static_cast<char*>(dst) + (r * dld + 8 * c) * 2) = load8_bf16<SRC>(p);
      } else {
        float* o = static_cast<float*>(dst) + r * dld + 8 * c;
        f32x4 a, b;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a[k] = load_f32<SRC>(X, r * ld + 8 * c + k);
          b[k] = load_f32<SRC>(X, r * ld + 8 * c + 4 + k);
        }
        *reinterpret_cast<f32x4*>(o) = a;
        *reinterpret_cast<f32x4*>(o + 4) = b;
      }
    } else {
      const float v = load_f32<SRC>(X, r * ld + c);
      if constexpr (DST == 0) static_cast<uint16_t*>(dst)[r * dld + c] = (uint16_t)f32_to_bf16_bits(v);
      else static_cast<float*>(dst)[r * dld + c] = v;
    }
  }
}

// Transposed staging copy of gathered rows for grouped updates: workgroup
// (block, quarter pair) finds its group by the block prefix, then moves
// tokens 8 block .. +7 of features F .. F + kGQ * 256 - 1 as copy_rows_t8
// does, with each token's row looked up in rows (or taken in order); the
// loads of all its quarters are issued before the first is written.  Rows
// are 16-byte aligned (checked by the caller).
constexpr int kGQ = 4;
__global__ void __launch_bounds__(256) gather_rows_t8(GatherParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kGQ][8][256];
  const int t = threadIdx.x;
  const int nq = (P.fq + kGQ - 1) / kGQ;
  const int64_t gb = blockIdx.x / nq;
  const int F0 = (int)(blockIdx.x - gb * nq) * (kGQ * 256);
  int lo = 0, hi = P.ngroups;  // last group g with blk_prefix[g] <= gb
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.blk_prefix[mid] <= gb) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const int64_t b = gb - P.blk_prefix[g];
  {
    const int r = t >> 5, q = t & 31;
    const int64_t tok = 8 * b + r;
    const bool valid = tok < P.cnt[g];
    int64_t row = 0;
    if (valid) {
      const int64_t pos = P.beg[g] + tok;
      row = P.rows ? (int64_t)P.rows[pos] : pos;
    }
    const char* src = static_cast<const char*>(P.X) + row * P.ld * 2;
    u32x4 v[kGQ];
#pragma unroll
    for (int k = 0; k < kGQ; ++k) {
      const int f = F0 + k * 256 + 8 * q;
      v[k] = (valid && f < P.d) ? *reinterpret_cast<const u32x4*>(src + (int64_t)f * 2) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kGQ; ++k) *reinterpret_cast<u32x4*>(&tile[k][r][8 * q]) = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kGQ; ++k) {
    const int f = F0 + k * 256 + t;
    if (f < P.d) {
      u32x4 c;
#pragma unroll
      for (int p = 0; p < 4; ++p) c[p] = (uint32_t)tile[k][2 * p][t] | ((uint32_t)tile[k][2 * p + 1][t] << 16);
      *reinterpret_cast<u32x4*>(static_cast<char*>(P.dst) + ((P.blk[g] + b) * P.d + f) * 16) = c;
    }
  }
}

// The row table of a grouped update read in place (RowTableParams): one
// entry per thread, its group found by binary search over tstart.
__global__ void __launch_bounds__(256) row_table(RowTableParams P) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= P.total) return;
  int32_t v = kRowAbsent;
  if (i < P.tstart[P.ngroups]) {
    int lo = 0, hi = P.ngroups;  // last group g with tstart[g] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (P.tstart[mid] <= i) lo = mid;
      else hi = mid;
    }
    const int64_t t = i - P.tstart[lo];
    if (t < P.cnt[lo]) {
      const int64_t pos = P.beg[lo] + t;
      const int64_t row = P.rows ? (int64_t)P.rows[pos] : pos;
      if (row >= 0 && row < P.nrows) v = (int32_t)(row * P.row_bytes);
    }
  }
  P.tbl[i] = v;
}

}  // namespace

hipError_t launch_row_table(const RowTableParams& P, hipStream_t stream) {
  if (P.total <= 0) return hipSuccess;
  const int64_t wgs = (P.total + 255) / 256;
  if (wgs >= ((int64_t)1 << 31) || P.nrows * P.row_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_table, dim3((unsigned)wgs), dim3(256), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_gather_rows_t8(const GatherParams& P, hipStream_t stream) {
  const int64_t wgs = P.blk_prefix[P.ngroups] * ((P.fq + kGQ - 1) / kGQ);
  if (wgs <= 0) return hipSuccess;
  if (wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_t8, dim3((unsigned)wgs), dim3(256), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_copy_rows_t8(const void* X, int64_t ld, int64_t n, int64_t d, void* dst, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (d % 8 != 0) return hipErrorInvalidValue;
  const int64_t blocks8 = (n + 7) / 8;
  const bool vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0 &&
                   ((ld * 2) & 15) == 0;
  const int64_t nq = (d + kCQ * 256 - 1) / (kCQ * 256);
  const int64_t wgs = blocks8 * nq;
  if (vec && wgs < ((int64_t)1 << 31)) {
    hipLaunchKernelGGL(copy_rows_t8, dim3((unsigned)wgs), dim3(256), 0, stream, static_cast<const char*>(X), ld * 2,
                       static_cast<char*>(dst), n, (int)d, (int)nq);
  } else {
    const int64_t elems = blocks8 * 8 * d;
    int64_t blocks = (elems + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(copy_rows_t8_elem, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(X), ld, static_cast<uint16_t*>(dst), n, d, elems);
  }
  return hipGetLastError();
}

namespace {

int grid_for(int64_t items) {
  int64_t blocks = (items + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  return (int)(blocks > 0 ? blocks : 1);
}

template <int SRC>
hipError_t cast_t8(const void* X, int64_t ld, int64_t n, int64_t d, void* dst, hipStream_t stream) {
  constexpr int xes = SRC == kSrcF32 ? 4 : 2;
  const int64_t blocks8 = (n + 7) / 8;
  const bool vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0 &&
                   ((ld * xes) & 15) == 0;
  const int64_t nq = (d + kCQ * 256 - 1) / (kCQ * 256);
  const int64_t wgs = blocks8 * nq;
  if (vec && wgs < ((int64_t)1 << 31)) {
    hipLaunchKernelGGL(cast_rows_t8<SRC>, dim3((unsigned)wgs), dim3(256), 0, stream, static_cast<const char*>(X),
                       ld * xes, static_cast<char*>(dst), n, (int)d, (int)nq);
  } else {
    const int64_t elems = blocks8 * 8 * d;
    hipLaunchKernelGGL(cast_rows_t8_elem<SRC>, dim3(grid_for(elems)), dim3(256), 0, stream, X, ld,
                       static_cast<uint16_t*>(dst), n, d, elems);
  }
  return hipGetLastError();
}

template <int SRC, int DST>
hipError_t cast_rm(const void* X, int64_t ld, int64_t n, int64_t d, void* dst, int64_t dld, hipStream_t stream) {
  constexpr int xes = SRC == kSrcF32 ? 4 : 2;
  constexpr int des = DST == 0 ? 2 : 4;
  const bool vec = d % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(dst) & 15u) == 0 && ((ld * xes) & 15) == 0 && ((dld * des) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((cast_rows<SRC, DST, true>), dim3(grid_for(n * (d / 8))), dim3(256), 0, stream, X, ld, dst,
                       dld, n, d);
  else
    hipLaunchKernelGGL((cast_rows<SRC, DST, false>), dim3(grid_for(n * d)), dim3(256), 0, stream, X, ld, dst, dld,
                       n, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cast_rows(const void* X, int x_dtype, int64_t ld, int64_t n, int64_t d, void* dst, int dst_dtype,
                            int64_t dld, bool t8, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (t8) {
    if (dst_dtype != kSrcBF16 || d % 8 != 0) return hipErrorInvalidValue;
    if (x_dtype == kSrcF32) return cast_t8<kSrcF32>(X, ld, n, d, dst, stream);
    if (x_dtype == kSrcF16) return cast_t8<kSrcF16>(X, ld, n, d, dst, stream);
    return hipErrorInvalidValue;
  }
  if (dst_dtype == kSrcBF16) {
    if (x_dtype == kSrcF32) return cast_rm<kSrcF32, 0>(X, ld, n, d, dst, dld, stream);
    if (x_dtype == kSrcF16) return cast_rm<kSrcF16, 0>(X, ld, n, d, dst, dld, stream);
  } else if (dst_dtype == kSrcF32) {
    if (x_dtype == kSrcBF16) return cast_rm<kSrcBF16, 1>(X, ld, n, d, dst, dld, stream);
    if (x_dtype == kSrcF16) return cast_rm<kSrcF16, 1>(X, ld, n, d, dst, dld, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_copy_rows(const void* X, int64_t ld, int esize, int64_t n, int64_t d, void* dst, int64_t dld,
                            hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const bool vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0 &&
                   ((ld * esize) & 15) == 0 && ((dld * esize) & 15) == 0 && ((d * esize) & 15) == 0;
  if (vec) {
    const int64_t cpr = d * esize / 16;
    const int64_t total = n * cpr;
    if (total < ((int64_t)1 << 31)) {
      const int64_t blocks = (total + 255) / 256;
      hipLaunchKernelGGL(copy_rows_vec32, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const char*>(X),
                         ld * esize, static_cast<char*>(dst), dld * esize, (uint32_t)total, (uint32_t)cpr);
    } else {
      const int64_t blocks = 8192;
      hipLaunchKernelGGL(copy_rows_vec, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const char*>(X),
                         ld * esize, static_cast<char*>(dst), dld * esize, n, cpr);
    }
  } else {
    int64_t blocks = (n * d + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (esize == 2)
      hipLaunchKernelGGL(copy_rows_elem<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(X), ld, static_cast<uint16_t*>(dst), dld, n, d);
    else
      hipLaunchKernelGGL(copy_rows_elem<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         static_cast<const uint32_t*>(X), ld, static_cast<uint32_t*>(dst), dld, n, d);
  }
  return hipGetLastError();
}

}  // namespace hess
