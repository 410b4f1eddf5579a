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

}  // namespace

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
