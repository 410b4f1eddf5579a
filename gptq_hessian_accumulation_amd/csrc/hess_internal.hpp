// Internal interface between the C ABI layer (hess_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hess {

constexpr int kInBF16 = 0;  // == HESS_BF16
constexpr int kInF32 = 1;   // == HESS_F32

constexpr int kMaxGroups = 64;  // Hessians per grouped launch

struct SyrkGroup {
  float* S;           // d x d float32 Gram sum (row stride SyrkParams::lds)
  float* ws;          // split-partial workspace (split launches only)
  int64_t row_begin;  // this group's token rows: [row_begin, row_end) of X, or of rows[]
  int64_t row_end;
};

struct SyrkParams {
  const void* X;        // tokens x features, row stride ld elements
  const int32_t* rows;  // gather: token t of a group is X row rows[t]; nullptr = identity
  int64_t ld;
  int64_t lds;          // row stride of S
  int d;
  int nb;               // tile rows per dimension, ceil(d / B)
  int ntiles;           // nb (nb + 1) / 2 upper-triangle tiles
  int ngroups;
  int ks;               // token splits per tile (1 = add straight into S)
  int kchunk;           // tokens per split (multiple of 64)
  int flush_iters;      // K-iterations between accumulator flushes
  int total_items;
  int xcd_contig;       // map contiguous item ranges to one XCD
  int s_vec;            // S rows 16-byte aligned (float4 epilogue)
  int item_prefix[kMaxGroups + 1];
  SyrkGroup g[kMaxGroups];
};

int syrk_tile_edge(int wt);
hipError_t launch_syrk(const SyrkParams& P, int wt, int in_dtype, bool vec, hipStream_t stream);
hipError_t launch_syrk_reduce(float* S, int64_t lds, const float* ws, int d, int B, int nb, int ntiles, int ks,
                              hipStream_t stream);

// Materialize: H = neutralize(S * scale) + damp * I.
hipError_t launch_materialize(const float* S, int64_t lds, int d, float scale, float damp_percent, int neutralize,
                              float* H, uint8_t* dead, float* damp_dev, double* sum_scratch, hipStream_t stream);

// Local 16 x 16 block Grams: out[b] (+)= X_b^T X_b.
hipError_t launch_local_blocks(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* out,
                               int accumulate, hipStream_t stream);

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream);

}  // namespace hess
