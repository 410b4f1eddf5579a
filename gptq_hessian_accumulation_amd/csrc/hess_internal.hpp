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
  int64_t row_begin;  // this group's token rows: [row_begin, row_end) of X, or of rows[]
  int64_t row_end;
};

// One SYRK launch.  Single Hessian (ngroups == 1): the first full_tiles
// upper-triangle tiles (row-major order) are each done whole by one
// workgroup, in grid_full workgroups (a multiple of 8, mapped XCD by XCD);
// the remaining tiles are split into tail_parts token ranges of tail_kchunk
// tokens whose partials go to ws and are added by launch_syrk_reduce.
// Grouped (ngroups > 1): group e owns items [item_prefix[e], item_prefix[e+1]),
// one whole tile each.
struct SyrkParams {
  const void* X;        // tokens x features, row stride ld elements
  const int32_t* rows;  // gather: token t of a group is X row rows[t]; nullptr = identity
  int64_t ld;
  int64_t lds;          // row stride of S
  float* ws;            // tail partials, 128 x 128 floats per (tile, part)
  int d;
  int nb;               // tile rows per dimension, ceil(d / 128)
  int ntiles;           // nb (nb + 1) / 2 upper-triangle tiles
  int ngroups;
  int flush_iters;      // K-iterations between accumulator flushes
  int full_tiles;
  int tail_parts;
  int tail_kchunk;      // multiple of 64
  int grid_full;
  int s_vec;            // S rows 16-byte aligned (float4 read-modify-write)
  int item_prefix[kMaxGroups + 1];
  SyrkGroup g[kMaxGroups];
};

// One launch of the 256-tile SYRK (bf16, 16-byte aligned rows, d % 8 == 0).
// Tiles order[0 .. dp_tiles) are done whole, one workgroup each (dp_tiles a
// multiple of 256).  Each of the other sk_tiles tiles is cut into `parts`
// aligned token ranges of part_len 32-token iterations (item = part *
// sk_tiles + tile); workgroup w < grid_sk does item w, and the items past grid_sk
// ("excess", excess_total iterations in all) are shared out evenly over the
// grid_sk workgroups as pieces.  Part 0 of a tile adds into S directly; the
// other parts and all pieces go to workspace slots, which a fixup kernel adds
// into S in a fixed order.
struct BigParams {
  const void* X;          // tokens x features, row stride ld elements; with t8, the transposed
                          // staging layout: 8-token blocks of ld 16-byte chunks (chunk f of
                          // block b = tokens 8b..8b+7 of feature f), n a multiple of 8
  int64_t ld;
  float* S;               // row stride lds
  int64_t lds;
  float* ws;              // 2 * grid_sk + (items - grid_sk) slots of 256 x 256 floats
  const int32_t* order;   // tile t -> (I << 16) | J, blocked order
  int64_t n;              // tokens
  int64_t excess_total;   // (items - grid_sk) * part_len
  int d;
  int nb;                 // 256-tiles per dimension
  int ntiles;
  int niter;              // 32-token iterations: ceil(n / 32)
  int dp_tiles;
  int sk_tiles;
  int parts;
  int part_len;
  int items;              // sk_tiles * parts
  int grid_sk;            // workgroups after the whole-tile ones (<= items)
  int t8;                 // X is in the transposed staging layout
};

// Longest float32 accumulation chain of the 256-tile kernel, in 32-token
// iterations (32,768 tokens): longer pieces of a tile are done as chunks of at
// most this many iterations, each chunk's sums added into the tile's
// destination.
constexpr int kBigChain = 1024;

hipError_t launch_syrk_big(const BigParams& P, hipStream_t stream);
hipError_t launch_syrk_big_fixup(const BigParams& P, hipStream_t stream);

// Grouped 256-tile launch on transposed staging: whole upper tiles of up to
// kBigMaxGroups Hessians of one width, each group's tokens at
// X + blk[g] 8-token blocks (blocks of d 16-byte chunks), n[g] tokens
// (a multiple of 8), sum into S[g] (row stride d).
constexpr int kBigMaxGroups = 64;
struct BigGroupParams {
  const void* X;
  const int32_t* sched;   // workgroup w's items: sched[sched[w] .. sched[w + 1]) (257 offsets first)
  // Rows read in place (tbl non-null): X is the row-major activations (row
  // stride P.ld), group g's token t is at byte offset tbl[blk[g] + t]
  // (blk[g] a multiple of 32; 0x80000000 past the group's rows and for
  // rows outside X; at least 256 entries after the last group's), and
  // xbytes (< 2^31) bounds every read
  const int32_t* tbl;
  int64_t xbytes;
  int nitems;             // ngroups * ntiles (item = group * ntiles + tile)
  int ngroups;
  int64_t blk[kBigMaxGroups];
  int64_t n[kBigMaxGroups];
  float* S[kBigMaxGroups];
};
// P supplies the geometry: order, d, nb, ntiles, ld = lds = d.
hipError_t launch_syrk_big_grouped(const BigParams& P, const BigGroupParams& G, hipStream_t stream);

// Transposed staging copy of gathered rows: group g's rows are
// rows[beg[g] .. beg[g] + cnt[g]) of X (or X rows beg[g] .. if rows is
// null), written as 8-token blocks starting at block blk[g] of dst, the last
// block zero-padded.  blk_prefix[g] = blocks of groups 0..g-1 (the grid).
struct GatherParams {
  const void* X;
  const int32_t* rows;
  void* dst;
  int64_t ld;
  int d;
  int fq;                 // 256-feature quarters per row: ceil(d / 256)
  int ngroups;
  int64_t beg[kBigMaxGroups];
  int64_t cnt[kBigMaxGroups];
  int64_t blk[kBigMaxGroups];
  int64_t blk_prefix[kBigMaxGroups + 1];
};
hipError_t launch_gather_rows_t8(const GatherParams& P, hipStream_t stream);

// Row table of a grouped update that reads the routed rows where they are:
// entry tstart[g] + t (t < cnt[g]) is the byte offset in X of group g's
// token t, the row rows[beg[g] + t] (or beg[g] + t if rows is null) times
// row_bytes; kRowAbsent for the padding of each group to a multiple of 32
// entries, for the entries from tstart[ngroups] up to total, and for a row
// outside [0, nrows).  nrows * row_bytes < 2^31.
constexpr int32_t kRowAbsent = (int32_t)0x80000000u;
constexpr int64_t kRowTableSlack = 256;   // entries after the last group's (read ahead by the SYRK)
struct RowTableParams {
  const int32_t* rows;
  int32_t* tbl;
  int64_t nrows;
  int64_t row_bytes;
  int64_t total;
  int ngroups;
  int64_t beg[kBigMaxGroups];
  int64_t cnt[kBigMaxGroups];
  int64_t tstart[kBigMaxGroups + 1];
};
hipError_t launch_row_table(const RowTableParams& P, hipStream_t stream);

// acc[j] += sum_t X[t][j]^2 (float32), j < d; part holds (max_splits + 32) x d
// floats: split partial sums, then sums of runs of 32 splits.  vec: X 16-byte aligned, ld * esize % 16 == 0
// and d a multiple of 16 / esize.
hipError_t launch_imatrix(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* part,
                          int max_splits, float* acc, hipStream_t stream);

// Thin batches straight into S (bf16 or float32 rows, X 16-byte aligned,
// ld * esize % 16 == 0, d % 8 == 0, n <= kSyrkThinMaxN): 64 x 64
// upper-triangle tiles, one workgroup each, no split and no workspace.
constexpr int64_t kSyrkThinMaxN = 512;
int64_t syrk_thin_tiles(int d);
hipError_t launch_syrk_thin(const void* X, int in_dtype, int64_t ld, int64_t n, int d, float* S, int64_t lds,
                            hipStream_t stream);

int syrk_tile_edge();
hipError_t launch_syrk(const SyrkParams& P, int in_dtype, bool vec, int grid, hipStream_t stream);
hipError_t launch_syrk_reduce(float* S, int64_t lds, const float* ws, int d, int nb, int full_tiles, int tail_tiles,
                              int parts, hipStream_t stream);

// Materialize: H = neutralize(S * scale) + damp * I.
hipError_t launch_materialize(const float* S, int64_t lds, int d, float scale, float damp_percent, int neutralize,
                              float* H, uint8_t* dead, float* damp_dev, double* sum_scratch, hipStream_t stream);

// Local 16 x 16 block Grams: out[b] (+)= X_b^T X_b, through per-workgroup
// partial sums in a scratch buffer of plan.part_bytes (slices x d/16 x 1 KB)
// added in a fixed order.
constexpr int64_t kLocalPartBytes = (int64_t)16 << 20;  // the scratch every plan fits in (d <= 262,144)
struct LocalPlan {
  int gx;            // 256-feature columns
  int64_t gy;        // token runs (scratch slices)
  int64_t tpw;       // tokens per run, a multiple of 32
  int64_t part_bytes;
};
LocalPlan local_plan(int64_t n, int d, int64_t part_bytes);
// Device address, on the current device, of the fixed kLocalPartBytes array
// used by the allocation-free local-block call (looked up once per device).
hipError_t local_static_scratch(float** out);
hipError_t launch_local_blocks(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* out,
                               int accumulate, const LocalPlan& plan, float* part, hipStream_t stream);

// Materialize of many Hessians of one width (all 16-byte aligned, d % 4 == 0)
// in two launches, bit for bit what launch_materialize gives each of them.
constexpr int kMatMaxGroups = 64;
struct MatGroup {
  const float* S;
  float* H;        // may equal S (in place)
  uint8_t* dead;
  float* damp;
  float scale;
};
struct MatGroupParams {
  int ngroups;
  int d;
  int64_t lds;
  float damp_percent;
  int neutralize;
  MatGroup g[kMatMaxGroups];
};
bool materialize_grouped_ok(const MatGroupParams& P);
hipError_t launch_materialize_grouped(const MatGroupParams& P, hipStream_t stream);
struct ZeroGroupParams {
  float* S[kMatMaxGroups];
  int64_t lds;
  int d;
  int vec;
};
hipError_t launch_zero_upper_grouped(float* const* S, int n, int64_t lds, int d, hipStream_t stream);

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream);
// Zero S's rows from column 256 * (row / 256) on: the upper triangle and every
// diagonal tile the SYRK kernels read or write.
hipError_t launch_zero_upper(float* S, int64_t lds, int d, hipStream_t stream);

// Error-propagating 4-bit quantization of W (rows x cols) with the factor U.
struct QuantParams {
  const float* W;
  int64_t ldw;
  int rows;
  int cols;
  const float* U;
  int64_t ldu;
  const uint8_t* dead;  // nullable: columns to zero first
  int group;            // <= 0 or >= cols: whole rows; else a divisor of 128
  float* Q;
  int64_t ldq;
  uint8_t* codes;
  int64_t ldc;
  float* scales;        // rows x groups
  double* loss;         // nullable
  int64_t nsamples;
  double* work;         // quant_workspace_doubles(rows, cols)
};
int64_t quant_workspace_doubles(int64_t rows, int64_t cols);
hipError_t launch_gptq_quantize(const QuantParams& P, hipStream_t stream);

// Upper Cholesky factor of the inverse: U (d x d float32, row stride ldu,
// zeros below the diagonal) with U^T U = H^-1, from the upper triangle of H
// (row stride ldh).  A and X are chol_padded(d)^2 float64 each, P is
// chol_padded(d) x 64 float64; info (device, nullable) receives 0 or 1 + the
// largest H column whose pivot failed.
int64_t chol_padded(int64_t d);
hipError_t launch_chol_inverse_upper(const float* H, int64_t ldh, int d, float* U, int64_t ldu, double* A, double* X,
                                     double* P, int* info, hipStream_t stream);

// Transposed staging copy (bf16): n rows of X (row stride ld) into 8-token
// blocks at dst, chunk f of block b = tokens 8b..8b+7 of feature f (16
// bytes), blocks of d chunks; rows n .. round_up(n, 8) - 1 are written as zeros.
hipError_t launch_copy_rows_t8(const void* X, int64_t ld, int64_t n, int64_t d, void* dst, hipStream_t stream);

// Converting staging copy: n rows of X (element type x_dtype: 0 bf16, 1
// float32, 2 fp16; row stride ld elements) into dst of type dst_dtype (0
// bf16, 1 float32), either row-major with row stride dld or (t8, bf16 only)
// in the transposed 8-token layout of launch_copy_rows_t8.  Narrowing rounds
// to nearest even; widening is exact.  Same-type pairs are not handled here.
hipError_t launch_cast_rows(const void* X, int x_dtype, int64_t ld, int64_t n, int64_t d, void* dst, int dst_dtype,
                            int64_t dld, bool t8, hipStream_t stream);

// Copy n rows of d elements (esize bytes each) from X (row stride ld) to dst (row stride dld).
hipError_t launch_copy_rows(const void* X, int64_t ld, int esize, int64_t n, int64_t d, void* dst, int64_t dld,
                            hipStream_t stream);

}  // namespace hess
