/*
 * hess.h -- calibration-Hessian accumulation on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libhess.so.  The library accumulates the GPTQ/QQQ calibration
 * Hessian H = (2/N) * sum_t x_t x_t^T of a linear layer's input activations
 * on one GPU, and builds the 16x16 per-block "local" Hessians.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Activations X are device memory, row-major tokens x features: element
 *   (t, j) is at X[t*ld + j], with ld >= d elements.  bf16 or float32.
 * - The Gram sum S, H_out, local blocks and dead masks are device memory.
 *   Pointers marked (host) are host memory.
 * - Every device operation is enqueued on the given HIP stream
 *   (hipStream_t passed as hess_stream_t; NULL is the null stream).  Apart
 *   from create and destroy calls, hess_timing and hess_add_batch_grouped(_ex),
 *   no call synchronizes with the host or allocates device memory, so those
 *   calls (batches, casts, flush, reset, materialize, adopt, imatrix, the
 *   Cholesky factor, the block quantize, and local blocks after the first
 *   call on a device, which allocates the device's partial-sum scratch) may
 *   be captured into a HIP graph.  hess_add_batch_grouped builds each launch's schedule on the
 *   host, sends it through a pinned buffer after the previous call's copy
 *   has finished, and sizes the device's gather buffer on first use: it is
 *   not for capture.  X must stay valid and unchanged until the stream has
 *   executed the call.
 * - A handle remembers the stream of its last call.  A call on a different
 *   stream first makes that stream wait for the previous one (an event), so
 *   updates of one Hessian never overlap.  Different handles are independent.
 *   Every call on a handle holds that handle's lock for its duration (grouped
 *   calls lock their handles in address order), so calls from several host
 *   threads never interleave; between threads, the order of the calls is the
 *   order in which they take the lock (GPTQModel PR 2979 serializes updates
 *   of one device's accumulator the same way, with a lock).
 * - Errors are returned as negative codes; the library never aborts and has
 *   no fallback paths.  hess_last_error() gives the calling thread's message
 *   for its last failed call.
 *
 * Page citations below refer to: GPTQModel PR 2979 "fix(qqq): per-device
 * Hessian partials for balanced multi-GPU calibration"; GPTQModel PR 2981
 * "fix(qqq): accumulate Hessian in-place per device to reduce memory";
 * NVIDIA Model-Optimizer PR 3002 page ("hessian_input_dtype"); GPTQModel
 * wiki "QQQ".
 */
#ifndef HESS_H
#define HESS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HESS_ABI_VERSION 1

typedef struct hess_s* hess_t;
typedef struct hess_imx_s* hess_imx_t;
typedef void* hess_stream_t; /* a hipStream_t */

/* Element types.  A handle's staging dtype (HESS_BF16 or HESS_F32) is the
 * type its products are formed in: bf16 products are exact in float32 and
 * summed in float32 (Model-Optimizer PR 3002 page, "What does this PR do?":
 * bfloat16 in, float32 out); float32 inputs are multiplied to float32
 * accuracy.  Activations may also be HESS_F16 (hess_add_batch_cast only). */
enum hess_dtype { HESS_BF16 = 0, HESS_F32 = 1, HESS_F16 = 2 };

enum hess_status {
  HESS_OK = 0,
  HESS_EINVAL = -1, /* invalid argument */
  HESS_ENOMEM = -2, /* device allocation failed (hess_create only) */
  HESS_EHIP = -3,   /* a HIP runtime or launch error; see hess_last_error() */
  HESS_ESTATE = -4, /* handle consumed by an in-place materialize */
  HESS_EALIGN = -5, /* X not aligned to its element size */
  HESS_ENOTPD = -6  /* a matrix to factor is not positive definite (reported by
                       bindings after reading hess_chol_inverse_upper's info) */
};

/* hess_materialize_ex flags */
#define HESS_NO_NEUTRALIZE 1u /* skip dead-column neutralization */

/* Library ABI version (HESS_ABI_VERSION). */
int hess_abi_version(void);

/* Static description of a status code. */
const char* hess_strerror(int code);

/* Message of the calling thread's last failed call ("" if none). */
const char* hess_last_error(void);

/*
 * hess_create -- a new, empty Hessian accumulator of width d.
 *
 * Allocates and zeroes the persistent float32 d x d Gram buffer once (GPTQModel
 * PR 2981, Changes: the per-device buffer is allocated once, as float32) plus
 * fixed scratch on the current HIP device: 16 MiB for split reductions, a
 * staging buffer for short batches (see hess_create_ex), and for bf16
 * handles with
 * d % 8 == 0 a small tile-order table.  Such handles also make sure the
 * device's shared 256-tile workspace holds (512 + ntiles % 256) slots of
 * 256 KiB, ntiles = nb (nb + 1) / 2 with nb = ceil(d / 256) (162 MiB at
 * d = 4096); that buffer lives until the process ends.  N = 0.
 *   d         number of input features (Hessian width), 1 <= d <= 65536.
 *   in_dtype  HESS_BF16 or HESS_F32: the staging dtype, i.e. the element
 *             type of every X given to hess_add_batch and the type that
 *             hess_add_batch_cast converts other activations to
 *             (Model-Optimizer PR 3002, hessian_input_dtype; GPTQModel PR
 *             3052, the staging_dtype accumulation setting).
 * Returns NULL on error (EINVAL / ENOMEM / EHIP; see hess_last_error()).
 * The handle owns its device memory until hess_destroy().
 */
hess_t hess_create(int64_t d, int in_dtype);

/* Size of a handle's staging buffer for short batches that hess_create
 * picks for handles with d >= 1024 (bytes); narrower handles get 64 MiB. */
#define HESS_STAGING_DEFAULT ((int64_t)1 << 30)

/*
 * hess_create_ex -- hess_create with the staging buffer's size chosen by the
 * caller: staging_bytes in [0, 16 GiB]; 0 (or too small for 256 rows)
 * disables staging for the handle, e.g. for Hessians only ever updated by
 * hess_add_batch_grouped.  hess_create picks 1 GiB (HESS_STAGING_DEFAULT)
 * for handles with d >= 1024, so that a staged flush is long enough for
 * the 256-tile kernel (209,664 tokens at d = 2560), and 64 MiB otherwise.
 * A smaller buffer saves memory at the cost of more, shorter flushes.
 * When a full buffer's flush would take the 256-tile kernel (bf16, d % 8 ==
 * 0, d >= 1,024 and enough tokens; see hess_set_tile_override), the staged
 * rows are kept in that kernel's operand layout: blocks of 8 tokens, each
 * 16-byte chunk holding the 8 tokens of one feature, every batch padded
 * with zero rows to a multiple of 8 (padding counts toward the capacity,
 * not toward N).  Such a handle's flushes always run on 256-tiles.
 */
hess_t hess_create_ex(int64_t d, int in_dtype, int64_t staging_bytes);

/* Frees the handle and its device memory after draining its last stream. */
int hess_destroy(hess_t h);

/*
 * hess_adopt -- dst takes a private copy of src's statistics: its Gram sum
 * becomes a copy of src's (after src's staged rows are folded in) and its
 * token count src's N; whatever dst held is dropped.  A follower that shares
 * a leader's inputs adopts the leader's Hessian as an independent float32
 * copy with the leader's sample count (GPTQModel PR 3052, "Shared-input
 * Hessian dedup: plan metadata, E2E validation, and telemetry", What Changed
 * > Phase 2 (looper Hessian dedup): adopt_hessian_from copies H and nsamples
 * and clears the follower's partials; updating one afterwards leaves the
 * other unchanged).
 * dst == src is a no-op.  EINVAL: null handle, different d (the pages'
 * column mismatch) or different accumulation settings: staging dtype or
 * staging buffer (its rows and layout fix how the sum is chunked), which the
 * same page's review (finding P2 and its fix) requires to match before a
 * Hessian is shared.  ESTATE: src was materialized in place.  Enqueued on
 * stream (both handles are ordered onto it).  Never allocates.
 */
int hess_adopt(hess_t dst, hess_t src, hess_stream_t stream);

/*
 * hess_add_batch -- S += X^T X and N += n_tokens, in place.
 *
 * One calibration batch (GPTQModel PR 2979, What Changed: add_batch computes
 * the Gram of the flattened activations and counts token vectors; PR 2981,
 * Changes: accumulated directly into the persistent buffer with no transient
 * d x d product).  Only the upper triangle of S (j >= i) is maintained.
 *   X         device, n_tokens x d row-major with row stride ld elements, of
 *             the handle's in_dtype, aligned to its element size.  When X is
 *             16-byte aligned and ld*elem_size is a multiple of 16 bytes the
 *             rows are read with 16-byte loads; otherwise a slower kernel
 *             with element loads is used.
 *   n_tokens  >= 0; 0 is a no-op (PR 2981, Validation: empty batches).
 *   ld        row stride in elements, >= d.
 *   stream    HIP stream the update is ordered on.
 * Errors: EINVAL (h NULL, n_tokens < 0, ld < d, X NULL with n_tokens > 0),
 * EALIGN (X not aligned to its element size), ESTATE, EHIP.  On error
 * nothing is enqueued and N is unchanged.
 */
int hess_add_batch(hess_t h, const void* X, int64_t n_tokens, int64_t ld, hess_stream_t stream);

/*
 * hess_add_batch_cast -- hess_add_batch for activations of any element type:
 * X is first put into the handle's staging dtype, then accumulated.
 *
 * fp16 and bf16 widen exactly to float32; float32 and fp16 round to the
 * nearest bf16, ties to even.  The staging dtype therefore decides the
 * result: one fp16 token of value 1 + 2^-10 gives a scaled diagonal of
 * 2 + 2^-8 + 2^-19 with float32 staging and exactly 2 with bf16 staging
 * (GPTQModel PR 3052, "Shared-input Hessian dedup", review finding P2;
 * Model-Optimizer PR 3002 page, "What does this PR do?": the bfloat16
 * hessian_input_dtype against the float32 default).
 *   x_dtype   HESS_F16, HESS_BF16 or HESS_F32.  Equal to the staging dtype:
 *             exactly hess_add_batch.  Otherwise the rows pass through the
 *             staging buffer, converted on the copy, in pieces that fit (a
 *             full buffer is folded into S first), so the handle needs a
 *             staging buffer (EINVAL with staging_bytes 0).
 *   other arguments and errors as hess_add_batch; X aligned to x_dtype's size.
 * Never allocates.
 */
int hess_add_batch_cast(hess_t h, const void* X, int x_dtype, int64_t n_tokens, int64_t ld, hess_stream_t stream);

/*
 * hess_materialize -- H_out = neutralize_dead(S * 2/N) + damp * I, where
 * damp = damp_percent * mean(diag) of the neutralized matrix.
 *
 * The final scale by 2 / total tokens (PR 2979, What Changed; wiki "QQQ",
 * Concepts > Quadratic error compensation), then steps 2 and 3 of the
 * quantization pass on that wiki page: neutralize dead input columns (a
 * column whose diagonal is exactly zero: its row and column stay zero and
 * its diagonal becomes 1), then add damp_percent * mean(diag(H)) to the
 * diagonal.  N = 0 gives (1 + damp_percent) * I.
 *   damp_percent  a fraction in [0, 1) (the pages' config validates (0, 1)).
 *   H_out         device, d x d float32, full symmetric matrix, row-major;
 *                 bitwise symmetric.  Must not alias S.
 * Enqueued on the handle's last-used stream.  S and N are unchanged, so
 * accumulation may continue and a later call sees the larger sum.
 */
int hess_materialize(hess_t h, float damp_percent, float* H_out);

/*
 * hess_materialize_ex -- hess_materialize with options.
 *   flags     0 or HESS_NO_NEUTRALIZE.
 *   H_out     device d x d float32, or NULL to materialize in place into the
 *             handle's own buffer (saves a second d x d allocation); after
 *             an in-place call the handle only accepts hess_reset,
 *             hess_token_count, hess_state_buffer and hess_destroy (ESTATE).
 *   dead_out  device, d bytes (1 = neutralized column), or NULL.
 *   damp_out  device, one float: the absolute damping added to the diagonal
 *             (wiki "QQQ", Implementation internals > Quantizer API and
 *             results: the returned damp is that value), or NULL.
 *   stream    HIP stream.
 */
int hess_materialize_ex(hess_t h, float damp_percent, unsigned flags, float* H_out,
                        uint8_t* dead_out, float* damp_out, hess_stream_t stream);

/*
 * hess_flush -- fold batches held in the handle's staging buffer into S.
 *
 * A batch shorter than about 2*d/elem_size tokens is not given its own pass
 * over the d x d sum: hess_add_batch copies its rows into a staging buffer
 * allocated by hess_create (64 MiB or 1 GiB, see hess_create_ex) and counts its tokens, and the staged
 * rows are added to S in one pass when the buffer fills, by
 * hess_materialize*, or by this call.  The Gram sum of the concatenated rows
 * equals the sum of the batches' Grams (GPTQModel PR 2981, Validation: add_batch
 * over several batches matches the closed form of their concatenation); only
 * the float32 rounding order differs.  Needed only before reading S through
 * hess_state_buffer.
 */
int hess_flush(hess_t h, hess_stream_t stream);

/* Tuning and test hook, process-wide: enable (1, default) or disable (0) the
 * staging of short batches. */
int hess_set_staging(int enable);

/*
 * hess_set_async_flush -- process-wide switch (default on) for handles
 * created afterwards: a handle with transposed staging whose halves each make
 * a long 256-tile flush splits its staging buffer in two; a full half is
 * folded into the sum on the handle's own stream, with fewer workgroups than
 * CUs, while the caller's stream goes on staging batches into the other half.
 * Calls that read or write the sum (materialize, flush, reset, adopt, long
 * batches, grouped calls) first make the caller's stream wait for it, so the
 * results are stream-ordered as before.  Under HIP graph capture the flush
 * stays on the capturing stream; capture a handle only after a flush,
 * materialize or reset of it, so that no asynchronous flush is pending.
 * Off: one buffer, every flush on the caller's stream.
 */
int hess_set_async_flush(int enable);

/* Test hook, process-wide: cap (bytes, > 0) on the rows gathered per
 * 256-tile grouped launch (hess_add_batch_grouped fills its gather buffer as
 * often as needed, splitting groups that do not fit); 0 (default) = the
 * whole buffer.  EINVAL for a negative value. */
int hess_set_group_chunk(int64_t bytes);

/* Process-wide: 256-tile grouped updates through hess_add_batch_grouped_ex
 * read each group's rows where they are in X (1, default) or gather them
 * into the per-device buffer first (0), as hess_add_batch_grouped always
 * does.  Both give the same bits. */
int hess_set_group_direct(int enable);

/* S = 0 (its upper triangle, where the sum lives; see hess_state_buffer),
 * N = 0 (enqueued on stream); also re-arms a consumed handle. */
int hess_reset(hess_t h, hess_stream_t stream);

/* Tokens accumulated so far (host int64; exact, counted on the host). */
int hess_token_count(hess_t h, int64_t* n_out);

/* Tuning and test hook, process-wide: force the edge of the upper-triangle
 * tiles used by hess_add_batch (0 = automatic choice per call, 64, 128, or
 * 256).  256-tiles apply to bf16 handles with d % 8 == 0 and 16-byte aligned
 * rows; 64-tiles (the thin-batch kernel, whose time is the read-modify-write
 * of S) to bf16 and float32 handles with d % 8 == 0 and 16-byte aligned rows
 * for passes of at most 512 tokens;
 * other calls keep 128-tiles.  The automatic choice takes 64-tiles for such
 * passes of at most 512 tokens, and 256-tiles at d >= 1,024 when a pass
 * (one batch, or one staging flush) gives each of the 256 workgroups at
 * least 300 iterations of 32 tokens.  The setting at hess_create also fixes
 * a handle's staging layout: 256 makes it the transposed one whenever the
 * handle stages, 128 keeps rows (see hess_create_ex). */
int hess_set_tile_override(int edge);

/*
 * hess_set_timing / hess_timing -- measurement aid.  While timing is on, each
 * SYRK pass of the handle (one per long batch and one per staging-buffer
 * flush, hess_add_batch's kernel) is bracketed by a pair of HIP events
 * recorded on the stream it is launched on.  hess_timing waits for the last
 * recorded event, then returns (host) the number of launches since timing was
 * switched on or last read, the tokens they processed and the sum of their
 * event-measured durations in milliseconds, and starts a new window.
 * hess_set_timing(h, on) also starts a new window.  Creating the events is
 * the only host-side allocation; no device memory is allocated.
 */
int hess_set_timing(hess_t h, int on);
int hess_timing(hess_t h, int64_t* launches, int64_t* tokens, double* ms);

/* Width and input type of a handle (host outputs). */
int hess_info(hess_t h, int64_t* d_out, int* in_dtype_out);

/*
 * hess_state_buffer -- the device address of the handle's float32 d x d
 * buffer: the Gram sum S (upper triangle valid; call hess_flush first so
 * staged batches are included) or, after an in-place materialize, H.
 * Read-only for callers except through this API.
 */
int hess_state_buffer(hess_t h, const float** S_out);

/*
 * hess_local_blocks -- out[b] += X_b^T X_b for every contiguous block of 16
 * features (Model-Optimizer PR 3002 page, "What does this PR do?",
 * local_hessian bullet: 16x16 per-block Hessians by a batched product that
 * reads bfloat16 and writes float32).  Unscaled; accumulates into out.
 *   X         device bf16, n_tokens x d row-major, ld = d.
 *   n_tokens  >= 0.
 *   d         multiple of block, >= block.
 *   block     must be 16.
 *   out       device float32 (d/16, 16, 16), row-major blocks.
 * Runs on the null stream.
 */
int hess_local_blocks(const void* X, int64_t n_tokens, int64_t d, int block, float* out);

/*
 * hess_local_blocks_ex -- hess_local_blocks with dtype, stride, stream and
 * accumulate (nonzero: out += ..., zero: out = ...).
 *   in_dtype  HESS_BF16 or HESS_F32 (float32 products are exact).
 *   ld        row stride of X in elements, >= d.
 * Sums go through per-workgroup partials added in a fixed order, so a call
 * gives the same bits every time (no atomics).  The partials live in a
 * per-device scratch that the first call on a device allocates (16 MiB, or
 * 1 KB per block beyond width 262,144) and later calls reuse; a call on
 * another stream than the previous one waits for it.
 */
int hess_local_blocks_ex(const void* X, int in_dtype, int64_t n_tokens, int64_t d, int64_t ld,
                         int block, float* out, int accumulate, hess_stream_t stream);

/*
 * hess_local_blocks_noalloc -- hess_local_blocks_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, same result bit for bit
 * (the same plan and summation order).
 *   - Allocates nothing: its partial sums live in a fixed 16 MiB array of
 *     device memory in the library, one per GPU, held until the process ends.
 *     The first call on a device looks up that array's address there.
 *   - d up to 262,144 (d/16 blocks of 1 KB must fit the array); wider
 *     returns HESS_EINVAL.
 *   - Every call on one GPU shares the array: calls that overlap on a GPU
 *     (concurrent streams, or another host thread) race and give wrong
 *     sums; order them.  Nothing in the array needs clearing between calls.
 */
int hess_local_blocks_noalloc(const void* X, int in_dtype, int64_t n_tokens, int64_t d, int64_t ld,
                              int block, float* out, int accumulate, hess_stream_t stream);

/*
 * hess_reset_grouped -- hess_reset of n_groups handles of one width in one
 * launch (per 64 handles): S_e = 0, N_e = 0, staged rows dropped.  For the
 * routed-expert Hessians of a MoE layer (Model-Optimizer PR 3002 page: the
 * option applies to every GPTQ Hessian, fused MoE experts included).
 *   hs        (host) n_groups distinct handles of equal d.
 * Stream-ordered like hess_reset; clears handles consumed in place too.
 */
int hess_reset_grouped(hess_t* hs, int n_groups, hess_stream_t stream);

/*
 * hess_materialize_grouped -- hess_materialize_ex of n_groups handles of one
 * width with the same damp_percent and flags, in two launches per 64 handles
 * (one writes every dead mask and damping, one every H), with the same bits
 * as n_groups separate hess_materialize_ex calls.
 *   hs        (host) n_groups distinct handles of equal d, none consumed.
 *   H_out     (host) array of n_groups device pointers: each a d x d float32
 *             output, or NULL for that handle in place (it is then consumed,
 *             as with hess_materialize_ex).  H_out itself must not be NULL.
 *   dead_out, damp_out  (host) arrays of device pointers (d bytes / one
 *             float each), or NULL arrays / NULL entries for the handles'
 *             own buffers.
 * Each handle's staged rows are folded in first.  Buffers that are not
 * 16-byte aligned, or d % 4 != 0, take one materialize per handle.
 */
int hess_materialize_grouped(hess_t* hs, int n_groups, float damp_percent, unsigned flags,
                             float* const* H_out, uint8_t* const* dead_out, float* const* damp_out,
                             hess_stream_t stream);

/*
 * hess_add_batch_grouped -- for each group e < n_groups:
 *   S_e += X[rows_e]^T X[rows_e],  N_e += |rows_e|,
 * in one launch.  One Hessian per routed expert over the tokens routed to it
 * (Model-Optimizer PR 3002 page: the option applies to every GPTQ Hessian,
 * fused MoE experts included; experts never share a Hessian).
 *   hs        (host) n_groups distinct handles of equal d and in_dtype.
 *   X         device, T x d row-major with row stride ld (all tokens).
 *   row_idx   device int32, offsets[n_groups] entries: rows of X grouped by
 *             expert; group e is row_idx[offsets[e] .. offsets[e+1]).  NULL
 *             means X's rows are already grouped (row_idx[i] = i).
 *   offsets   (host) int64, n_groups + 1 non-decreasing entries, offsets[0]=0.
 * All row indices must be in [0, T) where T is the caller's row count; the
 * library cannot check device contents.
 * bf16 handles with d % 8 == 0, d >= 1,024 and 16-byte aligned rows take
 * 256-tiles: the groups' rows are first gathered into a per-device buffer in
 * the transposed staging layout (8-row blocks per group), then one launch
 * adds whole upper tiles of every group.  The first such call on a device,
 * and any later one with more rows, allocates that buffer (after a device
 * synchronize if it replaces a smaller one): sum over groups of
 * ceil(rows / 8) * 8 * d * 2 bytes, at most 4 GiB; rows beyond it take
 * further fills (see hess_set_group_chunk).  The buffer lives until the
 * process ends.  Other handles take 128-tiles with rows gathered by the
 * kernel.
 */
int hess_add_batch_grouped(hess_t* hs, int n_groups, const void* X, int64_t ld,
                           const int32_t* row_idx, const int64_t* offsets, hess_stream_t stream);

/*
 * hess_add_batch_grouped_ex -- hess_add_batch_grouped with X's row count
 * n_rows (T) given, so that the 256-tile path need not gather: when
 * n_rows * ld * 2 < 2^31 bytes, the launch reads every group's rows in place
 * through a table of their offsets in X (1 KiB per 256 routed rows, built by
 * a small kernel in the per-device buffer, which then holds only the table
 * and the schedule), with the same operands in the same order as the
 * gathered path, so the same bits.  On that path a row index outside
 * [0, n_rows) reads as a zero row (it still counts toward N_e); every other
 * path requires them in range, as hess_add_batch_grouped does.
 * n_rows = -1: unknown (gathered path).
 * EINVAL also for n_rows < -1, and without row_idx for offsets[n_groups] >
 * n_rows.  Synchronization and allocation as hess_add_batch_grouped.
 */
int hess_add_batch_grouped_ex(hess_t* hs, int n_groups, const void* X, int64_t n_rows, int64_t ld,
                              const int32_t* row_idx, const int64_t* offsets, hess_stream_t stream);

/*
 * hess_gptq_quantize -- error-propagating 4-bit quantization of a weight
 * matrix with the upper Cholesky factor of the inverse damped Hessian (the
 * quantization pass's step 5: GPTQModel wiki "QQQ", Concepts > Quadratic
 * error compensation; 128-column blocks).
 *
 * Column i of W is quantized, its error divided by U[i][i] and propagated
 * into the columns not yet quantized through row i of U.  Quantizer (wiki
 * "QQQ", Whole-row and grouped weight quantization): symmetric, step
 * 2 max|w| / 15 per row (group_size -1) or per group of contiguous columns
 * taken when the group is reached; code clip(rint(w / step) + 8, 0, 15);
 * value step (code - 8).  Computed in float64 (inputs widened exactly).
 *   W       device float32, rows x cols (outputs x inputs), row stride ldw.
 *   U       device float32, cols x cols, row stride ldu: the factor from
 *           hess_chol_inverse_upper (only its upper triangle is read).
 *   dead    device bytes, cols, nullable: nonzero columns are zeroed first
 *           (the weight side of dead-column neutralization).
 *   group_size  -1 (whole rows), a divisor of 128, or >= cols (whole rows).
 *   Q       device float32 out, dequantized weights, row stride ldq; may be W
 *           itself (same stride).
 *   codes   device uint8 out, rows x cols, row stride ldc, values 0..15.
 *   scales  device float32 out, rows x groups (groups = 1 for whole rows).
 *   loss    device double out, nullable: sum over columns and rows of the
 *           squared error divided by U[i][i], over nsamples (wiki "QQQ",
 *           Implementation internals > Quantizer API and results).
 *   work    device workspace of hess_gptq_quantize_workspace(rows, cols)
 *           bytes, 16-byte aligned, owned by the caller.
 *   1 <= rows, cols <= 65536.  Errors: EINVAL (sizes, strides, group size,
 *   null pointers, overlaps, small workspace), EALIGN, EHIP.  Enqueued on
 *   stream; allocates nothing.
 */
int64_t hess_gptq_quantize_workspace(int64_t rows, int64_t cols); /* bytes, or -1 for bad sizes */
int hess_gptq_quantize(const float* W, int64_t rows, int64_t cols, int64_t ldw, const float* U, int64_t ldu,
                       const uint8_t* dead, int group_size, float* Q, int64_t ldq, uint8_t* codes, int64_t ldc,
                       float* scales, double* loss, int64_t nsamples, void* work, int64_t work_bytes,
                       hess_stream_t stream);

/*
 * hess_chol_inverse_upper -- the upper Cholesky factor of the inverse of a
 * damped Hessian: U upper triangular with a positive diagonal and
 * U^T U = H^-1 (the quantization pass's step 4 after neutralization and
 * damping: GPTQModel wiki "QQQ", Concepts > Quadratic error compensation).
 *
 * Computed in float64 (H widened exactly) by factoring the index-reversed H
 * and inverting that factor, then rounded once to float32.
 *   H      device float32, d x d, row stride ldh >= d; only its upper
 *          triangle (j >= i) is read (hess_materialize's output qualifies).
 *   U      device float32, d x d, row stride ldu >= d; every entry written
 *          (zeros below the diagonal).  U may be H itself (same stride: in
 *          place); no other overlap is allowed.
 *   work   device workspace of hess_chol_inverse_workspace(d) bytes, 16-byte
 *          aligned, owned by the caller, not overlapping H or U.
 *   info   device int, nullable: set to 0, or on failure to 1 + the largest
 *          column j of H whose pivot was not positive (H[j:, j:] is then not
 *          positive definite).  The pages raise the factorization error and
 *          retry nothing (wiki "QQQ", Pitfalls; damp_auto_increment is not
 *          applied): a failed factorization leaves NaN in U and says so in
 *          info, which the caller reads after the stream reaches this call.
 *   1 <= d <= 32768.  Errors: EINVAL (bad sizes, null pointers, workspace too
 *   small, overlaps), EALIGN, EHIP.  Enqueued on stream; allocates nothing.
 */
int64_t hess_chol_inverse_workspace(int64_t d); /* bytes, or -1 for a bad d */
int hess_chol_inverse_upper(const float* H, int64_t d, int64_t ldh, float* U, int64_t ldu, void* work,
                            int64_t work_bytes, int* info, hess_stream_t stream);

/*
 * imatrix statistic -- per-column float32 sums of squares of a layer's
 * inputs, acc[j] = sum over every token of X[t][j]^2.  The imatrix method
 * keeps this float32 statistic instead of a Gram matrix (NVIDIA
 * Model-Optimizer PR 3002 page, "What does this PR do?": a per-column sum of
 * squares, not a GEMM).  One streaming read of each batch.
 *
 * hess_imatrix_create -- an empty statistic of width d (1 <= d <= 2^24) for
 *   inputs of in_dtype (HESS_BF16 or HESS_F32) on the current device: d
 *   floats plus 1,024 x d floats of per-batch partial sums, allocated and
 *   zeroed once.  NULL on error (EINVAL / ENOMEM / EHIP).
 *   (1,056 x d floats of workspace in all: partials and their run sums.)
 * hess_imatrix_add_batch -- acc += column sums of squares of X (device,
 *   n_tokens x d row-major, row stride ld >= d, element-aligned), N +=
 *   n_tokens; n_tokens = 0 is a no-op.  Each batch is summed in float32 over
 *   up to 1,024 row runs whose partials are added in a fixed order.  Never
 *   allocates.  EINVAL / EALIGN / EHIP.
 * hess_imatrix_read -- copy acc (d floats) to the device buffer out,
 *   enqueued on stream; *n_out (host, may be NULL) = N, the tokens seen.
 * hess_imatrix_reset -- acc = 0, N = 0 (enqueued on stream).
 * hess_imatrix_destroy -- free the handle after draining its last stream.
 * A call on a different stream than the previous one waits for it (event).
 */
hess_imx_t hess_imatrix_create(int64_t d, int in_dtype);
int hess_imatrix_add_batch(hess_imx_t m, const void* X, int64_t n_tokens, int64_t ld, hess_stream_t stream);
int hess_imatrix_read(hess_imx_t m, float* out, int64_t* n_out, hess_stream_t stream);
int hess_imatrix_reset(hess_imx_t m, hess_stream_t stream);
int hess_imatrix_destroy(hess_imx_t m);

#ifdef __cplusplus
}
#endif

#endif /* HESS_H */
