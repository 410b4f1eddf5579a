// C ABI of libhess (declared in include/hess.h): handles, validation, stream
// ordering, the choice of kernel shape per call, and dispatch.
//
// A handle is one Hessian accumulator: the persistent float32 d x d Gram sum
// (allocated and zeroed once, as GPTQModel PR 2981 keeps one float32 buffer
// per device), the exact token count N kept on the host (PR 2979 counts
// flattened token vectors), and small fixed device buffers (dead mask, damp
// value, split workspace).  No call after hess_create allocates device memory.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <queue>
#include <vector>

#include "../../include/hess.h"
#include "hess_internal.hpp"

using namespace hess;

struct hess_s {
  // every call on the handle holds this lock (recursive: some calls call
  // others), so calls from several host threads do not interleave
  std::recursive_mutex mu;
  int64_t d = 0;
  int dtype = HESS_BF16;
  int device = 0;
  float* S = nullptr;        // d x d, row stride d
  uint8_t* dead = nullptr;   // d bytes
  float* damp = nullptr;     // 1 float
  float* ws = nullptr;       // split partials (may be null)
  int64_t ws_floats = 0;
  void* stage = nullptr;     // thin-batch staging rows (stage_cap x stage_ld elements)
  int64_t stage_cap = 0;     // tokens
  int64_t stage_ld = 0;      // row stride in elements (d rounded up to 8)
  int64_t stage_n = 0;       // tokens staged, not yet in S (with the zero rows of stage_t8)
  int64_t stage_real = 0;    // ... of which batch rows
  // bf16 staging in the transposed layout of the 256-tile kernel: 8-token
  // blocks of d 16-byte chunks (8 tokens of one feature), each batch padded
  // with zero rows to a multiple of 8; always flushed by that kernel
  bool stage_t8 = false;
  // Asynchronous flushes (transposed staging whose halves are each long
  // enough for the 256-tile kernel): the staging allocation is two halves of
  // stage_cap tokens.  A full half is folded in on the handle's own stream
  // (`side`) with fewer workgroups than CUs (async_wgs), which leaves CUs free for the
  // staging copies that go on into the other half on the caller's stream.
  // side_done[k] is recorded after half k's flush; busy[k]: that flush may
  // still be reading half k; pending: a side flush may still be writing S
  // (side_last is the newest).  Everything that touches S, or writes a busy
  // half, first makes its stream wait for those events.
  bool async = false;
  void* half[2] = {nullptr, nullptr};
  int cur = 0;
  hipStream_t side = nullptr;
  hipEvent_t side_done[2] = {nullptr, nullptr};
  hipEvent_t fork = nullptr;
  bool busy[2] = {false, false};
  bool pending = false;
  int side_last = 0;
  int64_t N = 0;
  bool consumed = false;     // in-place materialize done
  bool has_stream = false;
  hipStream_t last = nullptr;
  hipEvent_t ev = nullptr;
  // SYRK launch timing (hess_set_timing): event pairs around each launch of
  // the current window, and the tokens each launch processed
  bool timing = false;
  std::vector<hipEvent_t> tev;
  std::vector<int64_t> ttok;
  size_t tcount = 0;
  // 256-tile path: blocked order of the upper-triangle 256-tiles (device)
  int32_t* order256 = nullptr;
  int nb256 = 0;
  int ntiles256 = 0;
};

struct hess_imx_s {
  std::recursive_mutex mu;
  int64_t d = 0;
  int dtype = HESS_BF16;
  float* acc = nullptr;      // d floats: the running per-column sums of squares
  float* part = nullptr;     // kImxSplits x d floats: one batch's split partials
  int64_t N = 0;
  bool has_stream = false;
  hipStream_t last = nullptr;
  hipEvent_t ev = nullptr;
};

namespace {

// Stream-K workspace of the 256-tile path, one per device, shared by every
// handle on it and grown by hess_create to the largest width seen.  Launches
// that use it are ordered: a launch on another stream than the previous user
// first waits for that user's event.
struct BigWorkspace {
  std::mutex mu;
  float* ptr = nullptr;
  int64_t slots = 0;          // 256 x 256 float slots
  void* gptr = nullptr;       // grouped updates: gathered rows in transposed staging layout
  int64_t gbytes = 0;
  int32_t* hsched = nullptr;  // pinned host copy of a grouped launch's schedule
  hipEvent_t sched_ev = nullptr;
  bool sched_pending = false; // a copy out of hsched may still be running
  hipEvent_t ev = nullptr;
  bool used = false;
  hipStream_t last = nullptr;
};
constexpr int kMaxDevices = 64;
BigWorkspace g_big[kMaxDevices];

// Partial-sum scratch of the local blocks, one per device, allocated by the
// first call on the device (kLocalPartBytes, or more for widths past
// 262,144).  Calls on another stream than the previous user wait for its event.
struct LocalScratch {
  std::mutex mu;
  float* ptr = nullptr;
  int64_t bytes = 0;
  hipEvent_t ev = nullptr;
  bool used = false;
  hipStream_t last = nullptr;
};
LocalScratch g_local[kMaxDevices];

thread_local char g_err[512] = "";

using HLock = std::lock_guard<std::recursive_mutex>;

// The locks of several handles, taken in address order (so that two calls
// over overlapping sets of handles cannot deadlock); null entries are skipped.
struct GroupLock {
  std::vector<std::unique_lock<std::recursive_mutex>> held;
  GroupLock(hess_t* hs, int n) {
    std::vector<hess_t> v;
    for (int e = 0; hs && e < n; ++e)
      if (hs[e]) v.push_back(hs[e]);
    std::sort(v.begin(), v.end(), std::less<hess_t>());
    v.erase(std::unique(v.begin(), v.end()), v.end());
    for (hess_t h : v) held.emplace_back(h->mu);
  }
};
int g_tile_override = 0;  // 0 = automatic; 64, 128 or 256 force that SYRK tile edge where it applies
int64_t g_group_chunk = 0; // test hook: cap on the gathered bytes per grouped launch (0 = scratch size)
bool g_group_direct = true; // grouped 256-tile updates read the routed rows in place when X's size is known
bool g_staging = true;    // thin-batch staging enabled (process-wide)
bool g_async = true;      // asynchronous flushes for handles created from now on (process-wide)

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HESS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Order this call after the handle's previous call when the stream changes.
int order_stream(hess_t h, hipStream_t s) {
  if (h->has_stream && h->last != s) {
    hipError_t e = hipEventRecord(h->ev, h->last);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = hipStreamWaitEvent(s, h->ev, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  h->last = s;
  h->has_stream = true;
  return HESS_OK;
}

int esize(int dtype) { return dtype == HESS_F32 ? 4 : 2; }

// The vectorized loaders read whole units of 8 features with 16-byte loads:
// X and every row start 16-byte aligned, d a multiple of 8, and 64 rows of
// the stride addressable with 32-bit buffer offsets.
bool vec_ok(const void* p, int64_t ld, int64_t d, int es) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ((ld * es) & 15) == 0 && (d % 8) == 0 &&
         ld * es * 64 < ((int64_t)1 << 31);
}

constexpr int kCUs = 256;       // MI355X compute units: one SYRK workgroup each
constexpr int kTile = 128;      // SYRK tile edge
constexpr int64_t kWsSlots = 256;  // tail partial tiles a handle can hold
// K-iterations (64 tokens) per float32 accumulation chain: bf16 products are
// rounded once per 8 tokens, float32 products once per 2 tokens.
constexpr int kFlushItersBF16 = 64;
constexpr int kFlushItersF32 = 16;
int flush_iters(int dtype) { return dtype == HESS_F32 ? kFlushItersF32 : kFlushItersBF16; }

int grid8(int64_t items) { return (int)(((items + 7) / 8) * 8); }

// Work split of one batch of n tokens over the upper-triangle 128-tiles:
// whole tiles fill complete rounds of one workgroup per CU; tiles left for a
// last, partly empty round (or all tiles, when there are fewer tiles than
// CUs) are split into token ranges so that round is full, when the batch is
// long enough for the partials' extra traffic to pay off.
struct Plan {
  int nb, ntiles, full_tiles, tail_parts, tail_kchunk, grid_full, grid;
};

Plan plan_single(int64_t d, int64_t n, bool have_ws) {
  Plan p{};
  p.nb = (int)((d + kTile - 1) / kTile);
  p.ntiles = p.nb * (p.nb + 1) / 2;
  p.full_tiles = p.ntiles;
  p.tail_parts = 0;
  p.tail_kchunk = 0;
  const int full_rounds = p.ntiles / kCUs;
  const int tail = p.ntiles - full_rounds * kCUs;
  if (have_ws && tail > 0) {
    int parts = kCUs / tail;
    parts = (int)std::min<int64_t>(parts, n / 1024);               // >= 1024 tokens per part
    parts = (int)std::min<int64_t>(parts, kWsSlots / tail);         // workspace capacity
    if (parts >= 2) {
      const int64_t kchunk = ((n + parts - 1) / parts + 63) / 64 * 64;
      p.full_tiles = full_rounds * kCUs;
      p.tail_kchunk = (int)kchunk;
      p.tail_parts = (int)((n + kchunk - 1) / kchunk);
    }
  }
  p.grid_full = grid8(p.full_tiles);
  p.grid = p.grid_full;
  if (p.tail_parts > 0) p.grid += grid8((int64_t)(p.ntiles - p.full_tiles) * p.tail_parts);
  return p;
}

// Staging buffer: HESS_STAGING_DEFAULT bytes of rows per handle unless
// hess_create_ex says otherwise (a multiple of 64 tokens, at least 256).
int64_t stage_tokens(int64_t d, int es, int64_t bytes) {
  const int64_t row = ((d + 7) / 8 * 8) * es;
  int64_t cap = bytes / row / 64 * 64;
  return cap >= 256 ? cap : 0;
}

// A batch goes through the staging buffer when that moves fewer bytes than a
// pass over the upper-triangle sum: 2 n d esize (copy in and read back) is
// below 4 d^2, i.e. n < 2 d / esize.
bool stage_pays(const hess_s* h, int64_t n) {
  return g_staging && h->stage && n <= h->stage_cap && n * esize(h->dtype) < 2 * h->d;
}

constexpr int64_t kQuantMaxDim = 65536;  // largest rows / cols of hess_gptq_quantize
constexpr int64_t kCholMaxD = 32768;  // largest width of hess_chol_inverse_upper (16 GiB of workspace)
constexpr int64_t kImxSplits = 1024;  // row splits of one imatrix batch (partials per column)

// Calls on an imatrix handle from a new stream wait for the previous stream's work.
int imx_order_stream(hess_imx_t m, hipStream_t s) {
  if (m->has_stream && m->last != s) {
    hipError_t e = hipEventRecord(m->ev, m->last);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, m->ev, 0);
    if (e != hipSuccess) return hip_fail(e, "imatrix stream ordering");
  }
  m->has_stream = true;
  m->last = s;
  return HESS_OK;
}

// Timing events around one SYRK pass (hess_set_timing).
hipError_t timing_begin(hess_t h, hipStream_t s) {
  hipError_t e = hipSuccess;
  while (e == hipSuccess && h->tev.size() < 2 * (h->tcount + 1)) {
    hipEvent_t ev = nullptr;
    e = hipEventCreate(&ev);
    if (e == hipSuccess) h->tev.push_back(ev);
  }
  if (e != hipSuccess) return e;
  return hipEventRecord(h->tev[2 * h->tcount], s);
}

hipError_t timing_end(hess_t h, hipStream_t s, int64_t n) {
  const hipError_t e = hipEventRecord(h->tev[2 * h->tcount + 1], s);
  if (e != hipSuccess) return e;
  if (h->ttok.size() <= h->tcount) h->ttok.resize(h->tcount + 1);
  h->ttok[h->tcount++] = n;
  return hipSuccess;
}

// ---- 256-tile path ----
constexpr int kBig = 256;
constexpr int kBigKI = 32;               // tokens per iteration
constexpr int kBigMinD = 1024;           // automatic choice: widths at least this wide ...
constexpr int64_t kBigMinWork = 300;     // ... and at least this many iterations per workgroup
constexpr int64_t kGroupScratchMax = (int64_t)4 << 30;  // largest gather buffer of grouped updates, per device
// its tail holds one launch's schedule: 257 offsets and at most 64 groups x ntiles items (d <= 32768)
constexpr int64_t kGroupSchedBytes = (int64_t)(kCUs + 1 + kBigMaxGroups * (128 * 129 / 2)) * 4;
constexpr int64_t kGroupItemCost = 24;   // a tile chunk's prologue and output, in 32-token iterations

bool big_capable(int64_t d, int dtype) { return dtype == HESS_BF16 && d % 8 == 0 && d >= 8 && d <= 32768; }

// Upper-triangle tiles in blocked order: 4 x 4 super-tiles (row-major over
// the super-tiles, row-major inside each), so that consecutive tiles share
// few row and column panels.
std::vector<int32_t> blocked_order(int nb) {
  const int G = 4;
  std::vector<int32_t> o;
  for (int si = 0; si < nb; si += G)
    for (int sj = si; sj < nb; sj += G)
      for (int i = si; i < std::min(nb, si + G); ++i)
        for (int j = std::max(i, sj); j < std::min(nb, sj + G); ++j) o.push_back((i << 16) | j);
  return o;
}

// Workspace slots a launch can use: 2 grid_sk + excess items, grid_sk <= 256
// and excess items < sk_tiles = ntiles % 256.
int64_t big_slots(int ntiles) { return ntiles % kCUs ? 2 * kCUs + ntiles % kCUs : 0; }

// The 256-tile kernel has a fixed cost per launch (its parts' workspace
// round trip and fixup, its imbalance when tiles split into many parts), so
// it is chosen once each workgroup gets at least 300 iterations of 32
// tokens.  Measured on MI355X with N(0,1)-scaled bf16 data: width 2,560 with
// 52,224 tokens (350 per workgroup) takes 398 us against 436 us for four
// 128-tile passes of 13,056, and with 26,112 tokens (175 per workgroup) is
// slower than two 128-tile passes.
bool use_big(const hess_s* h, int64_t n, bool vec) {
  if (!h->order256 || !vec) return false;
  if (g_tile_override == kTile) return false;
  if (g_tile_override == kBig) return true;
  const int64_t niter = (n + kBigKI - 1) / kBigKI;
  return h->d >= kBigMinD && (int64_t)h->ntiles256 * niter >= kBigMinWork * kCUs;
}

// The timing events (hess_set_timing) bracket the main kernel, which does
// all the multiplications; the fixup that adds the stream-K pieces follows it.
//
// t8: X is a transposed staging buffer (ld = chunks per 8-token block, n a
// multiple of 8); n_real = rows that are batch rows, for the timing record.
//
// max_wgs caps the workgroups of the split tiles (a multiple of 8, at most
// 256); the asynchronous flush takes fewer than the CUs so that staging
// copies on another stream find free CUs.
int run_big(hess_t h, const void* X, int64_t n, int64_t ld, hipStream_t s, bool t8 = false, int64_t n_real = -1,
            int max_wgs = kCUs) {
  BigParams B;
  std::memset(&B, 0, sizeof(B));
  B.t8 = t8 ? 1 : 0;
  B.X = X;
  B.ld = ld;
  B.S = h->S;
  B.lds = h->d;
  B.order = h->order256;
  B.n = n;
  B.d = (int)h->d;
  B.nb = h->nb256;
  B.ntiles = h->ntiles256;
  B.niter = (int)((n + kBigKI - 1) / kBigKI);
  B.dp_tiles = (h->ntiles256 / kCUs) * kCUs;
  B.sk_tiles = h->ntiles256 - B.dp_tiles;
  B.parts = 1;
  B.part_len = B.niter;
  B.items = B.sk_tiles;
  B.grid_sk = 0;
  B.excess_total = 0;
  if (B.sk_tiles > 0) {
    // enough aligned parts per tile to give every CU one; the parts past the
    // first 256 (fewer than sk_tiles) are shared out as pieces
    B.parts = (int)std::min<int64_t>((max_wgs + B.sk_tiles - 1) / B.sk_tiles, B.niter);
    B.part_len = (B.niter + B.parts - 1) / B.parts;
    B.items = B.sk_tiles * B.parts;
    B.grid_sk = std::min(max_wgs, B.items);
    if (B.grid_sk >= 8) B.grid_sk -= B.grid_sk % 8;  // whole XCD rows
    B.excess_total = (int64_t)(B.items - B.grid_sk) * B.part_len;
  }
  const int64_t slots = 2 * (int64_t)B.grid_sk + (B.items - B.grid_sk);
  BigWorkspace& W = g_big[h->device];
  std::lock_guard<std::mutex> lock(W.mu);
  if (slots > W.slots) return fail(HESS_EHIP, "256-tile workspace too small");
  B.ws = W.ptr;
  hipError_t e = hipSuccess;
  if (W.used && W.last != s) {
    e = hipStreamWaitEvent(s, W.ev, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  if (h->timing) {
    e = timing_begin(h, s);
    if (e != hipSuccess) return hip_fail(e, "timing event");
  }
  e = launch_syrk_big(B, s);
  if (e != hipSuccess) return hip_fail(e, "256-tile SYRK launch");
  if (h->timing) {
    e = timing_end(h, s, n_real >= 0 ? n_real : n);
    if (e != hipSuccess) return hip_fail(e, "timing event");
  }
  e = launch_syrk_big_fixup(B, s);
  if (e != hipSuccess) return hip_fail(e, "256-tile fixup launch");
  e = hipEventRecord(W.ev, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  W.used = true;
  W.last = s;
  return HESS_OK;
}

// Thin batches added straight into S take the 64-tile kernel, whose time is
// the read-modify-write of S's upper triangle.
constexpr int kThinTile = 64;
bool use_thin(const hess_s* h, int64_t n, bool vec) {
  if (!vec || n > kSyrkThinMaxN) return false;
  return g_tile_override == 0 || g_tile_override == kThinTile;
}

int run_thin(hess_t h, const void* X, int64_t n, int64_t ld, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (h->timing) {
    e = timing_begin(h, s);
    if (e != hipSuccess) return hip_fail(e, "timing event");
  }
  e = launch_syrk_thin(X, h->dtype, ld, n, (int)h->d, h->S, h->d, s);
  if (e != hipSuccess) return hip_fail(e, "thin SYRK launch");
  if (h->timing) {
    e = timing_end(h, s, n);
    if (e != hipSuccess) return hip_fail(e, "timing event");
  }
  return HESS_OK;
}

// One SYRK pass of n rows of X into S, on stream s (already ordered).
int run_syrk(hess_t h, const void* X, int64_t n, int64_t ld, hipStream_t s) {
  const bool vec = vec_ok(X, ld, h->d, esize(h->dtype));
  if (use_thin(h, n, vec)) return run_thin(h, X, n, ld, s);
  if (use_big(h, n, vec)) return run_big(h, X, n, ld, s);
  const Plan pl = plan_single(h->d, n, h->ws != nullptr);
  SyrkParams P;
  std::memset(&P, 0, sizeof(P));
  P.X = X;
  P.rows = nullptr;
  P.ld = ld;
  P.lds = h->d;
  P.ws = h->ws;
  P.d = (int)h->d;
  P.nb = pl.nb;
  P.ntiles = pl.ntiles;
  P.ngroups = 1;
  P.flush_iters = flush_iters(h->dtype);
  P.full_tiles = pl.full_tiles;
  P.tail_parts = pl.tail_parts;
  P.tail_kchunk = pl.tail_kchunk;
  P.grid_full = pl.grid_full;
  P.s_vec = (h->d % 4) == 0;
  P.item_prefix[0] = 0;
  P.item_prefix[1] = pl.ntiles;
  P.g[0] = SyrkGroup{h->S, 0, n};
  hipError_t e = hipSuccess;
  if (h->timing) {
    e = timing_begin(h, s);
    if (e != hipSuccess) return hip_fail(e, "timing event");
  }
  e = launch_syrk(P, h->dtype, vec, pl.grid, s);
  if (e != hipSuccess) return hip_fail(e, "SYRK launch");
  if (h->timing) {
    e = timing_end(h, s, n);
    if (e != hipSuccess) return hip_fail(e, "timing event");
  }
  if (pl.tail_parts > 0) {
    e = launch_syrk_reduce(h->S, h->d, h->ws, (int)h->d, pl.nb, pl.full_tiles, pl.ntiles - pl.full_tiles,
                           pl.tail_parts, s);
    if (e != hipSuccess) return hip_fail(e, "split reduction launch");
  }
  return HESS_OK;
}

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

int pending_under_capture() {
  return fail(HESS_ESTATE, "an asynchronous staging flush is pending: flush, materialize or reset the handle "
              "before capturing it");
}

// Make s wait until the handle's asynchronous flushes are done (before s
// touches S): then every half is free again.
int join_side(hess_t h, hipStream_t s) {
  if (!h->pending) return HESS_OK;
  if (capturing(s)) return pending_under_capture();
  const hipError_t e = hipStreamWaitEvent(s, h->side_done[h->side_last], 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  h->pending = false;
  h->busy[0] = h->busy[1] = false;
  return HESS_OK;
}

// Make s wait until the current half may be written again.
int claim_half(hess_t h, hipStream_t s) {
  if (!h->busy[h->cur]) return HESS_OK;
  if (capturing(s)) return pending_under_capture();
  const hipError_t e = hipStreamWaitEvent(s, h->side_done[h->cur], 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  h->busy[h->cur] = false;
  return HESS_OK;
}

// Fold the staged rows into S, on s.
int flush_stage(hess_t h, hipStream_t s) {
  int rc = join_side(h, s);
  if (rc != HESS_OK || h->stage_n == 0) return rc;
  rc = h->stage_t8 ? run_big(h, h->stage, h->stage_n, h->d, s, true, h->stage_real)
                   : run_syrk(h, h->stage, h->stage_n, h->stage_ld, s);
  if (rc == HESS_OK) h->stage_n = h->stage_real = 0;
  return rc;
}

// Workgroups of an asynchronous flush (each holds a whole CU; the rest of
// the CUs run the staging copies).  Measured on MI355X at width 2,560 with a
// 187K-token flush and 180 staging copies of the next batches on the caller's
// stream: 1.73 ms one after the other, 1.96 ms side by side at 256 workgroups
// (the copies find no free CU), 1.56 / 1.52 / 1.43 ms at 224 / 208 / 192.
// A flush's cost per token grows as d^2 and a copy's as d, so wider handles
// leave fewer CUs to the copies: the ragged d=4096 Hessian took 6.55 ms with
// synchronous flushes and 6.57 / 6.38 / 6.23 / 7.00 ms with asynchronous ones
// at 192 / 216 / 224 / 240 workgroups (the headline at d=2560: 3.07 ms at
// 192, 3.21 at 224, 3.85 at 240).
int async_wgs(int64_t d) { return d <= 3072 ? 192 : 224; }

// A full half: fold it into S on the side stream (after everything enqueued
// on s so far) and go on staging into the other half.  Under graph capture
// the flush runs on s itself, with the same workgroups (the same token parts,
// so the same bits as outside a capture).
int flush_full_half(hess_t h, hipStream_t s) {
  if (!h->async) return flush_stage(h, s);
  if (capturing(s)) {
    int rc = join_side(h, s);
    if (rc != HESS_OK || h->stage_n == 0) return rc;
    rc = run_big(h, h->stage, h->stage_n, h->d, s, true, h->stage_real, async_wgs(h->d));
    if (rc == HESS_OK) h->stage_n = h->stage_real = 0;
    return rc;
  }
  hipError_t e = hipEventRecord(h->fork, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork, 0);
  if (e != hipSuccess) return hip_fail(e, "side stream ordering");
  const int rc = run_big(h, h->stage, h->stage_n, h->d, h->side, true, h->stage_real, async_wgs(h->d));
  if (rc != HESS_OK) return rc;
  e = hipEventRecord(h->side_done[h->cur], h->side);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  h->busy[h->cur] = true;
  h->pending = true;
  h->side_last = h->cur;
  h->cur ^= 1;
  h->stage = h->half[h->cur];
  h->stage_n = h->stage_real = 0;
  return HESS_OK;
}

// Grouped update on 256-tiles: the groups' rows are gathered into the
// device's scratch in the transposed staging layout (a multiple of 8 rows per
// group, zero-padded), then one launch takes whole upper tiles of every
// group.  Groups that do not fit are split; the scratch is refilled as many
// times as needed (each fill is one copy and one SYRK launch).
//
// direct (X's row count nrows known, nrows * ld * 2 < 2^31): no gather; the
// launch reads each group's rows where they are, through a table of their
// byte offsets in X (built per launch in the same buffer), with the same
// operands in the same order, so the same bits as the gathered path.
int grouped_big(hess_t* hs, int n_groups, const void* X, int64_t nrows, int64_t ld, const int32_t* row_idx,
                const int64_t* offsets, hipStream_t s) {
  const hess_t h0 = hs[0];
  const int64_t d = h0->d;
  BigWorkspace& W = g_big[h0->device];
  std::lock_guard<std::mutex> lock(W.mu);
  const bool direct = g_group_direct && nrows >= 0 && nrows * ld * 2 < ((int64_t)1 << 31);
  // the gather buffer (or row table): grown (never shrunk) to this call's
  // rows, up to 4 GiB
  int64_t need = 0;
  if (direct) {
    // each fill's table starts at the buffer's start; all groups' entries
    // bound any fill's
    for (int e = 0; e < n_groups; ++e) need += (offsets[e + 1] - offsets[e] + kBigKI - 1) / kBigKI * kBigKI;
    need = (need + kRowTableSlack) * 4 + kGroupSchedBytes;
  } else {
    for (int e = 0; e < n_groups; ++e) need += (offsets[e + 1] - offsets[e] + 7) / 8 * 8 * d * 2;
    need = std::min(need, kGroupScratchMax) + kGroupSchedBytes;
  }
  if (W.gbytes < need) {
    hipError_t e = hipSuccess;
    if (W.gptr) {
      e = hipDeviceSynchronize();
      if (e == hipSuccess) e = hipFree(W.gptr);
      W.gptr = nullptr;
      W.gbytes = 0;
    }
    if (e == hipSuccess) e = hipMalloc(&W.gptr, (size_t)need);
    if (e != hipSuccess) {
      W.gptr = nullptr;
      const int code = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? HESS_ENOMEM : HESS_EHIP;
      return fail(code, "grouped gather buffer (%lld bytes): %s", (long long)need, hipGetErrorString(e));
    }
    W.gbytes = need;
  }
  if (!W.hsched) {
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&W.hsched), (size_t)kGroupSchedBytes, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&W.sched_ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (W.hsched) (void)hipHostFree(W.hsched);
      W.hsched = nullptr;
      return hip_fail(e, "grouped schedule buffer");
    }
  }
  int64_t cap_bytes = W.gbytes - kGroupSchedBytes;
  if (g_group_chunk > 0) cap_bytes = std::min(cap_bytes, g_group_chunk);
  // 8-token blocks per fill (direct: whole groups, never split)
  const int64_t cap_blocks = direct ? ((int64_t)1 << 40) : cap_bytes / (d * 16);
  if (cap_blocks < 1) return fail(HESS_EINVAL, "grouped scratch smaller than one 8-row block");
  // pieces (group, first row, rows), largest groups first
  struct Piece { int e; int64_t beg, cnt; };
  std::vector<int> order;
  for (int e = 0; e < n_groups; ++e)
    if (offsets[e + 1] > offsets[e]) order.push_back(e);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return offsets[a + 1] - offsets[a] > offsets[b + 1] - offsets[b]; });
  std::vector<Piece> pieces;
  for (int e : order)
    for (int64_t b = offsets[e]; b < offsets[e + 1]; b += cap_blocks * 8)
      pieces.push_back({e, b, std::min(cap_blocks * 8, offsets[e + 1] - b)});
  hipError_t err = hipSuccess;
  if (W.used && W.last != s) {
    err = hipStreamWaitEvent(s, W.ev, 0);
    if (err != hipSuccess) return hip_fail(err, "hipStreamWaitEvent");
  }
  BigParams P;
  std::memset(&P, 0, sizeof(P));
  P.ld = direct ? ld : d;
  P.lds = d;
  P.order = h0->order256;
  P.d = (int)d;
  P.nb = h0->nb256;
  P.ntiles = h0->ntiles256;
  P.t8 = direct ? 0 : 1;
  size_t next = 0;
  while (next < pieces.size()) {
    // one fill: as many pieces as fit (at most kBigMaxGroups)
    GatherParams Gp;
    std::memset(&Gp, 0, sizeof(Gp));
    BigGroupParams Gb;
    std::memset(&Gb, 0, sizeof(Gb));
    int64_t blocks = 0;
    int k = 0;
    while (next < pieces.size() && k < kBigMaxGroups) {
      const Piece& pc = pieces[next];
      // 8-token blocks: gathered rows, or (direct) the table's entries in 8s,
      // a multiple of 32 entries per group
      const int64_t nblk = direct ? (pc.cnt + kBigKI - 1) / kBigKI * (kBigKI / 8) : (pc.cnt + 7) / 8;
      if (blocks + nblk > cap_blocks) break;
      Gp.beg[k] = pc.beg;
      Gp.cnt[k] = pc.cnt;
      Gp.blk[k] = blocks;
      Gp.blk_prefix[k] = blocks;
      Gb.blk[k] = direct ? blocks * 8 : blocks;
      Gb.n[k] = pc.cnt;
      Gb.S[k] = hs[pc.e]->S;
      blocks += nblk;
      ++k;
      ++next;
    }
    if (direct) {
      RowTableParams Tp;
      std::memset(&Tp, 0, sizeof(Tp));
      Tp.rows = row_idx;
      Tp.tbl = static_cast<int32_t*>(W.gptr);
      Tp.nrows = nrows;
      Tp.row_bytes = ld * 2;
      Tp.ngroups = k;
      for (int g = 0; g < k; ++g) {
        Tp.beg[g] = Gp.beg[g];
        Tp.cnt[g] = Gp.cnt[g];
        Tp.tstart[g] = Gp.blk[g] * 8;
      }
      Tp.tstart[k] = blocks * 8;
      Tp.total = blocks * 8 + kRowTableSlack;
      err = launch_row_table(Tp, s);
      if (err != hipSuccess) return hip_fail(err, "grouped row table launch");
    } else {
      Gp.blk_prefix[k] = blocks;
      Gp.X = X;
      Gp.rows = row_idx;
      Gp.dst = W.gptr;
      Gp.ld = ld;
      Gp.d = (int)d;
      Gp.fq = (int)((d + 255) / 256);
      Gp.ngroups = k;
      err = launch_gather_rows_t8(Gp, s);
      if (err != hipSuccess) return hip_fail(err, "grouped gather launch");
    }
    // the schedule: items longest first, each to the least-loaded workgroup
    // (cost: 32-token iterations plus a fixed cost for the tile's prologue
    // and output); workgroup w's items are kept in the order dealt
    const int nitems = k * P.ntiles;
    std::vector<std::vector<int32_t>> lists(kCUs);
    {
      std::vector<int> idx(k);
      for (int g = 0; g < k; ++g) idx[g] = g;
      std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return Gb.n[a] > Gb.n[b]; });
      using Slot = std::pair<int64_t, int>;
      std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> pq;
      for (int w = 0; w < kCUs; ++w) pq.push({0, w});
      for (int g : idx) {
        const int64_t iters = (Gb.n[g] + kBigKI - 1) / kBigKI;
        const int64_t cost = iters + kGroupItemCost * ((iters + kBigChain - 1) / kBigChain);
        for (int t = 0; t < P.ntiles; ++t) {
          Slot sl = pq.top();
          pq.pop();
          lists[sl.second].push_back(g * P.ntiles + t);
          pq.push({sl.first + cost, sl.second});
        }
      }
    }
    // the schedule goes through the pinned host buffer (once the previous
    // copy out of it has run) into the gather buffer's last bytes
    if (W.sched_pending) {
      err = hipEventSynchronize(W.sched_ev);
      if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
      W.sched_pending = false;
    }
    // slot s runs on workgroup (s / 32) + 8 (s % 32), i.e. slots 32x .. 32x+31
    // on XCD x: ties go to the lowest slot, so the first 256 items (the
    // largest groups' tiles in blocked order) reach the XCDs 32 at a time and
    // neighbouring tiles share panels in one L2
    int32_t* sched = W.hsched;
    sched[0] = kCUs + 1;
    for (int w = 0; w < kCUs; ++w) {
      const std::vector<int32_t>& li = lists[(w & 7) * 32 + (w >> 3)];
      std::copy(li.begin(), li.end(), sched + sched[w]);
      sched[w + 1] = sched[w] + (int32_t)li.size();
    }
    int32_t* dsched = reinterpret_cast<int32_t*>(static_cast<char*>(W.gptr) + W.gbytes - kGroupSchedBytes);
    err = hipMemcpyAsync(dsched, sched, (size_t)(kCUs + 1 + nitems) * sizeof(int32_t), hipMemcpyHostToDevice, s);
    if (err != hipSuccess) return hip_fail(err, "grouped schedule copy");
    err = hipEventRecord(W.sched_ev, s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    W.sched_pending = true;
    Gb.X = direct ? X : W.gptr;
    Gb.tbl = direct ? static_cast<const int32_t*>(W.gptr) : nullptr;
    Gb.xbytes = direct ? nrows * ld * 2 : 0;
    Gb.sched = dsched;
    Gb.ngroups = k;
    Gb.nitems = nitems;
    err = launch_syrk_big_grouped(P, Gb, s);
    if (err != hipSuccess) return hip_fail(err, "grouped 256-tile SYRK launch");
  }
  err = hipEventRecord(W.ev, s);
  if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
  W.used = true;
  W.last = s;
  return HESS_OK;
}

}  // namespace

extern "C" {

int hess_abi_version(void) { return HESS_ABI_VERSION; }

const char* hess_strerror(int code) {
  switch (code) {
    case HESS_OK: return "ok";
    case HESS_EINVAL: return "invalid argument";
    case HESS_ENOMEM: return "device allocation failed";
    case HESS_EHIP: return "HIP runtime error";
    case HESS_ESTATE: return "handle consumed by an in-place materialize";
    case HESS_EALIGN: return "misaligned input";
    case HESS_ENOTPD: return "matrix not positive definite";
    default: return "unknown status";
  }
}

const char* hess_last_error(void) { return g_err; }

int hess_set_tile_override(int edge) {
  if (edge != 0 && edge != 64 && edge != 128 && edge != 256)
    return fail(HESS_EINVAL, "tile override must be 0, 64, 128 or 256");
  g_tile_override = edge;
  return HESS_OK;
}

// Default staging at widths >= 1,024: 1 GiB, so that a flush is long
// enough for the 256-tile kernel (209,664 bf16 tokens at 2,560: one ragged
// calibration Hessian of ~375K tokens takes 2 passes).  Measured per Hessian
// on that workload: 4.8 ms with 64 MiB and 128-tile passes, 3.53 ms with
// 512 MiB (4 passes), 3.38-3.44 ms with 1 GiB, 3.52 ms with 2 GiB (one
// pass).  float32 rows at 4,096 (366K ragged tokens): 64.0 ms with 64 MiB,
// 54.3 with 256 MiB, 53.1-53.5 with 512 MiB or 1 GiB.  64 MiB otherwise.
int64_t default_staging(int64_t d) {
  return d >= 1024 ? HESS_STAGING_DEFAULT : ((int64_t)64 << 20);
}

hess_t hess_create(int64_t d, int in_dtype) { return hess_create_ex(d, in_dtype, default_staging(d)); }

hess_t hess_create_ex(int64_t d, int in_dtype, int64_t staging_bytes) {
  if (d < 1 || d > 65536) {
    fail(HESS_EINVAL, "d = %lld outside [1, 65536]", (long long)d);
    return nullptr;
  }
  if (in_dtype != HESS_BF16 && in_dtype != HESS_F32) {
    fail(HESS_EINVAL, "staging dtype %d is not HESS_BF16 or HESS_F32", in_dtype);
    return nullptr;
  }
  if (staging_bytes < 0 || staging_bytes > ((int64_t)16 << 30)) {
    fail(HESS_EINVAL, "staging_bytes = %lld outside [0, 16 GiB]", (long long)staging_bytes);
    return nullptr;
  }
  hess_t h = new (std::nothrow) hess_s();
  if (!h) {
    fail(HESS_ENOMEM, "host allocation failed");
    return nullptr;
  }
  h->d = d;
  h->dtype = in_dtype;
  hipError_t e = hipGetDevice(&h->device);
  const size_t sbytes = (size_t)d * (size_t)d * sizeof(float);
  if (e == hipSuccess) e = hipMalloc(&h->S, sbytes);
  if (e == hipSuccess) e = hipMalloc(&h->dead, (size_t)d);
  if (e == hipSuccess) e = hipMalloc(&h->damp, 64);
  // workspace for the partial tiles of a split last round
  if (e == hipSuccess) {
    h->ws_floats = kWsSlots * kTile * kTile;
    e = hipMalloc(&h->ws, (size_t)h->ws_floats * sizeof(float));
  }
  // staging rows for thin batches
  if (e == hipSuccess) {
    h->stage_cap = staging_bytes > 0 ? stage_tokens(d, esize(in_dtype), staging_bytes) : 0;
    h->stage_ld = (d + 7) / 8 * 8;
    if (h->stage_cap > 0) e = hipMalloc(&h->stage, (size_t)(h->stage_cap * h->stage_ld * esize(in_dtype)));
  }
  // 256-tile path: tile order and the device's shared stream-K workspace
  if (e == hipSuccess && big_capable(d, in_dtype)) {
    h->nb256 = (int)((d + kBig - 1) / kBig);
    const std::vector<int32_t> order = blocked_order(h->nb256);
    h->ntiles256 = (int)order.size();
    e = hipMalloc(&h->order256, order.size() * sizeof(int32_t));
    if (e == hipSuccess)
      e = hipMemcpy(h->order256, order.data(), order.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess && (h->device < 0 || h->device >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
      BigWorkspace& W = g_big[h->device];
      std::lock_guard<std::mutex> lock(W.mu);
      const int64_t need = big_slots(h->ntiles256);
      if (!W.ev) e = hipEventCreateWithFlags(&W.ev, hipEventDisableTiming);
      if (e == hipSuccess && W.slots < need) {
        if (W.ptr) {
          e = hipDeviceSynchronize();
          if (e == hipSuccess) e = hipFree(W.ptr);
          W.ptr = nullptr;
          W.slots = 0;
          W.used = false;
        }
        if (e == hipSuccess) e = hipMalloc(&W.ptr, (size_t)need * kBig * kBig * sizeof(float));
        if (e == hipSuccess) W.slots = need;
      }

    }
    // transposed staging when a full buffer's flush takes the 256-tile
    // kernel (with the tile override at create: 256 always, 128 never)
    if (h->stage_cap > 0 && g_tile_override != kTile) {
      const int64_t niter = h->stage_cap / kBigKI;
      h->stage_t8 = g_tile_override == kBig ||
                    (d >= kBigMinD && (int64_t)h->ntiles256 * niter >= kBigMinWork * kCUs);
    }
    // two halves flushed asynchronously when each half still makes a long
    // enough flush for the 256-tile kernel (and no tile is done whole)
    if (e == hipSuccess && h->stage_t8 && g_async && g_tile_override == 0 && h->ntiles256 < kCUs) {
      const int64_t hcap = stage_tokens(d, esize(in_dtype), staging_bytes / 2);
      if (hcap > 0 && (int64_t)h->ntiles256 * (hcap / kBigKI) >= kBigMinWork * kCUs) {
        h->async = true;
        h->stage_cap = hcap;
        h->half[0] = h->stage;
        h->half[1] = static_cast<char*>(h->stage) + hcap * h->stage_ld * esize(in_dtype);
        e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
        for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipEventCreateWithFlags(&h->side_done[k], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
      }
    }
  }
  if (e == hipSuccess) e = hipMemset(h->S, 0, sbytes);
  if (e == hipSuccess) e = hipMemset(h->damp, 0, 64);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    const int code = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? HESS_ENOMEM : HESS_EHIP;
    fail(code, "hess_create(d=%lld): %s", (long long)d, hipGetErrorString(e));
    (void)hipGetLastError();
    if (h->S) (void)hipFree(h->S);
    if (h->dead) (void)hipFree(h->dead);
    if (h->damp) (void)hipFree(h->damp);
    if (h->ws) (void)hipFree(h->ws);
    if (h->stage) (void)hipFree(h->stage);
    if (h->order256) (void)hipFree(h->order256);
    if (h->ev) (void)hipEventDestroy(h->ev);
    if (h->side) (void)hipStreamDestroy(h->side);
    for (hipEvent_t ev : h->side_done)
      if (ev) (void)hipEventDestroy(ev);
    if (h->fork) (void)hipEventDestroy(h->fork);
    delete h;
    return nullptr;
  }
  return h;
}

int hess_destroy(hess_t h) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  hipError_t e = hipSuccess;
  {
    // calls already inside the handle finish first; the caller must not
    // start new ones once it destroys the handle
    HLock lock(h->mu);
    if (h->has_stream) e = hipStreamSynchronize(h->last);
    if (h->side) {
      const hipError_t e2 = hipStreamSynchronize(h->side);
      if (e == hipSuccess) e = e2;
    }
  }
  if (h->side) {
    (void)hipStreamDestroy(h->side);
    for (hipEvent_t ev : h->side_done) (void)hipEventDestroy(ev);
    (void)hipEventDestroy(h->fork);
  }
  (void)hipFree(h->S);
  (void)hipFree(h->dead);
  (void)hipFree(h->damp);
  if (h->ws) (void)hipFree(h->ws);
  // the staging allocation starts at its first half (stage may point at the second)
  void* stage_base = h->async ? h->half[0] : h->stage;
  if (stage_base) (void)hipFree(stage_base);
  if (h->order256) (void)hipFree(h->order256);
  (void)hipEventDestroy(h->ev);
  for (hipEvent_t ev : h->tev) (void)hipEventDestroy(ev);
  delete h;
  return e == hipSuccess ? HESS_OK : hip_fail(e, "hess_destroy");
}

int hess_add_batch(hess_t h, const void* X, int64_t n_tokens, int64_t ld, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  if (h->consumed) return fail(HESS_ESTATE, "handle was materialized in place; hess_reset it first");
  if (n_tokens < 0) return fail(HESS_EINVAL, "n_tokens = %lld < 0", (long long)n_tokens);
  if (ld < h->d) return fail(HESS_EINVAL, "ld = %lld < d = %lld", (long long)ld, (long long)h->d);
  if (n_tokens == 0) return HESS_OK;
  if (!X) return fail(HESS_EINVAL, "X is NULL with n_tokens > 0");
  if (reinterpret_cast<uintptr_t>(X) % esize(h->dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
  if (rc != HESS_OK) return rc;
  if (stage_pays(h, n_tokens)) {
    // thin batch: append its rows to the staging buffer
    const int64_t rows = h->stage_t8 ? (n_tokens + 7) / 8 * 8 : n_tokens;
    if (h->stage_n + rows > h->stage_cap) {
      rc = flush_full_half(h, s);
      if (rc != HESS_OK) return rc;
    }
    rc = claim_half(h, s);
    if (rc != HESS_OK) return rc;
    char* dst = static_cast<char*>(h->stage) + h->stage_n * h->stage_ld * esize(h->dtype);
    hipError_t e = h->stage_t8 ? launch_copy_rows_t8(X, ld, n_tokens, h->d, dst, s)
                               : launch_copy_rows(X, ld, esize(h->dtype), n_tokens, h->d, dst, h->stage_ld, s);
    if (e != hipSuccess) return hip_fail(e, "staging copy launch");
    h->stage_n += rows;
    h->stage_real += n_tokens;
  } else {
    // long batch: its own SYRK pass, after whatever is staged
    rc = flush_stage(h, s);
    if (rc != HESS_OK) return rc;
    rc = run_syrk(h, X, n_tokens, ld, s);
    if (rc != HESS_OK) return rc;
  }
  h->N += n_tokens;
  return HESS_OK;
}

int hess_add_batch_cast(hess_t h, const void* X, int x_dtype, int64_t n_tokens, int64_t ld, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  if (x_dtype != HESS_BF16 && x_dtype != HESS_F32 && x_dtype != HESS_F16)
    return fail(HESS_EINVAL, "unknown activation dtype %d", x_dtype);
  if (x_dtype == h->dtype) return hess_add_batch(h, X, n_tokens, ld, stream);
  if (h->consumed) return fail(HESS_ESTATE, "handle was materialized in place; hess_reset it first");
  if (n_tokens < 0) return fail(HESS_EINVAL, "n_tokens = %lld < 0", (long long)n_tokens);
  if (ld < h->d) return fail(HESS_EINVAL, "ld = %lld < d = %lld", (long long)ld, (long long)h->d);
  if (n_tokens == 0) return HESS_OK;
  if (!X) return fail(HESS_EINVAL, "X is NULL with n_tokens > 0");
  const int xes = x_dtype == HESS_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(X) % xes != 0) return fail(HESS_EALIGN, "X not element-aligned");
  if (!h->stage) return fail(HESS_EINVAL, "converting activations needs the handle's staging buffer (staging_bytes > 0)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
  if (rc != HESS_OK) return rc;
  // the rows go through the staging buffer, converted on the copy, in pieces
  // that fit; a full buffer is folded into S first (8-row blocks in the
  // transposed layout keep the buffer's fill a multiple of 8)
  const int64_t unit = h->stage_t8 ? 8 : 1;
  for (int64_t off = 0; off < n_tokens;) {
    if (h->stage_cap - h->stage_n < unit) {
      rc = flush_full_half(h, s);
      if (rc != HESS_OK) return rc;
    }
    rc = claim_half(h, s);
    if (rc != HESS_OK) return rc;
    const int64_t space = h->stage_cap - h->stage_n;
    int64_t take = n_tokens - off < space ? n_tokens - off : space;
    if (take < n_tokens - off) take = take / unit * unit;
    const int64_t rows = (take + unit - 1) / unit * unit;
    char* dst = static_cast<char*>(h->stage) + h->stage_n * h->stage_ld * esize(h->dtype);
    hipError_t e = launch_cast_rows(static_cast<const char*>(X) + off * ld * xes, x_dtype, ld, take, h->d, dst,
                                    h->dtype, h->stage_ld, h->stage_t8, s);
    if (e != hipSuccess) return hip_fail(e, "converting staging copy launch");
    h->stage_n += rows;
    h->stage_real += take;
    off += take;
  }
  h->N += n_tokens;
  return HESS_OK;
}

int hess_add_batch_grouped(hess_t* hs, int n_groups, const void* X, int64_t ld, const int32_t* row_idx,
                           const int64_t* offsets, hess_stream_t stream) {
  return hess_add_batch_grouped_ex(hs, n_groups, X, -1, ld, row_idx, offsets, stream);
}

int hess_add_batch_grouped_ex(hess_t* hs, int n_groups, const void* X, int64_t n_rows, int64_t ld,
                              const int32_t* row_idx, const int64_t* offsets, hess_stream_t stream) {
  if (!hs || n_groups < 1) return fail(HESS_EINVAL, "need at least one handle");
  GroupLock lock(hs, n_groups);
  if (!offsets) return fail(HESS_EINVAL, "offsets is NULL");
  const hess_t h0 = hs[0];
  if (!h0) return fail(HESS_EINVAL, "null handle 0");
  for (int e = 0; e < n_groups; ++e) {
    if (!hs[e]) return fail(HESS_EINVAL, "null handle %d", e);
    if (hs[e]->d != h0->d || hs[e]->dtype != h0->dtype)
      return fail(HESS_EINVAL, "handle %d differs in width or input type from handle 0", e);
    if (hs[e]->consumed) return fail(HESS_ESTATE, "handle %d was materialized in place", e);
    for (int f = 0; f < e; ++f)
      if (hs[f] == hs[e]) return fail(HESS_EINVAL, "handle %d repeats handle %d", e, f);
  }
  if (offsets[0] != 0) return fail(HESS_EINVAL, "offsets[0] must be 0");
  for (int e = 0; e < n_groups; ++e)
    if (offsets[e + 1] < offsets[e]) return fail(HESS_EINVAL, "offsets decrease at %d", e);
  if (ld < h0->d) return fail(HESS_EINVAL, "ld < d");
  const int64_t total = offsets[n_groups];
  if (n_rows < -1) return fail(HESS_EINVAL, "n_rows = %lld < 0", (long long)n_rows);
  if (n_rows >= 0 && !row_idx && total > n_rows)
    return fail(HESS_EINVAL, "without row_idx the groups' %lld rows exceed n_rows = %lld", (long long)total,
                (long long)n_rows);
  if (total == 0) return HESS_OK;
  if (!X) return fail(HESS_EINVAL, "X is NULL");
  if (reinterpret_cast<uintptr_t>(X) % esize(h0->dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int e = 0; e < n_groups; ++e) {
    int rc = order_stream(hs[e], s);
    if (rc == HESS_OK) rc = join_side(hs[e], s);
    if (rc != HESS_OK) return rc;
  }
  const bool vec = vec_ok(X, ld, h0->d, esize(h0->dtype));
  if (vec && h0->order256 && h0->d >= kBigMinD && g_tile_override != kTile) {
    const int rc = grouped_big(hs, n_groups, X, n_rows, ld, row_idx, offsets, s);
    if (rc != HESS_OK) return rc;
    for (int e = 0; e < n_groups; ++e) hs[e]->N += offsets[e + 1] - offsets[e];
    return HESS_OK;
  }
  const int nb = (int)((h0->d + kTile - 1) / kTile);
  const int ntiles = nb * (nb + 1) / 2;
  // longest groups first, so their workgroups start in the first round
  std::vector<int> order;
  for (int e = 0; e < n_groups; ++e)
    if (offsets[e + 1] > offsets[e]) order.push_back(e);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return offsets[a + 1] - offsets[a] > offsets[b + 1] - offsets[b]; });
  for (size_t base = 0; base < order.size(); base += kMaxGroups) {
    const int cnt = (int)std::min<size_t>(kMaxGroups, order.size() - base);
    SyrkParams P;
    std::memset(&P, 0, sizeof(P));
    P.X = X;
    P.rows = row_idx;
    P.ld = ld;
    P.lds = h0->d;
    P.d = (int)h0->d;
    P.nb = nb;
    P.ntiles = ntiles;
    P.ngroups = cnt;
    P.flush_iters = flush_iters(h0->dtype);
    P.full_tiles = ntiles;
    P.grid_full = grid8(ntiles);
    P.s_vec = (h0->d % 4) == 0;
    P.item_prefix[0] = 0;
    for (int k = 0; k < cnt; ++k) {
      const int e = order[base + k];
      P.g[k] = SyrkGroup{hs[e]->S, offsets[e], offsets[e + 1]};
      P.item_prefix[k + 1] = P.item_prefix[k] + ntiles;
    }
    const int grid = cnt > 1 ? P.item_prefix[cnt] : P.grid_full;
    hipError_t err = launch_syrk(P, h0->dtype, vec, grid, s);
    if (err != hipSuccess) return hip_fail(err, "grouped SYRK launch");
  }
  for (int e = 0; e < n_groups; ++e) hs[e]->N += offsets[e + 1] - offsets[e];
  return HESS_OK;
}

int hess_materialize_ex(hess_t h, float damp_percent, unsigned flags, float* H_out, uint8_t* dead_out,
                        float* damp_out, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  if (h->consumed) return fail(HESS_ESTATE, "handle was materialized in place; hess_reset it first");
  if (!(damp_percent >= 0.0f && damp_percent < 1.0f))
    return fail(HESS_EINVAL, "damp_percent must be in [0, 1)");
  if (flags & ~HESS_NO_NEUTRALIZE) return fail(HESS_EINVAL, "unknown flags 0x%x", flags);
  if (H_out == h->S) return fail(HESS_EINVAL, "H_out aliases the Gram buffer; pass NULL for in place");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
  if (rc != HESS_OK) return rc;
  rc = flush_stage(h, s);
  if (rc != HESS_OK) return rc;
  const float scale = h->N > 0 ? (float)(2.0 / (double)h->N) : 0.0f;
  float* H = H_out ? H_out : h->S;
  uint8_t* dead = dead_out ? dead_out : h->dead;
  float* damp = damp_out ? damp_out : h->damp;
  hipError_t e = launch_materialize(h->S, h->d, (int)h->d, scale, damp_percent,
                                    (flags & HESS_NO_NEUTRALIZE) ? 0 : 1, H, dead, damp, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "materialize launch");
  if (!H_out) h->consumed = true;
  return HESS_OK;
}

int hess_materialize(hess_t h, float damp_percent, float* H_out) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  if (!H_out) return fail(HESS_EINVAL, "H_out is NULL (use hess_materialize_ex for in place)");
  return hess_materialize_ex(h, damp_percent, 0u, H_out, nullptr, nullptr, h->has_stream ? h->last : nullptr);
}

namespace {
// Handles of one grouped call: non-null, distinct, one width; ordered on s.
int check_group(hess_t* hs, int n_groups, hipStream_t s, bool allow_consumed) {
  if (!hs || n_groups < 1) return fail(HESS_EINVAL, "need at least one handle");
  for (int e = 0; e < n_groups; ++e) {
    if (!hs[e]) return fail(HESS_EINVAL, "null handle %d", e);
    if (hs[e]->d != hs[0]->d) return fail(HESS_EINVAL, "handle %d differs in width from handle 0", e);
    if (!allow_consumed && hs[e]->consumed) return fail(HESS_ESTATE, "handle %d was materialized in place", e);
    for (int f = 0; f < e; ++f)
      if (hs[f] == hs[e]) return fail(HESS_EINVAL, "handle %d repeats handle %d", e, f);
  }
  for (int e = 0; e < n_groups; ++e) {
    int rc = order_stream(hs[e], s);
    if (rc == HESS_OK) rc = join_side(hs[e], s);
    if (rc != HESS_OK) return rc;
  }
  return HESS_OK;
}
}  // namespace

int hess_reset_grouped(hess_t* hs, int n_groups, hess_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  GroupLock lock(hs, hs ? n_groups : 0);
  int rc = check_group(hs, n_groups, s, true);
  if (rc != HESS_OK) return rc;
  const int64_t d = hs[0]->d;
  for (int base = 0; base < n_groups; base += kMatMaxGroups) {
    const int cnt = std::min(kMatMaxGroups, n_groups - base);
    float* S[kMatMaxGroups];
    for (int k = 0; k < cnt; ++k) S[k] = hs[base + k]->S;
    hipError_t e = launch_zero_upper_grouped(S, cnt, d, (int)d, s);
    if (e != hipSuccess) return hip_fail(e, "grouped reset launch");
  }
  for (int e = 0; e < n_groups; ++e) {
    hs[e]->stage_n = hs[e]->stage_real = 0;
    hs[e]->N = 0;
    hs[e]->consumed = false;
  }
  return HESS_OK;
}

int hess_materialize_grouped(hess_t* hs, int n_groups, float damp_percent, unsigned flags, float* const* H_out,
                             uint8_t* const* dead_out, float* const* damp_out, hess_stream_t stream) {
  if (!(damp_percent >= 0.0f && damp_percent < 1.0f)) return fail(HESS_EINVAL, "damp_percent must be in [0, 1)");
  if (flags & ~HESS_NO_NEUTRALIZE) return fail(HESS_EINVAL, "unknown flags 0x%x", flags);
  if (!H_out) return fail(HESS_EINVAL, "H_out is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  GroupLock lock(hs, hs ? n_groups : 0);
  int rc = check_group(hs, n_groups, s, false);
  if (rc != HESS_OK) return rc;
  for (int e = 0; e < n_groups; ++e)
    if (H_out[e] == hs[e]->S) return fail(HESS_EINVAL, "H_out[%d] aliases its Gram buffer; pass NULL for in place", e);
  for (int e = 0; e < n_groups; ++e) {
    rc = flush_stage(hs[e], s);
    if (rc != HESS_OK) return rc;
  }
  const int64_t d = hs[0]->d;
  for (int base = 0; base < n_groups; base += kMatMaxGroups) {
    const int cnt = std::min(kMatMaxGroups, n_groups - base);
    MatGroupParams P;
    std::memset(&P, 0, sizeof(P));
    P.ngroups = cnt;
    P.d = (int)d;
    P.lds = d;
    P.damp_percent = damp_percent;
    P.neutralize = (flags & HESS_NO_NEUTRALIZE) ? 0 : 1;
    for (int k = 0; k < cnt; ++k) {
      const hess_t h = hs[base + k];
      P.g[k].S = h->S;
      P.g[k].H = H_out[base + k] ? H_out[base + k] : h->S;
      P.g[k].dead = (dead_out && dead_out[base + k]) ? dead_out[base + k] : h->dead;
      P.g[k].damp = (damp_out && damp_out[base + k]) ? damp_out[base + k] : h->damp;
      P.g[k].scale = h->N > 0 ? (float)(2.0 / (double)h->N) : 0.0f;
    }
    if (materialize_grouped_ok(P)) {
      hipError_t e = launch_materialize_grouped(P, s);
      if (e != hipSuccess) return hip_fail(e, "grouped materialize launch");
    } else {
      // unaligned buffers or d % 4 != 0: one materialize per Hessian
      for (int k = 0; k < cnt; ++k) {
        const hess_t h = hs[base + k];
        hipError_t e = launch_materialize(h->S, d, (int)d, P.g[k].scale, damp_percent, P.neutralize, P.g[k].H,
                                          P.g[k].dead, P.g[k].damp, nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "materialize launch");
      }
    }
  }
  for (int e = 0; e < n_groups; ++e)
    if (!H_out[e]) hs[e]->consumed = true;
  return HESS_OK;
}

int hess_reset(hess_t h, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
  if (rc == HESS_OK) rc = join_side(h, s);
  if (rc != HESS_OK) return rc;
  hipError_t e = launch_zero_upper(h->S, h->d, (int)h->d, s);
  if (e != hipSuccess) return hip_fail(e, "reset launch");
  h->stage_n = h->stage_real = 0;
  h->N = 0;
  h->consumed = false;
  return HESS_OK;
}

int hess_flush(hess_t h, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  if (h->consumed) return fail(HESS_ESTATE, "handle was materialized in place; hess_reset it first");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
  if (rc != HESS_OK) return rc;
  return flush_stage(h, s);
}

int hess_adopt(hess_t dst, hess_t src, hess_stream_t stream) {
  if (!dst || !src) return fail(HESS_EINVAL, "null handle");
  if (dst == src) return HESS_OK;
  hess_t pair[2] = {dst, src};
  GroupLock lock(pair, 2);
  if (dst->d != src->d) return fail(HESS_EINVAL, "width mismatch: %lld vs %lld", (long long)dst->d, (long long)src->d);
  // the staging type and the staging buffer (the chunking of the sum) decide
  // what the sum holds and its rounding order: only equal settings share
  if (dst->dtype != src->dtype || dst->stage_cap != src->stage_cap || dst->stage_t8 != src->stage_t8)
    return fail(HESS_EINVAL, "accumulation settings differ (staging dtype %d vs %d, staging rows %lld vs %lld)",
                dst->dtype, src->dtype, (long long)dst->stage_cap, (long long)src->stage_cap);
  if (src->consumed) return fail(HESS_ESTATE, "source was materialized in place; hess_reset it first");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(src, s);
  if (rc != HESS_OK) return rc;
  rc = order_stream(dst, s);
  if (rc != HESS_OK) return rc;
  rc = flush_stage(src, s);  // the source's sum is complete
  if (rc == HESS_OK) rc = join_side(dst, s);
  if (rc != HESS_OK) return rc;
  hipError_t e = hipMemcpyAsync(dst->S, src->S, (size_t)src->d * src->d * sizeof(float), hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "adopt copy");
  dst->stage_n = dst->stage_real = 0;  // the follower's own partials are dropped
  dst->N = src->N;
  dst->consumed = false;
  return HESS_OK;
}

int64_t hess_chol_inverse_workspace(int64_t d) {
  if (d < 1 || d > kCholMaxD) return -1;
  const int64_t dp = chol_padded(d);
  return (2 * dp * dp + dp * 64) * (int64_t)sizeof(double);
}

int hess_chol_inverse_upper(const float* H, int64_t d, int64_t ldh, float* U, int64_t ldu, void* work,
                            int64_t work_bytes, int* info, hess_stream_t stream) {
  if (d < 1 || d > kCholMaxD) return fail(HESS_EINVAL, "d = %lld outside [1, %lld]", (long long)d, (long long)kCholMaxD);
  if (!H || !U || !work) return fail(HESS_EINVAL, "null H, U or workspace");
  if (ldh < d || ldu < d) return fail(HESS_EINVAL, "row stride below d");
  if ((reinterpret_cast<uintptr_t>(H) & 3u) || (reinterpret_cast<uintptr_t>(U) & 3u))
    return fail(HESS_EALIGN, "H or U not float-aligned");
  if (reinterpret_cast<uintptr_t>(work) & 15u) return fail(HESS_EALIGN, "workspace not 16-byte aligned");
  const int64_t need = hess_chol_inverse_workspace(d);
  if (work_bytes < need)
    return fail(HESS_EINVAL, "workspace of %lld bytes, %lld needed", (long long)work_bytes, (long long)need);
  // U may be H itself (same stride); any other overlap is refused
  const uintptr_t h0 = reinterpret_cast<uintptr_t>(H), h1 = h0 + (uintptr_t)(((d - 1) * ldh + d) * 4);
  const uintptr_t u0 = reinterpret_cast<uintptr_t>(U), u1 = u0 + (uintptr_t)(((d - 1) * ldu + d) * 4);
  if (u0 < h1 && h0 < u1 && !(u0 == h0 && ldu == ldh)) return fail(HESS_EINVAL, "U overlaps H without being H");
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(work), w1 = w0 + (uintptr_t)need;
  if ((w0 < h1 && h0 < w1) || (w0 < u1 && u0 < w1)) return fail(HESS_EINVAL, "workspace overlaps H or U");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t dp = chol_padded(d);
  double* A = static_cast<double*>(work);
  hipError_t e = launch_chol_inverse_upper(H, ldh, (int)d, U, ldu, A, A + dp * dp, A + 2 * dp * dp, info, s);
  return e == hipSuccess ? HESS_OK : hip_fail(e, "Cholesky-of-inverse launch");
}

int64_t hess_gptq_quantize_workspace(int64_t rows, int64_t cols) {
  if (rows < 1 || rows > kQuantMaxDim || cols < 1 || cols > kQuantMaxDim) return -1;
  return quant_workspace_doubles(rows, cols) * (int64_t)sizeof(double);
}

namespace {
bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}
}  // namespace

int hess_gptq_quantize(const float* W, int64_t rows, int64_t cols, int64_t ldw, const float* U, int64_t ldu,
                       const uint8_t* dead, int group_size, float* Q, int64_t ldq, uint8_t* codes, int64_t ldc,
                       float* scales, double* loss, int64_t nsamples, void* work, int64_t work_bytes,
                       hess_stream_t stream) {
  if (rows < 1 || rows > kQuantMaxDim || cols < 1 || cols > kQuantMaxDim)
    return fail(HESS_EINVAL, "rows = %lld, cols = %lld outside [1, %lld]", (long long)rows, (long long)cols,
                (long long)kQuantMaxDim);
  if (!W || !U || !Q || !codes || !scales || !work) return fail(HESS_EINVAL, "null W, U, Q, codes, scales or workspace");
  if (ldw < cols || ldu < cols || ldq < cols || ldc < cols) return fail(HESS_EINVAL, "row stride below cols");
  if (!(group_size == -1 || (group_size >= 1 && (group_size >= cols || 128 % group_size == 0))))
    return fail(HESS_EINVAL, "group_size %d: -1, >= cols, or a divisor of 128", group_size);
  if (loss && nsamples < 1) return fail(HESS_EINVAL, "nsamples = %lld < 1", (long long)nsamples);
  if ((reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Q) |
       reinterpret_cast<uintptr_t>(scales)) & 3u)
    return fail(HESS_EALIGN, "W, U, Q or scales not float-aligned");
  if ((reinterpret_cast<uintptr_t>(work) & 15u) || (reinterpret_cast<uintptr_t>(loss) & 7u))
    return fail(HESS_EALIGN, "workspace not 16-byte or loss not 8-byte aligned");
  const int64_t need = hess_gptq_quantize_workspace(rows, cols);
  if (work_bytes < need)
    return fail(HESS_EINVAL, "workspace of %lld bytes, %lld needed", (long long)work_bytes, (long long)need);
  const int groups = (group_size <= 0 || group_size >= cols) ? 1 : (int)((cols + group_size - 1) / group_size);
  const int64_t wb = ((rows - 1) * ldw + cols) * 4, ub = ((cols - 1) * ldu + cols) * 4;
  const int64_t qb = ((rows - 1) * ldq + cols) * 4, cb = (rows - 1) * ldc + cols, sb = rows * groups * 4;
  // Q may be W itself (same stride: the working copy is taken first); nothing else may overlap
  if (overlaps(Q, qb, W, wb) && !(static_cast<const void*>(Q) == static_cast<const void*>(W) && ldq == ldw))
    return fail(HESS_EINVAL, "Q overlaps W without being W");
  const void* outs[3] = {Q, codes, scales};
  const int64_t outb[3] = {qb, cb, sb};
  for (int a = 0; a < 3; ++a) {
    if (overlaps(outs[a], outb[a], U, ub) || overlaps(outs[a], outb[a], work, need))
      return fail(HESS_EINVAL, "an output overlaps U or the workspace");
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], outb[a], outs[b], outb[b])) return fail(HESS_EINVAL, "outputs overlap");
  }
  if (overlaps(work, need, W, wb) || overlaps(work, need, U, ub)) return fail(HESS_EINVAL, "workspace overlaps W or U");
  QuantParams P{W, ldw, (int)rows, (int)cols, U, ldu, dead, group_size, Q, ldq, codes, ldc, scales, loss,
                nsamples, static_cast<double*>(work)};
  hipError_t e = launch_gptq_quantize(P, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HESS_OK : hip_fail(e, "block-quantize launch");
}

int hess_set_group_chunk(int64_t bytes) {
  if (bytes < 0) return fail(HESS_EINVAL, "group chunk must be >= 0");
  g_group_chunk = bytes;
  return HESS_OK;
}

int hess_set_group_direct(int enable) {
  g_group_direct = enable != 0;
  return HESS_OK;
}

int hess_set_staging(int enable) {
  g_staging = enable != 0;
  return HESS_OK;
}

int hess_set_async_flush(int enable) {
  g_async = enable != 0;
  return HESS_OK;
}

int hess_set_timing(hess_t h, int on) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  h->timing = on != 0;
  h->tcount = 0;
  return HESS_OK;
}

int hess_timing(hess_t h, int64_t* launches, int64_t* tokens, double* ms) {
  if (!h || !launches || !tokens || !ms) return fail(HESS_EINVAL, "null argument");
  HLock lock(h->mu);
  double total = 0.0;
  int64_t tok = 0;
  if (h->tcount > 0) {
    hipError_t e = hipEventSynchronize(h->tev[2 * h->tcount - 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    for (size_t i = 0; i < h->tcount; ++i) {
      float t = 0.0f;
      e = hipEventElapsedTime(&t, h->tev[2 * i], h->tev[2 * i + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      total += t;
      tok += h->ttok[i];
    }
  }
  *launches = (int64_t)h->tcount;
  *tokens = tok;
  *ms = total;
  h->tcount = 0;
  return HESS_OK;
}

int hess_token_count(hess_t h, int64_t* n_out) {
  if (!h || !n_out) return fail(HESS_EINVAL, "null argument");
  HLock lock(h->mu);
  *n_out = h->N;
  return HESS_OK;
}

int hess_info(hess_t h, int64_t* d_out, int* in_dtype_out) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  HLock lock(h->mu);
  if (d_out) *d_out = h->d;
  if (in_dtype_out) *in_dtype_out = h->dtype;
  return HESS_OK;
}

int hess_state_buffer(hess_t h, const float** S_out) {
  if (!h || !S_out) return fail(HESS_EINVAL, "null argument");
  HLock lock(h->mu);
  *S_out = h->S;
  return HESS_OK;
}

// Argument checks shared by the local-block entry points.
int local_check(const void* X, int in_dtype, int64_t n_tokens, int64_t d, int64_t ld, int block, const float* out) {
  if (in_dtype != HESS_BF16 && in_dtype != HESS_F32) return fail(HESS_EINVAL, "unknown input dtype %d", in_dtype);
  if (block != 16) return fail(HESS_EINVAL, "block must be 16");
  if (d < 16 || d % 16 != 0 || d > (1 << 30)) return fail(HESS_EINVAL, "d must be a positive multiple of 16");
  if (ld < d) return fail(HESS_EINVAL, "ld < d");
  if (n_tokens < 0) return fail(HESS_EINVAL, "n_tokens < 0");
  if (!out) return fail(HESS_EINVAL, "out is NULL");
  if (n_tokens > 0 && !X) return fail(HESS_EINVAL, "X is NULL with n_tokens > 0");
  if (reinterpret_cast<uintptr_t>(X) % esize(in_dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  return HESS_OK;
}

int hess_local_blocks_ex(const void* X, int in_dtype, int64_t n_tokens, int64_t d, int64_t ld, int block,
                         float* out, int accumulate, hess_stream_t stream) {
  int rc = local_check(X, in_dtype, n_tokens, d, ld, block, out);
  if (rc != HESS_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = n_tokens > 0 && vec_ok(X, ld, d, esize(in_dtype));
  // the plan fits kLocalPartBytes up to width 262,144 (one slice beyond)
  const int64_t part_cap = std::max<int64_t>(kLocalPartBytes, (d / 16) * 1024);
  const LocalPlan pl = local_plan(n_tokens, (int)d, part_cap);
  if (n_tokens == 0) {
    hipError_t e = launch_local_blocks(X, in_dtype, 0, (int)d, ld, vec, out, accumulate, pl, nullptr, s);
    return e == hipSuccess ? HESS_OK : hip_fail(e, "local blocks launch");
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HESS_EINVAL, "device %d out of range", dev);
  LocalScratch& L = g_local[dev];
  std::lock_guard<std::mutex> lock(L.mu);
  if (L.bytes < pl.part_bytes) {
    if (L.ptr) {
      e = hipDeviceSynchronize();
      if (e == hipSuccess) e = hipFree(L.ptr);
      L.ptr = nullptr;
      L.bytes = 0;
      L.used = false;
    }
    const int64_t want = std::max(pl.part_bytes, kLocalPartBytes);
    if (e == hipSuccess) e = hipMalloc(&L.ptr, (size_t)want);
    if (e == hipSuccess && !L.ev) e = hipEventCreateWithFlags(&L.ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      L.ptr = nullptr;
      const int code = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? HESS_ENOMEM : HESS_EHIP;
      return fail(code, "local-block scratch (%lld bytes): %s", (long long)want, hipGetErrorString(e));
    }
    L.bytes = want;
  }
  if (L.used && L.last != s) {
    e = hipStreamWaitEvent(s, L.ev, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  e = launch_local_blocks(X, in_dtype, n_tokens, (int)d, ld, vec, out, accumulate, pl, L.ptr, s);
  if (e != hipSuccess) return hip_fail(e, "local blocks launch");
  e = hipEventRecord(L.ev, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  L.used = true;
  L.last = s;
  return HESS_OK;
}

int hess_local_blocks_noalloc(const void* X, int in_dtype, int64_t n_tokens, int64_t d, int64_t ld, int block,
                              float* out, int accumulate, hess_stream_t stream) {
  int rc = local_check(X, in_dtype, n_tokens, d, ld, block, out);
  if (rc != HESS_OK) return rc;
  const LocalPlan pl = local_plan(n_tokens, (int)d, kLocalPartBytes);
  if (n_tokens > 0 && pl.part_bytes > kLocalPartBytes)
    return fail(HESS_EINVAL, "width %lld needs %lld bytes of partial sums; the allocation-free call holds %lld "
                "(widths up to 262,144)", (long long)d, (long long)pl.part_bytes, (long long)kLocalPartBytes);
  float* part = nullptr;
  hipError_t e = hipSuccess;
  if (n_tokens > 0) {
    e = local_static_scratch(&part);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress");
  }
  const bool vec = n_tokens > 0 && vec_ok(X, ld, d, esize(in_dtype));
  e = launch_local_blocks(X, in_dtype, n_tokens, (int)d, ld, vec, out, accumulate, pl, part,
                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HESS_OK : hip_fail(e, "local blocks launch");
}

int hess_local_blocks(const void* X, int64_t n_tokens, int64_t d, int block, float* out) {
  return hess_local_blocks_ex(X, HESS_BF16, n_tokens, d, d, block, out, 1, nullptr);
}

// ---- imatrix statistic: per-column float32 sums of squares ----

hess_imx_t hess_imatrix_create(int64_t d, int in_dtype) {
  if (d < 1 || d > ((int64_t)1 << 24)) {
    fail(HESS_EINVAL, "d = %lld outside [1, 2^24]", (long long)d);
    return nullptr;
  }
  if (in_dtype != HESS_BF16 && in_dtype != HESS_F32) {
    fail(HESS_EINVAL, "unknown input dtype %d", in_dtype);
    return nullptr;
  }
  hess_imx_t m = new (std::nothrow) hess_imx_s();
  if (!m) {
    fail(HESS_ENOMEM, "host allocation failed");
    return nullptr;
  }
  m->d = d;
  m->dtype = in_dtype;
  hipError_t e = hipMalloc(&m->acc, (size_t)d * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&m->part, (size_t)kImxSplits * d * sizeof(float));
  if (e == hipSuccess) e = hipMemset(m->acc, 0, (size_t)d * sizeof(float));
  if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    const int code = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? HESS_ENOMEM : HESS_EHIP;
    fail(code, "hess_imatrix_create(d=%lld): %s", (long long)d, hipGetErrorString(e));
    (void)hipGetLastError();
    if (m->acc) (void)hipFree(m->acc);
    if (m->part) (void)hipFree(m->part);
    if (m->ev) (void)hipEventDestroy(m->ev);
    delete m;
    return nullptr;
  }
  return m;
}

int hess_imatrix_destroy(hess_imx_t m) {
  if (!m) return fail(HESS_EINVAL, "null handle");
  hipError_t e = hipSuccess;
  {
    HLock lock(m->mu);
    if (m->has_stream) e = hipStreamSynchronize(m->last);
  }
  (void)hipFree(m->acc);
  (void)hipFree(m->part);
  (void)hipEventDestroy(m->ev);
  delete m;
  return e == hipSuccess ? HESS_OK : hip_fail(e, "hess_imatrix_destroy");
}

int hess_imatrix_add_batch(hess_imx_t m, const void* X, int64_t n_tokens, int64_t ld, hess_stream_t stream) {
  if (!m) return fail(HESS_EINVAL, "null handle");
  HLock lock(m->mu);
  if (n_tokens < 0) return fail(HESS_EINVAL, "n_tokens = %lld < 0", (long long)n_tokens);
  if (ld < m->d) return fail(HESS_EINVAL, "ld = %lld < d = %lld", (long long)ld, (long long)m->d);
  if (n_tokens == 0) return HESS_OK;
  if (!X) return fail(HESS_EINVAL, "X is NULL with n_tokens > 0");
  if (reinterpret_cast<uintptr_t>(X) % esize(m->dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = imx_order_stream(m, s);
  if (rc != HESS_OK) return rc;
  const bool vec = vec_ok(X, ld, m->d, esize(m->dtype));
  hipError_t e = launch_imatrix(X, m->dtype, n_tokens, (int)m->d, ld, vec, m->part, (int)kImxSplits, m->acc, s);
  if (e != hipSuccess) return hip_fail(e, "imatrix launch");
  m->N += n_tokens;
  return HESS_OK;
}

int hess_imatrix_read(hess_imx_t m, float* out, int64_t* n_out, hess_stream_t stream) {
  if (!m) return fail(HESS_EINVAL, "null handle");
  HLock lock(m->mu);
  if (!out) return fail(HESS_EINVAL, "out is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = imx_order_stream(m, s);
  if (rc != HESS_OK) return rc;
  hipError_t e = hipMemcpyAsync(out, m->acc, (size_t)m->d * sizeof(float), hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "imatrix read copy");
  if (n_out) *n_out = m->N;
  return HESS_OK;
}

int hess_imatrix_reset(hess_imx_t m, hess_stream_t stream) {
  if (!m) return fail(HESS_EINVAL, "null handle");
  HLock lock(m->mu);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = imx_order_stream(m, s);
  if (rc != HESS_OK) return rc;
  hipError_t e = launch_zero(m->acc, m->d, s);
  if (e != hipSuccess) return hip_fail(e, "imatrix reset launch");
  m->N = 0;
  return HESS_OK;
}

}  // extern "C"
