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
#include <vector>

#include "../../include/hess.h"
#include "hess_internal.hpp"

using namespace hess;

struct hess_s {
  int64_t d = 0;
  int dtype = HESS_BF16;
  int device = 0;
  float* S = nullptr;        // d x d, row stride d
  uint8_t* dead = nullptr;   // d bytes
  float* damp = nullptr;     // 1 float
  float* ws = nullptr;       // split partials (may be null)
  int64_t ws_floats = 0;
  int64_t N = 0;
  bool consumed = false;     // in-place materialize done
  bool has_stream = false;
  hipStream_t last = nullptr;
  hipEvent_t ev = nullptr;
};

namespace {

thread_local char g_err[512] = "";
int g_tile_override = 0;  // 0 = automatic; 128 or 192 forces a SYRK tile edge

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

// 16-byte row loads need X and every row start 16-byte aligned and whole
// 16-byte chunks of features (d a multiple of 8 elements).
bool vec_ok(const void* p, int64_t ld, int64_t d, int es) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ((ld * es) & 15) == 0 && ((d * es) & 15) == 0;
}

constexpr double kSimdRate = 2.1e12;  // sustained bf16 MFMA flop/s per SIMD
constexpr double kHbm = 6.5e12;       // sustained read+write bytes/s
constexpr int kCUs = 256;
// K-iterations (64 tokens) per float32 accumulation chain: bf16 products are
// rounded once per 8 tokens, fp32 split products once per 2 tokens.
constexpr int kFlushItersBF16 = 64;
constexpr int kFlushItersF32 = 16;
int flush_iters(int dtype) { return dtype == HESS_F32 ? kFlushItersF32 : kFlushItersBF16; }

struct Shape {
  int wt;
  int B;
  int nb;
  int ntiles;
};

Shape make_shape(int64_t d, int wt) {
  Shape s;
  s.wt = wt;
  s.B = syrk_tile_edge(wt);
  s.nb = (int)((d + s.B - 1) / s.B);
  s.ntiles = s.nb * (s.nb + 1) / 2;
  return s;
}

// Estimated time of one update of width d over `tokens` tokens split into
// `items` workgroups per tile set; a simple model (matrix-core time per
// workgroup round, S read-modify-write traffic) used only to pick a shape.
double estimate(const Shape& s, int64_t items, double tokens_per_item, int dtype) {
  const double eff = s.wt == 3 ? 0.85 : 0.6;
  const double mult = dtype == HESS_F32 ? 4.0 : 1.0;
  const double wave_tile = 32.0 * s.wt;
  const double t_wg = mult * 2.0 * wave_tile * wave_tile * tokens_per_item / (kSimdRate * eff);
  const double rounds = std::ceil((double)items / kCUs);
  const double compute = rounds * t_wg;
  const double mem = (double)s.ntiles * s.B * s.B * 8.0 / kHbm;
  return std::max(compute, mem) + 0.25 * std::min(compute, mem);
}

struct Plan {
  Shape shape;
  int ks;
  int64_t kchunk;
};

Plan plan_single(hess_t h, int64_t n, bool vec) {
  std::vector<int> wts;
  (void)vec;
  wts = {2};
  Plan best{};
  double best_t = 1e30;
  for (int wt : wts) {
    Shape s = make_shape(h->d, wt);
    // token splits: only for few tiles and long batches, within the workspace
    int ks_max = 1;
    if (h->ws && wt == 2 && n >= 8192) {
      const int64_t tile_floats = (int64_t)s.B * s.B;
      ks_max = (int)std::min<int64_t>(8, h->ws_floats / ((int64_t)s.ntiles * tile_floats));
      ks_max = std::min<int64_t>(ks_max, std::max<int64_t>(1, n / 4096));
    }
    for (int ks = 1; ks <= std::max(1, ks_max); ++ks) {
      const int64_t kchunk = ((n + ks - 1) / ks + 63) / 64 * 64;
      const int ks_eff = (int)((n + kchunk - 1) / kchunk);
      double t = estimate(s, (int64_t)s.ntiles * ks_eff, (double)kchunk, h->dtype);
      if (ks_eff > 1) t += 2.0 * ks_eff * s.ntiles * s.B * s.B * 4.0 / kHbm;  // partial write + read
      if (t < best_t) {
        best_t = t;
        best = Plan{s, ks_eff, kchunk};
      }
    }
  }
  return best;
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
    default: return "unknown status";
  }
}

const char* hess_last_error(void) { return g_err; }

int hess_set_tile_override(int edge) {
  if (edge != 0 && edge != 128 && edge != 192) return fail(HESS_EINVAL, "tile override must be 0, 128 or 192");
  g_tile_override = edge;
  return HESS_OK;
}

hess_t hess_create(int64_t d, int in_dtype) {
  if (d < 1 || d > 65536) {
    fail(HESS_EINVAL, "d = %lld outside [1, 65536]", (long long)d);
    return nullptr;
  }
  if (in_dtype != HESS_BF16 && in_dtype != HESS_F32) {
    fail(HESS_EINVAL, "unknown input dtype %d", in_dtype);
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
  // split workspace: only widths whose 128-edge tile count is small enough
  // to need token splits (256 partial tiles of 128 x 128 floats at most)
  if (e == hipSuccess) {
    const Shape s = make_shape(d, 2);
    if (s.ntiles < 160) {
      h->ws_floats = (int64_t)256 * 128 * 128;
      e = hipMalloc(&h->ws, (size_t)h->ws_floats * sizeof(float));
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
    if (h->ev) (void)hipEventDestroy(h->ev);
    delete h;
    return nullptr;
  }
  return h;
}

int hess_destroy(hess_t h) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  hipError_t e = hipSuccess;
  if (h->has_stream) e = hipStreamSynchronize(h->last);
  (void)hipFree(h->S);
  (void)hipFree(h->dead);
  (void)hipFree(h->damp);
  if (h->ws) (void)hipFree(h->ws);
  (void)hipEventDestroy(h->ev);
  delete h;
  return e == hipSuccess ? HESS_OK : hip_fail(e, "hess_destroy");
}

int hess_add_batch(hess_t h, const void* X, int64_t n_tokens, int64_t ld, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  if (h->consumed) return fail(HESS_ESTATE, "handle was materialized in place; hess_reset it first");
  if (n_tokens < 0) return fail(HESS_EINVAL, "n_tokens = %lld < 0", (long long)n_tokens);
  if (ld < h->d) return fail(HESS_EINVAL, "ld = %lld < d = %lld", (long long)ld, (long long)h->d);
  if (n_tokens == 0) return HESS_OK;
  if (!X) return fail(HESS_EINVAL, "X is NULL with n_tokens > 0");
  if (reinterpret_cast<uintptr_t>(X) % esize(h->dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = vec_ok(X, ld, h->d, esize(h->dtype));
  const Plan pl = plan_single(h, n_tokens, vec);
  int rc = order_stream(h, s);
  if (rc != HESS_OK) return rc;

  SyrkParams P;
  std::memset(&P, 0, sizeof(P));
  P.X = X;
  P.rows = nullptr;
  P.ld = ld;
  P.lds = h->d;
  P.d = (int)h->d;
  P.nb = pl.shape.nb;
  P.ntiles = pl.shape.ntiles;
  P.ngroups = 1;
  P.ks = pl.ks;
  P.kchunk = (int)std::min<int64_t>(pl.kchunk, 1 << 30);
  P.flush_iters = flush_iters(h->dtype);
  P.total_items = pl.shape.ntiles * pl.ks;
  P.xcd_contig = 1;
  P.s_vec = (h->d % 4) == 0;
  P.item_prefix[0] = 0;
  P.item_prefix[1] = P.total_items;
  P.g[0] = SyrkGroup{h->S, h->ws, 0, n_tokens};
  hipError_t e = launch_syrk(P, pl.shape.wt, h->dtype, vec, s);
  if (e != hipSuccess) return hip_fail(e, "SYRK launch");
  if (pl.ks > 1) {
    e = launch_syrk_reduce(h->S, h->d, h->ws, (int)h->d, pl.shape.B, pl.shape.nb, pl.shape.ntiles, pl.ks, s);
    if (e != hipSuccess) return hip_fail(e, "split reduction launch");
  }
  h->N += n_tokens;
  return HESS_OK;
}

int hess_add_batch_grouped(hess_t* hs, int n_groups, const void* X, int64_t ld, const int32_t* row_idx,
                           const int64_t* offsets, hess_stream_t stream) {
  if (!hs || n_groups < 1) return fail(HESS_EINVAL, "need at least one handle");
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
  if (total == 0) return HESS_OK;
  if (!X) return fail(HESS_EINVAL, "X is NULL");
  if (reinterpret_cast<uintptr_t>(X) % esize(h0->dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int e = 0; e < n_groups; ++e) {
    int rc = order_stream(hs[e], s);
    if (rc != HESS_OK) return rc;
  }
  const bool vec = vec_ok(X, ld, h0->d, esize(h0->dtype));
  // one shape for every group: pick it for the mean group length
  int nonempty = 0;
  for (int e = 0; e < n_groups; ++e) nonempty += offsets[e + 1] > offsets[e];
  const double mean_rows = (double)total / std::max(1, nonempty);
  int wt = 2;
  if (false) {
    const Shape s2 = make_shape(h0->d, 2), s3 = make_shape(h0->d, 3);
    const double t2 = estimate(s2, (int64_t)s2.ntiles * nonempty, mean_rows, h0->dtype);
    const double t3 = estimate(s3, (int64_t)s3.ntiles * nonempty, mean_rows, h0->dtype);
    wt = (g_tile_override == 192 || t3 < t2) ? 3 : 2;
  }
  const Shape sh = make_shape(h0->d, wt);
  // longest groups first, so the longest workgroups start in the first round
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
    P.nb = sh.nb;
    P.ntiles = sh.ntiles;
    P.ngroups = cnt;
    P.ks = 1;
    P.kchunk = 1 << 30;
    P.flush_iters = flush_iters(h0->dtype);
    P.xcd_contig = 0;
    P.s_vec = (h0->d % 4) == 0;
    P.item_prefix[0] = 0;
    for (int k = 0; k < cnt; ++k) {
      const int e = order[base + k];
      P.g[k] = SyrkGroup{hs[e]->S, nullptr, offsets[e], offsets[e + 1]};
      P.item_prefix[k + 1] = P.item_prefix[k] + sh.ntiles;
    }
    P.total_items = P.item_prefix[cnt];
    hipError_t err = launch_syrk(P, wt, h0->dtype, vec, s);
    if (err != hipSuccess) return hip_fail(err, "grouped SYRK launch");
  }
  for (int e = 0; e < n_groups; ++e) hs[e]->N += offsets[e + 1] - offsets[e];
  return HESS_OK;
}

int hess_materialize_ex(hess_t h, float damp_percent, unsigned flags, float* H_out, uint8_t* dead_out,
                        float* damp_out, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  if (h->consumed) return fail(HESS_ESTATE, "handle was materialized in place; hess_reset it first");
  if (!(damp_percent >= 0.0f && damp_percent < 1.0f))
    return fail(HESS_EINVAL, "damp_percent must be in [0, 1)");
  if (flags & ~HESS_NO_NEUTRALIZE) return fail(HESS_EINVAL, "unknown flags 0x%x", flags);
  if (H_out == h->S) return fail(HESS_EINVAL, "H_out aliases the Gram buffer; pass NULL for in place");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
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
  if (!H_out) return fail(HESS_EINVAL, "H_out is NULL (use hess_materialize_ex for in place)");
  return hess_materialize_ex(h, damp_percent, 0u, H_out, nullptr, nullptr, h->has_stream ? h->last : nullptr);
}

int hess_reset(hess_t h, hess_stream_t stream) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_stream(h, s);
  if (rc != HESS_OK) return rc;
  hipError_t e = launch_zero(h->S, h->d * h->d, s);
  if (e != hipSuccess) return hip_fail(e, "reset launch");
  h->N = 0;
  h->consumed = false;
  return HESS_OK;
}

int hess_token_count(hess_t h, int64_t* n_out) {
  if (!h || !n_out) return fail(HESS_EINVAL, "null argument");
  *n_out = h->N;
  return HESS_OK;
}

int hess_info(hess_t h, int64_t* d_out, int* in_dtype_out) {
  if (!h) return fail(HESS_EINVAL, "null handle");
  if (d_out) *d_out = h->d;
  if (in_dtype_out) *in_dtype_out = h->dtype;
  return HESS_OK;
}

int hess_state_buffer(hess_t h, const float** S_out) {
  if (!h || !S_out) return fail(HESS_EINVAL, "null argument");
  *S_out = h->S;
  return HESS_OK;
}

int hess_local_blocks_ex(const void* X, int in_dtype, int64_t n_tokens, int64_t d, int64_t ld, int block,
                         float* out, int accumulate, hess_stream_t stream) {
  if (in_dtype != HESS_BF16 && in_dtype != HESS_F32) return fail(HESS_EINVAL, "unknown input dtype %d", in_dtype);
  if (block != 16) return fail(HESS_EINVAL, "block must be 16");
  if (d < 16 || d % 16 != 0 || d > (1 << 30)) return fail(HESS_EINVAL, "d must be a positive multiple of 16");
  if (ld < d) return fail(HESS_EINVAL, "ld < d");
  if (n_tokens < 0) return fail(HESS_EINVAL, "n_tokens < 0");
  if (!out) return fail(HESS_EINVAL, "out is NULL");
  if (n_tokens > 0 && !X) return fail(HESS_EINVAL, "X is NULL with n_tokens > 0");
  if (reinterpret_cast<uintptr_t>(X) % esize(in_dtype) != 0) return fail(HESS_EALIGN, "X not element-aligned");
  const bool vec = n_tokens > 0 && vec_ok(X, ld, d, esize(in_dtype));
  hipError_t e = launch_local_blocks(X, in_dtype, n_tokens, (int)d, ld, vec, out, accumulate,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "local blocks launch");
  return HESS_OK;
}

int hess_local_blocks(const void* X, int64_t n_tokens, int64_t d, int block, float* out) {
  return hess_local_blocks_ex(X, HESS_BF16, n_tokens, d, d, block, out, 1, nullptr);
}

}  // extern "C"
