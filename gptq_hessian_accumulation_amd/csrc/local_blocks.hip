// Per-block 16 x 16 "local" Hessians on gfx950.
//
//   out[b] (+)= X[:, 16b:16b+16]^T X[:, 16b:16b+16]     for b < d/16
//
// The local_hessian statistic of the NVIDIA Model-Optimizer PR 3002 page
// ("What does this PR do?", local_hessian bullet): 16 x 16 per-block Gram
// matrices built by a batched product that reads bfloat16 and writes
// float32.  Unscaled; the blocks only weight candidate-scale errors.
//
// The work is a single streaming read of X (HBM-bound), in two kernels:
//  1. local_part: workgroup (x, y) takes the 256 features of column x (16
//     blocks, 4 per wave) over the y-th run of tokens and writes its 16
//     block sums to its own slice of a scratch buffer (no atomics).
//     32-token slabs are copied into LDS in their natural [token][feature]
//     layout with 16-byte nontemporal loads (one slab ahead in registers;
//     each byte is read once, and on MI355X the hint took a 32,768 x 4,096
//     bf16 update from 54.2 to 51.2 us).
//     - bf16: each wave reads its block operands with ds_read_b64_tr_b16,
//       which returns a feature's 4 consecutive tokens per lane; two such
//       reads give the 8 tokens a v_mfma_f32_16x16x32_bf16 lane needs.
//     - float32: v_mfma_f32_16x16x4_f32 with exact products, one float per
//       lane (token t0 + l/16, feature l%16 of the block).
//     In both the same register is the A and the B operand, because a
//     block's Gram pairs each feature with itself over the same tokens.
//     Each wave's sums pass through three accumulators (every 64 slabs of
//     bf16 or 16 of float32 into the second, every 32 of those into the
//     third), so no float32 chain grows long with the batch.
//  2. local_reduce: out[b] (+)= the slices' sums for block b, added in a
//     fixed grouped order (runs of 16, summed by four waves in parallel and
//     added in run order).  Every run gives the same bits.
//
// The scratch (slices x blocks x 1 KB) is at most kLocalPartBytes: the plan
// takes about 512 workgroups, fewer token runs when the blocks of a slice
// would not fit.

#include <mutex>

#include "hess_device.hpp"
#include "hess_internal.hpp"

// Partial sums of hess_local_blocks_noalloc: a fixed array in device memory,
// one copy per GPU the library runs on, held until the process ends.  Host
// code never passes this name to a kernel: it is a host-side stand-in, and
// the device address comes from hipGetSymbolAddress (local_static_scratch).
static __device__ __align__(256) float scratch[hess::kLocalPartBytes / sizeof(float)];

namespace hess {

namespace {

constexpr int kLThreads = 256;
constexpr int kLFeat = 256;                      // features per workgroup
constexpr int kLTok = 32;                        // tokens per slab
constexpr int kLChain2 = 32;                     // first-level sums per second-level chain

template <int IN>
struct LocalCfg;
template <>
struct LocalCfg<kInBF16> {
  static constexpr int ES = 2;                   // bytes per element
  static constexpr int ROW = kLFeat * 2 + 32;    // LDS bytes per token row (padded)
  static constexpr int CHAIN = 64;               // slabs per first-level chain (256 roundings)
};
template <>
struct LocalCfg<kInF32> {
  static constexpr int ES = 4;
  static constexpr int ROW = kLFeat * 4 + 64;    // rows 16 banks apart: a 64-lane read is conflict-free
  static constexpr int CHAIN = 16;               // slabs per first-level chain (128 roundings)
};

__device__ __forceinline__ s16x4 tr_read(const char* lds_base, int byte_off) {
  const HESS_LDS char* p = (const HESS_LDS char*)lds_base + byte_off;  // generic -> LDS address space
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((HESS_LDS s16x4*)p);
}

template <int IN, bool VEC>
__device__ __forceinline__ void local_body(const void* Xv, int64_t n, int d, int64_t ld, int64_t tok_per_wg,
                                           float* part, char* lds) {
  using C = LocalCfg<IN>;
  constexpr int ES = C::ES;
  constexpr int ROW = C::ROW;
  constexpr int CH = 16 / ES;                        // features per 16-byte chunk
  constexpr int CHUNKS = kLTok * kLFeat / CH;        // chunks per slab
  constexpr int CPT = CHUNKS / kLThreads;            // chunks per thread
  constexpr int STAGE = kLTok * ROW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int F0 = blockIdx.x * kLFeat;
  const int nblk = d / 16;
  const int64_t t_begin = (int64_t)blockIdx.y * tok_per_wg;
  const int64_t t_end = min(n, t_begin + tok_per_wg);
  const int nslab = t_begin < t_end ? (int)((t_end - t_begin + kLTok - 1) / kLTok) : 0;
  const char* X = static_cast<const char*>(Xv);

  u32x4 R[CPT];
  auto load = [&](int s) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kLThreads;
      const int row = c / (kLFeat / CH), colc = c % (kLFeat / CH);
      const int64_t t = t_begin + (int64_t)s * kLTok + row;
      const int f = F0 + colc * CH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < t_end && f < d) {
        const char* p = X + (t * ld + f) * ES;
        if (VEC && f + CH <= d) {
          v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          if constexpr (IN == kInBF16) {
            const uint16_t* e = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (f + k < d) w[k >> 1] |= (uint32_t)e[k] << (16 * (k & 1));
          } else {
            const uint32_t* e = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (f + k < d) w[k] = e[k];
          }
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      R[q] = v;
    }
  };
  auto store = [&](char* stage) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kLThreads;
      const int row = c / (kLFeat / CH), colc = c % (kLFeat / CH);
      *reinterpret_cast<u32x4*>(stage + row * ROW + colc * 16) = R[q];
    }
  };

  // three levels: slab sums chain in acc for C::CHAIN slabs, those sums in
  // acc2 for kLChain2 of them, and those in acc3, so that no float32 chain
  // grows long with the run of tokens (with identical values in a column,
  // every rounding of a long chain errs the same way)
  f32x4 acc[4], acc2[4], acc3[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc2[b] = acc[b];
    acc3[b] = acc[b];
  }

  // lane l: group g = l/16, i16 = l%16.  bf16: rows 8g + 4*half + r supplied
  // by lanes 4r + q at feature column 4q of the block; float32: token 4j + g,
  // feature i16 of the block
  const int g = lane >> 4, i16 = lane & 15;
  const int rsel = i16 >> 2, qsel = i16 & 3;

  auto compute = [&](const char* stage) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int blk = wave * 4 + bb;  // block within the workgroup
      if (F0 + blk * 16 >= d) continue;
      if constexpr (IN == kInBF16) {
        const int colb = blk * 32 + qsel * 8;  // bytes
        const s16x4 lo0 = tr_read(stage, (8 * g + rsel) * ROW + colb);
        const s16x4 lo1 = tr_read(stage, (8 * g + 4 + rsel) * ROW + colb);
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo0, lo1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[bb] = mfma16x16x32(a, a, acc[bb]);
      } else {
        // token 4 j + g of the slab: 4 j rows (j * ROW floats) past row g
        const float* col = reinterpret_cast<const float*>(stage + g * ROW) + blk * 16 + i16;
#pragma unroll
        for (int j = 0; j < kLTok / 4; ++j) {
          const float v = col[j * ROW];
          acc[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, v, acc[bb], 0, 0, 0);
        }
      }
    }
  };

  if (nslab > 0) {
    load(0);
    store(lds);
    __syncthreads();
  }
  for (int s = 0; s < nslab; ++s) {
    char* cur = lds + (s & 1) * STAGE;
    char* nxt = lds + ((s + 1) & 1) * STAGE;
    const bool more = s + 1 < nslab;
    if (more) load(s + 1);
    compute(cur);
    if ((s + 1) % C::CHAIN == 0 || !more) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        acc2[bb] += acc[bb];
        acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if ((s + 1) % (C::CHAIN * kLChain2) == 0 || !more) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          acc3[bb] += acc2[bb];
          acc2[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    if (more) store(nxt);
    __syncthreads();
  }

  // register r of lane l holds C[4*(l/16) + r][l%16] of each block
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int gb = F0 / 16 + wave * 4 + bb;
    if (gb >= nblk) continue;
    float* o = part + ((int64_t)blockIdx.y * nblk + gb) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[(4 * g + r) * 16 + i16] = acc3[bb][r];
  }
}

template <int IN, bool VEC>
__global__ void __launch_bounds__(kLThreads) local_part(const void* X, int64_t n, int d, int64_t ld,
                                                        int64_t tok_per_wg, float* part) {
  extern __shared__ __attribute__((aligned(16))) char hess_llds[];
  local_body<IN, VEC>(X, n, d, ld, tok_per_wg, part, hess_llds);
}

// out[b][e] (+)= sum over slices y = 0 .. nslice-1 of part[y][b][e], in a
// fixed order: runs of 16 slices summed in order, the runs of each group of
// 256 slices summed in order, then the groups, so no chain is longer than
// 16 + 16 + nslice / 256 additions.  Workgroup (b, q) takes elements
// 64 q .. 64 q + 63 of block b; its four waves sum runs r = wave, wave + 4, ...
// (each run's 16 loads in flight at once) into LDS, and the first wave adds
// them in run order.
constexpr int kRedRuns = 64;   // runs held in LDS: slices up to 1,024 per pass over them
__global__ void __launch_bounds__(256) local_reduce(const float* part, int nblk, int nslice, float* out,
                                                    int accumulate) {
  __shared__ float run[kRedRuns][64];
  const int b = blockIdx.x >> 2, e = (blockIdx.x & 3) * 64 + (threadIdx.x & 63), g = threadIdx.x >> 6;
  const float* p = part + (int64_t)b * 256 + e;
  const int64_t stride = (int64_t)nblk * 256;  // floats between slices
  float s = 0.0f;
  for (int y0 = 0; y0 < nslice; y0 += 16 * kRedRuns) {   // runs y0 / 16 .. y0 / 16 + kRedRuns - 1
    const int lim = min(nslice, y0 + 16 * kRedRuns);
    const int nrun = (lim - y0 + 15) / 16;
    for (int r = g; r < nrun; r += 4) {
      const int y1 = y0 + 16 * r;
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = y1 + k < lim ? p[(int64_t)(y1 + k) * stride] : 0.0f;
      float s1 = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (y1 + k < lim) s1 += v[k];
      run[r][threadIdx.x & 63] = s1;
    }
    __syncthreads();
    if (g == 0) {
      // groups of 16 runs (256 slices): s2 over a group's runs in order, then s += s2
      for (int r0 = 0; r0 < nrun; r0 += 16) {
        float s2 = 0.0f;
        for (int r = r0; r < min(nrun, r0 + 16); ++r) s2 += run[r][threadIdx.x];
        s += s2;
      }
    }
    __syncthreads();
  }
  if (g == 0) {
    float* o = out + (int64_t)b * 256 + e;
    *o = accumulate ? *o + s : s;
  }
}

__global__ void zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

}  // namespace

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t local_static_scratch(float** out) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static float* addr[kDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

LocalPlan local_plan(int64_t n, int d, int64_t part_bytes) {
  LocalPlan p{};
  const int64_t nblk = d / 16;
  p.gx = (d + kLFeat - 1) / kLFeat;
  // about 512 workgroups over the whole GPU, at least four slabs each, and
  // no more token runs than slices fit in the scratch.  Measured per
  // 32,768 x 4,096 update (partials + fixed-order reduction): 54.2 us at 512
  // workgroups, 58.2 at 1,024, 60 at 384, 73 at 256
  int64_t gy = (512 + p.gx - 1) / p.gx;
  const int64_t fit = part_bytes / (nblk * 1024);
  if (gy > fit) gy = fit;
  if (gy < 1) gy = 1;
  int64_t tpw = (n + gy - 1) / gy;
  tpw = ((tpw + kLTok - 1) / kLTok) * kLTok;
  if (tpw < 4 * kLTok) tpw = 4 * kLTok;
  p.tpw = tpw;
  p.gy = n > 0 ? (n + tpw - 1) / tpw : 0;
  p.part_bytes = p.gy * nblk * 1024;
  return p;
}

hipError_t launch_local_blocks(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* out,
                               int accumulate, const LocalPlan& pl, float* part, hipStream_t stream) {
  const int nblk = d / 16;
  if (n <= 0) {
    if (!accumulate) return launch_zero(out, (int64_t)nblk * 256, stream);
    return hipSuccess;
  }
  if (pl.gy < 1 || pl.gy >= 65536) return hipErrorInvalidValue;
  const int lds = 2 * kLTok * (in_dtype == kInF32 ? LocalCfg<kInF32>::ROW : LocalCfg<kInBF16>::ROW);
  const void* fn;
  if (in_dtype == kInBF16)
    fn = vec ? reinterpret_cast<const void*>(&local_part<kInBF16, true>)
             : reinterpret_cast<const void*>(&local_part<kInBF16, false>);
  else
    fn = vec ? reinterpret_cast<const void*>(&local_part<kInF32, true>)
             : reinterpret_cast<const void*>(&local_part<kInF32, false>);
  int64_t tpw = pl.tpw;
  void* args[] = {const_cast<void**>(&X), &n, &d, &ld, &tpw, &part};
  hipError_t e = hipLaunchKernel(fn, dim3(pl.gx, (unsigned)pl.gy), dim3(kLThreads), args, lds, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(local_reduce, dim3(4 * nblk), dim3(256), 0, stream, static_cast<const float*>(part), nblk,
                     (int)pl.gy, out, accumulate);
  return hipGetLastError();
}

}  // namespace hess
