// Per-block 16 x 16 "local" Hessians on gfx950.
//
//   out[b] (+)= X[:, 16b:16b+16]^T X[:, 16b:16b+16]     for b < d/16
//
// The local_hessian statistic of the NVIDIA Model-Optimizer PR 3002 page
// ("What does this PR do?", local_hessian bullet): 16 x 16 per-block Gram
// matrices built by a batched product that reads bfloat16 and writes
// float32.  Unscaled; the blocks only weight candidate-scale errors.
//
// The work is a single streaming read of X (HBM-bound): each workgroup takes
// 256 features (16 blocks, 4 per wave) of a run of tokens.  32-token slabs are
// copied into LDS in their natural [token][feature] layout with 16-byte loads
// (one load stage ahead in registers), and each wave reads its block operands
// with ds_read_b64_tr_b16, which returns a feature's 4 consecutive tokens per
// lane: two such reads give the 8 tokens a v_mfma_f32_16x16x32_bf16 lane
// needs.  The same register is both the A and the B operand, because a
// block's Gram pairs each feature with itself over the same tokens.  Each
// workgroup adds its 16 blocks into `out` with float32 atomics at the end.
//
// float32 inputs are split into hi + lo bf16 planes.  The hi*hi, the cross
// (hi*lo + lo*hi) and the lo*lo products go to three separate accumulators,
// combined smallest first at the end, so the small terms are never rounded
// against the large accumulator.

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kLThreads = 256;
constexpr int kLFeat = 256;                      // features per workgroup
constexpr int kLTok = 32;                        // tokens per slab
constexpr int kLRow = kLFeat * 2 + 32;           // LDS bytes per token row (padded)
constexpr int kLPlane = kLTok * kLRow;           // one bf16 plane of a slab

template <int IN>
struct LocalRegs;
template <>
struct LocalRegs<kInBF16> {
  u32x4 v[4];  // 4 chunks of 8 bf16
};
template <>
struct LocalRegs<kInF32> {
  u32x4 v[8];  // 8 chunks of 4 floats
};

__device__ __forceinline__ s16x4 tr_read(const char* lds_base, int byte_off) {
  const HESS_LDS char* p = (const HESS_LDS char*)lds_base + byte_off;  // generic -> LDS address space
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((HESS_LDS s16x4*)p);
}

template <int IN, bool VEC>
__device__ __forceinline__ void local_body(const void* Xv, int64_t n, int d, int64_t ld, int64_t tok_per_wg,
                                           float* out, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int F0 = blockIdx.x * kLFeat;
  const int64_t t_begin = (int64_t)blockIdx.y * tok_per_wg;
  const int64_t t_end = min(n, t_begin + tok_per_wg);
  if (t_begin >= t_end) return;
  const int nslab = (int)((t_end - t_begin + kLTok - 1) / kLTok);
  constexpr int ES = IN == kInF32 ? 4 : 2;
  constexpr int CH = 16 / ES;                        // features per 16-byte chunk
  constexpr int CHUNKS = kLTok * kLFeat / CH;        // chunks per slab
  constexpr int CPT = CHUNKS / kLThreads;            // chunks per thread
  constexpr int PLANES = IN == kInF32 ? 2 : 1;
  constexpr int STAGE = PLANES * kLPlane;
  const char* X = static_cast<const char*>(Xv);

  LocalRegs<IN> R;
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
          v = *reinterpret_cast<const u32x4*>(p);
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
      R.v[q] = v;
    }
  };
  auto store = [&](char* stage) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kLThreads;
      const int row = c / (kLFeat / CH), colc = c % (kLFeat / CH);
      if constexpr (IN == kInBF16) {
        *reinterpret_cast<u32x4*>(stage + row * kLRow + colc * 16) = R.v[q];
      } else {
        uint32_t h[4], l[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) split_bf16(__uint_as_float(R.v[q][k]), h[k], l[k]);
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2*>(stage + row * kLRow + colc * 8) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *reinterpret_cast<u32x2*>(stage + kLPlane + row * kLRow + colc * 8) =
            u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      }
    }
  };

  f32x4 acc[4], accx[4], accl[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    accx[b] = acc[b];
    accl[b] = acc[b];
  }

  // operand addressing: lane l, group g = l/16, i = l%16; rows 8g + 4*half + r
  // supplied by lanes 4r + q at feature column 4q of the block
  const int g = lane >> 4, i16 = lane & 15;
  const int rsel = i16 >> 2, qsel = i16 & 3;

  auto compute = [&](const char* stage) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int blk = wave * 4 + bb;  // block within the workgroup
      if (F0 + blk * 16 >= d) continue;
      const int colb = blk * 32 + qsel * 8;  // bytes
      const int off0 = (8 * g + rsel) * kLRow + colb;
      const int off1 = (8 * g + 4 + rsel) * kLRow + colb;
      s16x4 lo0 = tr_read(stage, off0), lo1 = tr_read(stage, off1);
      u32x4 a = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo0, lo1, 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (IN == kInBF16) {
        acc[bb] = mfma16x16x32(a, a, acc[bb]);
      } else {
        s16x4 l0 = tr_read(stage + kLPlane, off0), l1 = tr_read(stage + kLPlane, off1);
        u32x4 al = __builtin_bit_cast(u32x4, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
        accl[bb] = mfma16x16x32(al, al, accl[bb]);
        accx[bb] = mfma16x16x32(al, a, accx[bb]);
        accx[bb] = mfma16x16x32(a, al, accx[bb]);
        acc[bb] = mfma16x16x32(a, a, acc[bb]);
      }
    }
  };

  load(0);
  store(lds);
  __syncthreads();
  for (int s = 0; s < nslab; ++s) {
    char* cur = lds + (s & 1) * STAGE;
    char* nxt = lds + ((s + 1) & 1) * STAGE;
    const bool more = s + 1 < nslab;
    if (more) load(s + 1);
    compute(cur);
    if (more) store(nxt);
    __syncthreads();
  }

  if constexpr (IN == kInF32) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) acc[bb] = (accl[bb] + accx[bb]) + acc[bb];
  }
  // register r of lane l holds C[4*(l/16) + r][l%16] of each block
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int blk = wave * 4 + bb;
    const int gb = F0 / 16 + blk;
    if (gb * 16 >= d) continue;
    float* o = out + (int64_t)gb * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) unsafeAtomicAdd(o + (4 * g + r) * 16 + i16, acc[bb][r]);
  }
}

template <int IN, bool VEC>
__global__ void __launch_bounds__(kLThreads) local_kernel(const void* X, int64_t n, int d, int64_t ld,
                                                          int64_t tok_per_wg, float* out) {
  extern __shared__ __attribute__((aligned(16))) char hess_llds[];
  local_body<IN, VEC>(X, n, d, ld, tok_per_wg, out, hess_llds);
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

hipError_t launch_local_blocks(const void* X, int in_dtype, int64_t n, int d, int64_t ld, bool vec, float* out,
                               int accumulate, hipStream_t stream) {
  const int nblocks = d / 16;
  if (!accumulate) {
    hipError_t e = launch_zero(out, (int64_t)nblocks * 256, stream);
    if (e != hipSuccess) return e;
  }
  if (n <= 0) return hipSuccess;
  const int gx = (d + kLFeat - 1) / kLFeat;
  // about 1024 workgroups over the whole GPU, at least one slab each
  int64_t gy = (1024 + gx - 1) / gx;
  int64_t tpw = (n + gy - 1) / gy;
  tpw = ((tpw + kLTok - 1) / kLTok) * kLTok;
  if (tpw < 4 * kLTok) tpw = 4 * kLTok;
  gy = (n + tpw - 1) / tpw;
  const int planes = in_dtype == kInF32 ? 2 : 1;
  const int lds = 2 * planes * kLPlane;
  const void* fn;
  if (in_dtype == kInBF16)
    fn = vec ? reinterpret_cast<const void*>(&local_kernel<kInBF16, true>)
             : reinterpret_cast<const void*>(&local_kernel<kInBF16, false>);
  else
    fn = vec ? reinterpret_cast<const void*>(&local_kernel<kInF32, true>)
             : reinterpret_cast<const void*>(&local_kernel<kInF32, false>);
  void* args[] = {const_cast<void**>(&X), &n, &d, &ld, &tpw, &out};
  return hipLaunchKernel(fn, dim3(gx, (unsigned)gy), dim3(kLThreads), args, lds, stream);
}

}  // namespace hess
