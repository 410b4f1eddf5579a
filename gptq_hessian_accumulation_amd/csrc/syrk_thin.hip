// Symmetric rank-k update for thin batches (bf16 or float32 rows), shaped for
// memory bandwidth:
//
//   S[i][j] += sum_t X[t][i] * X[t][j]      for the upper-triangle tiles (j >= i)
//
// The same per-batch update as the other SYRK kernels (GPTQModel PR 2979,
// What Changed; PR 2981, Changes: in place into the persistent float32 sum),
// for batches of a few hundred tokens or fewer that are added straight into S
// (no staging buffer, or the caller's own flushes).  Such a batch does little
// arithmetic per element of S, so the read-modify-write of S's upper triangle
// (4 d (d + 1) bytes) sets the time:
//
//  * 64 x 64 tiles, one workgroup of 4 waves each (a 32 x 32 quadrant per
//    wave, 2 x 2 accumulators of v_mfma_f32_16x16x32_bf16, or of
//    v_mfma_f32_16x16x4_f32 for float32 rows): many small
//    workgroups resident per CU keep the most S traffic in flight, and the
//    tile count (2,080 at width 4,096) spreads evenly over the 256 CUs.
//  * The tile's S entries are requested right after the first step's
//    activation loads, before any arithmetic, so the S reads of all
//    resident workgroups overlap the products.  S is read and written in
//    whole 256-byte tile rows (16 lanes per row, 16 bytes each); the sums
//    go from the matrix-core layout to that one through LDS.  Measured at
//    width 4,096, this row layout moved S 1.2x faster than accessing it in
//    the accumulators' own layout (16 rows of 64 bytes per instruction).
//  * The activations of one 32-token step (two 32 x 64 panels, one on a
//    diagonal tile) go from memory into registers (one 16-byte load per
//    thread and panel for bf16, two for float32; the next step's issued
//    before this step's products) and through LDS, token-major with a padded
//    row.  bf16 operands (8 tokens of one feature) are read transposed with
//    ds_read_b64_tr_b16; a float32 operand is one word per lane.
//  * Buffer descriptors end at the batch's last row and features past d get
//    an out-of-range offset, so loads need no masks; S entries past d are
//    neither read nor written.

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kTE = 64;                 // tile edge
constexpr int kTS = 32;                 // tokens per step
constexpr int kRowPad = 144;            // LDS bytes per token row of a bf16 panel (128 used)
constexpr int kPanel = kTS * kRowPad;   // one bf16 panel of a step
constexpr int kRowPadF = 272;           // ... of a float32 panel (256 used)
constexpr int kPanelF = kTS * kRowPadF;
constexpr uint32_t kFar = 0x80000000u;  // an offset past any descriptor's range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t thin_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int nrec = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, nrec,
                                           0x00020000);
}

// Operand of a 16-feature block at LDS byte offset p (lane part included):
// two transposed 8-byte reads, tokens 8 g .. 8 g + 3 and 8 g + 4 .. 8 g + 7.
__device__ __forceinline__ u32x4 thin_operand(const char* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HESS_LDS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HESS_LDS s16x4*)(p + 4 * kRowPad));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return u32x4{a.x, a.y, b.x, b.y};
}

// LDS of one workgroup: the two panels of a step during the products, then
// the tile's 64 x 64 sums (row stride kAccLd floats) for the output.
constexpr int kAccLd = kTE + 4;
constexpr int kThinLds = kTE * kAccLd * 4 > 2 * kPanelF ? kTE * kAccLd * 4 : 2 * kPanelF;

// F32: float32 rows (4 features per 16-byte load, two loads per thread and
// panel; the panels hold the raw words, token-major, and each 4-token slice
// of a step is one v_mfma_f32_16x16x4_f32 per accumulator, exact products).
template <bool F32>
__global__ void __launch_bounds__(256) syrk_thin(const char* __restrict__ X, int64_t ld_bytes, int n, int d,
                                                 float* __restrict__ S, int64_t lds) {
  constexpr int kRow = F32 ? kRowPadF : kRowPad;
  constexpr int kPan = F32 ? kPanelF : kPanel;
  __shared__ __attribute__((aligned(16))) char lbuf[kThinLds];
  // workgroup b -> tile (I, J), I <= J: b = J (J + 1) / 2 + I
  const int b = blockIdx.x;
  int J = (int)((sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
  while (J * (J + 1) / 2 > b) --J;
  while ((J + 1) * (J + 2) / 2 <= b) ++J;
  const int I = b - J * (J + 1) / 2;
  const bool diag = I == J;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wr = w >> 1, wc = w & 1;

  // activation loads of a step, for panel I and (off the diagonal) panel J:
  // bf16, thread t moves features 8 (t % 8) .. +7 of token t / 8; float32,
  // features 4 (t % 16) .. +3 of tokens t / 16 and t / 16 + 16
  constexpr int kFeat = F32 ? 4 : 8, kEs = F32 ? 4 : 2, kLoads = F32 ? 2 : 1;
  const int tk = F32 ? t >> 4 : t >> 3, ch = F32 ? t & 15 : t & 7;
  const int fI = I * kTE + kFeat * ch, fJ = J * kTE + kFeat * ch;
  uint32_t vI[kLoads], vJ[kLoads];
#pragma unroll
  for (int h = 0; h < kLoads; ++h) {
    vI[h] = fI < d ? (uint32_t)((tk + 16 * h) * ld_bytes + fI * kEs) : kFar;
    vJ[h] = fJ < d ? (uint32_t)((tk + 16 * h) * ld_bytes + fJ * kEs) : kFar;
  }
  u32x4 xa[kLoads], xc[kLoads];
  auto load = [&](int k0) {
    const __amdgpu_buffer_rsrc_t r = thin_rsrc(X + (int64_t)k0 * ld_bytes, (int64_t)min(kTS, n - k0) * ld_bytes);
#pragma unroll
    for (int h = 0; h < kLoads; ++h) {
      xa[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vI[h], 0, 0));
      if (!diag) xc[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vJ[h], 0, 0));
    }
  };
#pragma unroll
  for (int h = 0; h < kLoads; ++h) xc[h] = u32x4{0u, 0u, 0u, 0u};
  load(0);

  // S entries of thread t: tile rows t / 16 + 16 k (k < 4), columns
  // 4 (t % 16) .. +3, so that 16 lanes cover one 256-byte tile row
  const __amdgpu_buffer_rsrc_t sr = thin_rsrc(S + (int64_t)I * kTE * lds, (int64_t)kTE * lds * 4);
  const int rlim = d - I * kTE, clim = d - J * kTE;
  const int sc = 4 * (t & 15);
  uint32_t so[4];
  float4 sv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = (t >> 4) + 16 * k;
    so[k] = (r < rlim && sc < clim) ? (uint32_t)(((int64_t)r * lds + J * kTE + sc) * 4) : kFar;
    sv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(sr, so[k], 0, 0));
  }

  // operand addresses.  bf16 (see thin_operand): 16-lane group g reads
  // tokens 8 g + (lane % 16) / 4, features f0 + 4 (lane % 4).  float32: lane
  // l reads token 4 s + l / 16 of slice s, feature f0 + l % 16.
  const int tl = F32 ? (lane >> 4) : 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int fl = F32 ? (lane & 15) : 4 * (lane & 3);
  const char* pa = lbuf + tl * kRow + (32 * wr + fl) * kEs;
  const char* pb = lbuf + (diag ? 0 : kPan) + tl * kRow + (32 * wc + fl) * kEs;
  char* const wI = lbuf + tk * kRow + ch * 16;
  char* const wJ = wI + kPan;

  // wave (wr, wc) sums the quadrant rows 32 wr .., columns 32 wc ..; on a
  // diagonal tile the below-diagonal quadrant is summed too (the same
  // values mirrored), so that every row of the tile is whole
  f32x4 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x4{};
  for (int k0 = 0; k0 < n; k0 += kTS) {
#pragma unroll
    for (int h = 0; h < kLoads; ++h) {
      *reinterpret_cast<u32x4*>(wI + 16 * h * kRow) = xa[h];
      if (!diag) *reinterpret_cast<u32x4*>(wJ + 16 * h * kRow) = xc[h];
    }
    __syncthreads();
    if (k0 + kTS < n) load(k0 + kTS);
    if constexpr (F32) {
      // the step's 8 slices sum into a fresh accumulator that is then added
      // to the running one, so no float32 chain exceeds 8 + n / 32 additions
      f32x4 st[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) st[rb][cb] = f32x4{};
#pragma unroll
      for (int sl = 0; sl < kTS / 4; ++sl) {
        float a[2], c[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          a[p] = *reinterpret_cast<const float*>(pa + 4 * sl * kRow + 16 * p * 4);
          c[p] = *reinterpret_cast<const float*>(pb + 4 * sl * kRow + 16 * p * 4);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            st[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(c[cb], a[rb], st[rb][cb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] += st[rb][cb];
    } else {
      u32x4 a[2], c[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        a[p] = thin_operand(pa + 32 * p);
        c[p] = thin_operand(pb + 32 * p);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma16x16x32(c[cb], a[rb], acc[rb][cb]);
    }
    __syncthreads();
  }
  // the sums through LDS into the row layout of the S accesses: lane l of
  // accumulator (rb, cb) holds row 32 wr + 16 rb + l % 16, columns
  // 32 wc + 16 cb + 4 (l / 16) .. +3
  float* At = reinterpret_cast<float*>(lbuf);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = 32 * wr + 16 * rb + (lane & 15), c = 32 * wc + 16 * cb + 4 * (lane >> 4);
      const f32x4 v = acc[rb][cb];
      *reinterpret_cast<float4*>(At + r * kAccLd + c) = float4{v[0], v[1], v[2], v[3]};
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 a = *reinterpret_cast<const float4*>(At + ((t >> 4) + 16 * k) * kAccLd + sc);
    const float4 x = sv[k];
    const float4 v{x.x + a.x, x.y + a.y, x.z + a.z, x.w + a.w};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sr, so[k], 0, 0);
  }
}

}  // namespace

int64_t syrk_thin_tiles(int d) {
  const int64_t nb = (d + kTE - 1) / kTE;
  return nb * (nb + 1) / 2;
}

hipError_t launch_syrk_thin(const void* X, int in_dtype, int64_t ld, int64_t n, int d, float* S, int64_t lds,
                            hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t tiles = syrk_thin_tiles(d);
  const int es = in_dtype == kInF32 ? 4 : 2;
  if (n > kSyrkThinMaxN || d % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15u) != 0 || ((ld * es) & 15) != 0 ||
      ld * es * kTS >= ((int64_t)1 << 31) || lds % 4 != 0 || lds * 4 * kTE >= ((int64_t)1 << 31) ||
      tiles >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  if (in_dtype == kInF32)
    hipLaunchKernelGGL(syrk_thin<true>, dim3((unsigned)tiles), dim3(256), 0, stream, static_cast<const char*>(X),
                       ld * es, (int)n, d, S, lds);
  else
    hipLaunchKernelGGL(syrk_thin<false>, dim3((unsigned)tiles), dim3(256), 0, stream, static_cast<const char*>(X),
                       ld * es, (int)n, d, S, lds);
  return hipGetLastError();
}

}  // namespace hess
