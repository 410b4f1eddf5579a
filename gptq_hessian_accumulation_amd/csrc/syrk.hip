// Symmetric rank-k update of the calibration Gram sum on gfx950 matrix cores.
//
//   S[i][j] += sum_t X[t][i] * X[t][j]      for the upper-triangle tiles (j >= i)
//
// This is the per-batch accumulation of the GPTQ/QQQ Hessian (GPTQModel PR 2979,
// What Changed: add_batch accumulates the Gram of the flattened activations;
// PR 2981, Changes: accumulated in place into the persistent float32 buffer,
// no transient d x d product), with bf16 inputs read directly and multiplied
// exactly into float32 (Model-Optimizer PR 3002 page, "What does this PR do?":
// bfloat16 in, float32 out).
//
// Structure of one workgroup (256 threads = 4 waves, 2 x 2):
//  * owns one B x B tile (I, J), I <= J, of S, B = 64*WT; each wave owns a
//    (32*WT) x (32*WT) sub-tile made of WT x WT blocks of 32 x 32;
//  * walks its token range in K-iterations of 64 tokens.  Each thread loads
//    8 tokens x 8 features with 16-byte row loads (coalesced along features),
//    transposes the 8 x 8 block in registers and writes 8 feature rows of
//    16 bytes into LDS, laid out [feature][token] with an XOR swizzle that
//    keeps both the writes and the matrix-core operand reads free of LDS
//    bank conflicts; two LDS stages overlap loads with the matrix cores;
//  * multiplies with v_mfma_f32_32x32x16_bf16 (B operand first, so each
//    accumulator holds a row segment of the block: float4 epilogue I/O);
//  * moves the matrix-core accumulators into a second float32 register set
//    every `flush_iters` iterations, so no float32 rounding chain is longer
//    than that many tokens whatever the batch size;
//  * adds the tile into S (read-modify-write, no transient buffer) or, when
//    the token range of a tile is split over several workgroups, writes a
//    partial tile that a reduction kernel adds into S in a fixed order.
// Diagonal tiles load one panel and skip the wave below the diagonal.
//
// float32 inputs are multiplied on the float32 matrix path
// (v_mfma_f32_32x32x2_f32, exact products): LDS holds the raw float32 words,
// [feature][token], and each lane feeds one token per instruction.  Their
// accumulators are flushed every 1024 tokens.  (A two-term bf16 split of
// float32 values leaves up to 2^-16 relative error per value, too coarse for
// float32 parity, and issuing its small lo*lo products as separate
// instructions rounds them away against the large accumulator.)

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;               // tokens per K-iteration

__device__ __forceinline__ int swz(int f) { return (f ^ (f >> 3)) & 7; }

template <int WT, int IN, bool VEC>
struct SyrkTraits {
  static constexpr int B = 64 * WT;                 // workgroup tile edge
  static constexpr int WTE = 32 * WT;               // wave tile edge
  // one feature row of a panel in LDS: 64 tokens of bf16, or of (hi|lo) words
  static constexpr int ROW_BYTES = IN == kInF32 ? kBK * 4 : kBK * 2;
  static constexpr int PANEL_BYTES = B * ROW_BYTES;
  static constexpr int STAGE_BYTES = 2 * PANEL_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int FG = B / 8;                  // 8-feature groups per panel
  static constexpr int UNITS_PER_PANEL = FG * 8;    // x 8 token groups
  static constexpr int MAX_UNITS = 2 * UNITS_PER_PANEL;
  static constexpr int UPT = (MAX_UNITS + kThreads - 1) / kThreads;
  static constexpr int ESIZE = IN == kInF32 ? 4 : 2;
};

// Registers holding one 8-token x 8-feature unit between its global load and
// its LDS store.  bf16: 8 rows of 8 bf16.  fp32: 8 rows of 8 floats.
template <int IN>
struct UnitRegs;
template <>
struct UnitRegs<kInBF16> {
  u32x4 row[8];
  uint32_t rmask;  // bit r: token row r is in range
  uint32_t cmask;  // bit c: feature c is in range
};
template <>
struct UnitRegs<kInF32> {
  u32x4 row[8][2];
  uint32_t rmask;
  uint32_t cmask;
};

template <int WT, int IN, bool VEC>
struct SyrkTile {
  using T = SyrkTraits<WT, IN, VEC>;

  // unit u -> (panel p, token group tg, feature group fg)
  __device__ __forceinline__ static void unit_coords(int u, int& p, int& tg, int& fg) {
    p = u / T::UNITS_PER_PANEL;
    const int r = u - p * T::UNITS_PER_PANEL;
    tg = r / T::FG;
    fg = r - tg * T::FG;
  }

  // Global -> registers for one unit.  Only issues loads: every address is
  // clamped into range (last valid token row, last valid feature) and the
  // validity masks travel with the registers, to be applied when the unit is
  // stored to LDS; nothing here waits for the loaded data.
  __device__ __forceinline__ static void load_unit(const SyrkParams& P, const int64_t (&xr)[8], int64_t k0,
                                                   int64_t k_end, int f0, UnitRegs<IN>& R) {
    const char* X = static_cast<const char*>(P.X);
    uint32_t rm = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) rm |= (k0 + r < k_end) ? (1u << r) : 0u;
    const int nvalid = P.d - f0;  // features of this unit in range (may be <= 0 or >= 8)
    R.rmask = nvalid > 0 ? rm : 0u;
    R.cmask = nvalid >= 8 ? 0xFFu : (nvalid > 0 ? ((1u << nvalid) - 1u) : 0u);
    if constexpr (VEC) {
      const int fc = nvalid > 0 ? f0 : 0;  // d % 8 == 0 here: a unit is all in or all out
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const u32x4* p = reinterpret_cast<const u32x4*>(X + (xr[r] * P.ld + fc) * T::ESIZE);
        if constexpr (IN == kInBF16) {
          R.row[r] = *p;
        } else {
          R.row[r][0] = p[0];
          R.row[r][1] = p[1];
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const char* rowp = X + xr[r] * P.ld * T::ESIZE;
        uint32_t w[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int fcl = min(f0 + c, P.d - 1);
          if constexpr (IN == kInBF16)
            w[c] = reinterpret_cast<const uint16_t*>(rowp)[fcl];
          else
            w[c] = reinterpret_cast<const uint32_t*>(rowp)[fcl];
        }
        if constexpr (IN == kInBF16) {
          R.row[r] = u32x4{w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16)};
        } else {
          R.row[r][0] = u32x4{w[0], w[1], w[2], w[3]};
          R.row[r][1] = u32x4{w[4], w[5], w[6], w[7]};
        }
      }
    }
  }

  // Token rows k0 .. k0+7 clamped into range, as row numbers of X (through
  // the gather index when there is one).
  __device__ __forceinline__ static void fetch_rows(const int32_t* rows, int64_t k0, int64_t k_end,
                                                    int32_t (&g)[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t t = k0 + r;
      const int64_t tc = t < k_end ? t : k_end - 1;
      g[r] = rows ? rows[tc] : 0;
    }
  }

  // Registers -> LDS for one unit: apply the validity masks, then write the
  // unit's 8 feature rows.  bf16: transpose the 8 x 8 block of 16-bit values;
  // a feature's 8 tokens are one 16-byte chunk.  fp32: a feature's 8 tokens
  // are two 16-byte chunks.  Chunk c of feature row f sits at chunk c ^ swz(f).
  __device__ __forceinline__ static void store_unit(char* stage, int p, int tg, int fg, const UnitRegs<IN>& R) {
    char* panel = stage + p * T::PANEL_BYTES;
    if constexpr (IN == kInBF16) {
      // 16-bit lane masks of the 8 columns: dword q holds columns 2q, 2q+1
      uint32_t cm[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        cm[q] = ((R.cmask >> (2 * q)) & 1u ? 0x0000FFFFu : 0u) | ((R.cmask >> (2 * q + 1)) & 1u ? 0xFFFF0000u : 0u);
      u32x4 rowm[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t rr = (R.rmask >> r) & 1u ? 0xFFFFFFFFu : 0u;
        rowm[r] = u32x4{R.row[r][0] & cm[0] & rr, R.row[r][1] & cm[1] & rr, R.row[r][2] & cm[2] & rr,
                        R.row[r][3] & cm[3] & rr};
      }
      u32x4 col[8];
      transpose8x8_b16(rowm, col);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int f = fg * 8 + i;
        *reinterpret_cast<u32x4*>(panel + f * T::ROW_BYTES + ((tg ^ swz(f)) << 4)) = col[i];
      }
    } else {
      uint32_t w[8][8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const bool ok = ((R.rmask >> r) & 1u) && ((R.cmask >> c) & 1u);
          w[r][c] = ok ? R.row[r][c >> 2][c & 3] : 0u;
        }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int f = fg * 8 + i;
        char* row = panel + f * T::ROW_BYTES;
        *reinterpret_cast<u32x4*>(row + (((2 * tg) ^ swz(f)) << 4)) = u32x4{w[0][i], w[1][i], w[2][i], w[3][i]};
        *reinterpret_cast<u32x4*>(row + (((2 * tg + 1) ^ swz(f)) << 4)) = u32x4{w[4][i], w[5][i], w[6][i], w[7][i]};
      }
    }
  }

  // bf16 operand for the 32 features [f0, f0+32), K16 step h (tokens 16h..16h+15).
  __device__ __forceinline__ static u32x4 read_operand(const char* panel, int f0, int h, int lane) {
    const int f = f0 + (lane & 31);
    const int c = 2 * h + (lane >> 5);
    return *reinterpret_cast<const u32x4*>(panel + f * T::ROW_BYTES + ((c ^ swz(f)) << 4));
  }

  // fp32: the words of tokens 16h + 8*(lane/32) + 0..7 of feature f0 + lane%32.
  __device__ __forceinline__ static void read_words(const char* panel, int f0, int h, int lane, u32x4& w0,
                                                    u32x4& w1) {
    const int f = f0 + (lane & 31);
    const int c = 4 * h + 2 * (lane >> 5);
    const char* row = panel + f * T::ROW_BYTES;
    w0 = *reinterpret_cast<const u32x4*>(row + ((c ^ swz(f)) << 4));
    w1 = *reinterpret_cast<const u32x4*>(row + (((c + 1) ^ swz(f)) << 4));
  }
};

template <int WT, int IN, bool VEC>
__device__ __forceinline__ void syrk_body(const SyrkParams& P, char* lds) {
  using T = SyrkTraits<WT, IN, VEC>;
  using K = SyrkTile<WT, IN, VEC>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // ---- work item -> (group, tile, token range) ----
  int item = blockIdx.x;
  if (P.xcd_contig) {
    // Consecutive workgroups go to the 8 XCDs in turn; give each XCD a
    // contiguous range of items so the tiles sharing panels share an L2.
    const int per = (P.total_items + 7) / 8;
    item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  }
  if (item >= P.total_items) return;
  int g = 0;
  while (g + 1 < P.ngroups && item >= P.item_prefix[g + 1]) ++g;
  const int local = item - P.item_prefix[g];
  const SyrkGroup G = P.g[g];
  const int tile = local % P.ntiles;
  const int split = local / P.ntiles;
  // tile -> (I, J), I <= J, row-major over the upper triangle
  int I = 0, rem = tile;
  while (rem >= P.nb - I) {
    rem -= P.nb - I;
    ++I;
  }
  const int J = I + rem;
  const bool diag = (I == J);
  const int64_t k_begin = G.row_begin + (int64_t)split * P.kchunk;
  const int64_t k_end = min(G.row_end, k_begin + (int64_t)P.kchunk);
  const int niter = (int)((k_end - k_begin + kBK - 1) / kBK);
  const int32_t* rows = P.rows;

  const int fa0 = I * T::B, fb0 = J * T::B;  // feature origin of panels A and B
  const bool wave_active = !(diag && wr > wc);  // below-diagonal wave of a diagonal tile

  constexpr int NB = WT * WT;
  f32x16 acc[NB];
  f32x16 mst[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    acc[b] = f32x16{};
    mst[b] = f32x16{};
  }

  const int npanels = diag ? 1 : 2;
  const int units = npanels * T::UNITS_PER_PANEL;
  UnitRegs<IN> R[T::UPT];

  // gather indices are fetched one K-iteration ahead of the rows they name
  int32_t gidx[T::UPT][8];
  auto fetch_iter = [&](int it) {
    if (!rows) return;
#pragma unroll
    for (int q = 0; q < T::UPT; ++q) {
      const int u = tid + q * kThreads;
      if (u < units) {
        int p, tg, fg;
        K::unit_coords(u, p, tg, fg);
        K::fetch_rows(rows, k_begin + (int64_t)it * kBK + tg * 8, k_end, gidx[q]);
      }
    }
  };
  auto load_iter = [&](int it) {
#pragma unroll
    for (int q = 0; q < T::UPT; ++q) {
      const int u = tid + q * kThreads;
      if (u < units) {
        int p, tg, fg;
        K::unit_coords(u, p, tg, fg);
        const int f0 = (p == 0 ? fa0 : fb0) + fg * 8;
        const int64_t k0 = k_begin + (int64_t)it * kBK + tg * 8;
        int64_t xr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int64_t tc = k0 + r < k_end ? k0 + r : k_end - 1;
          xr[r] = rows ? (int64_t)gidx[q][r] : tc;
        }
        K::load_unit(P, xr, k0, k_end, f0, R[q]);
      }
    }
  };
  auto store_iter = [&](char* stage) {
#pragma unroll
    for (int q = 0; q < T::UPT; ++q) {
      const int u = tid + q * kThreads;
      if (u < units) {
        int p, tg, fg;
        K::unit_coords(u, p, tg, fg);
        K::store_unit(stage, p, tg, fg, R[q]);
      }
    }
  };
  auto compute_iter = [&](const char* stage) {
    if (!wave_active) return;
    const char* pa = stage;
    const char* pb = diag ? stage : stage + T::PANEL_BYTES;
    const int fa = wr * T::WTE, fb = wc * T::WTE;
#pragma unroll
    for (int h = 0; h < kBK / 16; ++h) {
      if constexpr (IN == kInBF16) {
        u32x4 a[WT], b[WT];
#pragma unroll
        for (int i = 0; i < WT; ++i) a[i] = K::read_operand(pa, fa + 32 * i, h, lane);
#pragma unroll
        for (int j = 0; j < WT; ++j) b[j] = K::read_operand(pb, fb + 32 * j, h, lane);
#pragma unroll
        for (int i = 0; i < WT; ++i)
#pragma unroll
          for (int j = 0; j < WT; ++j) acc[i * WT + j] = mfma32x32x16(b[j], a[i], acc[i * WT + j]);
      } else {
        u32x4 a0[WT], a1[WT], b0[WT], b1[WT];
#pragma unroll
        for (int i = 0; i < WT; ++i) K::read_words(pa, fa + 32 * i, h, lane, a0[i], a1[i]);
#pragma unroll
        for (int j = 0; j < WT; ++j) K::read_words(pb, fb + 32 * j, h, lane, b0[j], b1[j]);
        // instruction s: lanes 0-31 multiply token 16h + s, lanes 32-63 token 16h + 8 + s
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int i = 0; i < WT; ++i)
#pragma unroll
            for (int j = 0; j < WT; ++j) {
              const float av = __uint_as_float(s < 4 ? a0[i][s] : a1[i][s - 4]);
              const float bv = __uint_as_float(s < 4 ? b0[j][s] : b1[j][s - 4]);
              acc[i * WT + j] = mfma32x32x2_f32(bv, av, acc[i * WT + j]);
            }
      }
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      mst[b] += acc[b];
      acc[b] = f32x16{};
    }
  };

  // ---- K loop: two LDS stages, registers prefetch one iteration ahead ----
  if (niter > 0) {
    fetch_iter(0);
    load_iter(0);
    if (niter > 1) fetch_iter(1);
    store_iter(lds);
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
      char* cur = lds + (it & 1) * T::STAGE_BYTES;
      char* nxt = lds + ((it + 1) & 1) * T::STAGE_BYTES;
      const bool more = it + 1 < niter;
      if (more) load_iter(it + 1);
      if (it + 2 < niter) fetch_iter(it + 2);
      compute_iter(cur);
      if (more) store_iter(nxt);
      if (P.flush_iters > 0 && ((it + 1) % P.flush_iters) == 0) flush();
      __syncthreads();
    }
  }
  flush();

  if (!wave_active) return;

  // ---- epilogue: lane holds row (l%32) of each block, columns 8q + 4h + e ----
  const int hsel = lane >> 5;
  const int rrow = lane & 31;
  if (P.ks == 1) {
    float* S = G.S;
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int row = fa0 + wr * T::WTE + 32 * i + rrow;
      if (row >= P.d) continue;
#pragma unroll
      for (int j = 0; j < WT; ++j) {
        const int colb = fb0 + wc * T::WTE + 32 * j + 4 * hsel;
        float* srow = S + (int64_t)row * P.lds;
        const f32x16& m = mst[i * WT + j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = colb + 8 * q;
          if (col + 4 <= P.d && P.s_vec) {
            float4 v = *reinterpret_cast<const float4*>(srow + col);
            v.x += m[4 * q + 0];
            v.y += m[4 * q + 1];
            v.z += m[4 * q + 2];
            v.w += m[4 * q + 3];
            *reinterpret_cast<float4*>(srow + col) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < P.d) srow[col + e] += m[4 * q + e];
          }
        }
      }
    }
  } else {
    // partial tile, tile-local row-major B x B, slot (split, tile)
    float* W = G.ws + ((int64_t)split * P.ntiles + tile) * (int64_t)(T::B * T::B);
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int row = wr * T::WTE + 32 * i + rrow;
#pragma unroll
      for (int j = 0; j < WT; ++j) {
        const int colb = wc * T::WTE + 32 * j + 4 * hsel;
        const f32x16& m = mst[i * WT + j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float4 v = {m[4 * q + 0], m[4 * q + 1], m[4 * q + 2], m[4 * q + 3]};
          *reinterpret_cast<float4*>(W + (int64_t)row * T::B + colb + 8 * q) = v;
        }
      }
    }
  }
}

// Reduction of split partial tiles: S_tile += ws[0] + ws[1] + ... in split
// order (a fixed order, so results do not depend on scheduling).
__global__ void __launch_bounds__(256) syrk_reduce_kernel(float* S, int64_t lds, const float* ws, int d, int B,
                                                          int nb, int ntiles, int ks) {
  const int tile = blockIdx.y;
  int I = 0, rem = tile;
  while (rem >= nb - I) {
    rem -= nb - I;
    ++I;
  }
  const int J = I + rem;
  const int64_t tile_elems = (int64_t)B * B;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < tile_elems;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(e / B), c = (int)(e % B);
    const int row = I * B + r, col = J * B + c;
    if (row >= d || col >= d) continue;
    if (I == J && r >= B / 2 && c < B / 2) continue;  // quadrant of the skipped wave: never written
    float acc = 0.f;
    for (int s = 0; s < ks; ++s) acc += ws[((int64_t)s * ntiles + tile) * tile_elems + e];
    S[(int64_t)row * lds + col] += acc;
  }
}

}  // namespace

#define HESS_SYRK_KERNEL(NAME, WT, IN, VEC, MINB)                                                 \
  __global__ void __launch_bounds__(kThreads, MINB) NAME(SyrkParams P) {                           \
    extern __shared__ __attribute__((aligned(16))) char hess_lds[];                                \
    syrk_body<WT, IN, VEC>(P, hess_lds);                                                           \
  }

HESS_SYRK_KERNEL(syrk_bf16_wt2_vec, 2, kInBF16, true, 2)
HESS_SYRK_KERNEL(syrk_bf16_wt2_gen, 2, kInBF16, false, 1)
HESS_SYRK_KERNEL(syrk_f32_wt2_vec, 2, kInF32, true, 1)
HESS_SYRK_KERNEL(syrk_f32_wt2_gen, 2, kInF32, false, 1)

namespace {
template <int WT, int IN>
int lds_bytes() {
  return SyrkTraits<WT, IN, true>::LDS_BYTES;
}

hipError_t set_lds_limit(const void* fn, int bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}
}  // namespace

int syrk_tile_edge(int wt) { return 64 * wt; }

hipError_t launch_syrk(const SyrkParams& P, int wt, int in_dtype, bool vec, hipStream_t stream) {
  const void* fn = nullptr;
  int lds = 0;
  if (in_dtype == kInBF16) {
    if (wt == 2 && vec) {
      fn = reinterpret_cast<const void*>(&syrk_bf16_wt2_vec);
      lds = lds_bytes<2, kInBF16>();
    } else if (wt == 2) {
      fn = reinterpret_cast<const void*>(&syrk_bf16_wt2_gen);
      lds = lds_bytes<2, kInBF16>();
    }
  } else if (in_dtype == kInF32 && wt == 2) {
    fn = vec ? reinterpret_cast<const void*>(&syrk_f32_wt2_vec) : reinterpret_cast<const void*>(&syrk_f32_wt2_gen);
    lds = lds_bytes<2, kInF32>();
  }
  if (!fn) return hipErrorInvalidValue;
  static bool attr_done[8] = {};
  const int key = (in_dtype == kInF32 ? 4 : 0) + (wt == 3 ? 2 : 0) + (vec ? 1 : 0);
  if (!attr_done[key]) {
    hipError_t e = set_lds_limit(fn, lds);
    if (e != hipSuccess) return e;
    attr_done[key] = true;
  }
  const int per = (P.total_items + 7) / 8;
  const int grid = P.xcd_contig ? per * 8 : P.total_items;
  void* args[] = {const_cast<SyrkParams*>(&P)};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, stream);
}

hipError_t launch_syrk_reduce(float* S, int64_t lds, const float* ws, int d, int B, int nb, int ntiles, int ks,
                              hipStream_t stream) {
  const int64_t elems = (int64_t)B * B;
  const int gx = (int)((elems + 255) / 256 < 64 ? (elems + 255) / 256 : 64);
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3(gx, ntiles), dim3(256), 0, stream, S, lds, ws, d, B, nb, ntiles, ks);
  return hipGetLastError();
}

}  // namespace hess
