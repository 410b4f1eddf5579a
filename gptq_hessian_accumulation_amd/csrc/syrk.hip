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
// One workgroup owns one 128 x 128 tile (I, J), I <= J, of S and a range of
// tokens.  Its 8 waves split into two roles (producer / consumer):
//  * 4 matrix-core waves (2 x 2, a 64 x 64 sub-tile each) read operands from
//    LDS and accumulate with v_mfma_f32_32x32x16_bf16 (B operand first, so
//    each accumulator holds a row segment).  Every `flush_iters` K-iterations
//    the accumulators are added into a second float32 register set, so no
//    float32 rounding chain is longer than that.
//  * 4 loader waves keep the X loads of the next two 64-token K-iterations in
//    flight at all times (the kernel is fed from L2 at up to ~15 TB/s and its
//    loads see ~1 us of latency under load), transpose each 8 x 8 block of
//    (token, feature) values in registers, and write [feature][token] panels
//    into LDS with an XOR swizzle that keeps both these writes and the operand
//    reads free of bank conflicts.  Two LDS stages, one barrier per iteration.
//    Every loader load is unconditional (iterations past the batch read an
//    empty range and the loop runs an even number of iterations), so each
//    wait is for exactly the data about to be stored.
//  * The matrix-core waves issue no X loads, so they read their part of the
//    S tile into the second register set when they start: the read half of
//    the read-modify-write hides behind the whole K loop.  At the end they
//    add the last accumulators and write S (or, for a tile whose token range
//    is split over several workgroups, a partial that a reduction kernel adds
//    into S in a fixed order).
// Diagonal tiles load one panel and leave the below-diagonal wave idle.
//
// X is read through raw buffer loads when it needs no gather and is 16-byte
// aligned: one descriptor per K-iteration whose range ends at the batch's
// last row, so rows past the batch and tiles past d (addressed out of range)
// read as zero and no masking is needed.  A gather (routed-expert rows) and
// unaligned X use global loads with clamped addresses and masks.
//
// float32 inputs are multiplied on the float32 matrix path
// (v_mfma_f32_32x32x2_f32, exact products): LDS holds the raw float32 words,
// [feature][token], and each lane feeds one token per instruction; their
// accumulators are flushed every 1024 tokens.  (A two-term bf16 split of
// float32 values leaves up to 2^-16 relative error per value, too coarse for
// float32 parity, and issuing its small lo*lo products as separate
// instructions rounds them away against the large accumulator.)

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kB = 128;                   // tile edge
constexpr int kBK = 64;                   // tokens per K-iteration
constexpr int kThreads = 512;             // 4 matrix-core waves + 4 loader waves
constexpr int kFG = kB / 8;               // 8-feature groups per panel
constexpr int kUnitsPerPanel = kFG * 8;   // x 8 token groups of 8

enum LoadMode { kBuffer = 0, kGatherVec = 1, kGeneric = 2 };

__device__ __forceinline__ int swz(int f) { return (f ^ (f >> 3)) & 7; }

template <int IN>
struct Traits {
  static constexpr int ES = IN == kInF32 ? 4 : 2;
  static constexpr int ROW_BYTES = kBK * ES;  // one feature row of a panel: 64 tokens
  static constexpr int PANEL_BYTES = kB * ROW_BYTES;
  static constexpr int STAGE_BYTES = 2 * PANEL_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
};

// One 8-token x 8-feature unit between its global load and its LDS store.
template <int IN>
struct Unit;
template <>
struct Unit<kInBF16> {
  u32x4 row[8];      // row r: token r, features 2p | 2p+1 << 16 in dword p
  uint32_t rmask;    // bit r: token in range (masked modes only)
  uint32_t cmask;    // bit c: feature in range (masked modes only)
};
template <>
struct Unit<kInF32> {
  u32x4 row[8][2];   // row r: 8 float32 features
  uint32_t rmask;
  uint32_t cmask;
};

// unit u -> (panel p, token group tg, feature group fg)
__device__ __forceinline__ void unit_coords(int u, int& p, int& tg, int& fg) {
  p = u / kUnitsPerPanel;
  const int r = u - p * kUnitsPerPanel;
  tg = r / kFG;
  fg = r - tg * kFG;
}

template <int IN>
__device__ __forceinline__ void load_unit_buffer(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t row_bytes,
                                                 Unit<IN>& R) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if constexpr (IN == kInBF16) {
      R.row[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, r * row_bytes, 0));
    } else {
      R.row[r][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, r * row_bytes, 0));
      R.row[r][1] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 16, r * row_bytes, 0));
    }
  }
}

// Global loads of one unit from rows xr[] (clamped into range by the caller)
// and features f0..f0+7 (clamped to d-1 here); the masks record what is real.
template <int IN, bool VEC>
__device__ __forceinline__ void load_unit_global(const char* X, int64_t ld, int d, const int64_t (&xr)[8],
                                                 uint32_t rmask, int f0, Unit<IN>& R) {
  constexpr int ES = Traits<IN>::ES;
  const int nvalid = d - f0;
  R.rmask = nvalid > 0 ? rmask : 0u;
  R.cmask = nvalid >= 8 ? 0xFFu : (nvalid > 0 ? ((1u << nvalid) - 1u) : 0u);
  if constexpr (VEC) {
    const int fc = nvalid > 0 ? f0 : 0;  // d % 8 == 0: a unit is all in or all out
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const u32x4* p = reinterpret_cast<const u32x4*>(X + (xr[r] * ld + fc) * ES);
      if constexpr (IN == kInBF16) {
        R.row[r] = p[0];
      } else {
        R.row[r][0] = p[0];
        R.row[r][1] = p[1];
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const char* rowp = X + xr[r] * ld * ES;
      uint32_t w[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int fcl = min(f0 + c, d - 1);
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

// Registers -> LDS for one unit (masks applied first when MASKED).  bf16: the
// 8 x 8 block of 16-bit values is transposed and a feature's 8 tokens are one
// 16-byte chunk; fp32: a feature's 8 tokens are two 16-byte chunks.  Chunk c
// of feature row f sits at chunk c ^ swz(f) of that row.
template <int IN, bool MASKED>
__device__ __forceinline__ void store_unit(char* panel, int tg, int fg, const Unit<IN>& R) {
  constexpr int RB = Traits<IN>::ROW_BYTES;
  if constexpr (IN == kInBF16) {
    u32x4 rowm[8];
    if constexpr (MASKED) {
      uint32_t cm[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        cm[q] = ((R.cmask >> (2 * q)) & 1u ? 0x0000FFFFu : 0u) | ((R.cmask >> (2 * q + 1)) & 1u ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t rr = (R.rmask >> r) & 1u ? 0xFFFFFFFFu : 0u;
        rowm[r] = u32x4{R.row[r][0] & cm[0] & rr, R.row[r][1] & cm[1] & rr, R.row[r][2] & cm[2] & rr,
                        R.row[r][3] & cm[3] & rr};
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) rowm[r] = R.row[r];
    }
    u32x4 col[8];
    transpose8x8_b16(rowm, col);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = fg * 8 + i;
      *reinterpret_cast<u32x4*>(panel + f * RB + ((tg ^ swz(f)) << 4)) = col[i];
    }
  } else {
    uint32_t w[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t v = R.row[r][c >> 2][c & 3];
        if constexpr (MASKED)
          w[r][c] = (((R.rmask >> r) & 1u) && ((R.cmask >> c) & 1u)) ? v : 0u;
        else
          w[r][c] = v;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = fg * 8 + i;
      char* row = panel + f * RB;
      *reinterpret_cast<u32x4*>(row + (((2 * tg) ^ swz(f)) << 4)) = u32x4{w[0][i], w[1][i], w[2][i], w[3][i]};
      *reinterpret_cast<u32x4*>(row + (((2 * tg + 1) ^ swz(f)) << 4)) = u32x4{w[4][i], w[5][i], w[6][i], w[7][i]};
    }
  }
}

// bf16 operand: features f0 + lane%32, tokens 16h + 8*(lane/32) + 0..7.
__device__ __forceinline__ u32x4 read_operand_bf16(const char* panel, int f0, int h, int lane) {
  const int f = f0 + (lane & 31);
  const int c = 2 * h + (lane >> 5);
  return *reinterpret_cast<const u32x4*>(panel + f * Traits<kInBF16>::ROW_BYTES + ((c ^ swz(f)) << 4));
}

// fp32: the words of tokens 16h + 8*(lane/32) + 0..7 of feature f0 + lane%32.
__device__ __forceinline__ void read_words_f32(const char* panel, int f0, int h, int lane, u32x4& w0, u32x4& w1) {
  const int f = f0 + (lane & 31);
  const int c = 4 * h + 2 * (lane >> 5);
  const char* row = panel + f * Traits<kInF32>::ROW_BYTES;
  w0 = *reinterpret_cast<const u32x4*>(row + ((c ^ swz(f)) << 4));
  w1 = *reinterpret_cast<const u32x4*>(row + (((c + 1) ^ swz(f)) << 4));
}

__device__ __forceinline__ void tile_ij(int tile, int nb, int& I, int& J) {
  int i = 0, rem = tile;
  while (rem >= nb - i) {
    rem -= nb - i;
    ++i;
  }
  I = i;
  J = i + rem;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(uint64_t base, int64_t bytes) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int nrec = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, nrec,
                                           0x00020000);
}

template <int IN, int MODE>
__device__ __forceinline__ void syrk_body(const SyrkParams& P, char* lds) {
  using T = Traits<IN>;
  constexpr bool MASKED = MODE != kBuffer;
  constexpr bool VEC = MODE != kGeneric;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform role
  const bool loader = wave >= 4;

  // ---- work item -> (group, tile, token range, output) ----
  int g = 0, tile = 0, slot = -1;
  int64_t k_begin = 0, k_end = 0;
  const int bid = blockIdx.x;
  if (P.ngroups > 1) {
    const int item = bid;
    if (item >= P.item_prefix[P.ngroups]) return;
    while (g + 1 < P.ngroups && item >= P.item_prefix[g + 1]) ++g;
    tile = item - P.item_prefix[g];
    k_begin = P.g[g].row_begin;
    k_end = P.g[g].row_end;
  } else if (bid < P.grid_full) {
    // full tiles: XCD x (= bid % 8) takes a contiguous run of tiles, which
    // share panels and so share that XCD's L2
    const int per = P.grid_full / 8;
    tile = (bid & 7) * per + (bid >> 3);
    if (tile >= P.full_tiles) return;
    k_begin = P.g[0].row_begin;
    k_end = P.g[0].row_end;
  } else {
    const int tail_items = (P.ntiles - P.full_tiles) * P.tail_parts;
    const int b = bid - P.grid_full;
    const int per = (tail_items + 7) / 8;
    const int item = (b & 7) * per + (b >> 3);
    if (item >= tail_items) return;
    const int t = item / P.tail_parts, part = item - t * P.tail_parts;
    tile = P.full_tiles + t;
    slot = item;
    k_begin = P.g[0].row_begin + (int64_t)part * P.tail_kchunk;
    k_end = min(P.g[0].row_end, k_begin + (int64_t)P.tail_kchunk);
  }
  int I, J;
  tile_ij(tile, P.nb, I, J);
  const bool diag = I == J;
  const int niter = (int)((k_end - k_begin + kBK - 1) / kBK);
  const int fa0 = I * kB, fb0 = J * kB;
  const int units = (diag ? 1 : 2) * kUnitsPerPanel;
  const bool rmw = slot < 0;

  // matrix-core waves
  const int wr = (wave >> 1) & 1, wc = wave & 1;
  const bool wave_active = !loader && !(diag && wr > wc);
  f32x16 acc[4], mst[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    acc[b] = f32x16{};
    mst[b] = f32x16{};
  }
  // loader waves: lane lu handles unit lu of every K-iteration.  All 256
  // lanes always issue their loads and stores (no divergent branch around
  // them, which would make the compiler wait for every outstanding load):
  // on a diagonal tile the second-panel units read an out-of-range offset
  // (zeros) and write them into the unused second panel.
  const int lu = loader ? tid - 256 : 0;
  const bool lactive = loader && lu < units;
  int up = 0, utg = 0, ufg = 0;
  unit_coords(lu, up, utg, ufg);
  const int uf0 = (up == 0 ? fa0 : fb0) + ufg * 8;
  const uint32_t row_bytes = (uint32_t)(P.ld * T::ES);
  const uint32_t voff =
      (lactive && uf0 < P.d) ? (uint32_t)(utg * 8) * row_bytes + (uint32_t)uf0 * T::ES : 0x80000000u;
  const char* X = static_cast<const char*>(P.X);
  const int32_t* rows = MODE == kBuffer ? nullptr : P.rows;
  Unit<IN> R0, R1;
  int32_t G0[8], G1[8];

  auto fetch_idx = [&](int it, int32_t (&G)[8]) {
    if (MODE == kBuffer || !rows) return;
    // iterations past the batch fetch (clamped) indices too: every load in
    // the loop is unconditional
    const int64_t k0 = k_begin + (int64_t)it * kBK + utg * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) G[r] = rows[k0 + r < k_end ? k0 + r : k_end - 1];
  };
  auto load_it = [&](int it, Unit<IN>& R, const int32_t (&G)[8]) {
    if constexpr (MODE == kBuffer) {
      // one descriptor per K-iteration, in scalar registers; its range ends
      // at the batch's last row, so later rows (and voff past d) read zero
      const int64_t k0 = k_begin + (int64_t)it * kBK;
      const int64_t valid = max((int64_t)0, min((int64_t)kBK, k_end - k0));  // 0 past the batch
      const uint64_t base = reinterpret_cast<uint64_t>(X) + (uint64_t)(k0 * P.ld * T::ES);
      load_unit_buffer<IN>(uniform_rsrc(base, valid * row_bytes), voff, row_bytes, R);
    } else {
      const int64_t k0 = k_begin + (int64_t)it * kBK + utg * 8;
      int64_t xr[8];
      uint32_t rm = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool ok = lactive && k0 + r < k_end;
        rm |= ok ? (1u << r) : 0u;
        xr[r] = rows ? (int64_t)G[r] : (ok ? k0 + r : k_end - 1);
      }
      load_unit_global<IN, VEC>(X, P.ld, P.d, xr, rm, uf0, R);
    }
  };
  auto store_it = [&](char* stage, const Unit<IN>& R) {
    store_unit<IN, MASKED>(stage + up * T::PANEL_BYTES, utg, ufg, R);
  };

  // S descriptor: the tile's rows that exist; columns past d in the last
  // row read zero, those in other rows are read but never written back
  const __amdgpu_buffer_rsrc_t srsrc =
      uniform_rsrc(reinterpret_cast<uint64_t>(P.g[g].S) + (uint64_t)((int64_t)fa0 * P.lds * 4),
                   (int64_t)min(kB, P.d - fa0) * P.lds * 4);
  // accumulator element (block i, j; register 4q + e) of this lane: tile row
  // wr*64 + 32i + lane%32, column wc*64 + 32j + 8q + 4*(lane/32) + e
  const int hsel = lane >> 5, rrow = lane & 31;

  // One K-iteration on the matrix cores.  The LDS operand reads of step
  // h+1 are issued before the instructions of step h, so their latency
  // overlaps the matrix-core work.
  auto compute_it = [&](const char* stage) {
    if (!wave_active) return;
    const char* pa = stage;
    const char* pb = diag ? stage : stage + T::PANEL_BYTES;
    const int fa = wr * 64, fb = wc * 64;
    if constexpr (IN == kInBF16) {
      u32x4 a[2][2], b[2][2];
      auto rd = [&](int h, u32x4 (&ar)[2], u32x4 (&br)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) ar[i] = read_operand_bf16(pa, fa + 32 * i, h, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) br[j] = read_operand_bf16(pb, fb + 32 * j, h, lane);
      };
      rd(0, a[0], b[0]);
#pragma unroll
      for (int h = 0; h < kBK / 16; ++h) {
        if (h + 1 < kBK / 16) rd(h + 1, a[(h + 1) & 1], b[(h + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's instructions
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i * 2 + j] = mfma32x32x16(b[h & 1][j], a[h & 1][i], acc[i * 2 + j]);
      }
    } else {
      u32x4 a0[2][2], a1[2][2], b0[2][2], b1[2][2];
      auto rd = [&](int h, u32x4 (&x0)[2], u32x4 (&x1)[2], u32x4 (&y0)[2], u32x4 (&y1)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) read_words_f32(pa, fa + 32 * i, h, lane, x0[i], x1[i]);
#pragma unroll
        for (int j = 0; j < 2; ++j) read_words_f32(pb, fb + 32 * j, h, lane, y0[j], y1[j]);
      };
      rd(0, a0[0], a1[0], b0[0], b1[0]);
#pragma unroll
      for (int h = 0; h < kBK / 16; ++h) {
        const int c = h & 1, n = (h + 1) & 1;
        if (h + 1 < kBK / 16) rd(h + 1, a0[n], a1[n], b0[n], b1[n]);
        __builtin_amdgcn_sched_barrier(0);
        // instruction s: lanes 0-31 multiply token 16h + s, lanes 32-63 token 16h + 8 + s
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float av = __uint_as_float(s < 4 ? a0[c][i][s] : a1[c][i][s - 4]);
              const float bv = __uint_as_float(s < 4 ? b0[c][j][s] : b1[c][j][s - 4]);
              acc[i * 2 + j] = mfma32x32x2_f32(bv, av, acc[i * 2 + j]);
            }
      }
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      mst[b] += acc[b];
      acc[b] = f32x16{};
    }
  };

  // The two roles run separate loops with the same number of barriers, so
  // each keeps only its own state in registers.  Odd iteration counts run
  // one more iteration over zeros.
  char* st0 = lds;
  char* st1 = lds + T::STAGE_BYTES;
  const int npad = (niter + 1) & ~1;
  if (loader) {
    // prologue: iterations 0 and 1 in flight, iteration 0 in LDS
    fetch_idx(0, G0);
    fetch_idx(1, G1);
    load_it(0, R0, G0);
    load_it(1, R1, G1);
    fetch_idx(2, G0);
    store_it(st0, R0);
    fetch_idx(3, G1);
    load_it(2, R0, G0);
    fetch_idx(4, G0);
    __syncthreads();
    // iteration it: store iteration it+1 (register set (it+1)&1) into the
    // stage the matrix cores are not reading, then reuse the set for the
    // loads of iteration it+3
    auto lstep = [&](int it, char* nxt, Unit<IN>& Rn, int32_t (&Gn)[8]) {
      store_it(nxt, Rn);
      load_it(it + 3, Rn, Gn);
      fetch_idx(it + 5, Gn);
      __syncthreads();
    };
    for (int it = 0; it < npad; it += 2) {
      lstep(it, st1, R1, G1);
      lstep(it + 1, st0, R0, G0);
    }
  } else {
    if (rmw && wave_active) {
      // all 16 loads issued back to back into a staging array, then moved
      // into the flush registers (first used at the first flush)
      float4 sv[16];
      if (P.s_vec) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int i = k >> 3, j = (k >> 2) & 1, q = k & 3;
          const int row = wr * 64 + 32 * i + rrow;
          const int col = fb0 + wc * 64 + 32 * j + 4 * hsel + 8 * q;
          sv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 srsrc, (uint32_t)(((int64_t)row * P.lds + col) * 4), 0, 0));
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int i = k >> 3, j = (k >> 2) & 1, q = k & 3;
          const int row = wr * 64 + 32 * i + rrow;
          const int col = fb0 + wc * 64 + 32 * j + 4 * hsel + 8 * q;
          const uint32_t off = (uint32_t)(((int64_t)row * P.lds + col) * 4);
          sv[k] = float4{__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, off, 0, 0)),
                         __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, off + 4, 0, 0)),
                         __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, off + 8, 0, 0)),
                         __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, off + 12, 0, 0))};
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int b = k >> 2, q = k & 3;
        mst[b][4 * q + 0] = sv[k].x;
        mst[b][4 * q + 1] = sv[k].y;
        mst[b][4 * q + 2] = sv[k].z;
        mst[b][4 * q + 3] = sv[k].w;
      }
    }
    __syncthreads();  // iteration 0 is in LDS
    int flush_left = P.flush_iters;
    auto cstep = [&](const char* cur) {
      compute_it(cur);
      if (--flush_left == 0) {
        flush();
        flush_left = P.flush_iters;
      }
      __syncthreads();
    };
    for (int it = 0; it < npad; it += 2) {
      cstep(st0);
      cstep(st1);
    }
    if (!wave_active) return;
    flush();
    float* W = rmw ? nullptr : P.ws + (int64_t)slot * (kB * kB);
    float* S = P.g[g].S;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wr * 64 + 32 * i + rrow;
        const int colb = wc * 64 + 32 * j + 4 * hsel;
        const f32x16& m = mst[i * 2 + j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v{m[4 * q + 0], m[4 * q + 1], m[4 * q + 2], m[4 * q + 3]};
          const int col = colb + 8 * q;
          if (!rmw) {
            *reinterpret_cast<float4*>(W + row * kB + col) = v;
            continue;
          }
          const int gr = fa0 + row, gc = fb0 + col;
          if (gr >= P.d) continue;
          float* srow = S + (int64_t)gr * P.lds;
          if (P.s_vec && gc + 4 <= P.d) {
            *reinterpret_cast<float4*>(srow + gc) = v;
          } else {
            if (gc + 0 < P.d) srow[gc + 0] = v.x;
            if (gc + 1 < P.d) srow[gc + 1] = v.y;
            if (gc + 2 < P.d) srow[gc + 2] = v.z;
            if (gc + 3 < P.d) srow[gc + 3] = v.w;
          }
        }
      }
  }
}

// Tiles split over several workgroups: S_tile += part_0 + part_1 + ... in
// part order (a fixed order, so results do not depend on scheduling).
__global__ void __launch_bounds__(256) syrk_reduce_kernel(float* S, int64_t lds, const float* ws, int d, int nb,
                                                          int full_tiles, int parts) {
  const int t = blockIdx.y;
  int I, J;
  tile_ij(full_tiles + t, nb, I, J);
  constexpr int E = kB * kB;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x) {
    const int r = e / kB, c = e % kB;
    const int row = I * kB + r, col = J * kB + c;
    if (row >= d || col >= d) continue;
    if (I == J && r >= kB / 2 && c < kB / 2) continue;  // never written
    float acc = 0.f;
    for (int p = 0; p < parts; ++p) acc += ws[((int64_t)t * parts + p) * E + e];
    S[(int64_t)row * lds + col] += acc;
  }
}

}  // namespace

#define HESS_SYRK_KERNEL(NAME, IN, MODE)                             \
  __global__ void __launch_bounds__(kThreads, 1) NAME(SyrkParams P) { \
    extern __shared__ __attribute__((aligned(16))) char hess_lds[];   \
    syrk_body<IN, MODE>(P, hess_lds);                                 \
  }

HESS_SYRK_KERNEL(syrk_bf16_buffer, kInBF16, kBuffer)
HESS_SYRK_KERNEL(syrk_bf16_gather, kInBF16, kGatherVec)
HESS_SYRK_KERNEL(syrk_bf16_generic, kInBF16, kGeneric)
HESS_SYRK_KERNEL(syrk_f32_buffer, kInF32, kBuffer)
HESS_SYRK_KERNEL(syrk_f32_gather, kInF32, kGatherVec)
HESS_SYRK_KERNEL(syrk_f32_generic, kInF32, kGeneric)

int syrk_tile_edge() { return kB; }

hipError_t launch_syrk(const SyrkParams& P, int in_dtype, bool vec, int grid, hipStream_t stream) {
  if (in_dtype != kInBF16 && in_dtype != kInF32) return hipErrorInvalidValue;
  const bool gather = P.rows != nullptr;
  const int mode = !vec ? kGeneric : gather ? kGatherVec : kBuffer;
  const void* table[2][3] = {
      {reinterpret_cast<const void*>(&syrk_bf16_buffer), reinterpret_cast<const void*>(&syrk_bf16_gather),
       reinterpret_cast<const void*>(&syrk_bf16_generic)},
      {reinterpret_cast<const void*>(&syrk_f32_buffer), reinterpret_cast<const void*>(&syrk_f32_gather),
       reinterpret_cast<const void*>(&syrk_f32_generic)}};
  const int di = in_dtype == kInF32 ? 1 : 0;
  const void* fn = table[di][mode];
  const int lds = di ? Traits<kInF32>::LDS_BYTES : Traits<kInBF16>::LDS_BYTES;
  static bool attr_done[2][3] = {};
  if (!attr_done[di][mode]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_done[di][mode] = true;
  }
  if (grid <= 0) return hipSuccess;
  void* args[] = {const_cast<SyrkParams*>(&P)};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, stream);
}

hipError_t launch_syrk_reduce(float* S, int64_t lds, const float* ws, int d, int nb, int full_tiles, int tail_tiles,
                              int parts, hipStream_t stream) {
  if (tail_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3(16, tail_tiles), dim3(256), 0, stream, S, lds, ws, d, nb, full_tiles,
                     parts);
  return hipGetLastError();
}

}  // namespace hess
