// Symmetric rank-k update of the calibration Gram sum with 256 x 256 tiles
// (bf16 activations, 16-byte aligned rows): the long-batch and staged-flush
// path of hess_add_batch.
//
//   S[i][j] += sum_t X[t][i] * X[t][j]      for the upper-triangle tiles (j >= i)
//
// This is the same per-batch update as the 128-tile kernel (GPTQModel PR 2979,
// What Changed; PR 2981, Changes: in place into the persistent float32 sum;
// Model-Optimizer PR 3002 page, "What does this PR do?": bfloat16 in, float32
// out), shaped for long batches on gfx950:
//
//  * A 256 x 256 tile halves the bytes each workgroup streams per flop
//    compared with a 128 x 128 tile.  Streaming activations from memory into
//    all 256 CUs tops out near 14 TB/s on this chip (a kernel whose reads hit
//    in L2 reaches ~24 TB/s), so at 128 x 128 the loads, not the matrix
//    cores, set the pace.
//  * 4 waves, one per SIMD, each own a 128 x 128 quadrant: 64 accumulators of
//    v_mfma_f32_16x16x32_bf16 (256 registers), one instruction per
//    accumulator per 32-token stage.  With activations of N(0,1) scale the
//    matrix cores are power-limited on this chip: measured with every other
//    cost removed, 16x16x32 sustains about 2.0 PFLOP/s where 32x32x16 gets
//    1.65 (half the accumulator traffic per flop; the clock stays higher).
//    The B operand goes first so that each lane's 4 results are consecutive
//    in a row of S (float4 output).
//  * Activations go from memory straight into LDS (buffer_load_dwordx4 with
//    the lds modifier): no registers hold loads and no VALU transposes them.
//    Row-major X: LDS keeps each 32-token stage token-major (a 512-byte row
//    of 256 features per token) with its 16-byte chunks XOR-swizzled; the
//    matrix operands (8 consecutive tokens of one feature) are read
//    transposed with ds_read_b64_tr_b16, two per operand.  The swizzle makes
//    the transposed reads free of bank conflicts and keeps the 64-lane DMA
//    writes 1 KB contiguous.  A staging buffer in the transposed layout
//    (8-token chunks of one feature, written so by the staging copy) lands
//    in LDS operand-ready: one ds_read_b128 per operand, 16 lanes reading
//    256 contiguous bytes.
//  * The loads are written as inline asm (m0 is an input operand) and
//    placed by hand among the matrix instructions of each iteration's second
//    half.  The compiler neither tracks nor waits for them; the kernel's own
//    s_waitcnt before each barrier and before the output are the only
//    waits, which is also what the loads need.
//  * Five LDS stages of 32 tokens (5 x 32 KB, all of the CU's LDS): the
//    loads of up to four iterations are in flight while one is multiplied;
//    one barrier per iteration.  The operands of the stage being multiplied
//    sit in one register set while the next stage's are read into the other
//    (2 x 64 registers).  The barrier is the bare s_barrier after an
//    explicit vmcnt wait for this wave's loads of the next stage.
//  * Loads never need masks: each iteration's buffer descriptor ends at the
//    batch's last row (rows past it read zero), features past d get an
//    out-of-range offset (zero), and iterations past a segment read an empty
//    range.
//  * Work is split stream-K: whole tiles while there are at least 256 of
//    them (one workgroup each, read-modify-write of S), then the remaining
//    tiles' 32-token iterations are divided evenly over up to 256
//    workgroups.  A workgroup's share crosses at most two tiles; each piece
//    that is not a whole tile is written to a workspace slot, and a fixup
//    kernel adds the pieces of each tile into S in a fixed order (results do
//    not depend on scheduling).  Workgroups on one XCD take consecutive work
//    of a blocked tile order, so they share activation panels in that XCD's L2.
//  * Diagonal tiles load one panel and leave the below-diagonal wave idle.
//  * Grouped launches (one Hessian per routed expert, Model-Optimizer PR 3002
//    page, "What does this PR do?") take whole tiles of many Hessians from a
//    host-built schedule, either on the experts' rows gathered into the
//    transposed layout or on the routed rows read where they are: the
//    row-major variant with each load's two row offsets taken from a table
//    (scalar loads one step ahead, outside the hand-counted load waits) and
//    the lane's feature offset added with saturation, so that a missing row
//    stays out of the descriptor's range and reads as zeros.  The operands
//    and their order are the same either way, so the sums are the same bits.
//
// A float32 accumulation chain here is at most kBigChain = 1,024 iterations
// (32,768 tokens) of one tile, whatever the batch length: each addition
// brings in one instruction's sum of 32 exact products (rounded once per 8),
// and a longer part or piece of a tile is cut into chunks whose sums are
// added into S or into the piece's workspace slot, one addition per chunk.

#include "hess_device.hpp"
#include "hess_internal.hpp"

namespace hess {

namespace {

constexpr int kT = 256;                      // tile edge
constexpr int kKI = 32;                      // tokens per stage
constexpr int kRowB = kT * 2;                // one token row of a panel: 512 bytes
constexpr int kPanelB = kKI * kRowB;         // 16 KB
constexpr int kStageB = 2 * kPanelB;         // 32 KB
constexpr int kDma = kStageB / 1024 / 4;     // 1-KB loads per wave per stage (8)
constexpr uint32_t kOOB = 0x80000000u;       // an offset past any descriptor's range
constexpr int kDist = 4;                     // iterations between a stage's load and its use
// s_waitcnt immediate: vmcnt(n), no wait on the other counters
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Physical 16-byte chunk of logical chunk c (8 features) in token row t of a
// row-major stage: c ^ 2 (t % 4) ^ 8 ((t / 8) % 2), an involution.  In a
// transposed read the 16 lanes of a group read 4 consecutive rows t and two
// adjacent chunks, which land in 8 distinct chunks of one 128-byte half of
// the bank space; the group 8 tokens further on lands in the other half.
__device__ __forceinline__ int chunk_pos(int t, int c) { return c ^ (2 * (t & 3)) ^ (8 * ((t >> 3) & 1)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, int64_t bytes) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int nrec = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, nrec,
                                           0x00020000);
}

// The same descriptor as four scalar words, for the load instruction written out.
__device__ __forceinline__ u32x4 rsrc_words(uint64_t base, int64_t bytes) {
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)base);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) & 0xffffu;
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  r[3] = 0x00020000u;
  return r;
}

// One 64-lane 16-byte load from memory into LDS at m0 + 16 * lane (zeros
// for offsets past the descriptor's range).  m0 is set by the compiler as
// an input operand; the s_nop covers the m0-write to LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16(const u32x4& r, uint32_t voff, uint32_t m0) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ u32x4 tr_pair(const char* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HESS_LDS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HESS_LDS s16x4*)(p + 4 * kRowB));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return u32x4{a.x, a.y, b.x, b.y};
}

// Longest float32 accumulation chain, in 32-token iterations (32,768 tokens,
// 4,096 roundings of an 8-product sum into the accumulator): a longer piece of
// a tile is cut into chunks of at most this many iterations, and each chunk's
// sums are added into the tile's destination.  Measured against the float64
// oracle on bf16 data with lognormal column scales, single chains of 16K
// tokens agree to about 1.1e-5 of the mean diagonal, 37K-token chains to
// 1.0e-5 and 65K-token chains to 1.75e-5; without a bound the error of one
// very long batch grows with its length.  Every chunk end is a read-modify-
// write of the tile's 256 KB by all workgroups at once (about 20 us per
// flush at width 2,560); the chunk ends are not staggered, because the
// workgroups of an XCD share activation panels in its L2 only while they
// stay at the same iteration (staggered ends measured 2.5% slower).
constexpr int kChain = kBigChain;

// Edge c of nch near-equal chunks of [k0, k1) (scalar).
__device__ __forceinline__ int chunk_edge(int k0, int k1, int c, int nch) {
  return __builtin_amdgcn_readfirstlane(k0 + (int)((int64_t)(k1 - k0) * c / nch));
}

// Excess pieces: workgroup w takes positions [excess_start(w), excess_start(w + 1))
// of the excess items laid end to end (part_len iterations each).
__device__ __forceinline__ int64_t excess_start(const BigParams& P, int w) {
  return (int64_t)w * P.excess_total / P.grid_sk;
}

// Row offsets through the constant address space: uniform loads of the row
// table become scalar loads, which the DMA pipeline's vector-memory count
// does not see.
typedef __attribute__((address_space(4))) const uint32_t cu32;

template <bool T8, bool Grouped, bool Idx = false>
__device__ __forceinline__ void big_body(const BigParams& P, const BigGroupParams* G) {
  __shared__ __attribute__((aligned(1024))) char st0[kStageB];
  __shared__ __attribute__((aligned(1024))) char st1[kStageB];
  __shared__ __attribute__((aligned(1024))) char st2[kStageB];
  __shared__ __attribute__((aligned(1024))) char st3[kStageB];
  __shared__ __attribute__((aligned(1024))) char st4[kStageB];

  // LDS addresses of the stages, for the load instructions' m0
  const uint32_t L0 = (uint32_t)reinterpret_cast<uintptr_t>((HESS_LDS char*)st0);
  const uint32_t L1 = (uint32_t)reinterpret_cast<uintptr_t>((HESS_LDS char*)st1);
  const uint32_t L2 = (uint32_t)reinterpret_cast<uintptr_t>((HESS_LDS char*)st2);
  const uint32_t L3 = (uint32_t)reinterpret_cast<uintptr_t>((HESS_LDS char*)st3);
  const uint32_t L4 = (uint32_t)reinterpret_cast<uintptr_t>((HESS_LDS char*)st4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const uint32_t row_bytes = (uint32_t)(P.ld * 2);

  // Operand of a 16-feature block f0..f0+15 of a panel for
  // v_mfma_f32_16x16x32_bf16: lane l holds feature f0 + l%16, tokens
  // 8 (l/16) .. +7 of the stage.
  //  * row-major stage: two transposed reads; in each, the 16 lanes of group
  //    g = l/16 read tokens 8 g + (l%16)/4 (+4 for the second read), features
  //    f0 + 4 (l%4) .. +3 (bytes 8 (l%2) of chunk (f0 + 4 (l%4)) / 8);
  //  * transposed stage: one 16-byte read of row l/16 (the l/16-th 8-token
  //    block), chunk f0 + l%16.
  const int tl = 8 * (lane >> 4) + ((lane & 15) >> 2);
  int offA[8], offB[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    offA[m] = tl * kRowB + (chunk_pos(tl, (128 * wr + 16 * m + 4 * (lane & 3)) >> 3) << 4) + 8 * (lane & 1);
    offB[m] = tl * kRowB + (chunk_pos(tl, (128 * wc + 16 * m + 4 * (lane & 3)) >> 3) << 4) + 8 * (lane & 1);
  }
  const int t8A = (lane >> 4) * 4096 + (128 * wr + (lane & 15)) * 16;
  const int t8B = (lane >> 4) * 4096 + (128 * wc + (lane & 15)) * 16;

  // one tile's iterations k0..k1-1 of the tokens at X (n of them) into S
  // slot_add: the slot already holds an earlier chunk of this piece; add to it
  // Idx: token t is X's row whose byte offset is tb[t] (a multiple of 32
  // entries per group, kOOB past the group's rows)
  auto segment = [&](int tile, int k0, int k1, int slot, bool slot_add, const void* X, int64_t n, float* S,
                     const int32_t* tb) {
    // accumulator (m, n): tile rows 128 wr + 16 m + (0..15), columns
    // 128 wc + 16 n + (0..15); lane l holds row 16 m + l%16, columns
    // 16 n + 4 (l/16) .. +3 (the column block is the instruction's first
    // operand, so each lane's four values are consecutive in a row of S)
    f32x4 acc[8][8];
    const int code = P.order[tile];
    const int I = code >> 16, J = code & 0xffff;
    const bool diag = I == J;
    // on a diagonal tile the below-diagonal quadrant's wave only loads
    const bool active = !(diag && wr == 1 && wc == 0);

    // DMA offsets: wave w loads 1-KB blocks gb = 8w + i of a stage (panel
    // gb / 16); lane j fills bytes 16j..16j+15.  Row-major X: block gb holds
    // token rows 2*(gb % 16) and +1, chunk j%32 of row t at chunk_pos(t, .).
    // Transposed staging: the panel is 4 rows (8-token blocks) of 256 16-byte
    // chunks (8 tokens of one feature); block gb holds features
    // 64*(gb % 4) .. +63 of row (gb % 16) / 4.
    uint32_t voff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int gb = kDma * wave + i;
      const int p = gb >> 4, b = gb & 15;
      if constexpr (T8) {
        const int c = b >> 2;
        const int f = (p ? J : I) * kT + 64 * (b & 3) + lane;
        voff[i] = (f < P.d && !(p && diag)) ? ((uint32_t)c * (uint32_t)P.ld + (uint32_t)f) * 16u : kOOB;
      } else if constexpr (Idx) {
        // the feature part only; the token's row offset is added per iteration
        const int t = 2 * b + (lane >> 5);
        const int f = (p ? J : I) * kT + 8 * chunk_pos(t, lane & 31);
        voff[i] = (f < P.d && !(p && diag)) ? (uint32_t)f * 2u : kOOB;
      } else {
        const int t = 2 * b + (lane >> 5);
        const int f = (p ? J : I) * kT + 8 * chunk_pos(t, lane & 31);  // chunk_pos is its own inverse
        voff[i] = (f < P.d && !(p && diag)) ? (uint32_t)t * row_bytes + (uint32_t)f * 2u : kOOB;
      }
    }
    // the iteration's tokens: rows (row-major X) or 8-token blocks of ld
    // chunks (transposed staging, n a multiple of 8)
    auto desc = [&](int j) {
      if constexpr (Idx) return rsrc_words(reinterpret_cast<uint64_t>(X), G->xbytes);
      const int64_t tok = (int64_t)j * kKI;
      const int64_t valid = j < k1 ? max((int64_t)0, min((int64_t)kKI, n - tok)) : 0;
      if constexpr (T8) {
        const uint64_t blk = (uint64_t)P.ld * 16u;
        return rsrc_words(reinterpret_cast<uint64_t>(X) + (uint64_t)(tok / 8) * blk,
                          ((valid + 7) / 8) * (int64_t)blk);
      } else {
        const uint64_t base = reinterpret_cast<uint64_t>(X) + (uint64_t)tok * row_bytes;
        return rsrc_words(base, valid * row_bytes);
      }
    };
    // load i of this wave's 8 for a stage at LDS address stage_lds, at byte
    // offsets off (per lane) of the descriptor r
    auto dma1 = [&](uint32_t stage_lds, const u32x4& r, int i, uint32_t off) {
      lds_dma16(r, off, stage_lds + (uint32_t)(wave * (kDma * 1024) + i * 1024));
    };
    // Idx: the row offsets of this wave's 16 tokens of iteration j (tokens
    // 16 (wave % 2) .. +15: load i covers tokens 2i and 2i + 1, one per half
    // wave), by scalar loads
    auto rows16 = [&](int j, uint32_t (&rw)[16]) {
      const cu32* q = (const cu32*)(tb + (int64_t)j * kKI + 16 * (wave & 1));
#pragma unroll
      for (int k = 0; k < 16; ++k) rw[k] = q[k];
    };
    // ... and the lanes' offsets for iteration j from them (past the segment:
    // every offset out of range); the saturating add keeps an out-of-range
    // part out of range
    auto offs = [&](int j, const uint32_t (&rw)[16], uint32_t (&vo)[kDma]) {
      const bool live = j < k1;
#pragma unroll
      for (int i = 0; i < kDma; ++i) {
        const uint32_t ra = live ? rw[2 * i] : kOOB, rb = live ? rw[2 * i + 1] : kOOB;
        vo[i] = __builtin_elementwise_add_sat(lane < 32 ? ra : rb, voff[i]);
      }
    };
    auto issue = [&](uint32_t stage_lds, const u32x4& r, const uint32_t (&vo)[kDma]) {
#pragma unroll
      for (int i = 0; i < kDma; ++i) dma1(stage_lds, r, i, vo[i]);
    };
    auto dma = [&](uint32_t stage_lds, int j) {
      if constexpr (Idx) {
        uint32_t rw[16], vo[kDma];
        rows16(j, rw);
        offs(j, rw, vo);
        issue(stage_lds, desc(j), vo);
      } else {
        issue(stage_lds, desc(j), voff);
      }
    };
    // operand j of a stage: A block j (j < 8, this wave's rows) or B block
    // j - 8 (its columns)
    const int t8Bd = t8B + (diag ? 0 : kPanelB);
    auto rd1 = [&](const char* stage, int j, u32x4 (&a)[8], u32x4 (&b)[8]) {
      const int m = j & 7;
      const char* pb = diag ? stage : stage + kPanelB;
      if constexpr (T8) {
        if (j < 8) a[m] = *reinterpret_cast<const u32x4*>(stage + t8A + m * 16 * 16);
        else b[m] = *reinterpret_cast<const u32x4*>(stage + t8Bd + m * 16 * 16);
      } else {
        if (j < 8) a[m] = tr_pair(stage + offA[m]);
        else b[m] = tr_pair(pb + offB[m]);
      }
    };
    // Iteration i (stage cur, operands xa, xb read during iteration i - 1):
    // wait for my loads of iteration i + 1 and meet the other waves (after
    // that barrier stage i + 1 is complete and nobody reads stage i - 1 any
    // more); then the 64 matrix instructions of stage i, with the 16 operand
    // reads of stage i + 1 (into ya, yb) and the 8 loads of iteration i + 4
    // into stage i - 1 placed among them by hand: after every 4 matrix
    // instructions one read, after every 8 one load.  A load instruction
    // waits at issue until the CU's address unit takes it; spread out this
    // way the wait holds up at most one matrix instruction.  Iterations past
    // the segment multiply the zeros their empty loads wrote.
    // Idx: rc holds the row offsets of iteration i + kDist (loaded one step
    // earlier); those of i + kDist + 1 go into rn
    auto step = [&](const char* nxt, uint32_t dtgt, int i, const u32x4 (&xa)[8], const u32x4 (&xb)[8],
                    u32x4 (&ya)[8], u32x4 (&yb)[8], const uint32_t (&rc)[16], uint32_t (&rn)[16]) {
      const u32x4 r = desc(k0 + i + kDist);
      uint32_t vo[kDma];
      if constexpr (Idx) {
        offs(k0 + i + kDist, rc, vo);
        rows16(k0 + i + kDist + 1, rn);
      } else {
#pragma unroll
        for (int q = 0; q < kDma; ++q) vo[q] = voff[q];
      }
      __builtin_amdgcn_sched_barrier(0);
      // my loads of iteration i + 1 have landed; those of i + 2 .. i + kDist - 1 stay in flight
      __builtin_amdgcn_s_waitcnt(vm_wait(kDma * (kDist - 2)));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (active) {
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int m = g >> 1, n = 4 * (g & 1);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[m][n + u] = mfma16x16x32(xb[n + u], xa[m], acc[m][n + u]);
          rd1(nxt, g, ya, yb);
          if (g & 1) dma1(dtgt, r, g >> 1, vo[g >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        issue(dtgt, r, vo);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{};

    // Idx: the row offsets of the first kDist iterations come in one vector
    // load (lane l: iteration k0 + l / 16, token 16 (wave % 2) + l % 16 of
    // it), covered by the wait below
    static_assert(kDist * 16 == 64, "one lane per row offset of the first kDist iterations");
    uint32_t pro = 0;
    if constexpr (Idx) {
      const uint32_t off = (uint32_t)((((k0 + (lane >> 4)) * kKI) + 16 * (wave & 1) + (lane & 15)) * 4);
      pro = __builtin_amdgcn_raw_buffer_load_b32(
          make_rsrc(reinterpret_cast<uint64_t>(tb), (int64_t)(k0 + kDist) * kKI * 4), off, 0, 0);
    }
    // the previous segment's output stores leave the count before these loads
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    const uint32_t Ls[5] = {L0, L1, L2, L3, L4};
    char* const St[5] = {st0, st1, st2, st3, st4};
#pragma unroll
    for (int q = 0; q < kDist; ++q) {
      if constexpr (Idx) {
        uint32_t rw[16], vo[kDma];
#pragma unroll
        for (int k = 0; k < 16; ++k) rw[k] = __builtin_amdgcn_readlane(pro, 16 * q + k);
        offs(k0 + q, rw, vo);
        issue(Ls[q], desc(k0 + q), vo);
      } else {
        dma(Ls[q], k0 + q);
      }
    }
    __builtin_amdgcn_s_waitcnt(vm_wait(kDma * (kDist - 1)));  // iteration k0 has landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 xa[8], xb[8], ya[8], yb[8];
    uint32_t ra[16], rb[16];
    if constexpr (Idx) rows16(k0 + kDist, ra);
    if (active) {
#pragma unroll
      for (int j = 0; j < 16; ++j) rd1(st0, j, xa, xb);
    }
    // ten iterations per trip: five stages, two operand register sets; the
    // exit is checked after every second iteration (an extra iteration
    // multiplies zeros)
    const int niter = k1 - k0;
    for (int i = 0;; i += 10) {
      step(St[1], Ls[kDist % 5], i, xa, xb, ya, yb, ra, rb);
      step(St[2], Ls[(1 + kDist) % 5], i + 1, ya, yb, xa, xb, rb, ra);
      if (i + 2 >= niter) break;
      step(St[3], Ls[(2 + kDist) % 5], i + 2, xa, xb, ya, yb, ra, rb);
      step(St[4], Ls[(3 + kDist) % 5], i + 3, ya, yb, xa, xb, rb, ra);
      if (i + 4 >= niter) break;
      step(St[0], Ls[(4 + kDist) % 5], i + 4, xa, xb, ya, yb, ra, rb);
      step(St[1], Ls[(5 + kDist) % 5], i + 5, ya, yb, xa, xb, rb, ra);
      if (i + 6 >= niter) break;
      step(St[2], Ls[(6 + kDist) % 5], i + 6, xa, xb, ya, yb, ra, rb);
      step(St[3], Ls[(7 + kDist) % 5], i + 7, ya, yb, xa, xb, rb, ra);
      if (i + 8 >= niter) break;
      step(St[4], Ls[(8 + kDist) % 5], i + 8, xa, xb, ya, yb, ra, rb);
      step(St[0], Ls[(9 + kDist) % 5], i + 9, ya, yb, xa, xb, rb, ra);
      if (i + 10 >= niter) break;
    }
    // drain the trailing loads; every wave is done with the stages
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (!active) return;

    // tile-local row and first column of accumulator (m, n) for this lane
    // (the lane index goes through an empty asm so that these per-lane
    // offsets are computed here, not hoisted out of the segment loop to sit
    // in registers through the main loop)
    int lv = lane;
    asm volatile("" : "+v"(lv));
    const int rr = 128 * wr + (lv & 15);
    const int cc = 128 * wc + 4 * (lv >> 4);
    if (slot >= 0) {
      float* W = P.ws + (int64_t)slot * (kT * kT);
      if (slot_add) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float4 o[8];
#pragma unroll
          for (int n = 0; n < 8; ++n) o[n] = *reinterpret_cast<const float4*>(W + (rr + 16 * m) * kT + cc + 16 * n);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const f32x4 a = acc[m][n];
            *reinterpret_cast<float4*>(W + (rr + 16 * m) * kT + cc + 16 * n) =
                float4{o[n].x + a[0], o[n].y + a[1], o[n].z + a[2], o[n].w + a[3]};
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const f32x4 a = acc[m][n];
            *reinterpret_cast<float4*>(W + (rr + 16 * m) * kT + cc + 16 * n) = float4{a[0], a[1], a[2], a[3]};
          }
      }
      return;
    }
    // whole tile: S += acc, branch-free.  Elements past d get an offset past
    // the descriptor's range: their loads read zero and their stores are
    // dropped.
    const __amdgpu_buffer_rsrc_t sr =
        make_rsrc(reinterpret_cast<uint64_t>(S) + (uint64_t)((int64_t)I * kT * P.lds * 4), (int64_t)kT * P.lds * 4);
    const int rlim = P.d - I * kT, clim = P.d - J * kT;  // tile-local row / column limits
    auto soff = [&](int m, int n) -> uint32_t {
      const int r = rr + 16 * m, c = cc + 16 * n;
      return (r < rlim && c < clim) ? (uint32_t)(((int64_t)r * P.lds + J * kT + c) * 4) : kOOB;
    };
    // 8 batches of 8 float4 (row block m); the loads of batch m + 1 are in
    // flight while batch m is added
    float4 sv[2][8];
    auto sload = [&](int m, float4 (&dst)[8]) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
        dst[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(sr, soff(m, n), 0, 0));
    };
    sload(0, sv[0]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m + 1 < 8) sload(m + 1, sv[(m + 1) & 1]);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float4 sx = sv[m & 1][n];
        const f32x4 a = acc[m][n];
        const float4 v{sx.x + a[0], sx.y + a[1], sx.z + a[2], sx.w + a[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sr, soff(m, n), 0, 0);
      }
    }
  };

  if constexpr (Grouped) {
    // Whole tiles of several Hessians (item = group * ntiles + tile); the
    // host deals them out (longest first, each to the least-loaded
    // workgroup) and lists each workgroup's items in G->sched.
    const int bid = blockIdx.x;
    const int i0 = __builtin_amdgcn_readfirstlane(G->sched[bid]);
    const int i1 = __builtin_amdgcn_readfirstlane(G->sched[bid + 1]);
    for (int ii = i0; ii < i1; ++ii) {
      const int item = __builtin_amdgcn_readfirstlane(G->sched[ii]);
      const int g = item / P.ntiles, t = item - g * P.ntiles;
      const int64_t ng = G->n[g];
      const int k1 = __builtin_amdgcn_readfirstlane((int)((ng + kKI - 1) / kKI));
      // the group's rows: its 8-token blocks in the gather buffer, or (Idx)
      // X's rows through its slice of the row table
      const char* Xg = Idx ? static_cast<const char*>(G->X)
                           : static_cast<const char*>(G->X) + G->blk[g] * (int64_t)P.ld * 16;
      const int32_t* tbg = Idx ? G->tbl + G->blk[g] : nullptr;
      // chains of at most kChain iterations, each chunk added into S
      const int nch = (k1 + kChain - 1) / kChain;
      for (int c = 0; c < nch; ++c)
        segment(__builtin_amdgcn_readfirstlane(t), chunk_edge(0, k1, c, nch), chunk_edge(0, k1, c + 1, nch), -1,
                false, Xg, ng, G->S[g], tbg);
    }
    return;
  }

  // work of this workgroup: one whole tile (the first dp_tiles tiles of the
  // order, XCD by XCD), or one aligned part of a tile plus a share of the
  // excess parts.  Items are numbered part-major (item = part * sk_tiles +
  // tile) and consecutive workgroups of an XCD take consecutive items, so an
  // XCD's workgroups read the same token range of neighbouring tiles' panels.
  // The pieces go through one loop with one call of segment, so that the
  // main loop exists once in the code.
  const int bid = blockIdx.x;
  const bool dp = bid < P.dp_tiles;
  const int b = bid - P.dp_tiles;
  const int w = dp ? 0 : (P.grid_sk % 8 == 0) ? (b & 7) * (P.grid_sk / 8) + (b >> 3) : b;
  int64_t q = 0, qend = 0;
  if (!dp && P.excess_total > 0) {
    q = excess_start(P, w);
    qend = excess_start(P, w + 1);
  }
  for (int piece = 0;; ++piece) {
    int tile, k0, k1, slot;
    if (piece == 0) {
      if (dp) {
        const int per = P.dp_tiles / 8;
        tile = (bid & 7) * per + (bid >> 3);
        k0 = 0;
        k1 = P.niter;
        slot = -1;
      } else {
        const int p = w / P.sk_tiles, t = w - p * P.sk_tiles;
        tile = P.dp_tiles + t;
        k0 = p * P.part_len;
        k1 = min(P.niter, k0 + P.part_len);
        slot = (P.parts == 1 || p == 0) ? -1 : w;
      }
    } else {
      if (q >= qend) break;
      const int e = (int)(q / P.part_len);
      const int off = (int)(q - (int64_t)e * P.part_len);
      const int len = (int)min(qend - (int64_t)e * P.part_len, (int64_t)P.part_len) - off;
      const int item = P.grid_sk + e;
      const int p = item / P.sk_tiles, t = item - p * P.sk_tiles;
      // iterations past the batch (the last part of a tile may be short)
      // read empty ranges and add zeros
      tile = P.dp_tiles + t;
      k0 = p * P.part_len + off;
      k1 = k0 + len;
      slot = P.grid_sk + w + e;
      q += len;
    }
    tile = __builtin_amdgcn_readfirstlane(tile);
    k0 = __builtin_amdgcn_readfirstlane(k0);
    k1 = __builtin_amdgcn_readfirstlane(k1);
    slot = __builtin_amdgcn_readfirstlane(slot);
    // chains of at most kChain iterations: the piece is cut into near-equal
    // chunks, each added into its destination (S, or the slot after the first)
    const int nch = (k1 - k0 + kChain - 1) / kChain;
    for (int c = 0; c < nch; ++c)
      segment(tile, chunk_edge(k0, k1, c, nch), chunk_edge(k0, k1, c + 1, nch), slot, c > 0, P.X, P.n, P.S, nullptr);
  }
}

__global__ void __launch_bounds__(256, 1) syrk_big_bf16(BigParams P) { big_body<false, false>(P, nullptr); }
__global__ void __launch_bounds__(256, 1) syrk_big_bf16_t8(BigParams P) { big_body<true, false>(P, nullptr); }

// Grouped launch on transposed staging: the tile geometry comes from P
// (order, d, nb, ntiles, ld = d, lds = d), the groups from G.
__global__ void __launch_bounds__(256, 1) syrk_big_t8_grouped(BigParams P, BigGroupParams G) {
  big_body<true, true>(P, &G);
}

// Grouped launch straight from the routed rows: group g's token t is the row
// of X at byte offset G.tbl[G.blk[g] + t] (ld = X's row stride), read into
// LDS as the row-major kernel reads a batch, so no gathered copy is made.
__global__ void __launch_bounds__(256, 1) syrk_big_rows_grouped(BigParams P, BigGroupParams G) {
  big_body<false, true, true>(P, &G);
}

// S_tile += the other parts and the pieces of tile t, in item order (pieces
// of one excess item in workgroup order): a fixed order, so results do not
// depend on scheduling.  Block (t, part) handles 1/16 of the tile: 1,024
// float4 of its 256 x 256 floats.
__global__ void __launch_bounds__(256) syrk_big_fixup(BigParams P) {
  // at most parts - 1 <= 255 main slots plus, over the tile's excess items,
  // at most grid_sk + (items of the tile) <= 512 pieces
  constexpr int kMaxSlots = 1024;
  __shared__ int slots[kMaxSlots];
  __shared__ int nslots;
  const int t = blockIdx.x;
  const int code = P.order[P.dp_tiles + t];
  const int I = code >> 16, J = code & 0xffff;
  // the tile's workspace slots, in summation order (one thread; the list is
  // the same for every element of the tile)
  if (threadIdx.x == 0) {
    int cnt = 0;
    for (int p = 0; p < P.parts; ++p) {
      const int item = p * P.sk_tiles + t;
      if (item < P.grid_sk) {
        // a main item; part 0 wrote S itself, empty parts wrote nothing
        if (p > 0 && p * P.part_len < P.niter && cnt < kMaxSlots) slots[cnt++] = item;
      } else {
        const int e = item - P.grid_sk;
        const int64_t lo = (int64_t)e * P.part_len, hi = lo + P.part_len;
        int w = (int)(lo * P.grid_sk / P.excess_total);
        while (w > 0 && excess_start(P, w) > lo) --w;
        int64_t ws = excess_start(P, w);
        for (; w < P.grid_sk && ws < hi; ++w) {
          const int64_t we = excess_start(P, w + 1);
          if (we > lo && we > ws && cnt < kMaxSlots) slots[cnt++] = P.grid_sk + w + e;
          ws = we;
        }
      }
    }
    nslots = cnt;
  }
  __syncthreads();
  const int cnt = nslots;
  if (cnt == 0) return;
  for (int k = 0; k < 4; ++k) {
    const int e4 = blockIdx.y * 1024 + k * 256 + threadIdx.x;  // float4 index in the tile
    const int r = e4 >> 6, c = (e4 & 63) * 4;
    if (I == J && r >= kT / 2 && c < kT / 2) continue;  // below the diagonal: never written
    const int gr = I * kT + r, gc = J * kT + c;
    if (gr >= P.d || gc >= P.d) continue;
    float4 a = *reinterpret_cast<const float4*>(P.ws + (int64_t)slots[0] * (kT * kT) + r * kT + c);
    for (int i = 1; i < cnt; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(P.ws + (int64_t)slots[i] * (kT * kT) + r * kT + c);
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    float4* o = reinterpret_cast<float4*>(P.S + (int64_t)gr * P.lds + gc);
    float4 sv = *o;
    sv.x += a.x;
    sv.y += a.y;
    sv.z += a.z;
    sv.w += a.w;
    *o = sv;
  }
}

}  // namespace

hipError_t launch_syrk_big(const BigParams& P, hipStream_t stream) {
  const int grid = P.dp_tiles + P.grid_sk;
  if (grid <= 0) return hipSuccess;
  if (P.t8)
    hipLaunchKernelGGL(syrk_big_bf16_t8, dim3(grid), dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL(syrk_big_bf16, dim3(grid), dim3(256), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_syrk_big_grouped(const BigParams& P, const BigGroupParams& G, hipStream_t stream) {
  if (G.nitems <= 0) return hipSuccess;
  if (G.tbl)
    hipLaunchKernelGGL(syrk_big_rows_grouped, dim3(256), dim3(256), 0, stream, P, G);
  else
    hipLaunchKernelGGL(syrk_big_t8_grouped, dim3(256), dim3(256), 0, stream, P, G);
  return hipGetLastError();
}

hipError_t launch_syrk_big_fixup(const BigParams& P, hipStream_t stream) {
  if (P.sk_tiles <= 0 || (P.parts == 1 && P.excess_total == 0)) return hipSuccess;
  hipLaunchKernelGGL(syrk_big_fixup, dim3(P.sk_tiles, 16), dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace hess
