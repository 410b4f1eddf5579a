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
//  * 4 waves, one per SIMD, each own a 128 x 128 quadrant: 16 accumulators of
//    v_mfma_f32_32x32x16_bf16 (256 registers).  The B operand goes first so
//    that each accumulator register holds part of a row (float4 output).
//  * Activations go from memory straight into LDS (buffer_load_dwordx4 with
//    the lds modifier): no registers hold loads and no VALU transposes them.
//    Row-major X: LDS keeps each 32-token stage token-major (a 512-byte row
//    of 256 features per token) with its 16-byte chunks XOR-swizzled; the
//    matrix operands (8 consecutive tokens of one feature) are read
//    transposed with ds_read_b64_tr_b16, two per operand.  The swizzle makes
//    both the 64-lane DMA writes (1 KB contiguous each) and the transposed
//    reads free of bank conflicts.  A staging buffer in the transposed
//    layout (8-token chunks of one feature, written so by the staging copy)
//    lands in LDS operand-ready: one ds_read_b128 per operand, 32 lanes
//    reading 512 contiguous bytes.
//  * The loads are written as inline asm (m0 is an input operand) and
//    placed by hand among the matrix instructions of each iteration's second
//    half.  The compiler neither tracks nor waits for them; the kernel's own
//    s_waitcnt before each barrier and before the output are the only
//    waits, which is also what the loads need.
//  * Five LDS stages of 32 tokens (5 x 32 KB, all of the CU's LDS): the
//    loads of up to four iterations are in flight while one is multiplied;
//    one barrier per iteration, placed between the two 16-token halves so
//    that the matrix cores keep running while a wave waits there and while
//    the next stage's first operands are read.  The barrier is the bare
//    s_barrier after an explicit vmcnt wait for this wave's loads of the
//    stage about to be read.
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
//
// A float32 accumulation chain here is one segment (at most the batch, and a
// staged flush is at most 13,056 tokens at width 2,560 or 8,192 at 4,096);
// each chain adds sums of 8 exact products.

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

// Logical 16-byte chunk (8 features) stored at physical chunk pc of token
// row t.  Forward: pc = c ^ 8*bit1(c) ^ 2*(t % 4).
__device__ __forceinline__ int chunk_at(int t, int pc) {
  const int q = pc ^ (2 * (t & 3));
  return q ^ (8 * ((q >> 1) & 1));
}

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

// Excess pieces: workgroup w takes positions [excess_start(w), excess_start(w + 1))
// of the excess items laid end to end (part_len iterations each).
__device__ __forceinline__ int64_t excess_start(const BigParams& P, int w) {
  return (int64_t)w * P.excess_total / P.grid_sk;
}

template <bool T8>
__device__ __forceinline__ void big_body(const BigParams& P) {
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

  // operand read offsets: lane l reads, for a 32-feature block fq of a panel,
  // token 8*(l/32) + (l%16)/4 (+4 for the second read) and features
  // 32 fq + 16*((l/16)%2) + 4*(l%4) .. +3
  const int tl = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int kl = (8 * ((lane >> 4) & 1)) ^ (2 * ((lane & 15) >> 2));
  const int el = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int bl = 8 * (lane & 1);
  int offA[4], offB[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    offA[m] = tl * kRowB + (((4 * (4 * wr + m) + el) ^ kl) << 4) + bl;
    offB[m] = tl * kRowB + (((4 * (4 * wc + m) + el) ^ kl) << 4) + bl;
  }
  // transposed staging: this lane's chunks in panels A and B (row l / 32)
  const int t8A = (lane >> 5) * 4096 + (128 * wr + (lane & 31)) * 16;
  const int t8B = (lane >> 5) * 4096 + (128 * wc + (lane & 31)) * 16;

  auto segment = [&](int tile, int k0, int k1, int slot) {
    f32x16 acc[4][4];
    const int code = P.order[tile];
    const int I = code >> 16, J = code & 0xffff;
    const bool diag = I == J;
    // on a diagonal tile the below-diagonal quadrant's wave only loads
    const bool active = !(diag && wr == 1 && wc == 0);

    // DMA offsets: wave w loads 1-KB blocks gb = 8w + i of a stage (panel
    // gb / 16); lane j fills bytes 16j..16j+15.  Row-major X: block gb holds
    // token rows 2*(gb % 16) and +1.  Transposed staging: the panel is 4
    // rows (8-token blocks) of 256 16-byte chunks (8 tokens of one feature);
    // block gb holds features 64*(gb % 4) .. +63 of row (gb % 16) / 4.
    uint32_t voff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int gb = kDma * wave + i;
      const int p = gb >> 4, b = gb & 15;
      if constexpr (T8) {
        const int c = b >> 2;
        const int f = (p ? J : I) * kT + 64 * (b & 3) + lane;
        voff[i] = (f < P.d && !(p && diag)) ? ((uint32_t)c * (uint32_t)P.ld + (uint32_t)f) * 16u : kOOB;
      } else {
        const int t = 2 * b + (lane >> 5);
        const int f = (p ? J : I) * kT + 8 * chunk_at(t, lane & 31);
        voff[i] = (f < P.d && !(p && diag)) ? (uint32_t)t * row_bytes + (uint32_t)f * 2u : kOOB;
      }
    }
    // the iteration's tokens: rows (row-major X) or 8-token blocks of ld
    // chunks (transposed staging, n a multiple of 8)
    auto desc = [&](int j) {
      const int64_t tok = (int64_t)j * kKI;
      const int64_t valid = j < k1 ? max((int64_t)0, min((int64_t)kKI, P.n - tok)) : 0;
      if constexpr (T8) {
        const uint64_t blk = (uint64_t)P.ld * 16u;
        return rsrc_words(reinterpret_cast<uint64_t>(P.X) + (uint64_t)(tok / 8) * blk,
                          ((valid + 7) / 8) * (int64_t)blk);
      } else {
        const uint64_t base = reinterpret_cast<uint64_t>(P.X) + (uint64_t)tok * row_bytes;
        return rsrc_words(base, valid * row_bytes);
      }
    };
    // load i of this wave's 8 for a stage at LDS address stage_lds
    auto dma1 = [&](uint32_t stage_lds, const u32x4& r, int i) {
      lds_dma16(r, voff[i], stage_lds + (uint32_t)(wave * (kDma * 1024) + i * 1024));
    };
    auto issue = [&](uint32_t stage_lds, const u32x4& r) {
#pragma unroll
      for (int i = 0; i < kDma; ++i) dma1(stage_lds, r, i);
    };
    auto dma = [&](uint32_t stage_lds, int j) { issue(stage_lds, desc(j)); };
    // operands of one 16-token half (ks) of a stage: A blocks of this wave's
    // rows, B blocks of its columns
    auto rd = [&](const char* stage, int ks, u32x4 (&a)[4], u32x4 (&b)[4]) {
      if constexpr (T8) {
        // one 16-byte read per operand: row 2 ks + l/32 of the panel, the
        // chunk of its feature (32 consecutive lanes read 512 contiguous bytes)
        const char* pa = stage + ks * 2 * 4096;
        const char* pb = (diag ? stage : stage + kPanelB) + ks * 2 * 4096;
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = *reinterpret_cast<const u32x4*>(pa + t8A + m * 32 * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) b[m] = *reinterpret_cast<const u32x4*>(pb + t8B + m * 32 * 16);
      } else {
        const char* pa = stage + ks * 16 * kRowB;
        const char* pb = (diag ? stage : stage + kPanelB) + ks * 16 * kRowB;
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = tr_pair(pa + offA[m]);
#pragma unroll
        for (int m = 0; m < 4; ++m) b[m] = tr_pair(pb + offB[m]);
      }
    };
    // operand j of one half: A block j (j < 4) or B block j - 4
    auto rd1 = [&](const char* stage, int ks, int j, u32x4 (&a)[4], u32x4 (&b)[4]) {
      const int m = j & 3;
      if constexpr (T8) {
        const char* pa = stage + ks * 2 * 4096;
        const char* pb = (diag ? stage : stage + kPanelB) + ks * 2 * 4096;
        if (j < 4) a[m] = *reinterpret_cast<const u32x4*>(pa + t8A + m * 32 * 16);
        else b[m] = *reinterpret_cast<const u32x4*>(pb + t8B + m * 32 * 16);
      } else {
        const char* pa = stage + ks * 16 * kRowB;
        const char* pb = (diag ? stage : stage + kPanelB) + ks * 16 * kRowB;
        if (j < 4) a[m] = tr_pair(pa + offA[m]);
        else b[m] = tr_pair(pb + offB[m]);
      }
    };
    auto mm = [&](const u32x4 (&a)[4], const u32x4 (&b)[4]) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = mfma32x32x16(b[n], a[m], acc[m][n]);
    };
    // 16 matrix instructions of one half, each followed by one of the 16
    // transposed reads of the other half's operands
    auto interleave = [&]() {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
    };
    // Iteration i (stage cur): the first half's operands (xa, xb) were read
    // during the previous iteration.  Multiply the first half while reading
    // the second; then wait for my loads of iteration i + 1 and meet the
    // other waves (after that barrier stage i + 1 is complete and nobody
    // reads stage i - 1 any more), and multiply the second half while
    // reading the first half of stage i + 1 and starting the loads of
    // iteration i + 4 into stage i - 1: after each pair of matrix
    // instructions one operand read and one load.  A load instruction waits
    // at issue until the CU's address unit takes it; spread out this way the
    // wait holds up at most one matrix instruction (issued back to back, the
    // four waves' 32 loads kept each wave from the matrix cores for ~350
    // cycles of every ~1,800).  The descriptor is built before the barrier.
    // Iterations past the segment multiply the zeros their empty loads wrote.
    u32x4 xa[4], xb[4], ya[4], yb[4];
    auto step = [&](const char* cur, const char* nxt, uint32_t dtgt, int i) {
      const u32x4 r = desc(k0 + i + 4);
      if (active) {
        rd(cur, 1, ya, yb);
        mm(xa, xb);
        interleave();
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): iterations i + 2 and i + 3 stay in flight
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (active) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int m = j >> 1, n = 2 * (j & 1);
          acc[m][n] = mfma32x32x16(yb[n], ya[m], acc[m][n]);
          acc[m][n + 1] = mfma32x32x16(yb[n + 1], ya[m], acc[m][n + 1]);
          rd1(nxt, 0, j, xa, xb);
          dma1(dtgt, r, j);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        issue(dtgt, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x16{};

    // the previous segment's output stores leave the count before these loads
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    dma(L0, k0);
    dma(L1, k0 + 1);
    dma(L2, k0 + 2);
    dma(L3, k0 + 3);
    __builtin_amdgcn_s_waitcnt(0x4F78);  // vmcnt(24): iteration k0 has landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (active) rd(st0, 0, xa, xb);
    for (int i = 0; i < k1 - k0; i += 5) {
      step(st0, st1, L4, i);
      step(st1, st2, L0, i + 1);
      step(st2, st3, L1, i + 2);
      step(st3, st4, L2, i + 3);
      step(st4, st0, L3, i + 4);
    }
    // drain the trailing (empty-range) loads; every wave is done with the stages
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (!active) return;

    // accumulator (m, n, register 4q + e) of this lane: tile row
    // 128 wr + 32 m + lane%32, column 128 wc + 32 n + 8 q + 4*(lane/32) + e
    // (the lane index goes through an empty asm so that these per-lane offsets
    // are computed here, not hoisted out of the segment loop to sit in
    // registers through the main loop)
    int lv = lane;
    asm volatile("" : "+v"(lv));
    const int rr = 128 * wr + (lv & 31);
    const int cc = 128 * wc + 4 * (lv >> 5);
    if (slot >= 0) {
      float* W = P.ws + (int64_t)slot * (kT * kT);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v{acc[m][n][4 * q], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]};
            *reinterpret_cast<float4*>(W + (rr + 32 * m) * kT + cc + 32 * n + 8 * q) = v;
          }
      return;
    }
    // whole tile: S += acc, branch-free.  Elements past d get an offset past
    // the descriptor's range: their loads read zero and their stores are
    // dropped.
    const __amdgpu_buffer_rsrc_t sr =
        make_rsrc(reinterpret_cast<uint64_t>(P.S) + (uint64_t)((int64_t)I * kT * P.lds * 4), (int64_t)kT * P.lds * 4);
    const int rlim = P.d - I * kT, clim = P.d - J * kT;  // tile-local row / column limits
    auto soff = [&](int m, int n, int q) -> uint32_t {
      const int r = rr + 32 * m, c = cc + 32 * n + 8 * q;
      return (r < rlim && c < clim) ? (uint32_t)(((int64_t)r * P.lds + J * kT + c) * 4) : kOOB;
    };
    // 8 batches of 8 float4 (row block m = k / 2, column blocks 2 (k % 2) and
    // +1); the loads of batch k + 1 are in flight while batch k is added
    float4 sv[2][8];
    auto sload = [&](int k, float4 (&dst)[8]) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        dst[u] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(sr, soff(k >> 1, 2 * (k & 1) + (u >> 2), u & 3), 0, 0));
    };
    sload(0, sv[0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k + 1 < 8) sload(k + 1, sv[(k + 1) & 1]);
      const int m = k >> 1;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int n = 2 * (k & 1) + (u >> 2), q = u & 3;
        const float4 sx = sv[k & 1][u];
        const float4 v{sx.x + acc[m][n][4 * q], sx.y + acc[m][n][4 * q + 1], sx.z + acc[m][n][4 * q + 2],
                       sx.w + acc[m][n][4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sr, soff(m, n, q), 0, 0);
      }
    }
  };

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
    if (k0 < k1) segment(tile, k0, k1, slot);
  }
}

__global__ void __launch_bounds__(256, 1) syrk_big_bf16(BigParams P) { big_body<false>(P); }
__global__ void __launch_bounds__(256, 1) syrk_big_bf16_t8(BigParams P) { big_body<true>(P); }

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

hipError_t launch_syrk_big_fixup(const BigParams& P, hipStream_t stream) {
  if (P.sk_tiles <= 0 || (P.parts == 1 && P.excess_total == 0)) return hipSuccess;
  hipLaunchKernelGGL(syrk_big_fixup, dim3(P.sk_tiles, 16), dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace hess
