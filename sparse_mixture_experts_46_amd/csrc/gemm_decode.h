// Grouped GEMM for decode-sized batches (at most 24 rows per expert on
// average), bf16 weights or weight-only INT8 weights (Q8).  The stream over
// the touched experts' weights is what bounds it (HBM).
//
// Q8: W = q * s, int8 codes q [Nout, Kdim] per group with one fp32 scale per
// output row.  q converts exactly to bf16 (|q| <= 127), the MFMAs
// (v_mfma_f32_16x16x32_bf16) accumulate x * q in fp32 and the epilogue
// multiplies by s.
//
//  * A block owns one 16-row tile and 16 kDecodeWaves output columns; each
//    of its waves computes 16 of those columns.
//  * The block's 16 activation rows are staged in LDS 512 K-columns at a
//    time by DMA (buffer_load ... lds, one 1 KB row per instruction, rows
//    16 bytes apart so the fragment reads of 16 rows hit 16 distinct bank
//    groups), double-buffered.  Every wave therefore reads the activations
//    once from LDS instead of each wave loading them from L2.
//  * Each wave streams only its 16 weight rows into registers (per lane and
//    64-wide K block: 16 bytes of int8 codes, or 32 bytes of bf16) in stages
//    of 4 blocks (8 for INT8 with one weight matrix), double-buffered, so the next
//    stage's weights are in flight while the current one is multiplied.
//    Each stage's weights are issued before the next activation chunk, so
//    waiting for them does not wait for that chunk.
//  * K is walked in 64-wide blocks; within a block, lane part p (lane / 16)
//    takes elements [16p, 16p + 16): the first 8 feed one MFMA and the last
//    8 the next.  The same permutation of K applies to both operands, so the
//    dot product is unchanged.  The last chunk may hold fewer than 8 blocks
//    (K a multiple of 64); its DMA offsets are clamped inside the row.
#pragma once

#include "gemm_common.h"
#include "gemm_pingpong.h"  // buf_dma16

namespace moe {

// Waves per decode workgroup; a tile is 16 rows x 16 kDecodeWaves columns.
constexpr int kDecodeWaves = 4;

// Tile order.  With at most one tile per workgroup (a grid that is a multiple
// of 8 and larger than the table) each XCD takes a contiguous eighth of the
// table, so the weight rows one XCD streams are neighbours.  Measured with 8
// experts, d = 4096, F = 14336 and 16 tokens (1792 tiles in the first GEMM):
// 0.320 ms on every run, against 0.32-0.37 ms in dispatch order.  With several
// tiles per workgroup the dispatch order (tile = block, then += grid) measured
// as fast or faster.
__device__ __forceinline__ TileWalk decode_walk(int total) {
  if ((gridDim.x & 7) == 0 && total < (int)gridDim.x) return tile_walk(total);
  TileWalk w;
  w.tile = blockIdx.x;
  w.step = gridDim.x;
  w.end = total;
  return w;
}

// int8 codes (|q| <= 127) to bf16, exactly: 8 codes packed in two words.
__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = i < 4 ? lo : hi;
    const int v = (int)(int8_t)((w >> (8 * (i & 3))) & 0xffu);
    // exact: an integer of magnitude <= 128 has at most 8 significant bits
    r[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint((float)v) >> 16));
  }
  return r;
}

template <bool DUAL, int EPI, bool Q8>
__global__ __launch_bounds__(64 * kDecodeWaves, DUAL ? 8 / kDecodeWaves : 16 / kDecodeWaves) void gemm_decode_kernel(GemmArgs p) {
  constexpr int NWV = kDecodeWaves, RPW = 16 / NWV, BNC = 16 * NWV;
  constexpr int KC = 512;          // K columns per staged activation chunk
  constexpr int RB = KC * 2 + 16;  // LDS bytes per staged activation row
  constexpr int BPB = Q8 ? 1 : 2;  // 16-byte weight loads per lane per 64-wide block
  // 64-wide blocks per weight stage: INT8 with one weight matrix takes 8,
  // with two (gate and up) 4 (measured: 8-block stages held the dual INT8
  // kernel to one sync-and-wait per activation chunk, 1.58 ms against 1.44
  // on the DeepSeek-shaped decode; the single-matrix kernel is 3 % faster
  // with 8)
  constexpr int SB = (Q8 && !DUAL) ? 8 : 4;
  constexpr int SPC = (KC / 64) / SB;  // weight stages per activation chunk
  constexpr int ESZ = Q8 ? 1 : 2;  // weight element bytes
  __shared__ __attribute__((aligned(16))) char abuf[2][16 * RB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = p.tile_base[p.G];
  const int row = lane & 15, part = lane >> 4;
  for (TileWalk tw = decode_walk(total); tw.tile < tw.end; tw.tile += tw.step) {
    const int tile = tw.tile;
    const TileInfo ti = resolve_tile(p, tile, 16, BNC);
    const int64_t Kd = p.Kdim;
    const int nblk = (int)(Kd / 64);               // 64-wide blocks in K
    const int nstage = (nblk + SB - 1) / SB;
    const uint32_t row_bytes = (uint32_t)Kd * 2;
    // wave w stages activation rows RPW w .. RPW w + RPW - 1 of the tile
    const char* arow_ptr[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      int lr = ti.mt * 16 + wave * RPW + i;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) ar = ti.row0 + lr;
      else {
        const int64_t gr = ti.row0 + lr;
        ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      }
      arow_ptr[i] = (const char*)((ti.shared ? p.a_shared : p.a) + ar * p.lda);
    }
    int n = ti.nt * BNC + wave * 16 + row;
    if (n >= ti.Nout) n = ti.Nout - 1;
    const int64_t wrow = ((ti.shared ? 0 : (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd + part * 16) * ESZ;
    const char* pb0 = (const char*)(ti.shared ? (const void*)p.bs0 : (const void*)p.b0) + wrow;
    const char* pb1 = DUAL ? (const char*)(ti.shared ? (const void*)p.bs1 : (const void*)p.b1) + wrow
                           : nullptr;
    // the INT8 scales and the bias of the lane's output column n (clamped:
    // the epilogue skips columns past Nout), loaded before the K loop so that
    // their latency hides under it
    float s0 = 1.f, s1 = 1.f, bias = 0.f;  // bf16 weights carry no scales
    if (Q8) {
      const int64_t si = ti.shared ? n : (int64_t)ti.g * p.Nout + n;
      s0 = (ti.shared ? p.scs0 : p.sc0)[si];
      if (DUAL) s1 = (ti.shared ? p.scs1 : p.sc1)[si];
    }
    if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
      bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + n]);

    auto issue_a = [&](int c, int buf) {
      uint32_t koff = (uint32_t)c * KC * 2 + (uint32_t)lane * 16;
      if (koff > row_bytes - 16) koff = row_bytes - 16;  // past K: a valid, unused 16 bytes
#pragma unroll
      for (int i = 0; i < RPW; ++i) buf_dma16(arow_ptr[i], koff, abuf[buf] + (wave * RPW + i) * RB);
    };
    uint4 b0[2][SB * BPB], b1[2][SB * BPB];
    auto issue_b = [&](int st, int set) {
      const int left = nblk - st * SB;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        if (j < left) {
#pragma unroll
          for (int u = 0; u < BPB; ++u) {
            const int64_t off = ((int64_t)(st * SB + j) * 64) * ESZ + u * 16;
            b0[set][j * BPB + u] = *(const uint4*)(pb0 + off);
            if (DUAL) b1[set][j * BPB + u] = *(const uint4*)(pb1 + off);
          }
        }
      }
    };

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int st, int buf, int set) {
      const int left = nblk - st * SB;
      const char* arow_l = abuf[buf] + row * RB + part * 32 + ((st % SPC) * SB) * 128;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        if (j < left) {
          const bf16x8_t fa0 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(arow_l + j * 128));
          const bf16x8_t fa1 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(arow_l + j * 128 + 16));
          bf16x8_t w0a, w0b, w1a, w1b;
          if (Q8) {
            const uint4 bb = b0[set][j];
            w0a = i8x8_to_bf16(bb.x, bb.y);
            w0b = i8x8_to_bf16(bb.z, bb.w);
            if (DUAL) {
              const uint4 cc = b1[set][j];
              w1a = i8x8_to_bf16(cc.x, cc.y);
              w1b = i8x8_to_bf16(cc.z, cc.w);
            }
          } else {
            w0a = __builtin_bit_cast(bf16x8_t, b0[set][2 * j]);
            w0b = __builtin_bit_cast(bf16x8_t, b0[set][2 * j + 1]);
            if (DUAL) {
              w1a = __builtin_bit_cast(bf16x8_t, b1[set][2 * j]);
              w1b = __builtin_bit_cast(bf16x8_t, b1[set][2 * j + 1]);
            }
          }
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, w0a, acc0, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, w0b, acc0, 0, 0, 0);
          if (DUAL) {
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, w1a, acc1, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, w1b, acc1, 0, 0, 0);
          }
        }
      }
    };

    constexpr int NA = RPW;  // activation DMA instructions per wave per chunk
    issue_a(0, 0);
    issue_b(0, 0);
    for (int st = 0; st < nstage; ++st) {
      const int c = st / SPC;
      const bool first = (st % SPC) == 0;
      // weights of stage st landed (and, at a chunk's first stage, its
      // activations: issued before stage st's weights); a later chunk's
      // activations may still be in flight
      if (first) wait_vmcnt<0>();
      else wait_vmcnt<NA>();
      if (first) __syncthreads();  // every wave's rows of chunk c; buffer (c+1)&1 free
      if (st + 1 < nstage) {
        if (st & 1) issue_b(st + 1, 0);
        else issue_b(st + 1, 1);
      }
      if (first && c + 1 < (nstage + SPC - 1) / SPC) issue_a(c + 1, (c + 1) & 1);
      if (st & 1) compute(st, c & 1, 1);
      else compute(st, c & 1, 0);
    }
    __syncthreads();  // the last buffer is read before the next tile stages into it

    // D layout (16x16): col = lane % 16, row = 4 * (lane / 16) + v
    const int col = ti.nt * BNC + wave * 16 + (lane & 15);
    if (col < ti.Nout) {
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ti.mt * 16 + 4 * part + v;
        if (r < ti.M) {
          const float o = DUAL ? silu_f(acc0[v] * s0) * (acc1[v] * s1)
                               : epi1<EPI>(acc0[v] * s0, bias);
          cbase[(ti.row0 + r) * (int64_t)ti.Nout + col] = f32_to_bf16(o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- INT4 --
// Weight-only INT4 (Q4): W = q * s with q in [-7, 7] stored as u = q + 8
// nibbles ([Nout, Kdim / 2] bytes per group of the grouped GEMM; the word
// layout of quant.hip) and one fp32 scale per 128 consecutive K of a row
// ([Nout, Kdim / 128]).  The tile, the activation staging and the weight
// double buffering are those of gemm_decode_kernel; K is walked in 128-wide
// groups, one scale each:
//  * lane part p (lane / 16) takes K [32p, 32p + 32) of a group: its 16-byte
//    load holds the 32 codes, four words of 8; word m feeds MFMA m with the
//    activations of K [32p + 8m, 32p + 8m + 8) (the same permutation of K on
//    both operands);
//  * ((word >> 4i) & 0x000F000F) | 0x43004300 is the bf16 pair (128 + u, 128
//    + u') of two codes, so a word becomes a bf16 fragment of w' = q + 136 in
//    7 integer instructions (3 shifts and 4 v_and_or_b32);
//  * per group the MFMAs give sum x w' and, against a fragment of ones,
//    S = sum x; the group adds s * (sum x w' - 136 S) = s * sum x q to the
//    fp32 output (every product is exact, the sums are fp32);
//  * a stage's codes are half the bytes of an INT8 stage over the same K, so
//    the codes are fetched two stages ahead (three register sets) to keep
//    as many bytes in flight, and the stage's scales as far ahead, by LDS
//    DMA into three per-wave LDS sets (one 4-byte DMA per lane and matrix);
//    every stage issues the same loads (indices clamped inside the row),
//    which keeps the wait counts exact.
// magic = 0x43004300 in a register the compiler cannot fold: (x & mask) |
// magic then selects one v_and_or_b32 with the mask in an SGPR (a gfx9 VOP3
// instruction takes at most one SGPR or literal, so with both constants
// literal it is split into v_and_b32 and v_or_b32).
__device__ __forceinline__ uint32_t q4_magic() {
  uint32_t m;
  asm("v_mov_b32 %0, 0x43004300" : "=v"(m));
  return m;
}
__device__ __forceinline__ bf16x8_t q4_word_to_bf16(uint32_t w, uint32_t magic) {
  uint4 r;
  r.x = (w & 0x000F000Fu) | magic;
  r.y = ((w >> 4) & 0x000F000Fu) | magic;
  r.z = ((w >> 8) & 0x000F000Fu) | magic;
  r.w = ((w >> 12) & 0x000F000Fu) | magic;
  return __builtin_bit_cast(bf16x8_t, r);
}

template <bool DUAL, int EPI>
__global__ __launch_bounds__(64 * kDecodeWaves, 8 / kDecodeWaves) void gemm_decode_q4_kernel(GemmArgs p) {
  constexpr int NWV = kDecodeWaves, RPW = 16 / NWV, BNC = 16 * NWV;
  constexpr int KC = 512;          // K columns per staged activation chunk
  constexpr int RB = KC * 2 + 16;  // LDS bytes per staged activation row
  constexpr int SG = KC / 128;     // 128-wide groups per weight stage (one stage per chunk)
  static_assert(SG == 4, "a stage's scales of 16 rows are one 4-byte DMA per lane");
  __shared__ __attribute__((aligned(16))) char abuf[2][16 * RB];
  // per wave, three stages of scales: [stage set][matrix][16 rows][SG groups]
  __shared__ __attribute__((aligned(16))) float sbuf[NWV][3][DUAL ? 2 : 1][16 * SG];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = p.tile_base[p.G];
  const int row = lane & 15, part = lane >> 4;
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                0x3F803F80u, 0x3F803F80u));
  const uint32_t magic = q4_magic();
  for (TileWalk tw = decode_walk(total); tw.tile < tw.end; tw.tile += tw.step) {
    const int tile = tw.tile;
    const TileInfo ti = resolve_tile(p, tile, 16, BNC);
    const int64_t Kd = p.Kdim;
    const int ngrp = (int)(Kd / 128);
    const int nstage = (ngrp + SG - 1) / SG;
    const uint32_t row_bytes = (uint32_t)Kd * 2;
    const char* arow_ptr[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      int lr = ti.mt * 16 + wave * RPW + i;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) ar = ti.row0 + lr;
      else {
        const int64_t gr = ti.row0 + lr;
        ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      }
      arow_ptr[i] = (const char*)((ti.shared ? p.a_shared : p.a) + ar * p.lda);
    }
    int n = ti.nt * BNC + wave * 16 + row;
    if (n >= ti.Nout) n = ti.Nout - 1;
    // codes: b_stride weights per routed group, two per byte
    const int64_t wrow = ((ti.shared ? 0 : (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd) / 2 +
                         part * 16;
    const char* pb0 = (const char*)(ti.shared ? (const void*)p.bs0 : (const void*)p.b0) + wrow;
    const char* pb1 = DUAL ? (const char*)(ti.shared ? (const void*)p.bs1 : (const void*)p.b1) + wrow
                           : nullptr;
    // the bias of the lane's output column n, loaded before the K loop
    float bias = 0.f;
    if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
      bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + n]);
    // scales: lane l fetches group l % 4 of a stage for row l / 4 of the
    // wave's 16 output rows
    int nd = ti.nt * BNC + wave * 16 + (lane >> 2);
    if (nd >= ti.Nout) nd = ti.Nout - 1;
    const int64_t srow = (ti.shared ? 0 : (int64_t)ti.g * p.Nout * ngrp) + (int64_t)nd * ngrp;
    const float* ps0 = (ti.shared ? p.scs0 : p.sc0) + srow;
    const float* ps1 = DUAL ? (ti.shared ? p.scs1 : p.sc1) + srow : nullptr;

    auto issue_a = [&](int c, int buf) {
      uint32_t koff = (uint32_t)c * KC * 2 + (uint32_t)lane * 16;
      if (koff > row_bytes - 16) koff = row_bytes - 16;  // past K: a valid, unused 16 bytes
#pragma unroll
      for (int i = 0; i < RPW; ++i) buf_dma16(arow_ptr[i], koff, abuf[buf] + (wave * RPW + i) * RB);
    };
    // codes two stages ahead (three register sets), scales as far ahead (three
    // LDS sets of the wave), the activation chunk one stage ahead (two LDS
    // buffers).  Scales come from HBM like the codes: fetched one stage ahead
    // into registers, their latency showed (d = 7168, 256 experts, 128 tokens:
    // first GEMM 1.21 ms, 0.88 ms with no scale loads at all).
    uint4 b0[3][SG], b1[3][SG];
    // vector loads of one stage's codes (both matrices) and of its scales
    constexpr int NBV = SG * (DUAL ? 2 : 1);
    constexpr int NS = DUAL ? 2 : 1;
    auto issue_b = [&](int st, int set) {
#pragma unroll
      for (int j = 0; j < SG; ++j) {
        // past the row: a valid group again, loaded and not used
        const int g = st * SG + j < ngrp ? st * SG + j : ngrp - 1;
        b0[set][j] = *(const uint4*)(pb0 + (int64_t)g * 64);
        if (DUAL) b1[set][j] = *(const uint4*)(pb1 + (int64_t)g * 64);
      }
    };
    auto issue_s = [&](int st, int set) {
      int g = st * SG + (lane & 3);
      if (g >= ngrp) g = ngrp - 1;  // past the row: loaded and not used
      lds_dma4(ps0 + g, &sbuf[wave][set][0][0]);
      if (DUAL) lds_dma4(ps1 + g, &sbuf[wave][set][DUAL ? 1 : 0][0]);
    };

    f32x4_t out0 = {0.f, 0.f, 0.f, 0.f}, out1 = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int st, int buf, int set) {
      const int left = ngrp - st * SG;
      const char* arow_l = abuf[buf] + row * RB + part * 64;
#pragma unroll
      for (int j = 0; j < SG; ++j) {
        if (j < left) {
          const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
          f32x4_t a0 = zero, a1 = zero, sx = zero;
          const float sc0 = sbuf[wave][set][0][row * SG + j];
          const float sc1 = DUAL ? sbuf[wave][set][DUAL ? 1 : 0][row * SG + j] : 0.f;
          const uint4 c0 = b0[set][j];
          const uint4 c1 = DUAL ? b1[set][j] : c0;
          const uint32_t w0[4] = {c0.x, c0.y, c0.z, c0.w};
          const uint32_t w1[4] = {c1.x, c1.y, c1.z, c1.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, *(const uint4*)(arow_l + j * 256 + m * 16));
            a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, q4_word_to_bf16(w0[m], magic), a0, 0, 0, 0);
            if (DUAL) a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, q4_word_to_bf16(w1[m], magic), a1, 0, 0, 0);
            sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, ones, sx, 0, 0, 0);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            out0[v] += sc0 * (a0[v] - 136.f * sx[v]);
            if (DUAL) out1[v] += sc1 * (a1[v] - 136.f * sx[v]);
          }
        }
      }
    };

    // Issue order: a(0), s(0), c(0), s(1), c(1), then per stage st: a(st+1),
    // s(st+2), c(st+2) (a: activation chunk, s: scales, c: codes), so at the
    // top of stage st only s(st+1) and c(st+1) may still be in flight.  Every
    // stage issues the same loads (indices clamped inside the row), which
    // keeps the wait counts exact.
    {
      issue_a(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      issue_s(0, 0);
      issue_b(0, 0);
      if (nstage > 1) {
        issue_s(1, 1);
        issue_b(1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      for (int st = 0; st < nstage; ++st) {
        if (st + 1 < nstage) wait_vmcnt<NS + NBV>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wave's rows of chunk st; buffer (st+1)&1 free
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < nstage) issue_a(st + 1, (st + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 2 < nstage) {
          const int set2 = (st + 2) % 3;
          if (set2 == 0) {
            issue_s(st + 2, 0);
            issue_b(st + 2, 0);
          } else if (set2 == 1) {
            issue_s(st + 2, 1);
            issue_b(st + 2, 1);
          } else {
            issue_s(st + 2, 2);
            issue_b(st + 2, 2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (a copy of the stage without the per-group tests, for full stages,
        // measured slower: the second GEMM's kernel lost a wave per SIMD)
        const int set = st % 3;
        if (set == 0) compute(st, st & 1, 0);
        else if (set == 1) compute(st, st & 1, 1);
        else compute(st, st & 1, 2);
      }
    }
    __syncthreads();  // the last buffer is read before the next tile stages into it

    // D layout (16x16): col = lane % 16, row = 4 * (lane / 16) + v
    const int col = ti.nt * BNC + wave * 16 + (lane & 15);
    if (col < ti.Nout) {
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ti.mt * 16 + 4 * part + v;
        if (r < ti.M) {
          const float o = DUAL ? silu_f(out0[v]) * out1[v] : epi1<EPI>(out0[v], bias);
          cbase[(ti.row0 + r) * (int64_t)ti.Nout + col] = f32_to_bf16(o);
        }
      }
    }
  }
}

}  // namespace moe
