// Grouped GEMM for decode-sized batches with weight-only INT8 weights.
//
// W = q * s: int8 codes q [Nout, Kdim] per group with one fp32 scale per
// output row.  q converts exactly to bf16 (|q| <= 127), the MFMAs
// (v_mfma_f32_16x16x32_bf16) accumulate x * q in fp32 and the epilogue
// multiplies by s.
//
//  * A block owns one 16-row tile and 64 output columns; each of its 4 waves
//    computes 16 of those columns.
//  * The block's 16 activation rows are staged in LDS 512 K-columns at a
//    time by DMA (buffer_load ... lds, one 1 KB row per instruction, rows
//    16 bytes apart so the fragment reads of 16 rows hit 16 distinct bank
//    groups), double-buffered.  Every wave therefore reads the activations
//    once from LDS instead of each wave loading them from L2.
//  * Each wave streams only its 16 weight rows into registers, 16 bytes per
//    lane per 64-wide K block (8 blocks per chunk), double-buffered across
//    chunks, so the next chunk's weights are in flight while the current one
//    is multiplied.
//  * K is walked in 64-wide blocks; within a block, lane part p (lane / 16)
//    takes elements [16p, 16p + 16): the first 8 feed one MFMA and the last
//    8 the next.  The same permutation of K applies to both operands, so the
//    dot product is unchanged.  The last chunk may hold fewer than 8 blocks
//    (K a multiple of 64); its DMA offsets are clamped inside the row.
#pragma once

#include "gemm_common.h"
#include "gemm_pingpong.h"  // buf_dma16
#include "gemm_skinny.h"    // i8x8_to_bf16

namespace moe {

template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_decode_q8_kernel(GemmArgs p) {
  constexpr int KC = 512;        // K columns per chunk
  constexpr int NB = KC / 64;    // 64-wide blocks per chunk
  constexpr int RB = KC * 2 + 16;  // LDS bytes per staged activation row
  __shared__ __attribute__((aligned(16))) char abuf[2][16 * RB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = p.tile_base[p.G];
  const int row = lane & 15, part = lane >> 4;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileInfo ti = resolve_tile(p, tile, 16, 64);
    const int64_t Kd = p.Kdim;
    const int nk = (int)((Kd + KC - 1) / KC);
    const uint32_t row_bytes = (uint32_t)Kd * 2;
    // wave w stages activation rows 4w .. 4w+3 of the tile
    const char* arow_ptr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int lr = ti.mt * 16 + wave * 4 + i;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) ar = ti.row0 + lr;
      else {
        const int64_t gr = ti.row0 + lr;
        ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      }
      arow_ptr[i] = (const char*)((ti.shared ? p.a_shared : p.a) + ar * p.lda);
    }
    int n = ti.nt * 64 + wave * 16 + row;
    if (n >= ti.Nout) n = ti.Nout - 1;
    const int64_t wrow = (ti.shared ? 0 : (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd + part * 16;
    const int8_t* pb0 = (const int8_t*)(ti.shared ? (const void*)p.bs0 : (const void*)p.b0) + wrow;
    const int8_t* pb1 = DUAL ? (const int8_t*)(ti.shared ? (const void*)p.bs1 : (const void*)p.b1) + wrow
                             : nullptr;

    auto issue_a = [&](int c, int buf) {
      uint32_t koff = (uint32_t)c * KC * 2 + (uint32_t)lane * 16;
      if (koff > row_bytes - 16) koff = row_bytes - 16;  // past K: a valid, unused 16 bytes
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_dma16(arow_ptr[i], koff, abuf[buf] + (wave * 4 + i) * RB);
    };
    uint4 b0[2][NB], b1[2][NB];
    auto issue_b = [&](int c, int set) {
      const int nbl = (int)((Kd - (int64_t)c * KC) / 64) < NB ? (int)((Kd - (int64_t)c * KC) / 64) : NB;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (j < nbl) {
          const int64_t off = (int64_t)c * KC + j * 64;
          b0[set][j] = *(const uint4*)(pb0 + off);
          if (DUAL) b1[set][j] = *(const uint4*)(pb1 + off);
        }
      }
    };

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c, int buf, int set) {
      const int nbl = (int)((Kd - (int64_t)c * KC) / 64) < NB ? (int)((Kd - (int64_t)c * KC) / 64) : NB;
      const char* arow_l = abuf[buf] + row * RB + part * 32;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (j < nbl) {
          const bf16x8_t fa0 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(arow_l + j * 128));
          const bf16x8_t fa1 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(arow_l + j * 128 + 16));
          const uint4 bb = b0[set][j];
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, i8x8_to_bf16(bb.x, bb.y), acc0, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, i8x8_to_bf16(bb.z, bb.w), acc0, 0, 0, 0);
          if (DUAL) {
            const uint4 cc = b1[set][j];
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, i8x8_to_bf16(cc.x, cc.y), acc1, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, i8x8_to_bf16(cc.z, cc.w), acc1, 0, 0, 0);
          }
        }
      }
    };

    issue_a(0, 0);
    issue_b(0, 0);
    for (int c = 0; c < nk; ++c) {
      const int cur = c & 1;
      wait_vmcnt<0>();   // chunk c: this wave's activation rows and weights landed
      __syncthreads();   // every wave's rows of chunk c; buffer cur ^ 1 no longer read
      if (c + 1 < nk) {
        issue_a(c + 1, cur ^ 1);
        if (cur) issue_b(c + 1, 0);
        else issue_b(c + 1, 1);
      }
      if (cur) compute(c, 1, 1);
      else compute(c, 0, 0);
    }
    __syncthreads();  // the last buffer is read before the next tile stages into it

    // D layout (16x16): col = lane % 16, row = 4 * (lane / 16) + v
    const int col = ti.nt * 64 + wave * 16 + (lane & 15);
    if (col < ti.Nout) {
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
      const int64_t si = ti.shared ? col : (int64_t)ti.g * p.Nout + col;
      const float s0 = (ti.shared ? p.scs0 : p.sc0)[si];
      const float s1 = DUAL ? (ti.shared ? p.scs1 : p.sc1)[si] : 0.f;
      float bias = 0.f;
      if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
        bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + col]);
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

}  // namespace moe
