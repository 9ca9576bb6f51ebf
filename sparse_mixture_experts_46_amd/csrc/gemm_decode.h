// Grouped GEMM for decode-sized batches (at most 24 rows per expert on
// average), bf16 weights or weight-only INT8 weights (Q8).  The stream over
// the touched experts' weights is what bounds it (HBM).
//
// Q8: W = q * s, int8 codes q [Nout, Kdim] per group with one fp32 scale per
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
//  * Each wave streams only its 16 weight rows into registers (per lane and
//    64-wide K block: 16 bytes of int8 codes, or 32 bytes of bf16) in stages
//    of 8 blocks (int8) or 4 blocks (bf16), double-buffered, so the next
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
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs p) {
  constexpr int KC = 512;          // K columns per staged activation chunk
  constexpr int RB = KC * 2 + 16;  // LDS bytes per staged activation row
  constexpr int BPB = Q8 ? 1 : 2;  // 16-byte weight loads per lane per 64-wide block
  constexpr int SB = Q8 ? 8 : 4;   // 64-wide blocks per weight stage
  constexpr int SPC = (KC / 64) / SB;  // weight stages per activation chunk
  constexpr int ESZ = Q8 ? 1 : 2;  // weight element bytes
  __shared__ __attribute__((aligned(16))) char abuf[2][16 * RB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = p.tile_base[p.G];
  const int row = lane & 15, part = lane >> 4;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileInfo ti = resolve_tile(p, tile, 16, 64);
    const int64_t Kd = p.Kdim;
    const int nblk = (int)(Kd / 64);               // 64-wide blocks in K
    const int nstage = (nblk + SB - 1) / SB;
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
    const int64_t wrow = ((ti.shared ? 0 : (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd + part * 16) * ESZ;
    const char* pb0 = (const char*)(ti.shared ? (const void*)p.bs0 : (const void*)p.b0) + wrow;
    const char* pb1 = DUAL ? (const char*)(ti.shared ? (const void*)p.bs1 : (const void*)p.b1) + wrow
                           : nullptr;

    auto issue_a = [&](int c, int buf) {
      uint32_t koff = (uint32_t)c * KC * 2 + (uint32_t)lane * 16;
      if (koff > row_bytes - 16) koff = row_bytes - 16;  // past K: a valid, unused 16 bytes
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_dma16(arow_ptr[i], koff, abuf[buf] + (wave * 4 + i) * RB);
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

    constexpr int NA = 4;  // activation DMA instructions per wave per chunk
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
    const int col = ti.nt * 64 + wave * 16 + (lane & 15);
    if (col < ti.Nout) {
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
      float s0 = 1.f, s1 = 1.f;  // bf16 weights carry no scales
      if (Q8) {
        const int64_t si = ti.shared ? col : (int64_t)ti.g * p.Nout + col;
        s0 = (ti.shared ? p.scs0 : p.sc0)[si];
        if (DUAL) s1 = (ti.shared ? p.scs1 : p.sc1)[si];
      }
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
