// Grouped GEMM, skinny kernel (decode: a few rows per expert).  One wave
// computes a 16-row x 16-column output block with v_mfma_f32_16x16x32_bf16;
// both operands come straight from global memory, 64 contiguous bytes per
// lane, so the kernel is a stream over the weights of the touched experts.
#pragma once

#include "gemm_common.h"

namespace moe {

// One wave computes a 16-row x 16-column output block.  Lane l holds row
// l % 16 and, for each 32-wide K step, the 8 elements at offset 8 * (l / 16):
// the MFMA operand layout, which also makes the four lanes of a row read 64
// contiguous bytes per load instruction.  Loads for UNR K steps are issued
// before their MFMAs so every wave keeps many bytes in flight.
template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs p) {
  constexpr int UNR = 16;
  const int lane = threadIdx.x & 63;
  const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int total = p.tile_base[p.G];
  const int row = lane & 15, q = lane >> 4;
  for (int tile = wave_g; tile < total; tile += nwaves) {
    const TileInfo ti = resolve_tile(p, tile, 16, 16);
    const int64_t Kd = p.Kdim;
    int lr = ti.mt * 16 + row;
    // lanes of rows past the group's end load nothing (their accumulator
    // rows are never stored); their A operand is zero
    const bool arow_ok = lr < ti.M;
    if (lr >= ti.M) lr = ti.M - 1;
    const uint16_t* pa;
    if (ti.shared) {
      pa = p.a_shared + (ti.row0 + lr) * p.lda;
    } else {
      const int64_t gr = ti.row0 + lr;
      const int64_t ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      pa = p.a + ar * p.lda;
    }
    int n = ti.nt * 16 + row;
    if (n >= ti.Nout) n = ti.Nout - 1;
    const uint16_t* pb0 = (ti.shared ? p.bs0 : p.b0 + (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd;
    const uint16_t* pb1 = DUAL ? (ti.shared ? p.bs1 : p.b1 + (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd
                               : nullptr;
    pa += q * 8; pb0 += q * 8;
    if (DUAL) pb1 += q * 8;

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int nk32 = (int)(Kd / 32);  // MFMA K steps
    int kc = 0;
    for (; kc + UNR <= nk32; kc += UNR) {
      uint4 a[UNR], b[UNR], c[UNR];
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int off = (kc + j) * 32;
        a[j] = arow_ok ? *(const uint4*)(pa + off) : make_uint4(0, 0, 0, 0);
        b[j] = *(const uint4*)(pb0 + off);
        if (DUAL) c[j] = *(const uint4*)(pb1 + off);
      }
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[j]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, b[j]), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, c[j]), acc1, 0, 0, 0);
      }
    }
    for (; kc < nk32; ++kc) {
      const int off = kc * 32;
      bf16x8_t fa = __builtin_bit_cast(bf16x8_t, arow_ok ? *(const uint4*)(pa + off) : make_uint4(0, 0, 0, 0));
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          fa, __builtin_bit_cast(bf16x8_t, *(const uint4*)(pb0 + off)), acc0, 0, 0, 0);
      if (DUAL)
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            fa, __builtin_bit_cast(bf16x8_t, *(const uint4*)(pb1 + off)), acc1, 0, 0, 0);
    }
    // D layout (16x16): col = lane % 16, row = 4*(lane/16) + v
    const int col = ti.nt * 16 + (lane & 15);
    if (col < ti.Nout) {
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
      float bias = 0.f;
      if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
        bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + col]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = ti.mt * 16 + 4 * q + v;
        if (r < ti.M) {
          float o = DUAL ? silu_f(acc0[v]) * acc1[v] : epi1<EPI>(acc0[v], bias);
          cbase[(ti.row0 + r) * (int64_t)ti.Nout + col] = f32_to_bf16(o);
        }
      }
    }
  }
}


// Weight-only INT8 variant: the weights are int8 codes q with one fp32 scale
// per output row, W = q * s.  q converts exactly to bf16 (|q| <= 127), the
// MFMAs accumulate x * q in fp32 and the epilogue multiplies by s.  Loads go
// by 64-wide K blocks: lane (row, part) reads the 16 codes at K offset
// 16 * part of the block (16 bytes) and the 16 matching activations (32
// bytes); the first 8 of each feed one MFMA and the last 8 the next.  That
// is a fixed permutation of K applied to both operands, so the dot product
// is unchanged.
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

// One 64-wide K block: two MFMAs per weight matrix (codes 0-7 with the first
// 8 activations, codes 8-15 with the next 8).
template <bool DUAL>
__device__ __forceinline__ void q8_block(uint4 a0, uint4 a1, uint4 b, uint4 c, f32x4_t& acc0,
                                         f32x4_t& acc1) {
  const bf16x8_t fa0 = __builtin_bit_cast(bf16x8_t, a0), fa1 = __builtin_bit_cast(bf16x8_t, a1);
  acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, i8x8_to_bf16(b.x, b.y), acc0, 0, 0, 0);
  acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, i8x8_to_bf16(b.z, b.w), acc0, 0, 0, 0);
  if (DUAL) {
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, i8x8_to_bf16(c.x, c.y), acc1, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, i8x8_to_bf16(c.z, c.w), acc1, 0, 0, 0);
  }
}

template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_q8_kernel(GemmArgs p) {
  constexpr int UNR = 8;  // 64-wide K blocks per batch of loads
  const int lane = threadIdx.x & 63;
  const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int total = p.tile_base[p.G];
  const int row = lane & 15, q = lane >> 4;
  for (int tile = wave_g; tile < total; tile += nwaves) {
    const TileInfo ti = resolve_tile(p, tile, 16, 16);
    const int64_t Kd = p.Kdim;
    int lr = ti.mt * 16 + row;
    const bool arow_ok = lr < ti.M;
    if (lr >= ti.M) lr = ti.M - 1;
    const uint16_t* pa;
    if (ti.shared) {
      pa = p.a_shared + (ti.row0 + lr) * p.lda;
    } else {
      const int64_t gr = ti.row0 + lr;
      const int64_t ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      pa = p.a + ar * p.lda;
    }
    int n = ti.nt * 16 + row;
    if (n >= ti.Nout) n = ti.Nout - 1;
    const int8_t* pb0 = (const int8_t*)(ti.shared ? (const void*)p.bs0 : (const void*)p.b0) +
                        (ti.shared ? 0 : (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd;
    const int8_t* pb1 = DUAL ? (const int8_t*)(ti.shared ? (const void*)p.bs1 : (const void*)p.b1) +
                                   (ti.shared ? 0 : (int64_t)ti.g * p.b_stride) + (int64_t)n * Kd
                             : nullptr;
    pa += q * 16;
    pb0 += q * 16;
    if (DUAL) pb1 += q * 16;

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int nb = (int)(Kd / 64);
    int kb = 0;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    for (; kb + UNR <= nb; kb += UNR) {
      uint4 a0[UNR], a1[UNR], b[UNR], c[UNR];
#pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int off = (kb + j) * 64;
        a0[j] = arow_ok ? *(const uint4*)(pa + off) : zero;
        a1[j] = arow_ok ? *(const uint4*)(pa + off + 8) : zero;
        b[j] = *(const uint4*)(pb0 + off);
        c[j] = DUAL ? *(const uint4*)(pb1 + off) : zero;
      }
#pragma unroll
      for (int j = 0; j < UNR; ++j) q8_block<DUAL>(a0[j], a1[j], b[j], c[j], acc0, acc1);
    }
    for (; kb < nb; ++kb) {
      const int off = kb * 64;
      const uint4 a0 = arow_ok ? *(const uint4*)(pa + off) : zero;
      const uint4 a1 = arow_ok ? *(const uint4*)(pa + off + 8) : zero;
      const uint4 b = *(const uint4*)(pb0 + off);
      const uint4 c = DUAL ? *(const uint4*)(pb1 + off) : zero;
      q8_block<DUAL>(a0, a1, b, c, acc0, acc1);
    }
    // D layout (16x16): col = lane % 16, row = 4*(lane/16) + v
    const int col = ti.nt * 16 + (lane & 15);
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
        const int r = ti.mt * 16 + 4 * q + v;
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
