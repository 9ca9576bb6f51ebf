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

}  // namespace moe
