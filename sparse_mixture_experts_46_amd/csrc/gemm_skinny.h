// Grouped GEMM, skinny kernel (decode: a few rows per expert).  One wave
// computes a 16-row x 16-column output block with v_mfma_f32_16x16x32_bf16;
// both operands come straight from global memory, 64 contiguous bytes per
// lane, so the kernel is a stream over the weights of the touched experts.
#pragma once

#include "gemm_common.h"

namespace moe {

// One wave computes a 16-row x 16-column output block.  Over a 128-wide K
// chunk, lane l (row l%16, quarter q = l/16) holds K elements
// [q*32, q*32+32) of its row in four 8-element slots; step j of the four
// MFMAs consumes slot j of A and of B, so both operands see the same K
// permutation and the product is unchanged.
template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int total = p.tile_base[p.G];
  const int row = lane & 15, q = lane >> 4;
  for (int tile = wave_g; tile < total; tile += nwaves) {
    const TileInfo ti = resolve_tile(p, tile, 16, 16);
    const int64_t Kd = p.Kdim;
    int lr = ti.mt * 16 + row;
    if (lr >= ti.M) lr = ti.M - 1;
    const uint16_t* pa;
    if (ti.shared) {
      pa = p.a_shared + (int64_t)lr * p.lda;
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
    pa += q * 32; pb0 += q * 32;
    if (DUAL) pb1 += q * 32;

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int nk = (int)(Kd / 128);
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
      uint4 a[8], b[8], c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (j >> 2) * 128 + (j & 3) * 8;
        a[j] = *(const uint4*)(pa + kc * 128 + off);
        b[j] = *(const uint4*)(pb0 + kc * 128 + off);
        if (DUAL) c[j] = *(const uint4*)(pb1 + kc * 128 + off);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[j]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, b[j]), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, c[j]), acc1, 0, 0, 0);
      }
    }
    for (; kc < nk; ++kc) {
      uint4 a[4], b[4], c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = *(const uint4*)(pa + kc * 128 + j * 8);
        b[j] = *(const uint4*)(pb0 + kc * 128 + j * 8);
        if (DUAL) c[j] = *(const uint4*)(pb1 + kc * 128 + j * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[j]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, b[j]), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, __builtin_bit_cast(bf16x8_t, c[j]), acc1, 0, 0, 0);
      }
    }
    if (Kd % 128) {  // a final 64-wide chunk: lane quarter q holds [q*16, q*16+16)
      const int64_t k0 = (int64_t)nk * 128 - q * 32 + q * 16;
      const uint16_t* qa = pa + k0;
      const uint16_t* qb = pb0 + k0;
      const uint16_t* qc = DUAL ? pb1 + k0 : nullptr;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t fa = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qa + j * 8));
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            fa, __builtin_bit_cast(bf16x8_t, *(const uint4*)(qb + j * 8)), acc0, 0, 0, 0);
        if (DUAL)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              fa, __builtin_bit_cast(bf16x8_t, *(const uint4*)(qc + j * 8)), acc1, 0, 0, 0);
      }
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


}  // namespace moe
