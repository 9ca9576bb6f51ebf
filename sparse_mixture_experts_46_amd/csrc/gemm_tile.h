// Grouped GEMM, tile kernel (prefill): C = A B^T per expert group on the
// gfx950 matrix cores, bf16 operands, fp32 accumulation.
//
//  * Persistent: one workgroup per CU walks the device-side tile table in a
//    fixed order; each XCD walks its own contiguous range of tiles (same
//    expert, neighbouring column tiles) that shares its L2.
//  * A BK-wide K slice of every A and B row of the tile goes straight from
//    global memory into LDS (global_load_lds_dwordx4, 16 bytes per lane, no
//    staging registers).  One wave instruction fills 1 KB of LDS: rows of
//    2*BK bytes, lane l -> row l / CH, physical chunk l % CH (CH = BK/8
//    chunks of 16 bytes).  The lane therefore fetches logical chunk
//    pc ^ swz(row), the XOR swizzle that spreads the fragment reads over the
//    LDS banks.
//  * STAGES-deep ring of LDS stages; loads for stage kt+STAGES-1 are issued
//    before computing stage kt, and one barrier per stage publishes it.
//  * v_mfma_f32_32x32x16_bf16 with the WEIGHT fragment as the first operand,
//    so the accumulator's row index runs along output columns: each lane
//    ends up with runs of 4 consecutive columns and stores 8 bytes at a time.
//  * SwiGLU (DUAL): the B tile holds BN/2 gate rows and the same BN/2 up
//    rows; silu(gate) * up is formed in registers.
#pragma once

#include "gemm_common.h"
#include "lds_dma.h"

namespace moe {

template <int CH, int SWZ>
__device__ __forceinline__ int swz(int row) {
  return (row >> SWZ) & (CH - 1);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int SWZ, bool DUAL, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_tile_kernel(GemmArgs p) {
  constexpr int NW = WM * WN;
  constexpr int CH = BK / 8;             // 16-byte chunks per staged row
  constexpr int RB = BK * 2;             // bytes per staged row
  constexpr int RPI = 1024 / RB;         // rows one wave instruction fills
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int BNo = DUAL ? BN / 2 : BN;  // output columns per tile
  constexpr int LA = BM / (NW * RPI), LB = BN / (NW * RPI);
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * RB;       // bytes per stage
  static_assert(BK == 32 || BK == 64 || BK == 128, "BK");
  static_assert(BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "tile/wave mismatch");
  static_assert(!DUAL || (FN % 2 == 0), "dual tile needs an even fragment count");
  static_assert(STAGES >= 2, "stages");
  extern __shared__ uint4 smem[];
  char* sbase = (char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int total = p.tile_base[p.G];
  const TileWalk walk = tile_walk(total);
  const int lrow = lane / CH, pch = lane % CH;

  // LDS rows (within a stage) whose fragments this lane reads
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * TM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int r;
    if (DUAL) {
      constexpr int FH = FN / 2;
      r = (j < FH) ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FH) * 32;
    } else {
      r = wn * TN + j * 32;
    }
    brow[j] = BM + r + (lane & 31);
  }
  const int khalf = lane >> 5;

  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    const TileInfo ti = resolve_tile(p, tile, BM, BNo);
    const int64_t Kd = p.Kdim;
    // ---- this lane's DMA sources: uniform base + per-lane byte offset
    const char* abase = (const char*)(ti.shared ? p.a_shared : p.a);
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (i * NW + wave) * RPI + lrow;
      int lr = ti.mt * BM + r;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) {
        ar = ti.row0 + lr;
      } else {
        const int64_t gr = ti.row0 + lr;
        ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      }
      aoff[i] = (uint32_t)((ar * p.lda + (pch ^ swz<CH, SWZ>(r)) * 8) * 2);
    }
    const char* bbase0 = (const char*)(ti.shared ? p.bs0 : p.b0 + (int64_t)ti.g * p.b_stride);
    const char* bbase1 = DUAL ? (const char*)(ti.shared ? p.bs1 : p.b1 + (int64_t)ti.g * p.b_stride)
                              : bbase0;
    uint32_t boff[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (i * NW + wave) * RPI + lrow;
      int n = ti.nt * BNo + ((DUAL && r >= BN / 2) ? r - BN / 2 : r);
      if (n >= ti.Nout) n = ti.Nout - 1;
      boff[i] = (uint32_t)(((int64_t)n * Kd + (pch ^ swz<CH, SWZ>(BM + r)) * 8) * 2);
    }

#define MOE_TILE_ISSUE(K0, BUF)                                                     \
    do {                                                                            \
      char* st_ = sbase + (BUF) * STAGE;                                            \
      const uint32_t kb_ = (uint32_t)(K0) * 2;                                      \
      _Pragma("unroll") for (int i = 0; i < LA; ++i)                                \
        lds_dma16(abase + aoff[i] + kb_, st_ + (i * NW + wave) * RPI * RB);         \
      _Pragma("unroll") for (int i = 0; i < LB; ++i) {                              \
        const int r_ = (i * NW + wave) * RPI;                                       \
        const char* bb_ = (DUAL && r_ >= BN / 2) ? bbase1 : bbase0;                 \
        lds_dma16(bb_ + boff[i] + kb_, st_ + (BM + r_) * RB);                       \
      }                                                                             \
    } while (0)

    f32x16_t acc[FN][FM];  // [weight fragment][token fragment]
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

    const int nk = (int)(Kd / BK);
    // prologue: stages 0 .. STAGES-2
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) MOE_TILE_ISSUE(s * BK, s);
    if (nk >= STAGES - 1) wait_vmcnt<(STAGES - 2) * (LA + LB)>();
    else wait_vmcnt<0>();
    __syncthreads();
    int buf = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const int pre = kt + STAGES - 1;
      int pbuf = buf + STAGES - 1;
      if (pbuf >= STAGES) pbuf -= STAGES;
      if (pre < nk) MOE_TILE_ISSUE(pre * BK, pbuf);
      const uint4* s = (const uint4*)(sbase + buf * STAGE);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + khalf;
        bf16x8_t fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[i] = __builtin_bit_cast(bf16x8_t, s[arow[i] * CH + (ch ^ swz<CH, SWZ>(arow[i]))]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[j] = __builtin_bit_cast(bf16x8_t, s[brow[j] * CH + (ch ^ swz<CH, SWZ>(brow[j]))]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
      }
      // the next stage must have landed: allow the younger stages in flight
      if (pre < nk) wait_vmcnt<(STAGES - 2) * (LA + LB)>();
      else wait_vmcnt<0>();
      __syncthreads();
      buf = (buf + 1 == STAGES) ? 0 : buf + 1;
    }
#undef MOE_TILE_ISSUE

    // ---- epilogue.  acc[j][i][v]: token row = i-th fragment row lane%32,
    // output column = j-th fragment column 8*(v/4) + 4*(lane/32) + v%4.
    uint16_t* cbase = ti.shared ? p.c_shared : p.c;
    const int64_t ldc = ti.Nout;
    constexpr int FO = DUAL ? FN / 2 : FN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = ti.mt * BM + wm * TM + i * 32 + (lane & 31);
      if (lr >= ti.M) continue;
      uint16_t* crow = cbase + (ti.row0 + lr) * ldc;
#pragma unroll
      for (int j = 0; j < FO; ++j) {
        const int cbase_col = ti.nt * BNo + (DUAL ? wn * (TN / 2) : wn * TN) + j * 32 + 4 * khalf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = cbase_col + 8 * q;
          if (col >= ti.Nout) continue;  // Nout % 64 == 0: a 4-column run is all in or all out
          float o[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int v = 4 * q + u;
            if (DUAL) {
              o[u] = silu_f(acc[j][i][v]) * acc[j + FN / 2][i][v];
            } else {
              float bias = 0.f;
              if (EPI != EPI_SILU_MUL && p.bias && !ti.shared)
                bias = bf16_to_f32(p.bias[(int64_t)ti.g * p.Nout + col + u]);
              o[u] = epi1<EPI>(acc[j][i][v], bias);
            }
          }
          uint2 pk;
          pk.x = pack_bf16x2(o[0], o[1]);
          pk.y = pack_bf16x2(o[2], o[3]);
          *(uint2*)(crow + col) = pk;
        }
      }
    }
  }
}

}  // namespace moe
