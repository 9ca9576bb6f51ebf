// Grouped GEMM, ping-pong tile kernel (prefill), the main prefill kernel.
//
// C = A B^T per expert group, bf16 operands, fp32 accumulation,
// v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand
// (so each lane ends with runs of 4 consecutive output columns).
//
//  * 8 waves in two groups: waves 0-3 and waves 4-7 (one of each per SIMD).
//    K advances in 32-wide sub-steps.  Every sub-step a wave runs a memory
//    phase M (read the sub-step's MFMA fragments from LDS into registers,
//    issue its share of a DMA) and a compute phase C (the MFMAs on those
//    registers).  The second group starts one s_barrier late, so on every
//    SIMD one wave computes while the other moves data.
//  * Global -> LDS with buffer_load ... lds (MUBUF, 16 bytes per lane, no
//    staging registers), in 64-wide K blocks: each wave instruction fetches
//    8 rows x 128 bytes, i.e. whole 128-byte lines.  Fetching half lines (a
//    32-wide block, 64 bytes per row) measured about half the per-CU load
//    throughput, which the 256 x 256 tile needs in full at the MFMA rate.
//    Lanes 0-31 take K 0..31 of the block and lanes 32-63 K 32..63, so one
//    instruction's 1 KB of LDS is [half][8 rows][64 B] and each 32-wide
//    sub-step reads one half.  Physical 16-byte chunk c of a row holds
//    logical chunk c ^ ((row >> 2) & 3), which spreads the fragment reads
//    over the banks.
//  * A and B have separate rings of DA and DB blocks.  Sub-step 2j issues
//    A(j+1) into the slot of A(j+1-DA); sub-step 2j+1 issues B(j+2) into the
//    slot of B(j+2-DB) and then waits for A(j+1) and B(j+1).  With DA >= 2
//    and DB >= 3 every overwritten slot was last read before the previous
//    barrier, and the weights get three sub-steps of lead.  Past the end of
//    K the last block is re-loaded (drained before the epilogue).
//  * Persistent: one workgroup per CU walks the device-side tile table; each
//    XCD works through its own contiguous range of tiles (same expert,
//    neighbouring column tiles) that shares its L2, in a fixed order or,
//    given walk counters, handing out the range's tiles one at a time so
//    that the XCD's workgroups stay on neighbouring tiles.
//  * SwiGLU (DUAL): the B tile holds BN/2 gate rows and the same BN/2 up
//    rows; silu(gate) * up is formed in registers.
#pragma once

#include <type_traits>

#include "gemm_common.h"
#include "gemm_tile.h"
#include "lds_dma.h"

namespace moe {

template <int BM, int BN, int WM, int WN, int DA, int DB, bool DUAL, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_pingpong_kernel(GemmArgs p) {
  static_assert(WM * WN == 8, "8 waves");
  static_assert(DA >= 2 && DB >= 3, "ring depths the slot reuse relies on");
  constexpr int NW = 8;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int BNo = DUAL ? BN / 2 : BN;
  constexpr int LA = BM / (NW * 8), LB = BN / (NW * 8);  // DMA instructions per wave per block
  static_assert(LA >= 1 && LB >= 1 && LA * NW * 8 == BM && LB * NW * 8 == BN, "tile rows");
  constexpr int ASLOT = BM * 128, BSLOT = BN * 128;  // bytes of one 64-wide K block
  extern __shared__ uint4 smem[];
  char* abuf = (char*)smem;
  char* bbuf = abuf + DA * ASLOT;
  const uint4* abuf4 = (const uint4*)abuf;
  const uint4* bbuf4 = (const uint4*)bbuf;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, so per-wave buffer resources and LDS bases live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave / WN, wn = wave % WN;
  const int total = p.tile_base[p.G];
  const TileWalk walk = tile_walk(total);
  // DMA lane map: K half, row within the instruction's 8, physical chunk
  const int dh = lane >> 5, drow = (lane & 31) >> 2, dch = lane & 3;
  const int khalf = lane >> 5;

  // Fragment rows, as uint4 indices inside a slot (half 0).  A fragment i of
  // wave-row wm holds tile rows i * (32 * WM) + 32 * wm + ...: the first half
  // of the fragments covers rows [0, BM / 2) on every wave, so a half-height
  // tile keeps all SIMDs equally busy.
  int aidx[FM], asw[FM], bidx[FN], bsw[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = i * (32 * WM) + wm * 32 + (lane & 31);
    aidx[i] = (r >> 3) * 64 + (r & 7) * 4;
    asw[i] = pp_swz(r);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int r;
    if (DUAL) {
      constexpr int FH = FN / 2;
      r = (j < FH) ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FH) * 32;
    } else {
      r = wn * TN + j * 32;
    }
    r += lane & 31;
    bidx[j] = (r >> 3) * 64 + (r & 7) * 4;
    bsw[j] = pp_swz(r);
  }

  // dynamic order: thread 0 takes the next tile from the counters and hands
  // it over in the first LDS word, which is free between tiles (no DMA in
  // flight, no fragment reads)
  const bool dyn = p.walk_ctr != nullptr && (gridDim.x & 7) == 0;
  DynWalk dw;
  volatile int* bcast = (volatile int*)smem;
  for (int tile = dyn ? dyn_first(dw, total) : walk.tile;;) {
    if (dyn && tile == -2) {
      if (tid == 0) *bcast = dyn_next(dw, p.walk_ctr);
      __syncthreads();
      tile = *bcast;
      __syncthreads();  // read by every wave before the DMA reuses the word
    }
    if (dyn ? tile < 0 : tile >= walk.end) break;
    const TileInfo ti = resolve_tile(p, tile, BM, BNo);
    const int64_t Kd = p.Kdim;
    const char* abase = (const char*)(ti.shared ? p.a_shared : p.a);
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (i * NW + wave) * 8 + drow;
      int lr = ti.mt * BM + r;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) ar = ti.row0 + lr;
      else {
        const int64_t gr = ti.row0 + lr;
        ar = p.a_rows ? (int64_t)(p.a_rows[gr] / p.a_div) : gr;
      }
      aoff[i] = (uint32_t)((ar * p.lda + dh * 32 + (dch ^ pp_swz(r)) * 8) * 2);
    }
    const char* bbase0 = (const char*)(ti.shared ? p.bs0 : p.b0 + (int64_t)ti.g * p.b_stride);
    const char* bbase1 = DUAL ? (const char*)(ti.shared ? p.bs1 : p.b1 + (int64_t)ti.g * p.b_stride)
                              : bbase0;
    uint32_t boff[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = (i * NW + wave) * 8 + drow;
      int n = ti.nt * BNo + ((DUAL && r >= BN / 2) ? r - BN / 2 : r);
      if (n >= ti.Nout) n = ti.Nout - 1;
      boff[i] = (uint32_t)(((int64_t)n * Kd + dh * 32 + (dch ^ pp_swz(r)) * 8) * 2);
    }
    const int nk = (int)(Kd / 64);
    // The tile body (MODE 0) for a full tile; (MODE 1) for a last tile of at
    // most BM / 2 rows, where only the first half of the A loads and of the
    // fragments run; (MODE 2) for a last tile of at most BM / 4 rows, where a
    // quarter of the A loads run and only the first group's waves, which hold
    // the tile's first BM / 4 rows in their first fragment, read fragments
    // and compute (the second group keeps every barrier); (MODE 3) for a last
    // tile of at most 3 BM / 4 rows, where three quarters of the A loads run
    // and the second group skips its second fragment (the last BM / 4 rows).
    auto run = [&](auto mode_c) {
      constexpr int MODE = decltype(mode_c)::value;
      constexpr int FMA = (MODE == 1 || MODE == 2) ? FM / 2 : FM;  // A fragments computed
      constexpr int LAA = MODE == 0 ? LA : MODE == 1 ? LA / 2 : MODE == 2 ? LA / 4 : 3 * LA / 4;
      const bool idle = MODE == 2 && grp == 1;
      // wave-uniform: whether this wave computes A fragment i
      auto frag_on = [&](int i) { return MODE != 3 || grp == 0 || i == 0; };
      auto issue_a = [&](int blk, int slot) {
        const uint32_t kb = (uint32_t)(blk < nk ? blk : nk - 1) * 128u;
        char* st = abuf + slot * ASLOT;
#pragma unroll
        for (int i = 0; i < LAA; ++i) buf_dma16(abase, aoff[i] + kb, st + (i * NW + wave) * 1024);
      };
      auto issue_b = [&](int blk, int slot) {
        const uint32_t kb = (uint32_t)(blk < nk ? blk : nk - 1) * 128u;
        char* st = bbuf + slot * BSLOT;
#pragma unroll
        for (int i = 0; i < LB; ++i) {
          const char* bb = (DUAL && (i * NW + wave) * 8 >= BN / 2) ? bbase1 : bbase0;
          buf_dma16(bb, boff[i] + kb, st + (i * NW + wave) * 1024);
        }
      };

      f32x16_t acc[FN][FMA];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FMA; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

      bf16x8_t fa[2][FMA], fb[2][FN];
      auto read_fragments = [&](int sa, int sb, int h) {
        if (idle) return;
        const uint4* sA = abuf4 + sa * (ASLOT / 16) + h * 32;
        const uint4* sB = bbuf4 + sb * (BSLOT / 16) + h * 32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int ch = ks * 2 + khalf;
#pragma unroll
          for (int i = 0; i < FMA; ++i)
            if (frag_on(i)) fa[ks][i] = __builtin_bit_cast(bf16x8_t, sA[aidx[i] + (ch ^ asw[i])]);
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[ks][j] = __builtin_bit_cast(bf16x8_t, sB[bidx[j] + (ch ^ bsw[j])]);
        }
      };
      // end of an M phase: fragments in registers, then the group barrier;
      // the C phase; its closing barrier
      auto finish_m_then_compute = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (!idle) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int i = 0; i < FMA; ++i)
                if (frag_on(i))
                  acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[j][i], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      };

      // prologue: B(0), A(0), B(1); block 0 landed everywhere before the loop
      issue_b(0, 0);
      issue_a(0, 0);
      issue_b(1, 1);
      wait_vmcnt<LB>();
      __syncthreads();
      if (grp == 1) __builtin_amdgcn_s_barrier();  // B runs one phase behind

      int sa = 0, sb = 0;  // slots of block j
      for (int j = 0; j < nk; ++j) {
        const int sa1 = sa + 1 == DA ? 0 : sa + 1;
        const int sb1 = sb + 1 == DB ? 0 : sb + 1;
        const int sb2 = sb1 + 1 == DB ? 0 : sb1 + 1;
        // ---- sub-step 2j: K 0..31 of block j; DMA share of A(j+1), issued
        // while the fragment reads are in flight
        read_fragments(sa, sb, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(j + 1, sa1);
        finish_m_then_compute();
        // ---- sub-step 2j+1: K 32..63 of block j; DMA share of B(j+2)
        read_fragments(sa, sb, 1);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(j + 2, sb2);
        wait_vmcnt<LB>();  // this wave's shares of A(j+1) and B(j+1) landed
        finish_m_then_compute();
        sa = sa1;
        sb = sb1;
      }
      if (grp == 0) __builtin_amdgcn_s_barrier();  // realign with B
      wait_vmcnt<0>();
      __syncthreads();

      // ---- epilogue: 4 consecutive output columns per lane, 8-byte stores
      uint16_t* cbase = ti.shared ? p.c_shared : p.c;
      const int64_t ldc = ti.Nout;
      constexpr int FO = DUAL ? FN / 2 : FN;
#pragma unroll
      for (int i = 0; i < FMA; ++i) {
        const int lr = ti.mt * BM + i * (32 * WM) + wm * 32 + (lane & 31);
        if (lr >= ti.M) continue;
        uint16_t* crow = cbase + (ti.row0 + lr) * ldc;
#pragma unroll
        for (int j = 0; j < FO; ++j) {
          const int cbase_col = ti.nt * BNo + (DUAL ? wn * (TN / 2) : wn * TN) + j * 32 + 4 * khalf;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = cbase_col + 8 * q;
            if (col >= ti.Nout) continue;
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
            if (DUAL && p.c_u) {  // also keep gate(x) and up(x) for the backward
              const int64_t ro = (ti.row0 + lr) * ldc + col;
              const f32x16_t& ga = acc[j][i];
              const f32x16_t& up = acc[j + FN / 2][i];
              *(uint2*)((ti.shared ? p.cs_u : p.c_u) + ro) =
                  make_uint2(pack_bf16x2(ga[4 * q], ga[4 * q + 1]), pack_bf16x2(ga[4 * q + 2], ga[4 * q + 3]));
              *(uint2*)((ti.shared ? p.cs_v : p.c_v) + ro) =
                  make_uint2(pack_bf16x2(up[4 * q], up[4 * q + 1]), pack_bf16x2(up[4 * q + 2], up[4 * q + 3]));
            }
          }
        }
      }
    };
    // half-height mode needs an even split of the A loads and fragments;
    // quarter-height mode also needs the first group's waves (0-3) to hold
    // exactly the tile's first BM / 4 rows in their first fragment
    constexpr bool kHalfOk = (FM % 2 == 0) && (LA % 2 == 0);
    constexpr bool kQuarterOk = kHalfOk && (LA % 4 == 0) && (BM * WN == 512);
    // three-quarter mode: with two fragments, the second group's second one
    // holds exactly the tile's last BM / 4 rows
    constexpr bool kThreeQOk = kQuarterOk && (FM == 2);
    const int left = ti.M - ti.mt * BM;
    if (kQuarterOk && left <= BM / 4) run(std::integral_constant<int, 2>{});
    else if (kHalfOk && left <= BM / 2) run(std::integral_constant<int, 1>{});
    else if (kThreeQOk && left <= 3 * BM / 4) run(std::integral_constant<int, 3>{});
    else run(std::integral_constant<int, 0>{});
    tile = dyn ? -2 : tile + walk.step;
  }
}

}  // namespace moe
