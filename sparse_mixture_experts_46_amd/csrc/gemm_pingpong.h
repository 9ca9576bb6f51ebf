// Grouped GEMM, ping-pong tile kernel (prefill), the main prefill kernel.
//
// C = A B^T per expert group, bf16 operands, fp32 accumulation,
// v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand
// (so each lane ends with runs of 4 consecutive output columns).
//
//  * 8 waves in two groups: waves 0-3 and waves 4-7 (one of each per SIMD).
//    Every k-step (one BK-wide LDS stage) a wave runs a memory phase M (read
//    the stage's MFMA fragments from LDS into registers, then issue its share
//    of the DMA for stage kt+STAGES-1) and a compute phase C (the MFMAs on
//    those registers).  The second group starts one s_barrier late, so on
//    every SIMD one wave computes while the other moves data.
//  * Global -> LDS with buffer_load ... lds (MUBUF, 16 bytes per lane, no
//    staging registers); one wave instruction fills 1 KB of a stage: rows of
//    2*BK bytes, lane l -> row l / CH, physical chunk l % CH, fetching logical
//    chunk (l % CH) ^ swz(row) (XOR swizzle, conflict-free fragment reads).
//  * STAGES-deep ring; loads for stage kt+STAGES-1 are issued during stage kt
//    and waited for STAGES-2 stages later, past the end of K the last slice is
//    re-loaded into the unused slot (drained before the epilogue).
//  * Persistent: one workgroup per CU walks the device-side tile table in a
//    fixed order; each XCD walks its own contiguous range of tiles (same
//    expert, neighbouring column tiles) that shares its L2.
//  * SwiGLU (DUAL): the B tile holds BN/2 gate rows and the same BN/2 up
//    rows; silu(gate) * up is formed in registers.
#pragma once

#include <type_traits>

#include "gemm_common.h"
#include "gemm_tile.h"

namespace moe {

// 16-byte-per-lane global -> LDS copy through a raw buffer resource.
__device__ __forceinline__ void buf_dma16(const void* base, uint32_t voff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, 0, 0, 0);
#endif
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int SWZ, bool DUAL, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_pingpong_kernel(GemmArgs p) {
  static_assert(WM * WN == 8, "8 waves");
  constexpr int NW = 8;
  constexpr int CH = BK / 8;
  constexpr int RB = BK * 2;
  constexpr int RPI = 1024 / RB;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int BNo = DUAL ? BN / 2 : BN;
  constexpr int LA = BM / (NW * RPI), LB = BN / (NW * RPI);
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * RB;
  constexpr int KS = BK / 16;
  static_assert(STAGES >= 3, "stages");
  extern __shared__ uint4 smem[];
  char* sbase = (char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, so per-wave buffer resources and LDS bases live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave / WN, wn = wave % WN;
  const int total = p.tile_base[p.G];
  const TileWalk walk = tile_walk(total);
  const int lrow = lane / CH, pch = lane % CH;

  // A fragment i of wave-row wm holds tile rows i * (32 * WM) + 32 * wm + ...:
  // the first half of the fragments covers rows [0, BM / 2) on every wave,
  // so a half-height tile keeps all SIMDs equally busy
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = i * (32 * WM) + wm * 32 + (lane & 31);
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
    const char* abase = (const char*)(ti.shared ? p.a_shared : p.a);
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = (i * NW + wave) * RPI + lrow;
      int lr = ti.mt * BM + r;
      if (lr >= ti.M) lr = ti.M - 1;
      int64_t ar;
      if (ti.shared) ar = ti.row0 + lr;
      else {
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
    const int nk = (int)(Kd / BK);
    // The tile body, for a full tile or (HALF) a last tile of at most BM / 2
    // rows: then only the first half of the A loads and of the fragments run.
    auto run = [&](auto half_c) {
      constexpr bool HALF = decltype(half_c)::value;
      constexpr int FMA = HALF ? FM / 2 : FM;  // A fragments computed
      constexpr int LAA = HALF ? LA / 2 : LA;  // A loads issued per stage
      constexpr int NLA = LAA + LB;
      auto issue = [&](int stage_k, int buf) {
        const int kk = stage_k < nk ? stage_k : nk - 1;
        char* st = sbase + buf * STAGE;
        const uint32_t kb = (uint32_t)(kk * BK) * 2;
#pragma unroll
        for (int i = 0; i < LAA; ++i) buf_dma16(abase, aoff[i] + kb, st + (i * NW + wave) * RPI * RB);
#pragma unroll
        for (int i = 0; i < LB; ++i) {
          const int r_ = (i * NW + wave) * RPI;
          const char* bb = (DUAL && r_ >= BN / 2) ? bbase1 : bbase0;
          buf_dma16(bb, boff[i] + kb, st + (BM + r_) * RB);
        }
      };

      f32x16_t acc[FN][FMA];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FMA; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

      // prologue: stages 0 .. STAGES-2
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) issue(s, s);
      wait_vmcnt<(STAGES - 2) * NLA>();  // stage 0 landed (own share)
      __syncthreads();
      if (grp == 1) __builtin_amdgcn_s_barrier();  // B runs one phase behind

      bf16x8_t fa[KS][FMA], fb[KS][FN];
      int buf = 0;
      for (int kt = 0; kt < nk; ++kt) {
        // ---- M phase: DMA share for stage kt+STAGES-1, fragments of stage kt
        int pbuf = buf + STAGES - 1;
        if (pbuf >= STAGES) pbuf -= STAGES;
        const uint4* s = (const uint4*)(sbase + buf * STAGE);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = ks * 2 + khalf;
#pragma unroll
          for (int i = 0; i < FMA; ++i)
            fa[ks][i] = __builtin_bit_cast(bf16x8_t, s[arow[i] * CH + (ch ^ swz<CH, SWZ>(arow[i]))]);
#pragma unroll
          for (int j = 0; j < FN; ++j)
            fb[ks][j] = __builtin_bit_cast(bf16x8_t, s[brow[j] * CH + (ch ^ swz<CH, SWZ>(brow[j]))]);
        }
        // this wave's share of stage kt+STAGES-1 (into the slot of stage
        // kt-1, which every wave finished reading before the last barrier),
        // issued while the fragment reads are still in flight
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + STAGES - 1, pbuf);
        // stage kt+1 (issued STAGES-2 phases ago) must have landed before the
        // next memory phase of either group
        wait_vmcnt<(STAGES - 2) * NLA>();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // ---- C phase
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FMA; ++i)
              acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[j][i], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        buf = (buf + 1 == STAGES) ? 0 : buf + 1;
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
          }
        }
      }
    };
    // half-height mode needs an even split of the A loads and fragments
    constexpr bool kHalfOk = (FM % 2 == 0) && (LA % 2 == 0);
    if (kHalfOk && ti.M - ti.mt * BM <= BM / 2) run(std::true_type{});
    else run(std::false_type{});
  }
}

}  // namespace moe
