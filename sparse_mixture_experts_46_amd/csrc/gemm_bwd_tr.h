// Grouped GEMMs of the backward pass, 256 x 256 tiles fed by DMA.
//
// The same problems as gemm_bwd_kernel (gemm_bwd.h: row groups and weight
// groups, K-contiguous or K-strided operands, the same epilogues), with no
// operand passing through registers:
//  * Every operand tile goes global -> LDS by DMA (buffer_load ... lds, 16
//    bytes per lane, 1 KB per wave instruction), two stages of 64-wide K.
//  * A K-contiguous tile is stored [row][64 K] (128 B per row, 16-byte chunk
//    c of row r at c ^ ((r >> 1) & 7)) and read with ds_read_b128, as in
//    gemm_bwd.h.
//  * A K-strided tile is stored as it lies in memory, [64 K][256 columns]
//    (512 B per K row, chunk c of K row k at c ^ ((k & 3) << 2)), and the
//    MFMA fragments (8 consecutive K of one column per lane) are formed by
//    gfx950's transposing LDS read, ds_read_b64_tr_b16.  Within each group
//    of 16 lanes, lane s supplies the address of 4 consecutive 16-bit
//    elements and lane i receives element i % 4 of lanes i / 4 + 4 j,
//    j = 0..3.  Lane s pointing at [k0 + s / 4][n0 + 4 (s % 4)] thus gives
//    lane i the 4 values K = k0 .. k0 + 3 of column n0 + i; two such reads
//    make the 8 K of a fragment.  The swizzle keeps the 4 K rows x 64 bytes
//    that 32 lanes read in one pass on distinct banks.
//  * Buffer descriptors sized to each group's extent make rows past the end
//    (a group's last row tile, a weight gradient's ragged K) read as zeros.
//  * 8 waves of 128 x 64 outputs (v_mfma_f32_32x32x16_bf16, weight fragment
//    first); waves 0-3 issue the A tile's DMA, waves 4-7 the B tile's.
//  * Ping-pong, as the forward's DMA kernel: waves 0-3 (tile rows 0-127)
//    and waves 4-7 (rows 128-255) put one wave on each SIMD; per 32-wide K
//    sub-step a wave reads its fragments (memory phase), then runs its 16
//    MFMAs (compute phase), and the second group runs one barrier behind,
//    so on every SIMD one wave computes while the other reads LDS.
//  * Epilogues: a weight gradient's bf16 tile and dh's activation backward
//    go through LDS (free after the K loop's last barrier), so global memory
//    sees whole rows of 128-byte lines; the other epilogues store 4 columns
//    per lane straight from the accumulators.
//  * SPLIT > 1 (with dual K): the K range (both halves) is cut into SPLIT
//    equal parts that are separate tiles; part 0 writes c, part q >= 1 the
//    plane q - 1 of c2 (the caller adds them).  A GEMM with few output
//    tiles gets SPLIT times the tiles, and the last round of the persistent
//    walk, which ragged groups leave partly empty, costs 1 / SPLIT of a
//    whole tile.
#pragma once

#include "gemm_bwd.h"
#include "gemm_tile.h"  // wait_vmcnt, lds_void_t

namespace moe {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// 16-byte DMA global -> LDS through a buffer descriptor of nrec bytes from
// base: offsets at or past nrec read as zero.
__device__ __forceinline__ void dma16_bounded(const void* base, uint32_t nrec, uint32_t voff,
                                              void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  // base and extent are wave-uniform: saying so keeps the descriptor in SGPRs
  // (else every load becomes a loop over the lanes' descriptors)
  const uint64_t b = (uint64_t)base;
  const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ub, (short)0, __builtin_amdgcn_readfirstlane((int)nrec), 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, 0, 0, 0);
#endif
}

// Chunk swizzle of a K-strided stage (32 chunks of 16 bytes per K row).
__device__ __forceinline__ int tr_swz(int k) { return (k & 3) << 2; }

// Byte offset, within a K-strided stage, of the 8 bytes at [k][n] (n % 4 == 0).
__device__ __forceinline__ uint32_t tr_off(int k, int n) {
  return (uint32_t)(k * 512 + (((n >> 3) ^ tr_swz(k)) << 4) + ((n & 4) << 1));
}

template <bool WG, bool BS, bool DUALB, bool DUALK, int EPI, int SPLIT = 1>
__global__ __launch_bounds__(512, 1) void gemm_bwd_tr_kernel(BwdArgs p, int total_tiles) {
  constexpr int BM = 256, BN = 256, BK = 64, CH = 8;
  constexpr int WN = 4, TM = 128, TN = 64, FM = 4, FN = 2;
  constexpr int BNo = DUALB ? BN / 2 : BN;
  constexpr bool A_STRIDED = WG;
  constexpr bool B_STRIDED = WG || BS;
  constexpr int OPB = 32768;      // bytes of one operand's stage
  constexpr int STB = 2 * OPB;    // bytes of one stage (A then B)
  static_assert(!(DUALB && B_STRIDED), "dual B needs the K-contiguous layout");
  static_assert(SPLIT == 1 || (DUALK && !WG), "split K applies to a dual-K row-group GEMM");
  extern __shared__ uint4 lds[];  // [2 stages][A | B]
  char* L = (char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool loads_a = wave < 4;
  const int qw = wave & 3;  // this wave's quarter of its operand's 32 DMA instructions
  const int khalf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
  const int total1 = WG ? total_tiles : p.tile_base[p.G];
  const int total = SPLIT * total1;
  const TileWalk walk = tile_walk(total);

  // first row (A) / column (B) of this wave's fragments within the tile
  // (the activation epilogues: fragment j of the 4 wave columns covers tile
  // columns 128 j .. 128 j + 127, which the epilogue stages one j at a time)
  constexpr bool ACT = EPI == BEPI_SWIGLU_BWD || EPI == BEPI_GELU_BWD;
  static_assert(!(ACT && (DUALB || WG || SPLIT > 1 || FN != 2)), "activation epilogues: row groups, one B");
  int am[FM], bn[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) am[i] = wm * TM + i * 32;
#pragma unroll
  for (int j = 0; j < FN; ++j)
    bn[j] = DUALB ? (j < FN / 2 ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FN / 2) * 32)
                  : (ACT ? j * 128 + wn * 32 : wn * TN + j * 32);

  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    const int part = SPLIT > 1 ? tile / total1 : 0;  // split K: which part
    const BwdTile ti = bwd_tile(p, WG, tile - part * total1, BM, BN);
    const int Ktot = WG ? ti.rows : (DUALK ? 2 * p.Kdim : p.Kdim);
    const int nk = SPLIT > 1 ? Ktot / BK / SPLIT : (Ktot + BK - 1) / BK;
    const int kt0 = part * nk;  // first K step of this tile's part

    // ---- this wave's DMA source: base, extent and per-lane offsets
    const char* base0;
    const char* base1;  // dual K: second half; dual B: up rows
    uint32_t nrec, soff_step;
    const bool strided = loads_a ? A_STRIDED : B_STRIDED;
    uint32_t voff[8];
    {
      int64_t ld;
      if (loads_a) {
        ld = p.lda;
        const char* a0 = (const char*)(ti.shared ? p.a_shared : p.a);
        const char* a1 = DUALK ? (const char*)(ti.shared ? p.a2_shared : p.a2) : a0;
        // row groups: the tile's first row; weight groups: the group's first row
        const int64_t r0 = (ti.shared ? 0 : ti.row0) + (WG ? 0 : (int64_t)ti.mt * BM);
        base0 = a0 + r0 * ld * 2;
        base1 = a1 + r0 * ld * 2;
        const int64_t rows_left = WG ? ti.rows : ti.rows - (int64_t)ti.mt * BM;
        nrec = (uint32_t)(rows_left * ld * 2);
      } else {
        ld = p.ldb;
        if (WG) {
          const int64_t r0 = ti.shared ? 0 : ti.row0;
          base0 = (const char*)(ti.shared ? p.bs0 : p.b0) + r0 * ld * 2;
          base1 = base0;
          nrec = (uint32_t)((int64_t)ti.rows * ld * 2);
        } else {
          const int64_t goff = ti.shared ? 0 : (int64_t)ti.g * p.b_stride * 2;
          base0 = (const char*)(ti.shared ? p.bs0 : p.b0) + goff;
          base1 = (DUALB || DUALK) ? (const char*)(ti.shared ? p.bs1 : p.b1) + goff : base0;
          // one weight matrix: [nout, Kdim] (K-contiguous) or [Kdim, nout]
          nrec = (uint32_t)((int64_t)ti.nout * p.Kdim * 2);
        }
      }
      soff_step = strided ? (uint32_t)(BK * ld * 2) : (uint32_t)(BK * 2);
      const int org = loads_a ? (WG ? ti.mt * BM : 0) : ti.nt * (WG ? BN : BNo);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = qw * 8 + u;  // instruction: 1 KB of the operand's stage
        if (!strided) {
          // 8 tile rows x 8 chunks; dual B: instructions 16.. hold the up rows
          const int r = t * 8 + (lane >> 3);
          const int c = (lane & 7) ^ ((r >> 1) & 7);
          int64_t row;
          if (loads_a) row = r;  // relative to the tile's first row
          else row = org + ((DUALB && r >= BN / 2) ? r - BN / 2 : r);
          voff[u] = (uint32_t)(row * ld * 2 + c * 16);
        } else {
          // 2 K rows x 32 chunks
          const int k = t * 2 + (lane >> 5);
          const int c = (lane & 31) ^ tr_swz(k);
          voff[u] = (uint32_t)((int64_t)k * ld * 2 + (int64_t)(org + c * 8) * 2);
        }
      }
    }
    // the K step moves the descriptor's base (and shrinks its extent), so the
    // range check stays on the group's own rows
    auto issue = [&](int kt, int buf) {
      int kk = kt + kt0;
      const char* b = base0;
      if (DUALK && kk * BK >= p.Kdim) {
        kk -= p.Kdim / BK;
        b = base1;
      }
      const uint32_t step = (uint32_t)kk * soff_step;
      const uint32_t nk_rec = nrec > step ? nrec - step : 0u;
      char* dst = L + buf * STB + (loads_a ? 0 : OPB);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = qw * 8 + u;
        const char* bb = (DUALB && !loads_a && t >= 16) ? base1 : b;
        dma16_bounded(bb + step, nk_rec, voff[u], dst + t * 1024);
      }
    };

    f32x16_t acc[FN][FM];  // [weight fragment][token fragment]
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

    // fragment of a K-contiguous stage: rows r0 + lane % 32, K chunk ch
    auto frag_c = [&](const char* S, int r0, int ch) -> bf16x8_t {
      const int r = r0 + (lane & 31);
      return __builtin_bit_cast(bf16x8_t, *(const uint4*)(S + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4)));
    };
    // fragment of a K-strided stage: columns n0 + lane % 32, K = 16 ks + 8 (lane / 32) + 0..7
    auto frag_t = [&](const char* S, int n0, int ks) -> bf16x8_t {
      const int k = ks * 16 + 8 * (g16 >> 1) + (i16 >> 2);
      const int n = n0 + 16 * (g16 & 1) + 4 * (i16 & 3);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(S + tr_off(k, n)));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(S + tr_off(k + 4, n)));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // fragments of K slice ks of a stage
    auto read_frags = [&](int stage, int ks, bf16x8_t* xa, bf16x8_t* xb) {
      const char* SA = L + stage * STB;
      const char* SB = SA + OPB;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        xa[i] = A_STRIDED ? frag_t(SA, am[i], ks) : frag_c(SA, am[i], ks * 2 + khalf);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        xb[j] = B_STRIDED ? frag_t(SB, bn[j], ks) : frag_c(SB, bn[j], ks * 2 + khalf);
    };
    // Ping-pong over 32-wide K sub-steps, as the forward's DMA kernel:
    // group 0 (waves 0-3: tile rows 0-127, the A operand's DMA) and group 1
    // (waves 4-7: rows 128-255, B's DMA) put one wave on each SIMD.  A
    // sub-step is a memory phase (read the sub-step's fragments; in a
    // block's first sub-step also issue this wave's share of the next
    // block's DMA; in its second wait for that share) and a compute phase
    // (the MFMAs), each closed by a barrier.  Group 1 starts one barrier
    // late, so on every SIMD one wave computes while the other moves data.
    // Block kt+1 goes into the slot of block kt-1, whose last reads (group
    // 1's memory phase of kt-1's second sub-step) ended before the barrier
    // that precedes the issue.  Every wave passes the same number of
    // barriers: 1 + 4 nk + 1.
    const int grp = wave >> 2;
    bf16x8_t fa[2][FM], fb[2][FN];
    if (nk > 0) issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    if (grp == 1) __builtin_amdgcn_s_barrier();
    auto finish_m_then_compute = [&]() {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): fragments in registers
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[h][j], fa[h][i], acc[j][i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      // sub-step 0: K 0..31 of block kt; this wave's DMA share of block kt+1
      read_frags(cur, 0, fa[0], fb[0]);
      read_frags(cur, 1, fa[1], fb[1]);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
      finish_m_then_compute();
      // sub-step 1: K 32..63; this wave's share of block kt+1 landed
      read_frags(cur, 2, fa[0], fb[0]);
      read_frags(cur, 3, fa[1], fb[1]);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      finish_m_then_compute();
    }
    if (grp == 0) __builtin_amdgcn_s_barrier();  // realign the groups

    // ---- epilogue (as gemm_bwd_kernel); split K: parts 1.. write c2's planes
    BwdArgs pe = p;
    if (SPLIT > 1 && part > 0) {
      pe.c = (char*)p.c2 + (part - 1) * p.c2_plane;
      pe.c_shared = (char*)p.c2_shared + (part - 1) * p.c2_plane_shared;
    }
    if constexpr (ACT) {
      // Through LDS, 128 columns at a time: every wave puts its fragment j
      // of dh there as fp32 [256 rows][128] (16-byte chunk c of row r at
      // c ^ (r & 31)); then each thread takes 8 consecutive columns of a row,
      // so u, v, du, dv and h move as whole 128-byte lines.  No wave reads
      // the stages after the K loop's last barrier, so the first pass needs
      // no barrier before it writes.
      float* E = (float*)L;
      const int cp = tid & 15;  // this thread's 8 columns of the pass: 8 cp .. 8 cp + 7
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = am[i] + (lane & 31);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int c = wn * 8 + 2 * qq + khalf;
            *(float4*)(E + r * 128 + ((c ^ (r & 31)) << 2)) =
                make_float4(acc[j][i][4 * qq], acc[j][i][4 * qq + 1], acc[j][i][4 * qq + 2],
                            acc[j][i][4 * qq + 3]);
          }
        }
        __syncthreads();
        const int col = ti.nt * BN + j * 128 + 8 * cp;
        // 32 rows per pass of the 512 threads; 4 rows' u (and v) loaded
        // before any of their results is stored (which may be in place)
#pragma unroll
        for (int b = 0; b < 8; b += 4) {
          uint4 uu[4], vv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = ti.mt * BM + (b + q) * 32 + (tid >> 4);
            if (m < ti.rows && col < ti.nout)
              act_bwd_load8<EPI>(p, ti, (ti.row0 + m) * p.ldc + col, uu[q], vv[q]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = (b + q) * 32 + (tid >> 4);
            const int m = ti.mt * BM + r;
            if (m >= ti.rows || col >= ti.nout) continue;
            const float4 d0 = *(const float4*)(E + r * 128 + (((2 * cp) ^ (r & 31)) << 2));
            const float4 d1 = *(const float4*)(E + r * 128 + (((2 * cp + 1) ^ (r & 31)) << 2));
            const float g[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            act_bwd_store8<EPI>(p, ti, (ti.row0 + m) * p.ldc + col, g, uu[q], vv[q]);
          }
        }
        __syncthreads();  // E read by all before it is refilled (next pass, next tile's DMA)
      }
      continue;
    }
    const int mlim = WG ? p.Mout : ti.rows;
    if constexpr (WG && EPI == BEPI_STORE) {
      // Weight gradients through LDS: the tile as bf16 [256][256] (16-byte
      // chunk c of row r at c ^ (r & 31)), then 32 threads per row store
      // whole 512-byte rows.  The stages are free after the K loop's last
      // barrier.
      uint16_t* E = (uint16_t*)L;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = am[i] + (lane & 31);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int c = (bn[j] >> 3) + qq;
            *(uint2*)(E + r * 256 + ((c ^ (r & 31)) << 3) + 4 * khalf) =
                make_uint2(pack_bf16x2(acc[j][i][4 * qq], acc[j][i][4 * qq + 1]),
                           pack_bf16x2(acc[j][i][4 * qq + 2], acc[j][i][4 * qq + 3]));
          }
        }
      __syncthreads();
      uint16_t* C = (uint16_t*)(ti.shared ? p.c_shared : p.c) +
                    (ti.shared ? 0 : (int64_t)ti.g * p.c_gstride);
      const int cp = tid & 31;
      const int col = ti.nt * BN + 8 * cp;
#pragma unroll 4
      for (int rp = 0; rp < 16; ++rp) {
        const int r = rp * 16 + (tid >> 5);
        const int m = ti.mt * BM + r;
        if (m < mlim && col < ti.nout)
          *(uint4*)(C + (int64_t)m * p.ldc + col) = *(const uint4*)(E + r * 256 + ((cp ^ (r & 31)) << 3));
      }
      __syncthreads();  // E read by all before the next tile's DMA
      continue;
    }
    constexpr int FO = DUALB ? FN / 2 : FN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = ti.mt * BM + am[i] + (lane & 31);
      if (m >= mlim) continue;
      const int64_t rowoff = WG ? (ti.shared ? 0 : (int64_t)ti.g * p.c_gstride) + (int64_t)m * p.ldc
                                : (ti.row0 + m) * p.ldc;
#pragma unroll
      for (int j = 0; j < FO; ++j) {
        const int cb = ti.nt * BNo + (DUALB ? wn * (TN / 2) : wn * TN) + j * 32 + 4 * khalf;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int col = cb + 8 * qq;
          if (col >= ti.nout) continue;
          const int64_t o = rowoff + col;
          float r0[4], r1[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            r0[u] = acc[j][i][4 * qq + u];
            r1[u] = DUALB ? acc[j + FN / 2][i][4 * qq + u] : 0.f;
          }
          bwd_epilogue4<EPI, WG>(pe, ti, o, col, r0, r1);
        }
      }
    }
  }
}

}  // namespace moe
