// Grouped GEMMs of the backward pass.
//
// Two ways of cutting the work into groups (experts; group n_routed, when
// present, is the shared expert over all T tokens):
//  * Row groups (the recompute of the first expert GEMM, and the data
//    gradients): C = A B^T over each group's rows, as in the forward.  A is
//    K-contiguous ([rows, K], optionally gathered through a_rows).  B is
//    either K-contiguous ([Nout, K] per group, the forward layout) or
//    K-strided ([K, Nout] per group: a weight used transposed, e.g.
//    dh = do W2 with W2 stored [d, F]).
//  * Weight groups (the weight gradients): C_g = A_g^T B_g, the contraction
//    running over the group's rows, so both operands are K-strided
//    ([rows, Mout] and [rows, Nout], either optionally gathered) and K is
//    ragged.  A group with no rows gets C_g = 0.
//
// bf16 kernel (gfx950 matrix cores, v_mfma_f32_32x32x16_bf16, fp32
// accumulation): R x R output tiles (R = 128: 4 waves of 64 x 64; R = 256:
// 8 waves of 128 x 64), K in 64-wide steps.  The first half of the waves
// stage the A tile and the second half the B tile, global -> registers ->
// LDS, the next step's loads in flight while the current one is multiplied
// (two LDS buffers, one barrier per step).  A K-contiguous tile
// row goes as 16-byte chunks.  A K-strided tile is read as 8 x 8 blocks (8 K
// rows of 8 contiguous elements, each load a 16-byte run of one K row),
// transposed in registers, and written as 8 K-contiguous 16-byte chunks.
// Either way LDS holds [tile row][64 K] with the chunk XOR swizzle, so the
// fragment reads are the same for every layout.  Weight fragment first in
// the MFMA, so each lane ends with runs of 4 consecutive output columns.
//
// fp32 kernel: one thread per output element, plain fp32 dot products over
// the same addressing (used for fp32 layers, which are small).
#pragma once

#include "gemm_common.h"

namespace moe {

enum {
  BEPI_STORE = 0,       // C (act dtype), plus the routed bias of the column if given
  BEPI_STORE_F32 = 1,   // C in fp32 whatever the operand dtype
  BEPI_UV = 2,          // dual B: gate columns -> c, up columns -> c2
  BEPI_SWIGLU_BWD = 3,  // acc = dh; u = c, v = c2 -> du -> c, dv -> c2, silu(u) v -> c3
  BEPI_GELU_BWD = 4,    // acc = dh; u = c -> dh gelu'(u) -> c, gelu(u) -> c3
};

struct BwdArgs {
  const int32_t* offset;     // [n_routed + 1] row offsets of the routed groups
  int n_routed;
  int64_t shared_rows;       // rows of the shared group (0 = none)
  const int32_t* tile_base;  // row groups: tile table [G + 1]
  int G;
  // A: row groups [rows, Kdim]; weight groups [rows, Mout] (read transposed)
  const void* a;
  const void* a2;            // dual K: A of the second half of K
  const int32_t* a_rows;     // nullable gather: row r -> a[a_rows[r] / a_div]
  int a_div;
  int64_t lda;
  const void* a_shared;
  const void* a2_shared;
  // B: row groups [Nout, Kdim] or, strided, [Kdim, Nout] per group (b_stride
  // apart); weight groups [rows, Nout] (read transposed)
  const void* b0;
  const void* b1;            // dual B: up rows; dual K: B of the second half
  int64_t b_stride;
  int64_t ldb;
  const void* bs0;
  const void* bs1;
  const int32_t* b_rows;     // weight groups: nullable gather of B's rows
  int b_div;
  int Mout;                  // weight groups: output rows per group
  int Nout, Nout_shared;
  int Kdim;                  // row groups: K (per half with dual K)
  const void* bias;          // [n_routed, Nout] (BEPI_STORE, row groups)
  void* c;
  void* c2;
  void* c3;
  void* c_shared;
  void* c2_shared;
  void* c3_shared;
  // split K (gemm_bwd_tr_kernel, SPLIT > 1): part q >= 1 of the K range
  // writes c2 (c2_shared) + (q - 1) * these bytes
  int64_t c2_plane, c2_plane_shared;
  int64_t ldc;
  int64_t c_gstride;         // weight groups: elements between groups' outputs
  // nullable (BEPI_SWIGLU_BWD / BEPI_GELU_BWD): read u (and v) from here
  // instead of c (c2); the results still go to c, c2, c3
  const void* cin;
  const void* cin2;
  const void* cin_shared;
  const void* cin2_shared;
};

// The sigmoids of both derivatives through one exp and the hardware
// reciprocal (v_rcp_f32, within 1 ulp), as the forward's silu and gelu,
// instead of a correctly rounded division or tanhf: with s = sigmoid(2 z),
// tanh z = 2 s - 1, 1 + tanh z = 2 s and 1 - tanh^2 z = 4 s (1 - s).
__device__ __forceinline__ float silu_grad_f(float u) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-u));
  return s * (1.0f + u * (1.0f - s));
}

__device__ __forceinline__ float gelu_tanh_grad_f(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * c * (u + 0.044715f * u * u * u)));
  return s + 2.0f * u * s * (1.0f - s) * c * (1.0f + 3.0f * 0.044715f * u * u);
}

// Tile of a grouped problem.
struct BwdTile {
  int g, mt, nt;
  bool shared;
  int64_t row0;  // first row of the group in the row space (0 for the shared group)
  int rows;      // rows of the group (row groups: M; weight groups: K)
  int nout;
};

__device__ __forceinline__ BwdTile bwd_tile(const BwdArgs& p, bool wgroups, int tile, int BM, int BN) {
  BwdTile t;
  int local;
  if (wgroups) {
    // stripes of 4 row tiles, the row index fastest: the 32 tiles one XCD
    // runs together form a 4 x 8 block, which reads 4 slabs of A and 8 of B
    // per K step (a 2 x 16 or 16 x 2 run reads 18)
    const int mtiles = (p.Mout + BM - 1) / BM, ntiles = (p.Nout + BN - 1) / BN;
    t.g = tile / (mtiles * ntiles);
    local = tile - t.g * mtiles * ntiles;
    constexpr int H = 4;
    const int stripe = local / (H * ntiles), first = stripe * H;
    const int sh = mtiles - first < H ? mtiles - first : H;
    const int w = local - stripe * H * ntiles;
    t.mt = first + w % sh;
    t.nt = w / sh;
  } else {
    t.g = find_group(p.tile_base, p.G, tile);
    local = tile - p.tile_base[t.g];
  }
  t.shared = (t.g == p.n_routed);
  t.row0 = t.shared ? 0 : p.offset[t.g];
  t.rows = t.shared ? (int)p.shared_rows : (int)(p.offset[t.g + 1] - p.offset[t.g]);
  t.nout = (t.shared && !wgroups) ? p.Nout_shared : p.Nout;
  if (!wgroups) {
    const int mtiles = (t.rows + BM - 1) / BM;
    t.mt = local % mtiles;
    t.nt = local / mtiles;
  }
  return t;
}

// Element offset of row r of a group's operand (gathered or not).
__device__ __forceinline__ int64_t bwd_row(const BwdTile& t, const int32_t* rows_map, int div,
                                           int64_t ld, int r) {
  if (t.shared) return (int64_t)r * ld;
  const int64_t gr = t.row0 + r;
  if (!rows_map) return gr * ld;
  const int32_t v = rows_map[gr];
  return (int64_t)(div == 1 ? v : v / div) * ld;
}

__device__ __forceinline__ int bwd_swz(int row) { return (row >> 1) & 7; }

// Epilogue of 4 consecutive output columns col .. col+3 at element offset o
// (r0: the accumulators; r1: the up half of a dual-B tile).
//
// The activation-backward epilogues (BEPI_SWIGLU_BWD / BEPI_GELU_BWD) in two
// halves: the bf16 u (and v) of 4 columns, then du (dv) and h from them.  The
// results may overwrite u and v in place, so a caller that loads several
// runs before storing any keeps the loads from waiting on the stores.
template <int EPI>
__device__ __forceinline__ void act_bwd_load4(const BwdArgs& p, const BwdTile& ti, int64_t o, uint2& uu,
                                              uint2& vv) {
  const uint16_t* Ur = (const uint16_t*)(p.cin ? (ti.shared ? p.cin_shared : p.cin)
                                                : (ti.shared ? p.c_shared : p.c));
  uu = *(const uint2*)(Ur + o);
  if (EPI == BEPI_SWIGLU_BWD) {
    const uint16_t* Vr = (const uint16_t*)(p.cin2 ? (ti.shared ? p.cin2_shared : p.cin2)
                                                   : (ti.shared ? p.c2_shared : p.c2));
    vv = *(const uint2*)(Vr + o);
  } else {
    vv = make_uint2(0u, 0u);
  }
}

template <int EPI>
__device__ __forceinline__ void act_bwd_store4(const BwdArgs& p, const BwdTile& ti, int64_t o,
                                               const float (&r0)[4], const uint2& uu, const uint2& vv) {
  uint16_t* U = (uint16_t*)(ti.shared ? p.c_shared : p.c);
  uint16_t* H = (uint16_t*)(ti.shared ? p.c3_shared : p.c3);
  const float u[4] = {__uint_as_float(uu.x << 16), __uint_as_float(uu.x & 0xffff0000u),
                      __uint_as_float(uu.y << 16), __uint_as_float(uu.y & 0xffff0000u)};
  float du[4], h[4];
  if (EPI == BEPI_SWIGLU_BWD) {
    uint16_t* V = (uint16_t*)(ti.shared ? p.c2_shared : p.c2);
    const float v[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                        __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
    float dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = silu_f(u[e]);
      h[e] = sg * v[e];
      dv[e] = r0[e] * sg;
      du[e] = r0[e] * v[e] * silu_grad_f(u[e]);
    }
    *(uint2*)(V + o) = make_uint2(pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = gelu_tanh_f(u[e]);
      du[e] = r0[e] * gelu_tanh_grad_f(u[e]);
    }
  }
  *(uint2*)(U + o) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
  *(uint2*)(H + o) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
}

// The same on 8 columns (16-byte runs).
template <int EPI>
__device__ __forceinline__ void act_bwd_load8(const BwdArgs& p, const BwdTile& ti, int64_t o, uint4& uu,
                                              uint4& vv) {
  const uint16_t* Ur = (const uint16_t*)(p.cin ? (ti.shared ? p.cin_shared : p.cin)
                                                : (ti.shared ? p.c_shared : p.c));
  uu = *(const uint4*)(Ur + o);
  if (EPI == BEPI_SWIGLU_BWD) {
    const uint16_t* Vr = (const uint16_t*)(p.cin2 ? (ti.shared ? p.cin2_shared : p.cin2)
                                                   : (ti.shared ? p.c2_shared : p.c2));
    vv = *(const uint4*)(Vr + o);
  } else {
    vv = make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int EPI>
__device__ __forceinline__ void act_bwd_store8(const BwdArgs& p, const BwdTile& ti, int64_t o,
                                               const float (&r0)[8], const uint4& uu, const uint4& vv) {
  uint16_t* U = (uint16_t*)(ti.shared ? p.c_shared : p.c);
  uint16_t* H = (uint16_t*)(ti.shared ? p.c3_shared : p.c3);
  const uint32_t uw[4] = {uu.x, uu.y, uu.z, uu.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
  uint32_t du[4], dv[4], h[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float u2[2] = {__uint_as_float(uw[c] << 16), __uint_as_float(uw[c] & 0xffff0000u)};
    float du2[2], dv2[2], h2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float g = r0[2 * c + e];
      if (EPI == BEPI_SWIGLU_BWD) {
        const float v = __uint_as_float(e ? (vw[c] & 0xffff0000u) : (vw[c] << 16));
        const float sg = silu_f(u2[e]);
        h2[e] = sg * v;
        dv2[e] = g * sg;
        du2[e] = g * v * silu_grad_f(u2[e]);
      } else {
        h2[e] = gelu_tanh_f(u2[e]);
        du2[e] = g * gelu_tanh_grad_f(u2[e]);
        dv2[e] = 0.f;
      }
    }
    du[c] = pack_bf16x2(du2[0], du2[1]);
    dv[c] = pack_bf16x2(dv2[0], dv2[1]);
    h[c] = pack_bf16x2(h2[0], h2[1]);
  }
  if (EPI == BEPI_SWIGLU_BWD)
    *(uint4*)((uint16_t*)(ti.shared ? p.c2_shared : p.c2) + o) = make_uint4(dv[0], dv[1], dv[2], dv[3]);
  *(uint4*)(U + o) = make_uint4(du[0], du[1], du[2], du[3]);
  *(uint4*)(H + o) = make_uint4(h[0], h[1], h[2], h[3]);
}

template <int EPI, bool WG>
__device__ __forceinline__ void bwd_epilogue4(const BwdArgs& p, const BwdTile& ti, int64_t o, int col,
                                              float (&r0)[4], const float (&r1)[4]) {
  if (EPI == BEPI_STORE_F32) {
    float* C = (float*)(ti.shared ? p.c_shared : p.c);
    *(float4*)(C + o) = make_float4(r0[0], r0[1], r0[2], r0[3]);
  } else if (EPI == BEPI_STORE) {
    uint16_t* C = (uint16_t*)(ti.shared ? p.c_shared : p.c);
    if (p.bias && !ti.shared && !WG) {
      const uint16_t* b = (const uint16_t*)p.bias + (int64_t)ti.g * p.Nout + col;
#pragma unroll
      for (int u = 0; u < 4; ++u) r0[u] += bf16_to_f32(b[u]);
    }
    *(uint2*)(C + o) = make_uint2(pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]));
  } else if (EPI == BEPI_UV) {
    uint16_t* C = (uint16_t*)(ti.shared ? p.c_shared : p.c);
    uint16_t* C2 = (uint16_t*)(ti.shared ? p.c2_shared : p.c2);
    *(uint2*)(C + o) = make_uint2(pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]));
    *(uint2*)(C2 + o) = make_uint2(pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3]));
  } else {  // BEPI_SWIGLU_BWD / BEPI_GELU_BWD: r0 = dh
    uint2 uu, vv;
    act_bwd_load4<EPI>(p, ti, o, uu, vv);
    act_bwd_store4<EPI>(p, ti, o, r0, uu, vv);
  }
}

// Column j of an 8 x 8 block of 16-bit elements whose row i is in[i]:
// element j of every in[i], in order of i.  Word c of a row holds elements
// 2c (low half) and 2c + 1 (high half).
__device__ __forceinline__ uint32_t word_b32(const uint4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint4 transpose8x8_col_b16(const uint4 (&in)[8], int j) {
  const int c = j >> 1;
  uint32_t o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t lo = word_b32(in[2 * v], c), hi = word_b32(in[2 * v + 1], c);
    o[v] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// R: tile side (R x R outputs; 2R threads, R / 32 waves, half of them
// staging A and half B).  WG: weight groups (else row groups).  BS: row
// groups with a K-strided B.  DUALB: B rows split gate/up (row groups,
// K-contiguous B).  DUALK: K runs over (a, b0) then (a2, b1).
template <int R, bool WG, bool BS, bool DUALB, bool DUALK, int EPI>
__global__ __launch_bounds__(2 * R, R == 128 ? 2 : 1) void gemm_bwd_kernel(BwdArgs p,
                                                                         int total_tiles) {
  constexpr int BM = R, BN = R, BK = 64, CH = 8;
  constexpr int NW = R / 32;                    // waves
  constexpr int WM = 2, WN = NW / 2;            // wave grid
  constexpr int TM = BM / WM, TN = BN / WN;     // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;     // 32 x 32 fragments per wave
  constexpr int BNo = DUALB ? BN / 2 : BN;
  constexpr int RG = R / 8;                     // 8-row groups per operand tile
  constexpr bool A_STRIDED = WG;
  constexpr bool B_STRIDED = WG || BS;
  static_assert(R == 128 || R == 256, "tile side");
  static_assert(!(DUALB && B_STRIDED), "dual B needs the K-contiguous layout");
  static_assert(!DUALB || FN % 2 == 0, "dual B pairs gate and up fragments");
  extern __shared__ uint4 lds[];  // [2][(BM + BN) * CH]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool loads_a = wave < NW / 2;
  const int q = tid & (R - 1);
  const int khalf = lane >> 5;
  const int total = WG ? total_tiles : p.tile_base[p.G];
  const TileWalk walk = tile_walk(total);

  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * TM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int r = DUALB ? (j < FN / 2 ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FN / 2) * 32)
                        : wn * TN + j * 32;
    brow[j] = BM + r + (lane & 31);
  }

  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    const BwdTile ti = bwd_tile(p, WG, tile, BM, BN);
    const int Ktot = WG ? ti.rows : (DUALK ? 2 * p.Kdim : p.Kdim);
    const int nk = (Ktot + BK - 1) / BK;
    // this thread's operand, wave-uniform
    const char* base0;  // first (or only) K half
    const char* base1;  // second K half (dual K) or the up rows (dual B)
    int64_t ld;
    if (loads_a) {
      base0 = (const char*)(ti.shared ? p.a_shared : p.a);
      base1 = DUALK ? (const char*)(ti.shared ? p.a2_shared : p.a2) : base0;
      ld = p.lda;
    } else {
      const int64_t goff = (ti.shared || WG) ? 0 : (int64_t)ti.g * p.b_stride * 2;
      base0 = (const char*)(ti.shared ? p.bs0 : p.b0) + goff;
      base1 = (DUALK || DUALB) ? (const char*)(ti.shared ? p.bs1 : p.b1) + goff : base0;
      ld = p.ldb;
    }
    const bool strided = loads_a ? A_STRIDED : B_STRIDED;
    // tile-row origin of this thread's operand and its row limit
    const int r_org = loads_a ? ti.mt * BM : ti.nt * (WG ? BN : BNo);
    const int r_lim = loads_a ? (WG ? p.Mout : ti.rows) : ti.nout;

    // K-contiguous operand: chunk c = q + R i -> tile row (q >> 3) + RG i, chunk q & 7
    int64_t roff[8];
    if (!strided) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tr = (q >> 3) + RG * i;
        if (loads_a) {
          int lr = r_org + tr;
          if (lr >= r_lim) lr = r_lim - 1;
          roff[i] = bwd_row(ti, p.a_rows, p.a_div, ld, lr) * 2;
        } else {
          // dual B: tile rows [0, BN/2) gate rows, [BN/2, BN) the same up rows
          int n = r_org + ((DUALB && tr >= BN / 2) ? tr - BN / 2 : tr);
          if (n >= r_lim) n = r_lim - 1;
          roff[i] = (int64_t)n * ld * 2;
        }
      }
    }
    // K-strided operand: 8 x 8 block, tile rows rg*8 .. +7, K rows kg*8 .. +7
    const int rg = q % RG, kg = q / RG;
    int col0 = r_org + rg * 8;
    if (col0 > r_lim - 8) col0 = r_lim - 8;  // past the edge: valid memory, never stored

    uint4 st[8];
    auto load = [&](int kt) {
      int k0 = kt * BK;
      const char* bs = base0;
      if (DUALK && k0 >= p.Kdim) {
        k0 -= p.Kdim;
        bs = base1;
      }
      if (!strided) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const char* src = ((DUALB && !loads_a && (q >> 3) + RG * i >= BN / 2) ? base1 : bs) + roff[i];
          st[i] = *(const uint4*)(src + (int64_t)(k0 + (q & 7) * 8) * 2);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + kg * 8 + i;
          if (WG) {
            if (k < ti.rows) {
              const int32_t* map = loads_a ? p.a_rows : p.b_rows;
              const int div = loads_a ? p.a_div : p.b_div;
              st[i] = *(const uint4*)(bs + (bwd_row(ti, map, div, ld, k) + col0) * 2);
            } else {
              st[i] = make_uint4(0u, 0u, 0u, 0u);
            }
          } else {
            st[i] = *(const uint4*)(bs + ((int64_t)k * ld + col0) * 2);
          }
        }
      }
    };
    auto store = [&](int buf) {
      uint4* L = lds + buf * (BM + BN) * CH + (loads_a ? 0 : BM * CH);
      if (!strided) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tr = (q >> 3) + RG * i, ch = q & 7;
          L[tr * CH + (ch ^ bwd_swz(tr))] = st[i];
        }
      } else {
        // column j of the 8 x 8 block is tile row rg*8 + j at K chunk kg,
        // written as soon as it is formed
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tr = rg * 8 + j;
          L[tr * CH + (kg ^ bwd_swz(tr))] = transpose8x8_col_b16(st, j);
        }
      }
    };

    f32x16_t acc[FN][FM];  // [weight fragment][token fragment]
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.f;

    if (nk > 0) {
      load(0);
      store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) load(kt + 1);
      const uint4* s = lds + (kt & 1) * (BM + BN) * CH;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + khalf;
        bf16x8_t fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[i] = __builtin_bit_cast(bf16x8_t, s[arow[i] * CH + (ch ^ bwd_swz(arow[i]))]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[j] = __builtin_bit_cast(bf16x8_t, s[brow[j] * CH + (ch ^ bwd_swz(brow[j]))]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
      }
      if (kt + 1 < nk) store((kt + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue.  acc[j][i][v]: output row = fragment i row lane % 32,
    // output column = fragment j column 8 * (v / 4) + 4 * (lane / 32) + v % 4.
    const int mlim = WG ? p.Mout : ti.rows;
    constexpr int FO = DUALB ? FN / 2 : FN;
    constexpr bool ACT = EPI == BEPI_SWIGLU_BWD || EPI == BEPI_GELU_BWD;
    static_assert(!(ACT && DUALB), "the activation epilogues take one B operand");
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = ti.mt * BM + wm * TM + i * 32 + (lane & 31);
      if (m >= mlim) continue;
      const int64_t rowoff = WG ? (ti.shared ? 0 : (int64_t)ti.g * p.c_gstride) + (int64_t)m * p.ldc
                                : (ti.row0 + m) * p.ldc;
      if constexpr (ACT) {
        // all of this row's u (and v) runs first, then the stores
        uint2 uu[FO][4], vv[FO][4];
#pragma unroll
        for (int j = 0; j < FO; ++j)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int col = ti.nt * BNo + wn * TN + j * 32 + 4 * khalf + 8 * qq;
            if (col < ti.nout) act_bwd_load4<EPI>(p, ti, rowoff + col, uu[j][qq], vv[j][qq]);
          }
#pragma unroll
        for (int j = 0; j < FO; ++j)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int col = ti.nt * BNo + wn * TN + j * 32 + 4 * khalf + 8 * qq;
            if (col >= ti.nout) continue;
            float r0[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) r0[u] = acc[j][i][4 * qq + u];
            act_bwd_store4<EPI>(p, ti, rowoff + col, r0, uu[j][qq], vv[j][qq]);
          }
        continue;
      }
#pragma unroll
      for (int j = 0; j < FO; ++j) {
        const int cb = ti.nt * BNo + (DUALB ? wn * (TN / 2) : wn * TN) + j * 32 + 4 * khalf;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int col = cb + 8 * qq;
          if (col >= ti.nout) continue;  // nout % 64 == 0: a 4-column run is all in or all out
          const int64_t o = rowoff + col;
          float r0[4], r1[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            r0[u] = acc[j][i][4 * qq + u];
            r1[u] = DUALB ? acc[j + FN / 2][i][4 * qq + u] : 0.f;
          }
          bwd_epilogue4<EPI, WG>(p, ti, o, col, r0, r1);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 --
// One thread per output element of 16 x 16 tiles (the row-group tile table
// is built with bm = bno = 16); the same addressing and epilogues in fp32.
template <bool WG, bool BS, bool DUALB, bool DUALK, int EPI>
__global__ __launch_bounds__(256) void gemm_bwd_f32_kernel(BwdArgs p, int total_tiles) {
  const int total = WG ? total_tiles : p.tile_base[p.G];
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const BwdTile ti = bwd_tile(p, WG, tile, 16, 16);
    const int m = ti.mt * 16 + (threadIdx.x >> 4);
    const int n = ti.nt * 16 + (threadIdx.x & 15);
    const int mlim = WG ? p.Mout : ti.rows;
    if (m >= mlim || n >= ti.nout) continue;
    float s0 = 0.f, s1 = 0.f;
    const float* A0 = (const float*)(ti.shared ? p.a_shared : p.a);
    if (WG) {
      const float* B0 = (const float*)(ti.shared ? p.bs0 : p.b0);
      for (int k = 0; k < ti.rows; ++k)
        s0 += A0[bwd_row(ti, p.a_rows, p.a_div, p.lda, k) + m] *
              B0[bwd_row(ti, p.b_rows, p.b_div, p.ldb, k) + n];
    } else {
      const int64_t goff = ti.shared ? 0 : (int64_t)ti.g * p.b_stride;
      const float* B0 = (const float*)(ti.shared ? p.bs0 : p.b0) + goff;
      const float* B1 = (DUALB || DUALK) ? (const float*)(ti.shared ? p.bs1 : p.b1) + goff : B0;
      const int64_t ar = bwd_row(ti, p.a_rows, p.a_div, p.lda, m);
      for (int k = 0; k < p.Kdim; ++k) {
        const float a = A0[ar + k];
        s0 += a * (BS ? B0[(int64_t)k * p.ldb + n] : B0[(int64_t)n * p.ldb + k]);
        if (DUALB) s1 += a * B1[(int64_t)n * p.ldb + k];
      }
      if (DUALK) {
        const float* A2 = (const float*)(ti.shared ? p.a2_shared : p.a2);
        for (int k = 0; k < p.Kdim; ++k)
          s0 += A2[ar + k] * (BS ? B1[(int64_t)k * p.ldb + n] : B1[(int64_t)n * p.ldb + k]);
      }
    }
    const int64_t o = WG ? (ti.shared ? 0 : (int64_t)ti.g * p.c_gstride) + (int64_t)m * p.ldc + n
                         : (ti.row0 + m) * p.ldc + n;
    float* C = (float*)(ti.shared ? p.c_shared : p.c);
    if (EPI == BEPI_STORE || EPI == BEPI_STORE_F32) {
      if (EPI == BEPI_STORE && p.bias && !ti.shared && !WG)
        s0 += ((const float*)p.bias)[(int64_t)ti.g * p.Nout + n];
      C[o] = s0;
    } else if (EPI == BEPI_UV) {
      C[o] = s0;
      ((float*)(ti.shared ? p.c2_shared : p.c2))[o] = s1;
    } else {
      float* H = (float*)(ti.shared ? p.c3_shared : p.c3);
      const float u = C[o];
      if (EPI == BEPI_SWIGLU_BWD) {
        float* V = (float*)(ti.shared ? p.c2_shared : p.c2);
        const float v = V[o], sg = silu_f(u);
        H[o] = sg * v;
        V[o] = s0 * sg;
        C[o] = s0 * v * silu_grad_f(u);
      } else {
        H[o] = gelu_tanh_f(u);
        C[o] = s0 * gelu_tanh_grad_f(u);
      }
    }
  }
}

}  // namespace moe
