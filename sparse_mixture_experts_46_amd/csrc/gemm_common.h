// Grouped-GEMM plumbing shared by the tile (prefill) and skinny (decode)
// kernels: the argument block, the device-side tile table and epilogues.
//
// A group g is one expert: rows [offset[g], offset[g+1]) of the
// expert-contiguous row space and weights W_g of shape [Nout, Kdim] with K
// contiguous, so every GEMM is C = A B^T with both operands K-contiguous.
// Group N (when present) is the shared expert over all T tokens.
#pragma once

#include "moe_common.h"

namespace moe {

enum { EPI_SILU_MUL = 0, EPI_GELU = 1, EPI_BIAS = 2 };

struct GemmArgs {
  const uint16_t* a;        // routed A rows (x_perm / h), or x when a_rows
  const int32_t* a_rows;    // nullable gather map: row r -> a[a_rows[r] / a_div]
  int a_div;
  int64_t lda;
  const int32_t* offset;    // [n_routed + 1] row offsets of the routed groups
  int n_routed;
  int64_t shared_rows;      // rows of the shared group (0 = none)
  const uint16_t* a_shared; // A of the shared group
  const uint16_t* b0;       // routed weights (gate / single), [n_routed, Nout, Kdim]
  const uint16_t* b1;       // routed up weights (SwiGLU)
  int64_t b_stride;         // Nout * Kdim
  const uint16_t* bs0;      // shared weights
  const uint16_t* bs1;
  int Nout, Nout_shared, Kdim;
  const uint16_t* bias;     // routed bias [n_routed, Nout] (nullable)
  uint16_t* c;              // routed output [rows, Nout]
  uint16_t* c_shared;       // shared output [shared_rows, Nout_shared]
  const int32_t* tile_base; // [G + 1]
  int G;
};

template <int EPI>
__device__ __forceinline__ float epi1(float acc, float bias) {
  if (EPI == EPI_GELU) return gelu_tanh_f(acc + bias);
  return acc + bias;
}

// Resolve tile -> (group, first row, rows, output columns, A/B/C pointers).
struct TileInfo {
  int g, M, Nout, mt, nt;
  bool shared;
  int64_t row0;
};

__device__ __forceinline__ TileInfo resolve_tile(const GemmArgs& p, int tile, int BM, int BNo) {
  TileInfo ti;
  ti.g = find_group(p.tile_base, p.G, tile);
  const int local = tile - p.tile_base[ti.g];
  ti.shared = (ti.g == p.n_routed);
  ti.row0 = ti.shared ? 0 : p.offset[ti.g];
  ti.M = ti.shared ? (int)p.shared_rows : (int)(p.offset[ti.g + 1] - ti.row0);
  ti.Nout = ti.shared ? p.Nout_shared : p.Nout;
  const int mtiles = (ti.M + BM - 1) / BM;
  ti.mt = local % mtiles;
  ti.nt = local / mtiles;
  (void)BNo;
  return ti;
}


// ------------------------------------------------------------ tile setup --
// tile_base[g] = sum_{g' < g} ceil(M_g'/BM) * ceil(Nout_g'/BNo), for two
// tilings at once (first and second GEMM).  One block of 1024 threads.
__global__ __launch_bounds__(1024) void tile_setup_kernel(
    const int32_t* __restrict__ offset, int n_routed, int64_t shared_rows,
    int bm1, int bno1, int nout1, int nout1_s, int bm2, int bno2, int nout2,
    int nout2_s, int32_t* __restrict__ base1, int32_t* __restrict__ base2) {
  __shared__ int32_t s1[2048], s2[2048];
  const int G = n_routed + (shared_rows > 0 ? 1 : 0);
  for (int g = threadIdx.x; g < 2048; g += 1024) {
    int32_t t1 = 0, t2 = 0;
    if (g < G) {
      int64_t M = g < n_routed ? (int64_t)(offset[g + 1] - offset[g]) : shared_rows;
      int n1 = g < n_routed ? nout1 : nout1_s, n2 = g < n_routed ? nout2 : nout2_s;
      t1 = (int32_t)(((M + bm1 - 1) / bm1) * ((n1 + bno1 - 1) / bno1));
      t2 = (int32_t)(((M + bm2 - 1) / bm2) * ((n2 + bno2 - 1) / bno2));
    }
    s1[g] = t1; s2[g] = t2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // G <= 1025: a short serial scan is enough
    int32_t r1 = 0, r2 = 0;
    for (int g = 0; g < G; ++g) {
      base1[g] = r1; base2[g] = r2;
      r1 += s1[g]; r2 += s2[g];
    }
    base1[G] = r1; base2[G] = r2;
  }
}


}  // namespace moe
