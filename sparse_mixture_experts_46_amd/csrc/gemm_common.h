// Grouped-GEMM plumbing shared by the tile (prefill) and decode
// kernels: the argument block, the device-side tile table and epilogues.
//
// A group g is one expert: rows [offset[g], offset[g+1]) of the
// expert-contiguous row space and weights W_g of shape [Nout, Kdim] with K
// contiguous, so every GEMM is C = A B^T with both operands K-contiguous.
// Group N (when present) is the shared expert over all T tokens.
#pragma once

#include "moe_common.h"
#include "moe_internal.h"  // TileSpecs

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
  int split_bm;             // 0: one launch covers every row; else see main_rows()
  int region;               // 0: main rows of each group, 1: the tail rows
  // weight-only INT8 / INT4 (decode kernels only): b0/b1/bs0/bs1 then hold
  // int8 codes or packed INT4 codes and these their scales: INT8 one per
  // output row, [n_routed, Nout] / [Nout]; INT4 one per 128 K of a row,
  // [n_routed, Nout, Kdim / 128] / [Nout, Kdim / 128]
  int qbits;  // 0: weights in bf16, 8: INT8, 4: INT4
  const float* sc0;
  const float* sc1;
  const float* scs0;
  const float* scs1;
  // nullable (ping-pong kernel only, with a grid that is a multiple of 8): 8
  // zeroed counters, one per XCD, for the dynamic tile order
  int32_t* walk_ctr;
  // nullable (SwiGLU first GEMM, ping-pong kernel only): also store the
  // gate and up products A W1^T and A W3^T, routed [rows, Nout] / shared
  uint16_t* c_u;
  uint16_t* c_v;
  uint16_t* cs_u;
  uint16_t* cs_v;
};

// Rows [0, main_rows) of a group go to the main launch, in tiles of split_bm
// rows whose last one is at least half full; the remaining rows (fewer than
// split_bm / 2) go to the tail launch, which uses small tiles.  Without a
// split the main launch covers every row.
__host__ __device__ __forceinline__ int main_rows(int M, int split_bm) {
  if (split_bm <= 0) return M;
  const int full = M / split_bm, rem = M % split_bm;
  const int cov = (full + (2 * rem >= split_bm ? 1 : 0)) * split_bm;
  return cov < M ? cov : M;
}

__host__ __device__ __forceinline__ void region_rows(int M, int split_bm, int region, int* first,
                                                     int* count) {
  const int cov = main_rows(M, split_bm);
  *first = region == 0 ? 0 : cov;
  *count = region == 0 ? cov : M - cov;
}

template <int EPI>
__device__ __forceinline__ float epi1(float acc, float bias) {
  if (EPI == EPI_GELU) return gelu_tanh_f(acc + bias);
  return acc + bias;
}

// Order in which a persistent workgroup visits the tile table.  Workgroups
// are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8).
// With at least as many tiles as workgroups, each round of nb tiles is cut
// into 8 contiguous runs, one per XCD, so an XCD works on neighbouring tiles
// (same expert, adjacent columns) that share its L2 while all XCDs stay on
// the same stretch of the table.  With fewer tiles than workgroups the tiles
// are cut into 8 contiguous ranges of ceil(total / 8), so every XCD has work.
struct TileWalk {
  int tile, step, end;
};
__device__ __forceinline__ TileWalk tile_walk(int total) {
  const int nb = gridDim.x, bid = blockIdx.x;
  TileWalk w;
  w.step = nb;
  w.end = total;
  if ((nb & 7) != 0) {
    w.tile = bid;
  } else if (total >= nb) {
    w.tile = (bid & 7) * (nb >> 3) + (bid >> 3);
  } else {  // one round: at most one tile per workgroup
    const int per = (total + 7) >> 3, x = bid & 7;
    w.tile = x * per + (bid >> 3);
    w.end = (x + 1) * per < total ? (x + 1) * per : total;
  }
  return w;
}

// Dynamic order (kernels given 8 zeroed counters): the tile table is cut
// into 8 contiguous ranges of equal tile count, range x for XCD x.  A
// workgroup's first tile is the (bid >> 3)-th of its XCD's range; after
// that it takes the next untaken tile of that range from the XCD's counter,
// so the workgroups of one XCD always hold neighbouring tiles (the same
// expert's rows and weight columns, sharing the XCD's L2) however long each
// tile took.  A workgroup whose range is used up takes tiles from the next
// XCDs' ranges in turn; -1 when every range is used up.  Which workgroup
// computes a tile does not change the tile's result.
struct DynWalk {
  int x, nb8, probe, total;
};
__device__ __forceinline__ int dyn_lo(int total, int x) { return (int)(((int64_t)total * x) >> 3); }
__device__ __forceinline__ int dyn_first(DynWalk& w, int total) {
  w.x = blockIdx.x & 7;
  w.nb8 = gridDim.x >> 3;
  w.probe = 0;
  w.total = total;
  const int t = dyn_lo(total, w.x) + (int)(blockIdx.x >> 3);
  return t < dyn_lo(total, w.x + 1) ? t : -2;  // -2: ask the counters
}
// One thread of the workgroup calls this.
__device__ __forceinline__ int dyn_next(DynWalk& w, int32_t* ctr) {
  while (w.probe < 8) {
    const int y = (w.x + w.probe) & 7;
    const int t = dyn_lo(w.total, y) + w.nb8 + atomicAdd(&ctr[y], 1);
    if (t < dyn_lo(w.total, y + 1)) return t;
    ++w.probe;
  }
  return -1;
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
  const int64_t g0 = ti.shared ? 0 : p.offset[ti.g];
  const int Mg = ti.shared ? (int)p.shared_rows : (int)(p.offset[ti.g + 1] - g0);
  int first, count;
  region_rows(Mg, p.split_bm, p.region, &first, &count);
  ti.row0 = g0 + first;
  ti.M = count;
  ti.Nout = ti.shared ? p.Nout_shared : p.Nout;
  const int mtiles = (ti.M + BM - 1) / BM;
  ti.mt = local % mtiles;
  ti.nt = local / mtiles;
  (void)BNo;
  return ti;
}

// ------------------------------------------------------------ tile setup --
// base[k][g] = sum_{g' < g} tiles of group g' under spec k (k < nspec); tables
// are (n_routed + 2) apart, and base[k][G] is the total.  Also zeroes nctr
// walk counters at ctr.  Called by every thread of one block of 1024
// threads; rows(g) gives the rows of group g (the shared group is n_routed).
template <class Rows>
__device__ __forceinline__ void build_tile_tables(Rows rows, int n_routed, int64_t shared_rows,
                                                  const TileSpecs& specs, int nspec,
                                                  int32_t* __restrict__ base,
                                                  int32_t* __restrict__ ctr, int nctr) {
  __shared__ int32_t cnt[4][1040];
  if ((int)threadIdx.x < nctr) ctr[threadIdx.x] = 0;
  const int G = n_routed + (shared_rows > 0 ? 1 : 0);
  for (int g = threadIdx.x; g < G; g += 1024) {
    const int M = g < n_routed ? rows(g) : (int)shared_rows;
    for (int k = 0; k < nspec; ++k) {
      const TileSpec& sp = specs.s[k];
      int first, count;
      region_rows(M, sp.split_bm, sp.region, &first, &count);
      const int n = g < n_routed ? sp.nout : sp.nout_s;
      cnt[k][g] = ((count + sp.bm - 1) / sp.bm) * ((n + sp.bno - 1) / sp.bno);
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nspec) {  // G <= 1025: a short serial scan per table
    const int k = threadIdx.x;
    int32_t* b = base + (int64_t)k * (n_routed + 2);
    int32_t r = 0;
    for (int g = 0; g < G; ++g) {
      b[g] = r;
      r += cnt[k][g];
    }
    b[G] = r;
  }
}

// The tables from the dispatch offsets (the FFN's own launch).  One block
// of 1024 threads.
static __global__ __launch_bounds__(1024) void tile_setup_kernel(
    const int32_t* __restrict__ offset, int n_routed, int64_t shared_rows, TileSpecs specs,
    int nspec, int32_t* __restrict__ base, int32_t* __restrict__ ctr = nullptr, int nctr = 0) {
  build_tile_tables([&](int g) { return (int)(offset[g + 1] - offset[g]); }, n_routed,
                    shared_rows, specs, nspec, base, ctr, nctr);
}

}  // namespace moe
