// Dispatch: per-expert counts, capacity clamp in token order, the layout of
// the kept (token, slot) pairs in expert-contiguous rows, and the gather of
// the kept tokens into those rows.
//
// Pages (by title and section):
//   mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战": 2.3 (capacity
//     floor(K/N * CF * S); tokens over an expert's capacity are dropped and
//     reach the next layer through the residual path), section 三 (MoELayer:
//     for each expert, the ascending list of tokens that chose it is cut to
//     `capacity` and those rows are gathered; the per-expert loop is to be
//     replaced by grouped matrix multiplication).
//
// Token order without atomics on the ranks: every block of 256 tokens
// builds, in LDS, one bit per (expert, token) for the tokens that chose the
// expert.  The in-block rank of a pair is the popcount of the expert's bits
// below its token; the rank across blocks adds an exclusive scan of the
// per-block counts.  Everything is integer and deterministic.
#include "gemm_common.h"  // build_tile_tables
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int DT = kDispatchTokens;   // tokens per block
constexpr int DW = DT / 32;           // 32-bit words per expert bitmap

// A token's K expert ids, loaded once (independent loads, not one dependent
// load per comparison), and the mask of its slots whose id is out of range
// or repeats an earlier slot's id.
struct TokenIds {
  int32_t e[kMaxTopK];
  uint32_t bad;
};
__device__ __forceinline__ TokenIds load_token(const int32_t* __restrict__ idx, int64_t t, int N,
                                               int K) {
  TokenIds r;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) r.e[k] = k < K ? idx[t * K + k] : -1;
  r.bad = 0u;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    bool bad = r.e[k] < 0 || r.e[k] >= N;
#pragma unroll
    for (int k2 = 0; k2 < k; ++k2) bad = bad || r.e[k2] == r.e[k];
    if (k < K && bad) r.bad |= 1u << k;
  }
  return r;
}

// Fills the block's bitmap from the tokens' ids (tk of token t, valid if
// t < T).
__device__ __forceinline__ void build_bitmap(const TokenIds& tk, int64_t T, int N, int K,
                                             uint32_t* bm, int64_t t, int local, int nthreads) {
  for (int i = threadIdx.x; i < N * DW; i += nthreads) bm[i] = 0u;
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
      if (k < K && !((tk.bad >> k) & 1u))
        atomicOr(&bm[tk.e[k] * DW + (local >> 5)], 1u << (local & 31));
  }
  __syncthreads();
}

__global__ __launch_bounds__(DT) void dispatch_hist_kernel(
    const int32_t* __restrict__ idx, int64_t T, int N, int K,
    int32_t* __restrict__ blk_count, int32_t* __restrict__ blk_bad) {
  extern __shared__ uint32_t bm[];
  __shared__ int nbad;
  const int local = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * DT + local;
  if (local == 0) nbad = 0;
  const TokenIds tk = t < T ? load_token(idx, t, N, K) : TokenIds{};
  build_bitmap(tk, T, N, K, bm, t, local, DT);
  if (t < T) {
    const int mybad = __popc(tk.bad);
    if (mybad) atomicAdd(&nbad, mybad);  // integer: order-independent
  }
  for (int e = local; e < N; e += DT) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < DW; ++w) c += __popc(bm[e * DW + w]);
    blk_count[(int64_t)blockIdx.x * N + e] = c;
  }
  __syncthreads();
  if (local == 0) blk_bad[blockIdx.x] = nbad;
}

// Exclusive scan of skept[0..N) (N <= 1024) by a block of 1024 threads, with
// scan[] as LDS scratch: offset[e] (global) and, if soff is given, the same
// in LDS; offset[N] = the total, which every thread gets back.
__device__ __forceinline__ int32_t scan_kept(const int32_t* skept, int32_t* scan, int N,
                                             int32_t* __restrict__ offset, int32_t* soff) {
  const int tid = threadIdx.x;
  const int32_t v = tid < N ? skept[tid] : 0;
  scan[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t add = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  if (tid < N) {
    offset[tid] = scan[tid] - v;
    if (soff) soff[tid] = scan[tid] - v;
  }
  const int32_t total = scan[1023];
  if (tid == 0) offset[N] = total;
  __syncthreads();
  return total;
}

// Experts with at least one kept row, counted by a block of 1024 threads
// (N <= 1024: one expert per thread); every thread gets the count.
__device__ __forceinline__ int count_touched(const int32_t* skept, int N) {
  const int tid = threadIdx.x;
  return __syncthreads_count(tid < N && skept[tid] > 0);
}

// counters = {kept rows, dropped pairs, bad ids, touched experts}
__device__ __forceinline__ void write_counters(int32_t* __restrict__ counters, int32_t total,
                                               int64_t T, int K, int64_t bad, int touched) {
  counters[0] = total;
  counters[1] = (int32_t)(T * K - total);
  counters[2] = (int32_t)bad;
  counters[3] = touched;
}

// One block of 1024 threads: per-expert exclusive scan over blocks (token
// order), capacity clamp, exclusive scan of kept rows over experts.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t* __restrict__ blk_count, const int32_t* __restrict__ blk_bad,
    int64_t nblk, int64_t T, int N, int K, int64_t cap,
    int32_t* __restrict__ blk_base, int32_t* __restrict__ kept_out,
    int32_t* __restrict__ offset, int32_t* __restrict__ counters, TilePlan plan) {
  __shared__ int32_t skept[kMaxExperts];
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < N; e += 1024) {
    // eight block counts loaded before they are scanned: one dependent load
    // per block made this latency-bound
    int32_t run = 0;
    int64_t b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blk_count[(b + u) * N + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        blk_base[(b + u) * N + e] = run;
        run += c[u];
      }
    }
    for (; b < nblk; ++b) {
      int32_t c = blk_count[b * N + e];
      blk_base[b * N + e] = run;
      run += c;
    }
    int32_t kp = (int64_t)run < cap ? run : (int32_t)cap;
    skept[e] = kp;
    if (kept_out) kept_out[e] = kp;
  }
  __syncthreads();
  const int32_t total = scan_kept(skept, scan, N, offset, nullptr);
  const int touched = count_touched(skept, N);
  if (counters) {  // bad ids: per-thread strided sums, then thread 0 adds them
    int64_t bad = 0;
    for (int64_t b = tid; b < nblk; b += 1024) bad += blk_bad[b];
    scan[tid] = (int32_t)bad;  // scan[] is free again after scan_kept
    __syncthreads();
    if (tid == 0) {
      int64_t all = 0;
      const int nt = nblk < 1024 ? (int)nblk : 1024;
      for (int i = 0; i < nt; ++i) all += scan[i];
      write_counters(counters, total, T, K, all, touched);
    }
    __syncthreads();
  }
  if (plan.nspec > 0)  // the expert FFN's tile tables, from the kept counts
    build_tile_tables([&](int g) { return skept[g]; }, plan.n_routed, plan.shared_rows, plan.specs,
                      plan.nspec, plan.base, plan.ctr, plan.nctr);
}

// Rows of token t's slots: rank among the tokens that chose the expert =
// base[e] (earlier blocks; 0 if base is null) + the bits of this block's
// bitmap below the token; kept iff rank < cap, at row off[e] + rank.
__device__ __forceinline__ void assign_token(const TokenIds& tk, int64_t t,
                                             int local, int N, int K, int64_t cap,
                                             const uint32_t* bm, const int32_t* base,
                                             const int32_t* off, int32_t* __restrict__ pair_row,
                                             int32_t* __restrict__ row_pair,
                                             uint8_t* __restrict__ dropped) {
  const int w = local >> 5;
  const uint32_t below = (1u << (local & 31)) - 1u;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= K) continue;
    const int64_t pr = t * K + k;
    const int e = tk.e[k];
    const bool bad = (tk.bad >> k) & 1u;
    int32_t row = -1;
    if (!bad) {
      int r = 0;
      for (int w2 = 0; w2 < w; ++w2) r += __popc(bm[e * DW + w2]);
      r += __popc(bm[e * DW + w] & below);
      int64_t rank = (int64_t)(base ? base[e] : 0) + r;
      if (rank < cap) {
        row = off[e] + (int32_t)rank;
        row_pair[row] = (int32_t)pr;
      }
    }
    pair_row[pr] = row;
    if (dropped) dropped[pr] = row < 0 ? 1 : 0;
  }
}

__global__ __launch_bounds__(DT) void dispatch_assign_kernel(
    const int32_t* __restrict__ idx, int64_t T, int N, int K, int64_t cap,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offset,
    int32_t* __restrict__ pair_row, int32_t* __restrict__ row_pair,
    uint8_t* __restrict__ dropped) {
  extern __shared__ uint32_t bm[];
  const int local = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * DT + local;
  const TokenIds tk = t < T ? load_token(idx, t, N, K) : TokenIds{};
  build_bitmap(tk, T, N, K, bm, t, local, DT);
  if (t >= T) return;
  assign_token(tk, t, local, N, K, cap, bm, blk_base + (int64_t)blockIdx.x * N, offset, pair_row,
               row_pair, dropped);
}

// All of the above in one block of 1024 threads when every token fits one
// dispatch block (T <= DT): the bitmap is built once, block bases are zero,
// and the offsets stay in LDS for the assignment.  Saves two launches on
// decode-sized batches.
__global__ __launch_bounds__(1024) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int64_t T, int N, int K, int64_t cap,
    int32_t* __restrict__ kept_out, int32_t* __restrict__ offset,
    int32_t* __restrict__ counters, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ row_pair, uint8_t* __restrict__ dropped, TilePlan plan) {
  extern __shared__ uint32_t bm[];
  __shared__ int32_t skept[kMaxExperts];
  __shared__ int32_t soff[kMaxExperts];
  __shared__ int32_t scan[1024];
  __shared__ int nbad;
  const int local = threadIdx.x;
  const int64_t t = local < DT ? (int64_t)local : T;  // threads past DT: no token
  if (local == 0) nbad = 0;
  const TokenIds tk = t < T ? load_token(idx, t, N, K) : TokenIds{};
  build_bitmap(tk, T, N, K, bm, t, local, 1024);
  if (t < T) {
    const int mybad = __popc(tk.bad);
    if (mybad) atomicAdd(&nbad, mybad);  // integer: order-independent
  }
  for (int e = local; e < N; e += 1024) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < DW; ++w) c += __popc(bm[e * DW + w]);
    const int32_t kp = (int64_t)c < cap ? c : (int32_t)cap;
    skept[e] = kp;
    if (kept_out) kept_out[e] = kp;
  }
  __syncthreads();
  const int32_t total = scan_kept(skept, scan, N, offset, soff);
  const int touched = count_touched(skept, N);
  if (local == 0 && counters) write_counters(counters, total, T, K, nbad, touched);
  if (t < T) assign_token(tk, t, local, N, K, cap, bm, nullptr, soff, pair_row, row_pair, dropped);
  if (plan.nspec > 0)  // the expert FFN's tile tables, from the kept counts
    build_tile_tables([&](int g) { return skept[g]; }, plan.n_routed, plan.shared_rows, plan.specs,
                      plan.nspec, plan.base, plan.ctr, plan.nctr);
}

// x_perm[r] = x[row_pair[r] / K] for r < offset[N]; 16-byte chunks.
__global__ __launch_bounds__(256) void permute_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ row_pair,
    const int32_t* __restrict__ offset, int N, int K, int chunks,
    uint4* __restrict__ x_perm) {
  const int total = offset[N];
  for (int r = blockIdx.x; r < total; r += gridDim.x) {
    const int64_t src = row_pair[r] / K;
    const uint4* s = x + src * chunks;
    uint4* dst = x_perm + (int64_t)r * chunks;
    for (int c = threadIdx.x; c < chunks; c += 256) dst[c] = s[c];
  }
}

}  // namespace

int64_t dispatch_num_blocks(int64_t T) { return (T + DT - 1) / DT; }

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int N, int K,
                           int64_t capacity, int32_t* blk_count,
                           int32_t* blk_base, int32_t* blk_bad,
                           int32_t* kept, int32_t* offset, int32_t* pair_row,
                           int32_t* row_pair, uint8_t* dropped,
                           int32_t* counters, hipStream_t stream, const TilePlan* plan) {
  const int64_t nblk = dispatch_num_blocks(T);
  const size_t smem = (size_t)N * DW * sizeof(uint32_t);
  const int64_t cap = capacity < 0 ? T : capacity;
  TilePlan tp = {};
  if (plan) {
    // the tables' groups are the dispatch's experts
    if (plan->n_routed != N || plan->nspec < 0 || plan->nspec > 4) return hipErrorInvalidValue;
    tp = *plan;
  }
  if (nblk == 1) {
    dispatch_small_kernel<<<1, 1024, smem, stream>>>(idx, T, N, K, cap, kept, offset, counters,
                                                     pair_row, row_pair, dropped, tp);
    return hipGetLastError();
  }
  dispatch_hist_kernel<<<(unsigned)nblk, DT, smem, stream>>>(idx, T, N, K, blk_count, blk_bad);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dispatch_scan_kernel<<<1, 1024, 0, stream>>>(blk_count, blk_bad, nblk, T, N, K, cap,
                                               blk_base, kept, offset, counters, tp);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  dispatch_assign_kernel<<<(unsigned)nblk, DT, smem, stream>>>(
      idx, T, N, K, cap, blk_base, offset, pair_row, row_pair, dropped);
  return hipGetLastError();
}

hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* row_pair,
                          const int32_t* offset, int N, int K, int d,
                          int64_t max_rows, void* x_perm, hipStream_t stream) {
  const int chunks = d * elem_bytes / 16;
  int64_t grid = max_rows < 4096 ? max_rows : 4096;
  if (grid < 1) grid = 1;
  permute_kernel<<<(unsigned)grid, 256, 0, stream>>>((const uint4*)x, row_pair, offset, N, K,
                                                     chunks, (uint4*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
