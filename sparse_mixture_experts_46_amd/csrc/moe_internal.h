// Internal launch interface between the C-ABI host layer (moe_api.cpp) and
// the kernel translation units.  Every launcher enqueues on `stream`, never
// synchronises, and returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Router noise of one call (the generator is described in rng.h).
struct RouterNoise {
  const float* tensor;  // [T, N] standard-normal draws of the caller, or nullptr
  float std;            // scale of the draws
  int philox;           // 1: draws made in the kernels (tensor is then nullptr)
  uint64_t seed, offset;
};

// ---------------------------------------------------------------- router --
// Tokens handled by one block of the top-K kernel (multiple of 4).
int router_tokens_per_block(int64_t T);
int64_t router_num_blocks(int64_t T);

// K splits of the logits GEMM for this shape (partials [splits, T, N]).
int router_num_splits(int64_t T, int d, int N, bool x_bf16);

// Whether the logits run as a bf16 GEMM against the exact three-part split
// of W_r (bf16 x, d a multiple of 64), and the bytes of that split's planes
// [3][N][d] bf16 (0 otherwise).
bool router_gemm_path(int64_t T, int d, int N, bool x_bf16);
size_t router_planes_bytes(int64_t T, int d, int N, bool x_bf16);

// logits = x W_r^T + b_r.  With several K splits the partial products go to
// part [splits, T, N] and (reduce_splits) a reduction writes logits;
// otherwise a top-K kernel adds them.  With one split the logits are written
// directly (part unused).  planes: scratch of router_planes_bytes (nullable
// when that is 0).
hipError_t launch_router_logits(const void* x, bool x_bf16, const float* w_r, const float* b_r,
                                uint16_t* planes, float* part, float* logits, int64_t T, int d,
                                int N, hipStream_t stream, bool reduce_splits);

// Whether router_topk_kernel adds the K splits itself (from 1024 tokens:
// with fewer, one wave per token adding many splits is latency-bound, and
// the separate reduction spreads them wider).
bool router_topk_adds_splits(int64_t T, int nsplit);

// Selection, gates and per-block partial statistics on logits + noise.std *
// (the noise draws), when noise_on(noise):
//   part_p [nblk, N] fp32, part_cnt [nblk, N] int32,
//   part_z [nblk, 3] fp32 (sum of squared logits, of squared log-sum-exp, of
//   routing entropy)
// With nsplit > 1 the logits are first reduced from the K-split partials
// part (launch_router_logits without its reduction) plus b_r and written to
// logits; with nsplit == 1 logits holds them already.
hipError_t launch_router_topk(float* logits, const float* part, int nsplit, const float* b_r,
                              const RouterNoise& noise, const float* b_sel, int32_t* idx,
                              float* gate, float* part_p, int32_t* part_cnt, float* part_z,
                              int64_t T, int N, int K, int gate_mode, hipStream_t stream);

// Few experts with bf16 x above kRouterSmallT tokens (router_fused_path:
// N <= 16): logits, top-K, gates and the per-block partials (as
// launch_router_topk) in one kernel, without K splits or planes;
// launch_router_stats follows.
bool router_fused_path(int64_t T, int N, bool x_bf16);
hipError_t launch_router_fused(const void* x, const float* w_r, const float* b_r,
                               const RouterNoise& noise, const float* b_sel, float* logits,
                               int32_t* idx, float* gate, float* part_p, int32_t* part_cnt,
                               float* part_z, int64_t T, int d, int N, int K, int gate_mode,
                               hipStream_t stream);

// Small batches (router_small_path): one workgroup reduces the logit splits
// (part from launch_router_logits without its reduction; nsplit =
// router_num_splits), selects, gates and writes the statistics.  Null
// count / f / p / loss are skipped.
constexpr int64_t kRouterSmallT = 64;
bool router_small_path(int64_t T, int N);
hipError_t launch_router_small(const float* part, int nsplit, const float* b_r,
                               const RouterNoise& noise, const float* b_sel, float* logits, int32_t* idx,
                               float* gate, int64_t T, int N, int K, int gate_mode, float alpha,
                               int32_t* count, float* f, float* p, float* loss, float* entropy,
                               float* b_sel_out, float bias_rate, hipStream_t stream);

// part_fp: [ceil(N / 64)] fp32 scratch (per-expert-block sums of f_e * p_e)
// Every output nullable; b_sel_out gets one auxiliary-loss-free step of
// b_sel (nullable = 0) and may alias it.
hipError_t launch_router_stats(const float* part_p, const int32_t* part_cnt,
                               const float* part_z, float* part_fp, int64_t nblk, int64_t T,
                               int N, int K, float alpha, int32_t* count,
                               float* f, float* p, float* loss, float* entropy,
                               const float* b_sel, float* b_sel_out, float bias_rate,
                               hipStream_t stream);

// ----------------------------------------------------------- tile tables --
// One tiling of the expert groups: tile height bm, bno output columns per
// tile, output widths of the routed / shared groups, and the row region (see
// main_rows in gemm_common.h).
struct TileSpec {
  int bm, bno, nout, nout_s, split_bm, region;
};

struct TileSpecs {
  TileSpec s[4];
};

// The tile tables of one expert-FFN launch: nspec tilings (0: none), tables
// (n_routed + 2) apart from base, and nctr walk counters at ctr to zero.
// The dispatch kernels build them at their end when given one, which saves
// the FFN its own table launch.
struct TilePlan {
  TileSpecs specs;
  int nspec;
  int n_routed;
  int64_t shared_rows;
  int32_t* base;
  int32_t* ctr;
  int nctr;
};

// -------------------------------------------------------------- dispatch --
constexpr int kDispatchTokens = 256;  // tokens per dispatch block
constexpr int kWalkCounters = 16;     // tile-walk counters of the two grouped GEMMs (8 each)
int64_t dispatch_num_blocks(int64_t T);

// plan (nullable): tile tables to build from the kept counts (see TilePlan)
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int N, int K,
                           int64_t capacity, int32_t* blk_count,
                           int32_t* blk_base, int32_t* blk_bad,
                           int32_t* kept, int32_t* offset, int32_t* pair_row,
                           int32_t* row_pair, uint8_t* dropped,
                           int32_t* counters, hipStream_t stream,
                           const TilePlan* plan = nullptr);

hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* row_pair,
                          const int32_t* offset, int N, int K, int d,
                          int64_t max_rows, void* x_perm, hipStream_t stream);

// ------------------------------------------------------------ expert FFN --
// One group of the grouped GEMMs: rows [row0, row0 + M) of the A operand,
// weights of `Nout x Kdim` (row-major, K contiguous).
struct FfnProblem {
  int64_t T;
  int d, N, K, F, F_shared;
  int act;          // moe_act_t
  bool bf16;
  const void* a;    // x_perm, or x when a_rows != nullptr
  const int32_t* a_rows;
  const int32_t* offset;  // [N+1] device
  const void *w1, *w3, *w2, *b1, *b2;
  const void *ws1, *ws3, *ws2;
  const void* x_shared;
  void* h;          // [(T*K + T_shared), max(F, F_shared)] intermediate
  void* y_perm;     // [T*K, d]
  void* y_shared;   // [T, d]
  int32_t* tile_base;  // [3 * (N + 2) + kWalkCounters] scratch: three tile tables, walk counters
  // nullable, SwiGLU: also store gate(x) = A W1^T and up(x) = A W3^T
  // ([T*K + T_shared, F], shared rows after the routed ones) when the first
  // GEMM runs the ping-pong kernel (ffn_saves_uv)
  void* save_u;
  void* save_v;
  // weight-only INT8 (w1/w3/w2/ws* hold int8 codes, per-output-row scales)
  // or INT4 (packed codes, one scale per 128 K of a row)
  bool int8, int4;
  const float *w1_scale, *w3_scale, *w2_scale, *ws1_scale, *ws3_scale, *ws2_scale;
};

// INT8 / INT4 weights are supported where the decode kernel runs: at most
// this many routed rows per expert on average.
bool ffn_int8_supported(int64_t T, int K, int N);

// Whether launch_expert_ffn stores gate(x) and up(x) when asked (bf16
// SwiGLU layers whose first GEMM runs the ping-pong kernel).
bool ffn_saves_uv(int64_t T, int K, int N, int act, bool bf16);

size_t ffn_workspace_bytes(int64_t T, int d, int N, int K, int F, int F_shared,
                           bool bf16);
// The tile tables launch_expert_ffn(p) uses; false when it uses none (fp32
// layers).
bool plan_expert_ffn_tiles(const FfnProblem& p, TilePlan* plan);

// ev (nullable, else 4 nullable events): recorded before the first grouped
// GEMM, after it, after the main launch of the second grouped GEMM and after
// its tail launch.  tables_ready: the tables of plan_expert_ffn_tiles(p) were
// built on the stream already (by the dispatch), so they are not built again.
hipError_t launch_expert_ffn(const FfnProblem& p, hipStream_t stream, const hipEvent_t* ev,
                             bool tables_ready = false);

// ----------------------------------------------------------- quantization --
// w bf16 [rows, cols] -> q int8 [rows, cols], scale fp32 [rows]; cols % 8 == 0
hipError_t launch_quantize_int8(const void* w, int64_t rows, int cols, int8_t* q, float* scale,
                                hipStream_t stream);
// w bf16 [rows, cols] -> q [rows, cols / 2] packed INT4 codes, scale fp32
// [rows, cols / 128]; cols % 128 == 0
hipError_t launch_quantize_int4(const void* w, int64_t rows, int cols, uint8_t* q, float* scale,
                                hipStream_t stream);

// --------------------------------------------------------------- combine --
hipError_t launch_combine(const void* y_perm, const int32_t* pair_row,
                          const float* gate, const void* y_shared, void* y,
                          int64_t T, int d, int K, bool bf16,
                          hipStream_t stream);

// -------------------------------------------------------------- backward --
// The backward pass (backward.hip).  Every GEMM operand and output is in the
// layer dtype unless noted; rows = T*K routed rows then T shared rows.
hipError_t launch_combine_backward(const void* dy, const void* y_perm, const float* gate,
                                   const int32_t* pair_row, int64_t T, int K, int d, bool bf16,
                                   void* d_perm, float* dgate, hipStream_t stream);

// part: [router_bwd_num_blocks(T), N] fp32 scratch; db_r nullable.
int64_t router_bwd_num_blocks(int64_t T);
hipError_t launch_router_backward(const float* logits, const RouterNoise& noise,
                                  const int32_t* idx, const int32_t* pair_row, const float* dgate,
                                  const int32_t* count, int64_t T, int N, int K, int gate_mode,
                                  float alpha, float c_aux, float c_z, float c_zlse,
                                  float* dlogits, float* part, float* db_r, hipStream_t stream);

// dW_r = dlogits^T x; part: [router_dw_splits(T, N), N, d] fp32 scratch (unused
// with one split).  T > 0.
int router_dw_splits(int64_t T, int N);
hipError_t launch_router_dw(const float* dl, const void* x, bool bf16, int64_t T, int N, int d,
                            float* part, float* dw_r, hipStream_t stream);

// dx = sum of the token's kept rows of dx_perm (+ the planes2 planes of
// dx_perm2, [planes2][T*K, d]) (+ dx_shared (+ the planes of dx_shared2,
// [planes2][T, d])) (+ dl W_r); the second buffers are nullable.
hipError_t launch_dx(const void* dx_perm, const int32_t* pair_row, int K, const void* dx_shared,
                     const float* dl, const float* w_r, int N, int64_t T, int d, bool bf16,
                     void* dx, hipStream_t stream, const void* dx_perm2 = nullptr,
                     const void* dx_shared2 = nullptr, int planes2 = 0);

struct FfnBwdProblem {
  int64_t T;
  int d, N, K, F, F_shared;
  int act;  // moe_act_t
  bool bf16;
  const void* x;            // [T, d] layer input (rows gathered through row_pair / K)
  const int32_t* row_pair;  // [T*K]
  const int32_t* offset;    // [N+1]
  const void *w1, *w3, *w2, *b1;
  const void *ws1, *ws3, *ws2;
  const void* d_perm;       // [T*K, d] gradient of each kept row's expert output
  const void* dy;           // [T, d] gradient of the shared expert's output
  void* dx_perm;            // [T*K, d] out: gradient of each kept row's input
  void* dx_shared;          // [T, d] out (shared expert only)
  // nullable: with them (SwiGLU, 256-row tiles) dx_perm / dx_shared get the
  // first of ffn_backward_dx_parts parts of the K sum (du W1 + dv W3) and
  // these, [parts - 1][rows, d], the others; the caller adds them
  void* dx_perm2;
  void* dx_shared2;
  // nullable: gate(x) and up(x) saved by the forward (layout of save_u /
  // save_v); with them the first GEMM is not recomputed
  const void* u_in;
  const void* v_in;
  void *dw1, *dw3, *dw2, *db1, *db2, *dws1, *dws3, *dws2;  // out
  void* ws;                 // ffn_backward_workspace_bytes
  // nullable, else 5 nullable events recorded after the recompute, the dh
  // GEMM, dw2, dx_perm and dw1 (dw3)
  const hipEvent_t* ev;
};
size_t ffn_backward_workspace_bytes(int64_t T, int d, int N, int K, int F, int F_shared, bool bf16);
// Parts (1, 2 or 4) in which launch_expert_ffn_backward, given dx_perm2 /
// dx_shared2, computes dx_perm for this shape (1: it leaves them unwritten).
int ffn_backward_dx_parts(int64_t T, int N, int K, int F, int d, int act, bool bf16);
hipError_t launch_expert_ffn_backward(const FfnBwdProblem& p, hipStream_t stream);

// Fill n bytes at p with zeros (a kernel, so it can be captured in a graph).
hipError_t launch_zero(void* p, size_t n, hipStream_t stream);

}  // namespace moe
