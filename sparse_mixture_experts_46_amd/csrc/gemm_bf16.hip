// Expert FFNs as grouped GEMMs on the gfx950 matrix cores (bf16 in, fp32
// accumulate).
//
// Pages (by title and section):
//   mzlw.cn "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战", section 三:
//     Expert.forward = down( silu(gate(x)) * up(x) ); the MoELayer runs one
//     expert at a time over its gathered rows and notes that production code
//     should use grouped matrix multiplication instead.
//   learnagent.wiki "混合专家模型（Mixture of Experts, MoE）", 运行示例: the GELU
//     expert Linear(h, 2h) -> GELU -> Linear(2h, h) with biases.
//   mstx.cn "MoE 如何替代 FFN？…", section 5: a shared expert that every
//     token passes through (DeepSeek-MoE); it runs here as one extra group.
//
// Host side: tile-shape choice per layer shape, the device tile tables, and
// the two launches (gate/up with the fused activation, then down).  The
// kernels are in gemm_pingpong.h and gemm_tile.h (prefill) and gemm_decode.h
// (decode).
#include "gemm_common.h"
#include "gemm_pingpong.h"
#include "gemm_decode.h"
#include "gemm_tile.h"
#include "host_device.h"
#include "moe_internal.h"

namespace moe {

// ============================================================== host =====
namespace {

int num_cus() { return device_cus(); }

// wg_per_cu: resident workgroups per CU the grid is sized for
template <int BM, int BN, int BK, int WM, int WN, int ST, int SW, bool DUAL, int EPI>
hipError_t run_tile(const GemmArgs& a, int64_t max_tiles, hipStream_t s, int wg_per_cu = 1) {
  auto kern = gemm_tile_kernel<BM, BN, BK, WM, WN, ST, SW, DUAL, EPI>;
  const size_t smem = (size_t)ST * (BM + BN) * BK * 2;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_dynamic_lds_once((const void*)kern, (int)smem, lds_set);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)num_cus() * wg_per_cu;
  if (max_tiles < grid) grid = ((max_tiles + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  kern<<<(unsigned)grid, WM * WN * 64, smem, s>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int DA, int DB, bool DUAL, int EPI>
hipError_t run_pingpong(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  auto kern = gemm_pingpong_kernel<BM, BN, WM, WN, DA, DB, DUAL, EPI>;
  // DA blocks of A and DB blocks of B, 64 K-columns (128 bytes) per row
  const size_t smem = (size_t)DA * BM * 128 + (size_t)DB * BN * 128;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_dynamic_lds_once((const void*)kern, (int)smem, lds_set);
  if (e != hipSuccess) return e;
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = ((max_tiles + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  kern<<<(unsigned)grid, 512, smem, s>>>(a);
  return hipGetLastError();
}

// Decode sizes: one workgroup per 16-row x 16 kDecodeWaves-column tile (the
// tile table is built with those dims), up to 64 waves' worth of workgroups
// per CU, a multiple of 8 (see decode_walk); bf16, INT8 or INT4 weights.
template <bool DUAL, int EPI>
hipError_t run_decode(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  int64_t grid = max_tiles;
  const int64_t cap = (int64_t)num_cus() * (64 / kDecodeWaves);
  if (grid > cap) grid = cap;
  grid = (grid + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  constexpr int nt = 64 * kDecodeWaves;
  if (a.qbits == 4)
    gemm_decode_q4_kernel<DUAL, EPI><<<(unsigned)grid, nt, 0, s>>>(a);
  else if (a.qbits == 8)
    gemm_decode_kernel<DUAL, EPI, true><<<(unsigned)grid, nt, 0, s>>>(a);
  else
    gemm_decode_kernel<DUAL, EPI, false><<<(unsigned)grid, nt, 0, s>>>(a);
  return hipGetLastError();
}

// Tile shapes by the expected rows per expert.
enum Kind { K_DECODE = 0, K_SMALL = 1, K_MID = 2, K_BIG = 3, K_TAIL = 4, K_TAIL64 = 5 };

constexpr double kDecodeRows = 24.0;  // rows per expert up to which the decode kernel runs

Kind pick_kind(double rows_per_expert) {
  if (rows_per_expert <= kDecodeRows) return K_DECODE;
  if (rows_per_expert <= 96.0) return K_SMALL;
  // 256-row tiles move fewer operand bytes per flop than 128-row ones; they
  // pay off from ~160 rows per expert on (DeepSeek-shaped prefill, ~256 rows
  // per expert: 9.6 ms with them against 10.5 ms with 128-row tiles, padding
  // included)
  if (rows_per_expert <= 160.0) return K_MID;
  return K_BIG;
}

// (BM, BN) per kind; BNo = BN/2 for the dual (SwiGLU gate/up) GEMM.
void kind_dims(Kind k, bool dual, int* bm, int* bno) {
  switch (k) {
    case K_DECODE: *bm = 16; *bno = 16 * kDecodeWaves; return;
    case K_SMALL:  *bm = 64; *bno = dual ? 128 : 256; return;
    case K_MID:    *bm = 128; *bno = dual ? 128 : 256; return;
    case K_TAIL:   *bm = 32; *bno = dual ? 32 : 64; return;
    case K_TAIL64: *bm = 64; *bno = dual ? 32 : 64; return;
    default:       *bm = 256; *bno = dual ? 128 : 256; return;
  }
}

template <bool DUAL, int EPI>
hipError_t run_kind(Kind k, const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  switch (k) {
    case K_DECODE: return run_decode<DUAL, EPI>(a, max_tiles, s);
    // swizzles: (row >> 1) & 7 for 128-byte rows, (row >> 2) & 3 for 64-byte
    // rows: conflict-free fragment reads on the 64-bank LDS
    case K_SMALL:  return run_tile<64, 256, 64, 1, 4, 2, 1, DUAL, EPI>(a, max_tiles, s);
    // 8 waves, 64 x 64 each (128 KB of LDS)
    case K_MID:    return run_pingpong<128, 256, 2, 4, 2, 3, DUAL, EPI>(a, max_tiles, s);
    // small tiles for the few leftover rows of each group, two workgroups per
    // CU, K in slices of 128 (256 contiguous bytes per weight row): many
    // workgroups share the weight stream of the touched experts
    // (256-byte LDS rows: swizzle row & 15)
    case K_TAIL:   return run_tile<32, 64, 128, 1, DUAL ? 1 : 2, 3, 0, DUAL, EPI>(a, max_tiles, s, 2);
    // the same for K not a multiple of 128
    case K_TAIL64: return run_tile<64, 64, 64, 2, DUAL ? 1 : 2, 2, 1, DUAL, EPI>(a, max_tiles, s, 1);
    // 8 waves, 64 x 128 each, ping-pong between the two waves of each SIMD;
    // two 32 KB A blocks and three 32 KB B blocks fill the 160 KB of LDS
    default:       return run_pingpong<256, 256, 4, 2, 2, 3, DUAL, EPI>(a, max_tiles, s);
  }
}

int64_t max_tiles_for(int64_t rows, int G, int bm, int64_t cols, int bno) {
  // sum over groups of ceil(M_g/bm) <= rows/bm + G
  return (rows / bm + G) * ((cols + bno - 1) / bno);
}

}  // namespace

hipError_t launch_ffn_f32(const FfnProblem& p, hipStream_t stream);

bool ffn_int8_supported(int64_t T, int K, int N) {
  return pick_kind((double)(T * K) / (double)N) == K_DECODE;
}

bool ffn_saves_uv(int64_t T, int K, int N, int act, bool bf16) {
  const Kind k = pick_kind((double)(T * K) / (double)N);
  return bf16 && act == 0 && (k == K_MID || k == K_BIG);
}

size_t ffn_workspace_bytes(int64_t T, int d, int N, int K, int F, int F_shared, bool bf16) {
  (void)d; (void)N;
  const size_t el = bf16 ? 2 : 4;
  const int Fm = F > F_shared ? F : F_shared;
  size_t h = ((size_t)T * K + (F_shared > 0 ? (size_t)T : 0)) * (size_t)Fm * el;
  return (h + 255) / 256 * 256;
}

namespace {

// The tilings of one bf16 expert-FFN launch.
struct FfnShape {
  bool swiglu, split2;
  Kind k, tk;
  int64_t rows, srows;
  int G;
  int bm1, bno1, bm2, bno2, tbm, tbno, sbm2;
};

FfnShape ffn_shape(const FfnProblem& p) {
  FfnShape f;
  f.swiglu = (p.act == 0);
  f.rows = p.T * p.K;
  f.srows = p.F_shared > 0 ? p.T : 0;
  f.G = p.N + (f.srows > 0 ? 1 : 0);
  const double rpe = (double)f.rows / (double)p.N;
  f.k = pick_kind(rpe);
  // With the largest tiles and many rows per expert (> 640) the second GEMM
  // has only d / 256 column tiles per row tile, so a partial last row tile
  // per expert can add a whole round of workgroups.  There each group's rows
  // are split: the main launch covers whole 256-row tiles (the last one at
  // least half full) and a tail launch of small tiles the remainder (< 128
  // rows).  With fewer rows per expert most experts would have a tail, each
  // streaming that expert's weights a second time.  The first GEMM, with its
  // many column tiles, always runs in one launch: a tail launch would stream
  // the touched experts' gate/up weights a second time, which costs more
  // than the partial tiles it saves.
  f.split2 = (f.k == K_BIG) && rpe > 640.0;
  kind_dims(f.k, f.swiglu, &f.bm1, &f.bno1);
  kind_dims(f.k, false, &f.bm2, &f.bno2);
  f.tk = (p.F % 128 == 0) ? K_TAIL : K_TAIL64;  // K of GEMM 2 is F
  kind_dims(f.tk, false, &f.tbm, &f.tbno);
  f.sbm2 = f.split2 ? f.bm2 : 0;
  return f;
}

}  // namespace

bool plan_expert_ffn_tiles(const FfnProblem& p, TilePlan* plan) {
  if (!p.bf16) return false;
  const FfnShape f = ffn_shape(p);
  *plan = {};
  plan->specs.s[0] = {f.bm1, f.bno1, p.F, p.F_shared, 0, 0};
  plan->specs.s[1] = {f.bm2, f.bno2, p.d, p.d, f.sbm2, 0};
  plan->specs.s[2] = {f.tbm, f.tbno, p.d, p.d, f.sbm2, 1};
  plan->nspec = f.split2 ? 3 : 2;
  plan->n_routed = p.N;
  plan->shared_rows = f.srows;
  plan->base = p.tile_base;
  // walk counters after the three tables: 8 for each ping-pong launch
  plan->ctr = p.tile_base + 3 * (p.N + 2);
  plan->nctr = kWalkCounters;
  return true;
}

hipError_t launch_expert_ffn(const FfnProblem& p, hipStream_t stream, const hipEvent_t* ev,
                             bool tables_ready) {
  auto mark = [&](int i) -> hipError_t {
    return (ev && ev[i]) ? hipEventRecord(ev[i], stream) : hipSuccess;
  };
  hipError_t err;
  if (!p.bf16) {
    if ((err = mark(0)) != hipSuccess) return err;
    if ((err = launch_ffn_f32(p, stream)) != hipSuccess) return err;
    for (int i = 1; i < 4; ++i)
      if ((err = mark(i)) != hipSuccess) return err;
    return hipSuccess;
  }
  const FfnShape f = ffn_shape(p);
  const bool swiglu = f.swiglu, split2 = f.split2;
  const Kind k = f.k, tk = f.tk;
  const int64_t rows = f.rows, srows = f.srows;
  const int G = f.G;
  const int bm1 = f.bm1, bno1 = f.bno1, bm2 = f.bm2, bno2 = f.bno2, tbm = f.tbm, tbno = f.tbno;
  const int sbm2 = f.sbm2;
  int32_t* base[3];
  for (int i = 0; i < 3; ++i) base[i] = p.tile_base + i * (p.N + 2);
  int32_t* ctr = p.tile_base + 3 * (p.N + 2);
  if (!tables_ready) {
    TilePlan plan;
    plan_expert_ffn_tiles(p, &plan);
    tile_setup_kernel<<<1, 1024, 0, stream>>>(p.offset, p.N, srows, plan.specs, plan.nspec,
                                              plan.base, plan.ctr, plan.nctr);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  const int Fm = p.F > p.F_shared ? p.F : p.F_shared;
  uint16_t* h = (uint16_t*)p.h;
  uint16_t* h_shared = h + (size_t)rows * Fm;

  // ---- GEMM 1: h = act(A W1^T [+ b1]) [* (A W3^T)]
  GemmArgs g1 = {};
  g1.a = (const uint16_t*)p.a;
  g1.a_rows = p.a_rows;
  g1.a_div = p.K;
  g1.lda = p.d;
  g1.offset = p.offset;
  g1.n_routed = p.N;
  g1.shared_rows = srows;
  g1.a_shared = (const uint16_t*)p.x_shared;
  g1.b0 = (const uint16_t*)p.w1;
  g1.b1 = (const uint16_t*)p.w3;
  g1.b_stride = (int64_t)p.F * p.d;
  g1.bs0 = (const uint16_t*)p.ws1;
  g1.bs1 = (const uint16_t*)p.ws3;
  g1.Nout = p.F;
  g1.Nout_shared = p.F_shared;
  g1.Kdim = p.d;
  g1.bias = (const uint16_t*)p.b1;
  g1.c = h;
  g1.c_shared = h_shared;
  g1.tile_base = base[0];
  g1.walk_ctr = ctr;
  g1.G = G;
  g1.split_bm = 0;
  g1.region = 0;
  if (p.save_u && p.save_v && swiglu && (k == K_MID || k == K_BIG)) {
    g1.c_u = (uint16_t*)p.save_u;
    g1.c_v = (uint16_t*)p.save_v;
    g1.cs_u = g1.c_u + (size_t)rows * p.F;  // shared rows after the routed ones (F_shared == F)
    g1.cs_v = g1.c_v + (size_t)rows * p.F;
  }
  if (p.int8 || p.int4) {
    if (k != K_DECODE) return hipErrorNotSupported;  // checked on the host before
    g1.qbits = p.int4 ? 4 : 8;
    g1.sc0 = p.w1_scale;
    g1.sc1 = p.w3_scale;
    g1.scs0 = p.ws1_scale;
    g1.scs1 = p.ws3_scale;
  }
  if ((err = mark(0)) != hipSuccess) return err;
  const int64_t mt1 = max_tiles_for(rows + srows, G, bm1, Fm, bno1);
  err = swiglu ? run_kind<true, EPI_SILU_MUL>(k, g1, mt1, stream)
               : run_kind<false, EPI_GELU>(k, g1, mt1, stream);
  if (err != hipSuccess) return err;
  if ((err = mark(1)) != hipSuccess) return err;

  // ---- GEMM 2: y = h W2^T [+ b2]
  GemmArgs g2 = {};
  g2.a = h;
  g2.a_rows = nullptr;
  g2.a_div = 1;
  g2.lda = Fm;
  g2.offset = p.offset;
  g2.n_routed = p.N;
  g2.shared_rows = srows;
  g2.a_shared = h_shared;
  g2.b0 = (const uint16_t*)p.w2;
  g2.b1 = nullptr;
  g2.b_stride = (int64_t)p.d * p.F;
  g2.bs0 = (const uint16_t*)p.ws2;
  g2.bs1 = nullptr;
  g2.Nout = p.d;
  g2.Nout_shared = p.d;
  g2.Kdim = p.F;  // (F_shared is either 0 or F: checked on the host)
  g2.bias = (const uint16_t*)p.b2;
  g2.c = (uint16_t*)p.y_perm;
  g2.c_shared = (uint16_t*)p.y_shared;
  g2.tile_base = base[1];
  g2.walk_ctr = ctr + 8;
  g2.G = G;
  g2.split_bm = sbm2;
  g2.region = 0;
  if (p.int8 || p.int4) {
    g2.qbits = p.int4 ? 4 : 8;
    g2.sc0 = p.w2_scale;
    g2.scs0 = p.ws2_scale;
  }
  const int64_t mt2 = max_tiles_for(rows + srows, G, bm2, p.d, bno2);
  err = run_kind<false, EPI_BIAS>(k, g2, mt2, stream);
  if (err != hipSuccess) return err;
  if ((err = mark(2)) != hipSuccess) return err;
  if (split2) {
    GemmArgs t2 = g2;
    t2.tile_base = base[2];
    t2.walk_ctr = nullptr;  // the tail's tile kernel walks in the fixed order
    t2.region = 1;
    // a tail is shorter than half a main tile
    const int64_t tt2 = (int64_t)G * ((sbm2 / 2 + tbm - 1) / tbm) * ((p.d + tbno - 1) / tbno);
    err = run_kind<false, EPI_BIAS>(tk, t2, tt2, stream);
    if (err != hipSuccess) return err;
  }
  return mark(3);
}

}  // namespace moe
