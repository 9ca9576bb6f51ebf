// libmoe C ABI: argument checks, workspace layout and the launch sequence
// of the MoE layer forward.  Host code only; kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

moe_status_t check_config(const moe_config_t* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->d <= 0 || c->N <= 0 || c->K <= 0 || c->F <= 0 || c->F_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->K > c->N) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_SWIGLU && c->act != MOE_ACT_GELU_TANH) return MOE_ERR_INVALID_ARG;
  if (c->gate < MOE_GATE_RENORM_ALL || c->gate > MOE_GATE_PROB_NO_RENORM) return MOE_ERR_INVALID_ARG;
  if (c->flags & ~(uint32_t)MOE_FLAG_NOISE_PHILOX) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->aux_alpha)) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->noise_std) || !std::isfinite(c->bias_rate)) return MOE_ERR_INVALID_ARG;
  if (c->weight_format != MOE_WEIGHTS_DTYPE && c->weight_format != MOE_WEIGHTS_INT8 &&
      c->weight_format != MOE_WEIGHTS_INT4)
    return MOE_ERR_INVALID_ARG;
  if (c->weight_format != MOE_WEIGHTS_DTYPE &&
      (c->dtype != MOE_BF16 || c->act != MOE_ACT_SWIGLU || !ffn_int8_supported(c->T, c->K, c->N)))
    return MOE_ERR_UNSUPPORTED;
  // INT4 scales cover 128 consecutive K of a row: both GEMMs' K must be whole groups
  if (c->weight_format == MOE_WEIGHTS_INT4 && (c->d % 128 || c->F % 128 || c->F_shared % 128))
    return MOE_ERR_UNSUPPORTED;
  if (c->N > MOE_MAX_EXPERTS || c->K > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (c->d % 64 || c->F % 64 || c->F_shared % 64) return MOE_ERR_UNSUPPORTED;
  if (c->F_shared != 0 && (c->F_shared != c->F || c->act != MOE_ACT_SWIGLU)) return MOE_ERR_UNSUPPORTED;
  if (c->T > (int64_t(1) << 24)) return MOE_ERR_UNSUPPORTED;
  if (c->T * c->K > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_BF16) {
    // the grouped GEMMs address x, h and one expert's weights with 32-bit
    // byte offsets from a single base
    const int64_t lim = int64_t(1) << 32;
    const int64_t fm = c->F > c->F_shared ? c->F : c->F_shared;
    const int64_t h_rows = c->T * c->K + (c->F_shared > 0 ? c->T : 0);
    if (2 * c->T * (int64_t)c->d >= lim) return MOE_ERR_UNSUPPORTED;
    if (2 * h_rows * fm >= lim) return MOE_ERR_UNSUPPORTED;
    if (2 * (int64_t)c->F * c->d >= lim || 2 * (int64_t)c->F_shared * c->d >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

size_t elem_bytes(const moe_config_t* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

// ---- workspace layouts -----------------------------------------------------
struct RouterWs {
  size_t split, logits, part_p, part_cnt, part_z, part_fp, planes, total;
};
RouterWs router_ws(const moe_config_t* c) {
  RouterWs w;
  const int64_t nb = router_num_blocks(c->T);
  size_t o = 0;
  const int ns = router_num_splits(c->T, c->d, c->N, c->dtype == MOE_BF16);
  w.split = o;  // logit partials, one [T, N] slab per K split (only if > 1 split)
  o = align_up(o + (ns > 1 ? (size_t)ns * c->T * c->N * 4 : 0));
  w.logits = o; o = align_up(o + (size_t)c->T * c->N * 4);
  w.part_p = o; o = align_up(o + (size_t)nb * c->N * 4);
  w.part_cnt = o; o = align_up(o + (size_t)nb * c->N * 4);
  w.part_z = o; o = align_up(o + (size_t)nb * 3 * 4);
  w.part_fp = o; o = align_up(o + (size_t)((c->N + 63) / 64) * 4);
  w.planes = o; o = align_up(o + router_planes_bytes(c->T, c->d, c->N, c->dtype == MOE_BF16));
  w.total = o;
  return w;
}

struct DispatchWs {
  size_t blk_count, blk_base, blk_bad, total;
};
DispatchWs dispatch_ws(const moe_config_t* c) {
  DispatchWs w;
  const int64_t nb = dispatch_num_blocks(c->T);
  size_t o = 0;
  w.blk_count = o; o = align_up(o + (size_t)nb * c->N * 4);
  w.blk_base = o; o = align_up(o + (size_t)nb * c->N * 4);
  w.blk_bad = o; o = align_up(o + (size_t)nb * 4);
  w.total = o;
  return w;
}

struct FfnWs {
  size_t tile_base, h, total;
};
FfnWs ffn_ws(const moe_config_t* c) {
  FfnWs w;
  size_t o = 0;
  w.tile_base = o; o = align_up(o + ((size_t)3 * (c->N + 2) + kWalkCounters) * 4);
  w.h = o; o = align_up(o + ffn_workspace_bytes(c->T, c->d, c->N, c->K, c->F, c->F_shared,
                                                c->dtype == MOE_BF16));
  w.total = o;
  return w;
}

struct LayerWs {
  RouterWs r;
  DispatchWs dsp;
  FfnWs f;
  size_t router, dispatch, ffn;
  size_t idx, gate, kept, offset, pair_row, row_pair, counters, y_perm, y_shared;
  size_t total;
};
LayerWs layer_ws(const moe_config_t* c) {
  LayerWs w;
  w.r = router_ws(c);
  w.dsp = dispatch_ws(c);
  w.f = ffn_ws(c);
  const size_t pairs = (size_t)c->T * c->K;
  const size_t eb = elem_bytes(c);
  size_t o = 0;
  w.router = o; o = align_up(o + w.r.total);
  w.dispatch = o; o = align_up(o + w.dsp.total);
  w.ffn = o; o = align_up(o + w.f.total);
  w.idx = o; o = align_up(o + pairs * 4);
  w.gate = o; o = align_up(o + pairs * 4);
  w.kept = o; o = align_up(o + (size_t)c->N * 4);
  w.offset = o; o = align_up(o + (size_t)(c->N + 1) * 4);
  w.pair_row = o; o = align_up(o + pairs * 4);
  w.row_pair = o; o = align_up(o + pairs * 4);
  w.counters = o; o = align_up(o + 4 * 4);
  w.y_perm = o; o = align_up(o + pairs * (size_t)c->d * eb);
  w.y_shared = o; o = align_up(o + (c->F_shared > 0 ? (size_t)c->T * c->d * eb : 0));
  w.total = o;
  return w;
}

// Backward: router scratch (db_r block sums, dW_r split partials), the
// expert FFN backward scratch, and the layer's intermediates.
struct RouterBwdWs {
  size_t part_db, part_dw, total;
};
RouterBwdWs router_bwd_ws(const moe_config_t* c) {
  RouterBwdWs w;
  size_t o = 0;
  w.part_db = o; o = align_up(o + (size_t)router_bwd_num_blocks(c->T) * c->N * 4);
  const int ns = router_dw_splits(c->T, c->N);
  w.part_dw = o; o = align_up(o + (ns > 1 ? (size_t)ns * c->N * c->d * 4 : 0));
  w.total = o;
  return w;
}

struct BwdWs {
  RouterBwdWs r;
  size_t router, ffn, d_perm, dgate, dlogits, dx_perm, dx_shared, dx_perm2, dx_shared2, total;
};
BwdWs bwd_ws(const moe_config_t* c) {
  BwdWs w;
  w.r = router_bwd_ws(c);
  const size_t pairs = (size_t)c->T * c->K;
  const size_t eb = c->dtype == MOE_BF16 ? 2 : 4;
  size_t o = 0;
  w.router = o; o = align_up(o + w.r.total);
  w.ffn = o; o = align_up(o + ffn_backward_workspace_bytes(c->T, c->d, c->N, c->K, c->F,
                                                           c->F_shared, c->dtype == MOE_BF16));
  w.d_perm = o; o = align_up(o + pairs * c->d * eb);
  w.dgate = o; o = align_up(o + pairs * 4);
  w.dlogits = o; o = align_up(o + (size_t)c->T * c->N * 4);
  w.dx_perm = o; o = align_up(o + pairs * c->d * eb);
  w.dx_shared = o; o = align_up(o + (c->F_shared > 0 ? (size_t)c->T * c->d * eb : 0));
  // the other parts of a split dx_perm (dx_shared): up to 3 planes
  w.dx_perm2 = o; o = align_up(o + 3 * pairs * c->d * eb);
  w.dx_shared2 = o; o = align_up(o + (c->F_shared > 0 ? 3 * (size_t)c->T * c->d * eb : 0));
  w.total = o;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The router noise of this call: the caller's draws (w->noise), draws made
// in the kernels (MOE_FLAG_NOISE_PHILOX), or none.
RouterNoise router_noise(const moe_config_t* c, const moe_weights_t* w) {
  RouterNoise n = {};
  n.tensor = w->noise;
  n.std = c->noise_std;
  n.philox = (c->flags & MOE_FLAG_NOISE_PHILOX) ? 1 : 0;
  n.seed = c->noise_seed;
  n.offset = c->noise_offset;
  return n;
}

moe_status_t check_weights_router(const moe_config_t* c, const moe_weights_t* w) {
  if (!w || !w->w_r) return MOE_ERR_INVALID_ARG;
  // one source of noise at a time
  if ((c->flags & MOE_FLAG_NOISE_PHILOX) && w->noise) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_weights_ffn(const moe_config_t* c, const moe_weights_t* w) {
  if (!w || !w->w1 || !w->w2) return MOE_ERR_INVALID_ARG;
  if (c->act == MOE_ACT_SWIGLU && !w->w3) return MOE_ERR_INVALID_ARG;
  if (c->act == MOE_ACT_SWIGLU && (w->b1 || w->b2)) return MOE_ERR_UNSUPPORTED;
  if (c->F_shared > 0 && (!w->ws1 || !w->ws3 || !w->ws2)) return MOE_ERR_INVALID_ARG;
  if (c->weight_format != MOE_WEIGHTS_DTYPE) {
    if (!w->w1_scale || !w->w3_scale || !w->w2_scale) return MOE_ERR_INVALID_ARG;
    if (c->F_shared > 0 && (!w->ws1_scale || !w->ws3_scale || !w->ws2_scale))
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

void set_weights(FfnProblem& p, const moe_config_t* c, const moe_weights_t* w) {
  p.w1 = w->w1; p.w3 = w->w3; p.w2 = w->w2; p.b1 = w->b1; p.b2 = w->b2;
  p.ws1 = w->ws1; p.ws3 = w->ws3; p.ws2 = w->ws2;
  p.int8 = c->weight_format == MOE_WEIGHTS_INT8;
  p.int4 = c->weight_format == MOE_WEIGHTS_INT4;
  p.w1_scale = w->w1_scale; p.w3_scale = w->w3_scale; p.w2_scale = w->w2_scale;
  p.ws1_scale = w->ws1_scale; p.ws3_scale = w->ws3_scale; p.ws2_scale = w->ws2_scale;
}

// ---- stages ----------------------------------------------------------------
moe_status_t do_router(const moe_config_t* c, const moe_weights_t* w, const void* x,
                       int32_t* idx, float* gate, float* logits, const moe_stats_t* st,
                       void* ws, hipStream_t s) {
  const RouterWs L = router_ws(c);
  float* lg = logits ? logits : at<float>(ws, L.logits);
  const bool bf16 = c->dtype == MOE_BF16;
  int32_t* count = st ? st->count : nullptr;
  float* f = st ? st->f : nullptr;
  float* p = st ? st->p : nullptr;
  float* loss = st ? st->loss : nullptr;
  float* entropy = st ? st->entropy : nullptr;
  float* b_out = st ? st->b_sel_out : nullptr;
  if (router_fused_path(c->T, c->N, bf16)) {
    hipError_t e = launch_router_fused(x, w->w_r, w->b_r, router_noise(c, w), w->b_sel, lg, idx,
                                       gate, at<float>(ws, L.part_p), at<int32_t>(ws, L.part_cnt),
                                       at<float>(ws, L.part_z), c->T, c->d, c->N, c->K, c->gate,
                                       s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (count || f || p || loss || entropy || b_out) {
      e = launch_router_stats(at<float>(ws, L.part_p), at<int32_t>(ws, L.part_cnt),
                              at<float>(ws, L.part_z), at<float>(ws, L.part_fp),
                              router_num_blocks(c->T), c->T, c->N, c->K, c->aux_alpha, count, f,
                              p, loss, entropy, w->b_sel, b_out, c->bias_rate, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  if (router_small_path(c->T, c->N)) {
    hipError_t e = launch_router_logits(x, bf16, w->w_r, w->b_r, at<uint16_t>(ws, L.planes),
                                        at<float>(ws, L.split), lg, c->T, c->d, c->N, s,
                                        /*reduce_splits=*/false);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = launch_router_small(at<float>(ws, L.split), router_num_splits(c->T, c->d, c->N, bf16),
                            w->b_r, router_noise(c, w), w->b_sel, lg, idx, gate, c->T, c->N,
                            c->K, c->gate, c->aux_alpha, count, f, p, loss, entropy, b_out,
                            c->bias_rate, s);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  // the K-split partials are added by the top-K kernel from 1024 tokens on,
  // else by a reduction of their own
  const int ns = router_num_splits(c->T, c->d, c->N, bf16);
  const bool fused = router_topk_adds_splits(c->T, ns);
  hipError_t e = launch_router_logits(x, bf16, w->w_r, w->b_r, at<uint16_t>(ws, L.planes),
                                      at<float>(ws, L.split), lg, c->T, c->d, c->N, s,
                                      /*reduce_splits=*/!fused);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_router_topk(lg, at<float>(ws, L.split), fused ? ns : 1,
                         w->b_r, router_noise(c, w), w->b_sel, idx, gate, at<float>(ws, L.part_p),
                         at<int32_t>(ws, L.part_cnt), at<float>(ws, L.part_z), c->T, c->N, c->K,
                         c->gate, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (count || f || p || loss || entropy || b_out) {
    e = launch_router_stats(at<float>(ws, L.part_p), at<int32_t>(ws, L.part_cnt),
                            at<float>(ws, L.part_z), at<float>(ws, L.part_fp),
                            router_num_blocks(c->T), c->T, c->N, c->K, c->aux_alpha, count, f, p,
                            loss, entropy, w->b_sel, b_out, c->bias_rate, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// plan (nullable): the expert FFN's tile tables, built at the dispatch's end
moe_status_t do_dispatch(const moe_config_t* c, const int32_t* idx, const moe_dispatch_t* o,
                         void* ws, hipStream_t s, const TilePlan* plan = nullptr) {
  const DispatchWs L = dispatch_ws(c);
  hipError_t e = launch_dispatch(idx, c->T, c->N, c->K, c->capacity, at<int32_t>(ws, L.blk_count),
                                 at<int32_t>(ws, L.blk_base), at<int32_t>(ws, L.blk_bad), o->kept,
                                 o->offset, o->pair_row, o->row_pair, o->dropped, o->counters, s,
                                 plan);
  return hip_status(e);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

int64_t moe_capacity(int32_t K, int32_t N, int64_t T, double cf) {
  if (K < 1 || N < 1 || T < 0 || std::isnan(cf)) return -1;
  if (cf < 0) return T;
  const double scaled = cf * 1e9;
  if (scaled > 9.0e18) return -1;
  const __int128 num = (__int128)std::llround(scaled);
  const __int128 q = ((__int128)K * num * (__int128)T) / ((__int128)N * (__int128)1000000000);
  return (int64_t)q;
}

moe_status_t moe_router_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = router_ws(cfg).total;
  return MOE_OK;
}

moe_status_t moe_dispatch_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = dispatch_ws(cfg).total;
  return MOE_OK;
}

moe_status_t moe_ffn_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = ffn_ws(cfg).total;
  return MOE_OK;
}

moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = layer_ws(cfg).total;
  return MOE_OK;
}

moe_status_t moe_router_topk(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                             int32_t* topk_idx, float* topk_gate, float* logits,
                             const moe_stats_t* stats, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights_router(cfg, w)) != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < router_ws(cfg).total) return MOE_ERR_WORKSPACE;
  return do_router(cfg, w, x, topk_idx, topk_gate, logits, stats, ws, (hipStream_t)stream);
}

moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* topk_idx, const void* x,
                          const moe_dispatch_t* out, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  if (!topk_idx || !out->offset || !out->pair_row || !out->row_pair) return MOE_ERR_INVALID_ARG;
  if (out->x_perm && !x) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < dispatch_ws(cfg).total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  st = do_dispatch(cfg, topk_idx, out, ws, s);
  if (st != MOE_OK) return st;
  if (out->x_perm) {
    hipError_t e = launch_permute(x, (int)elem_bytes(cfg), out->row_pair, out->offset, cfg->N,
                                  cfg->K, cfg->d, cfg->T * cfg->K, out->x_perm, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, const moe_weights_t* w, const void* a,
                            const int32_t* a_rows, const int32_t* offset, void* y_perm,
                            const void* x_shared, void* y_shared, void* ws, size_t ws_bytes,
                            void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights_ffn(cfg, w)) != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!a || !offset || !y_perm) return MOE_ERR_INVALID_ARG;
  if (cfg->F_shared > 0 && (!x_shared || !y_shared)) return MOE_ERR_INVALID_ARG;
  // without a gather map the first GEMM addresses x_perm [T*K, d] from one
  // base with 32-bit byte offsets (x [T, d] and h are bounded by check_config)
  if (cfg->dtype == MOE_BF16 && !a_rows &&
      2 * cfg->T * (int64_t)cfg->K * cfg->d >= (int64_t(1) << 32))
    return MOE_ERR_UNSUPPORTED;
  const FfnWs L = ffn_ws(cfg);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  FfnProblem p = {};
  p.T = cfg->T; p.d = cfg->d; p.N = cfg->N; p.K = cfg->K; p.F = cfg->F;
  p.F_shared = cfg->F_shared; p.act = cfg->act; p.bf16 = cfg->dtype == MOE_BF16;
  p.a = a; p.a_rows = a_rows; p.offset = offset;
  set_weights(p, cfg, w);
  p.x_shared = x_shared; p.y_perm = y_perm; p.y_shared = y_shared;
  p.h = at<void>(ws, L.h);
  p.tile_base = at<int32_t>(ws, L.tile_base);
  return hip_status(launch_expert_ffn(p, (hipStream_t)stream, nullptr));
}

moe_status_t moe_combine(const moe_config_t* cfg, const void* y_perm, const int32_t* pair_row,
                         const float* topk_gate, const void* y_shared, void* y, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!y_perm || !pair_row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_perm, pair_row, topk_gate, y_shared, y, cfg->T, cfg->d,
                                   cfg->K, cfg->dtype == MOE_BF16, (hipStream_t)stream));
}

moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               const moe_layer_out_t* out, void* ws, size_t ws_bytes,
                               const moe_trace_t* trace, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_weights_router(cfg, w)) != MOE_OK) return st;
  if ((st = check_weights_ffn(cfg, w)) != MOE_OK) return st;
  if (!out) return MOE_ERR_INVALID_ARG;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !out->y) return MOE_ERR_INVALID_ARG;
  const LayerWs L = layer_ws(cfg);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) -> moe_status_t {
    if (trace && trace->ev[i]) return hip_status(hipEventRecord((hipEvent_t)trace->ev[i], s));
    return MOE_OK;
  };

  int32_t* idx = out->topk_idx ? out->topk_idx : at<int32_t>(ws, L.idx);
  float* gate = out->topk_gate ? out->topk_gate : at<float>(ws, L.gate);
  moe_dispatch_t d = out->dispatch;
  d.x_perm = nullptr;
  if (!d.kept) d.kept = at<int32_t>(ws, L.kept);
  if (!d.offset) d.offset = at<int32_t>(ws, L.offset);
  if (!d.pair_row) d.pair_row = at<int32_t>(ws, L.pair_row);
  if (!d.row_pair) d.row_pair = at<int32_t>(ws, L.row_pair);
  if (!d.counters) d.counters = at<int32_t>(ws, L.counters);

  if ((st = mark(0)) != MOE_OK) return st;
  st = do_router(cfg, w, x, idx, gate, out->logits, &out->stats, at<void>(ws, L.router), s);
  if (st != MOE_OK) return st;
  const FfnWs FL = ffn_ws(cfg);
  unsigned char* fws = at<unsigned char>(ws, L.ffn);
  FfnProblem p = {};
  p.T = cfg->T; p.d = cfg->d; p.N = cfg->N; p.K = cfg->K; p.F = cfg->F;
  p.F_shared = cfg->F_shared; p.act = cfg->act; p.bf16 = cfg->dtype == MOE_BF16;
  p.a = x; p.a_rows = d.row_pair; p.offset = d.offset;  // rows gathered in the GEMM
  set_weights(p, cfg, w);
  p.x_shared = x;
  p.y_perm = out->y_perm ? out->y_perm : at<void>(ws, L.y_perm);
  p.save_u = out->u;
  p.save_v = out->v;
  p.y_shared = cfg->F_shared > 0 ? at<void>(ws, L.y_shared) : nullptr;
  p.h = fws + FL.h;
  p.tile_base = (int32_t*)(fws + FL.tile_base);
  // the dispatch builds the FFN's tile tables at its end (one launch fewer)
  TilePlan plan;
  const bool planned = plan_expert_ffn_tiles(p, &plan);

  if ((st = mark(1)) != MOE_OK) return st;
  st = do_dispatch(cfg, idx, &d, at<void>(ws, L.dispatch), s, planned ? &plan : nullptr);
  if (st != MOE_OK) return st;

  hipEvent_t fev[4] = {};
  if (trace)
    for (int i = 0; i < 4; ++i) fev[i] = (hipEvent_t)trace->ev[2 + i];
  if (launch_expert_ffn(p, s, fev, planned) != hipSuccess) return MOE_ERR_HIP;
  if (launch_combine(p.y_perm, d.pair_row, gate, p.y_shared, out->y, cfg->T, cfg->d, cfg->K,
                     p.bf16, s) != hipSuccess)
    return MOE_ERR_HIP;
  return mark(6);
}

moe_status_t moe_quantize_int8(const void* w, int64_t rows, int32_t cols, int8_t* q, float* scale,
                               void* stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (cols % 64) return MOE_ERR_UNSUPPORTED;
  if (rows * (int64_t)cols >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_int8(w, rows, cols, q, scale, (hipStream_t)stream));
}

moe_status_t moe_quantize_int4(const void* w, int64_t rows, int32_t cols, uint8_t* q, float* scale,
                               void* stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (cols % 128) return MOE_ERR_UNSUPPORTED;
  if (rows * (int64_t)cols >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_int4(w, rows, cols, q, scale, (hipStream_t)stream));
}

int32_t moe_layer_saves_uv(const moe_config_t* cfg) {
  if (check_config(cfg) != MOE_OK || cfg->weight_format != MOE_WEIGHTS_DTYPE) return 0;
  return ffn_saves_uv(cfg->T, cfg->K, cfg->N, cfg->act, cfg->dtype == MOE_BF16) ? 1 : 0;
}

// ---- backward ---------------------------------------------------------------
moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (cfg->weight_format != MOE_WEIGHTS_DTYPE) return MOE_ERR_UNSUPPORTED;
  *bytes = bwd_ws(cfg).total;
  return MOE_OK;
}

moe_status_t moe_combine_backward(const moe_config_t* cfg, const void* dy, const void* y_perm,
                                  const float* topk_gate, const int32_t* pair_row, void* d_perm,
                                  float* dgate, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!dy || !y_perm || !topk_gate || !pair_row || !d_perm || !dgate) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_backward(dy, y_perm, topk_gate, pair_row, cfg->T, cfg->K,
                                            cfg->d, cfg->dtype == MOE_BF16, d_perm, dgate,
                                            (hipStream_t)stream));
}

moe_status_t moe_router_backward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                 const float* logits, const int32_t* topk_idx,
                                 const int32_t* pair_row, const float* dgate,
                                 const int32_t* count, moe_loss_grad_t lg, float* dlogits,
                                 float* dw_r, float* db_r, void* ws, size_t ws_bytes,
                                 void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!w || !dw_r) return MOE_ERR_INVALID_ARG;
  if ((cfg->flags & MOE_FLAG_NOISE_PHILOX) && w->noise) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(lg.aux) || !std::isfinite(lg.z) || !std::isfinite(lg.z_lse))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (cfg->T == 0) {
    if (launch_zero(dw_r, (size_t)cfg->N * cfg->d * 4, s) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_zero(db_r, db_r ? (size_t)cfg->N * 4 : 0, s));
  }
  if (!x || !logits || !topk_idx || !pair_row || !dgate || !count || !dlogits)
    return MOE_ERR_INVALID_ARG;
  const RouterBwdWs R = router_bwd_ws(cfg);
  if (!ws || ws_bytes < R.total) return MOE_ERR_WORKSPACE;
  if (launch_router_backward(logits, router_noise(cfg, w), topk_idx, pair_row, dgate, count,
                             cfg->T, cfg->N, cfg->K, cfg->gate, cfg->aux_alpha, lg.aux, lg.z,
                             lg.z_lse, dlogits, at<float>(ws, R.part_db), db_r, s) != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(launch_router_dw(dlogits, x, cfg->dtype == MOE_BF16, cfg->T, cfg->N, cfg->d,
                                     at<float>(ws, R.part_dw), dw_r, s));
}

namespace {
moe_status_t check_grads_ffn(const moe_config_t* c, const moe_grads_t* g) {
  if (!g || !g->dw1 || !g->dw2) return MOE_ERR_INVALID_ARG;
  if (c->act == MOE_ACT_SWIGLU && !g->dw3) return MOE_ERR_INVALID_ARG;
  if (c->F_shared > 0 && (!g->dws1 || !g->dws3 || !g->dws2)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Zero every weight gradient (T == 0: no rows, so every gradient is 0).
moe_status_t zero_grads(const moe_config_t* c, const moe_grads_t* g, hipStream_t s) {
  const size_t eb = c->dtype == MOE_BF16 ? 2 : 4;
  const size_t fd = (size_t)c->F * c->d;
  const size_t fs = (size_t)c->F_shared * c->d;
  struct { void* p; size_t n; } z[] = {
      {g->dw1, c->N * fd * eb}, {g->dw3, c->N * fd * eb}, {g->dw2, c->N * fd * eb},
      {g->db1, (size_t)c->N * c->F * eb}, {g->db2, (size_t)c->N * c->d * eb},
      {g->dws1, fs * eb}, {g->dws3, fs * eb}, {g->dws2, fs * eb}};
  for (auto& e : z)
    if (launch_zero(e.p, e.n, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t do_ffn_backward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                             const int32_t* row_pair, const int32_t* offset, const void* d_perm,
                             const void* dy, void* dx_perm, void* dx_shared,
                             const moe_grads_t* g, void* ws, hipStream_t s,
                             const hipEvent_t* ev = nullptr, void* dx_perm2 = nullptr,
                             void* dx_shared2 = nullptr, const void* u_in = nullptr,
                             const void* v_in = nullptr) {
  FfnBwdProblem p = {};
  p.T = cfg->T; p.d = cfg->d; p.N = cfg->N; p.K = cfg->K; p.F = cfg->F;
  p.F_shared = cfg->F_shared; p.act = cfg->act; p.bf16 = cfg->dtype == MOE_BF16;
  p.x = x; p.row_pair = row_pair; p.offset = offset;
  p.w1 = w->w1; p.w3 = w->w3; p.w2 = w->w2; p.b1 = w->b1;
  p.ws1 = w->ws1; p.ws3 = w->ws3; p.ws2 = w->ws2;
  p.d_perm = d_perm; p.dy = dy; p.dx_perm = dx_perm; p.dx_shared = dx_shared;
  p.dx_perm2 = dx_perm2; p.dx_shared2 = dx_shared2;
  p.u_in = u_in; p.v_in = v_in;
  p.dw1 = g->dw1; p.dw3 = g->dw3; p.dw2 = g->dw2;
  // bias gradients only for layers that have the biases
  p.db1 = w->b1 ? g->db1 : nullptr;
  p.db2 = w->b2 ? g->db2 : nullptr;
  p.dws1 = g->dws1; p.dws3 = g->dws3; p.dws2 = g->dws2;
  p.ws = ws;
  p.ev = ev;
  if (launch_expert_ffn_backward(p, s) != hipSuccess) return MOE_ERR_HIP;
  const size_t eb = p.bf16 ? 2 : 4;
  if (!w->b1 && g->db1 && launch_zero(g->db1, (size_t)cfg->N * cfg->F * eb, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (!w->b2 && g->db2 && launch_zero(g->db2, (size_t)cfg->N * cfg->d * eb, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}
}  // namespace

moe_status_t moe_expert_ffn_backward(const moe_config_t* cfg, const moe_weights_t* w,
                                     const void* x, const int32_t* row_pair,
                                     const int32_t* offset, const void* d_perm, const void* dy,
                                     void* dx_perm, void* dx_shared, const moe_grads_t* grads,
                                     void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->weight_format != MOE_WEIGHTS_DTYPE) return MOE_ERR_UNSUPPORTED;
  if ((st = check_weights_ffn(cfg, w)) != MOE_OK) return st;
  if ((st = check_grads_ffn(cfg, grads)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (cfg->T == 0) return zero_grads(cfg, grads, s);
  if (!x || !row_pair || !offset || !d_perm || !dx_perm) return MOE_ERR_INVALID_ARG;
  if (cfg->F_shared > 0 && (!dy || !dx_shared)) return MOE_ERR_INVALID_ARG;
  const size_t need = ffn_backward_workspace_bytes(cfg->T, cfg->d, cfg->N, cfg->K, cfg->F,
                                                   cfg->F_shared, cfg->dtype == MOE_BF16);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return do_ffn_backward(cfg, w, x, row_pair, offset, d_perm, dy, dx_perm,
                         cfg->F_shared > 0 ? dx_shared : nullptr, grads, ws, s);
}

moe_status_t moe_dispatch_backward(const moe_config_t* cfg, const void* dx_perm,
                                   const int32_t* pair_row, const void* dx_shared,
                                   const float* dlogits, const float* w_r, void* dx,
                                   void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!dx_perm || !pair_row || !dx || (dlogits && !w_r)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dx(dx_perm, pair_row, cfg->K, dx_shared, dlogits, w_r, cfg->N, cfg->T,
                              cfg->d, cfg->dtype == MOE_BF16, dx, (hipStream_t)stream));
}

moe_status_t moe_layer_backward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                const moe_saved_t* sv, const void* dy, moe_loss_grad_t lg,
                                const moe_grads_t* g, void* ws, size_t ws_bytes,
                                const moe_bwd_trace_t* trace, void* stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->weight_format != MOE_WEIGHTS_DTYPE) return MOE_ERR_UNSUPPORTED;
  if ((st = check_weights_router(cfg, w)) != MOE_OK) return st;
  if ((st = check_weights_ffn(cfg, w)) != MOE_OK) return st;
  if ((st = check_grads_ffn(cfg, g)) != MOE_OK) return st;
  if (!g->dw_r) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(lg.aux) || !std::isfinite(lg.z) || !std::isfinite(lg.z_lse))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (cfg->T == 0) {
    if ((st = zero_grads(cfg, g, s)) != MOE_OK) return st;
    if (launch_zero(g->dw_r, (size_t)cfg->N * cfg->d * 4, s) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_zero(g->db_r, g->db_r ? (size_t)cfg->N * 4 : 0, s));
  }
  if (!x || !dy || !g->dx || !sv) return MOE_ERR_INVALID_ARG;
  if (!sv->logits || !sv->topk_idx || !sv->topk_gate || !sv->count || !sv->offset ||
      !sv->pair_row || !sv->row_pair || !sv->y_perm)
    return MOE_ERR_INVALID_ARG;
  const BwdWs B = bwd_ws(cfg);
  if (!ws || ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  const bool bf16 = cfg->dtype == MOE_BF16;
  void* d_perm = at<void>(ws, B.d_perm);
  float* dgate = at<float>(ws, B.dgate);
  float* dl = g->dlogits ? g->dlogits : at<float>(ws, B.dlogits);
  void* dx_perm = at<void>(ws, B.dx_perm);
  void* dx_shared = cfg->F_shared > 0 ? at<void>(ws, B.dx_shared) : nullptr;
  auto mark = [&](int i) -> moe_status_t {
    if (trace && trace->ev[i]) return hip_status(hipEventRecord((hipEvent_t)trace->ev[i], s));
    return MOE_OK;
  };
  if ((st = mark(0)) != MOE_OK) return st;
  if (launch_combine_backward(dy, sv->y_perm, sv->topk_gate, sv->pair_row, cfg->T, cfg->K, cfg->d,
                              bf16, d_perm, dgate, s) != hipSuccess)
    return MOE_ERR_HIP;
  if ((st = mark(1)) != MOE_OK) return st;
  void* rws = at<void>(ws, B.router);
  if (launch_router_backward(sv->logits, router_noise(cfg, w), sv->topk_idx, sv->pair_row,
                             dgate, sv->count, cfg->T, cfg->N, cfg->K, cfg->gate, cfg->aux_alpha,
                             lg.aux, lg.z, lg.z_lse, dl, at<float>(rws, B.r.part_db), g->db_r,
                             s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_router_dw(dl, x, bf16, cfg->T, cfg->N, cfg->d, at<float>(rws, B.r.part_dw), g->dw_r,
                       s) != hipSuccess)
    return MOE_ERR_HIP;
  if ((st = mark(2)) != MOE_OK) return st;
  hipEvent_t fev[5] = {};
  if (trace)
    for (int i = 0; i < 5; ++i) fev[i] = (hipEvent_t)trace->ev[3 + i];
  // dx_perm in up to four parts of its K sum, which the dx kernel adds
  void* dx_perm2 = at<void>(ws, B.dx_perm2);
  void* dx_shared2 = cfg->F_shared > 0 ? at<void>(ws, B.dx_shared2) : nullptr;
  // the forward's gate(x) and up(x), where it stores them: no recompute
  const bool have_uv = sv->u && sv->v &&
                       ffn_saves_uv(cfg->T, cfg->K, cfg->N, cfg->act, cfg->dtype == MOE_BF16);
  st = do_ffn_backward(cfg, w, x, sv->row_pair, sv->offset, d_perm, dy, dx_perm, dx_shared, g,
                       at<void>(ws, B.ffn), s, fev, dx_perm2, dx_shared2,
                       have_uv ? sv->u : nullptr, have_uv ? sv->v : nullptr);
  if (st != MOE_OK) return st;
  if ((st = mark(8)) != MOE_OK) return st;
  // the FFN backward fills the other parts only when it splits
  const int parts = ffn_backward_dx_parts(cfg->T, cfg->N, cfg->K, cfg->F, cfg->d, cfg->act,
                                          cfg->dtype == MOE_BF16);
  if (launch_dx(dx_perm, sv->pair_row, cfg->K, dx_shared, dl, w->w_r, cfg->N, cfg->T, cfg->d, bf16,
                g->dx, s, parts > 1 ? dx_perm2 : nullptr, parts > 1 ? dx_shared2 : nullptr,
                parts - 1) != hipSuccess)
    return MOE_ERR_HIP;
  return mark(9);
}

}  // extern "C"
