/*
 * moe.h: C ABI of libmoe, the forward pass of a token-choice
 * Mixture-of-Experts FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   - router linear layer, logits = x W_r^T (+ b_r): mzlw.cn "MoE 混合专家模型
 *     稀疏激活的架构原理与负载均衡挑战" 2.1; learnagent.wiki "混合专家模型
 *     （Mixture of Experts, MoE）" 结构 2.
 *   - top-K selection and gates renormalised over the chosen K: wmrh.cn
 *     explainer ("MoE 的核心思想") section 公式表达重点; mzlw.cn section 三
 *     (MoERouter); learnagent.wiki 运行示例.
 *   - selection-only per-expert bias: learnagent.wiki 结构 4.
 *   - Switch auxiliary loss alpha*N*sum f_i p_i: mzlw.cn 2.2; router
 *     z-loss: wmrh.cn section Router Z-Loss.
 *   - training-time router noise (noise_std times a standard-normal draw
 *     added to every logit before top-K, gates and the balance loss):
 *     mzlw.cn section 三 (MoERouter.forward); the auxiliary-loss-free bias
 *     update: learnagent.wiki 结构 4; routing entropy as a monitored
 *     quantity: mstx.cn, the list of new challenges.
 *   - capacity floor(K/N*CF*S) and token dropping: mzlw.cn 2.3.
 *   - per-expert FFN (SwiGLU: mzlw.cn section 三, Expert; GELU:
 *     learnagent.wiki 运行示例), shared expert: mstx.cn "MoE 如何替代
 *     FFN？…" section 5; grouped GEMM instead of the per-expert loop: the
 *     comment in mzlw.cn section 三, MoELayer.forward.
 *   - gate-weighted combine y = sum_k g_k E_k(x): wmrh.cn 公式表达重点;
 *     learnagent.wiki 结构 3.
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is a DEVICE pointer (HIP device memory of the
 *     current device), row-major, densely packed, 16-byte aligned.  The
 *     caller owns every buffer, including the workspace; the library
 *     allocates nothing.  Its only process-wide state is write-once facts
 *     per device (the compute-unit count, whether a kernel's LDS limit was
 *     raised), held in atomics: any host thread may call any entry point
 *     for any device.  Calls that share an output or workspace buffer must
 *     be ordered by the caller (same stream, or events).
 *   - `stream` is a hipStream_t (may be NULL = default stream).  Work is
 *     enqueued asynchronously; no entry point synchronises the host.
 *   - bf16 tensors are IEEE bfloat16 (uint16 storage).  The router weight,
 *     router biases, logits, gates and statistics are always fp32.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and return MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED /
 *     MOE_ERR_WORKSPACE.  A failed kernel launch returns MOE_ERR_HIP.
 *     T == 0 is valid and enqueues nothing.
 *   - Ties between equal router scores go to the lower expert index; the
 *     K chosen experts of a token are listed by decreasing score.
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bitwise-identical outputs (no floating-point atomics).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, K > N, negative size, ...       */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the library's limits        */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required   */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed   */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_ACT_SWIGLU = 0,     /* down( silu(x W1^T) * (x W3^T) )                 */
  MOE_ACT_GELU_TANH = 1   /* down( gelu_tanh(x W1^T + b1) ) + b2             */
} moe_act_t;

typedef enum {
  MOE_WEIGHTS_DTYPE = 0,  /* expert weights in cfg->dtype                       */
  MOE_WEIGHTS_INT8 = 1,   /* expert weights as int8 codes q with one fp32 scale
                             per output row s (W = q * s), from
                             moe_quantize_int8; bf16 SwiGLU layers at decode
                             sizes only (T*K/N <= 24), else UNSUPPORTED     */
  MOE_WEIGHTS_INT4 = 2    /* expert weights as packed 4-bit codes with one fp32
                             scale per 128 consecutive input columns of a row
                             (W = q * s), from moe_quantize_int4; as INT8, and
                             d, F, F_shared multiples of 128               */
} moe_weight_format_t;

typedef enum {
  MOE_GATE_RENORM_ALL = 0,     /* softmax over all N, divided by the top-K sum */
  MOE_GATE_SOFTMAX_TOPK = 1,   /* softmax of the K chosen logits (same value)  */
  MOE_GATE_PROB_NO_RENORM = 2  /* softmax over all N, not renormalised         */
} moe_gate_t;

/* Limits of the library (MOE_ERR_UNSUPPORTED outside them):
 *   1 <= N <= 1024, 1 <= K <= min(N, 16), d % 64 == 0, F % 64 == 0,
 *   F_shared % 64 == 0, T <= 2^24, bf16 layers need d, F >= 64.
 *   bf16 layers also need every grouped-GEMM operand addressed from one
 *   base to fit in 4 GiB (the kernels use 32-bit byte offsets):
 *   2*T*d < 2^32 (x) and 2*(T*K + T_shared)*max(F, F_shared) < 2^32 (the
 *   intermediate h; T_shared = T with a shared expert), and one expert's
 *   weight matrix 2*F*d < 2^32; moe_expert_ffn given x_perm (a_rows NULL)
 *   also needs 2*T*K*d < 2^32.                                           */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

typedef struct {
  int64_t T;          /* tokens (rows of x)                                  */
  int32_t d;          /* model width                                         */
  int32_t N;          /* routed experts                                      */
  int32_t K;          /* experts chosen per token                            */
  int32_t F;          /* routed expert intermediate width                    */
  int32_t F_shared;   /* shared expert intermediate width, 0 = no shared     */
  int32_t dtype;      /* moe_dtype_t of x, expert weights, expert biases, y  */
  int32_t act;        /* moe_act_t                                           */
  int32_t gate;       /* moe_gate_t                                          */
  int64_t capacity;   /* rows each expert may keep; < 0 = unlimited          */
  float aux_alpha;    /* alpha of the Switch auxiliary loss                  */
  uint32_t flags;     /* MOE_FLAG_* bits; others must be 0                   */
  float noise_std;    /* scale of the router noise (used only with
                         moe_weights_t.noise or MOE_FLAG_NOISE_PHILOX;
                         mzlw.cn section 三 uses 0.1)                         */
  float bias_rate;    /* step of the selection-bias update written to
                         moe_stats_t.b_sel_out (used only with it)           */
  int32_t weight_format; /* moe_weight_format_t of w1, w3, w2, ws1, ws3, ws2 */
  uint64_t noise_seed;   /* MOE_FLAG_NOISE_PHILOX: key of the generator      */
  uint64_t noise_offset; /* MOE_FLAG_NOISE_PHILOX: stream of this call (e.g.
                            the training step); one offset per call         */
} moe_config_t;

/* Router noise drawn inside the kernels (training-time noisy top-K, mzlw.cn
 * section 三, MoERouter.forward): the router works on
 * logits + noise_std * z from selection on, with z[t, e] standard-normal
 * number t*N + e of the stream (noise_seed, noise_offset) of Philox-4x32-10
 * (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
 * 1, 2, 3", SC 2011) and the Box-Muller transform: number i comes from
 * block i/4 (counter words: block low, block high, offset low, offset high;
 * key words: seed low, seed high), whose outputs (x0, x1) and (x2, x3) give
 * numbers 4b..4b+3 as (r cos a, r sin a), u1 = (x_even + 1) 2^-32,
 * u2 = x_odd 2^-32, r = sqrt(-2 ln u1), a = 2 pi u2, evaluated in double
 * precision and rounded once to float.  The backward pass draws the same
 * numbers again.  Not together with moe_weights_t.noise (INVALID_ARG).     */
#define MOE_FLAG_NOISE_PHILOX 1u

/* Weights.  Router: w_r [N, d] fp32, b_r [N] fp32 (nullable; also carries any
 * fixed per-expert logit offset), b_sel [N] fp32 selection-only bias
 * (nullable).  Experts, in linear-layer layout [out, in], dtype cfg->dtype:
 * w1 [N, F, d] (SwiGLU gate, or the GELU input projection), w3 [N, F, d]
 * (SwiGLU up; NULL for GELU), w2 [N, d, F] (down), b1 [N, F] and b2 [N, d]
 * (GELU only, nullable).  Shared expert (SwiGLU, only when F_shared > 0):
 * ws1 [F_shared, d], ws3 [F_shared, d], ws2 [d, F_shared].
 * noise [T, N] fp32 (nullable): this step's standard-normal draws, from
 * the caller's generator.  With it the router works on
 * logits + noise_std * noise from selection on (top-K, gates and every
 * statistic); the logits output still holds the noise-free logits.
 * With weight_format MOE_WEIGHTS_INT8, w1/w3/w2/ws1/ws3/ws2 hold int8 codes
 * in the same layouts and the *_scale arrays their per-output-row fp32
 * scales: w1_scale, w3_scale [N, F], w2_scale [N, d], ws1_scale,
 * ws3_scale [F_shared], ws2_scale [d] (all required then, else ignored).
 * With MOE_WEIGHTS_INT4 they hold moe_quantize_int4's packed codes (half a
 * byte per weight, rows of in/2 bytes) and the *_scale arrays one fp32 scale
 * per 128 input columns: w1_scale, w3_scale [N, F, d/128], w2_scale
 * [N, d, F/128], ws1_scale, ws3_scale [F_shared, d/128], ws2_scale
 * [d, F_shared/128].                                                      */
typedef struct {
  const float* w_r;
  const float* b_r;
  const float* b_sel;
  const void* w1;
  const void* w3;
  const void* w2;
  const void* b1;
  const void* b2;
  const void* ws1;
  const void* ws3;
  const void* ws2;
  const float* noise;
  const float* w1_scale;
  const float* w3_scale;
  const float* w2_scale;
  const float* ws1_scale;
  const float* ws3_scale;
  const float* ws2_scale;
} moe_weights_t;

/* Router statistics (each pointer nullable):
 *   count [N] int32: pairs (token, slot) that chose expert e, before capacity
 *   f     [N] fp32 : count / (T*K)
 *   p     [N] fp32 : mean over tokens of softmax(logits)_e
 *   loss  [3] fp32 : { aux = alpha*N*sum_e f_e p_e,
 *                      z = mean_t sum_e logits_te^2,
 *                      z_lse = mean_t logsumexp(logits_t)^2 }
 *   entropy [1] fp32 : mean_t of -sum_e P_te log P_te, P_t = softmax(logits_t)
 *   b_sel_out [N] fp32 : the selection bias after one auxiliary-loss-free
 *                      step: b_sel[e] + bias_rate * sign(T*K/N - count[e])
 *                      (b_sel NULL counts as 0).  May alias weights.b_sel:
 *                      it is written after selection has read it.
 * "logits" here are the ones the router works on (with noise if given).  */
typedef struct {
  int32_t* count;
  float* f;
  float* p;
  float* loss;
  float* entropy;
  float* b_sel_out;
} moe_stats_t;

/* Dispatch outputs.  A "pair" is (token t, slot k), flattened as t*K + k.
 *   kept     [N]    int32 rows kept by each expert = min(count, capacity)
 *   offset   [N+1]  int32 exclusive scan of kept; expert e owns rows
 *                   [offset[e], offset[e+1]) in ascending token order;
 *                   offset[N] = total kept rows                 (required)
 *   pair_row [T*K]  int32 row of each pair, -1 if dropped      (required)
 *   row_pair [T*K]  int32 pair id (t*K+k) of each row; entries at and
 *                   after offset[N] are left untouched          (required)
 *   dropped  [T*K]  uint8 1 if the pair was dropped (capacity or bad id)
 *   counters [4]    int32 { kept rows, dropped pairs, pairs with an
 *                   out-of-range or repeated expert id, experts with >= 1
 *                   kept row }
 *   x_perm   [T*K, d] dtype: x_perm[r] = x[row_pair[r] / K] for r < offset[N]
 * Each pointer marked nullable in moe_dispatch may be NULL.               */
typedef struct {
  int32_t* kept;
  int32_t* offset;
  int32_t* pair_row;
  int32_t* row_pair;
  uint8_t* dropped;
  int32_t* counters;
  void* x_perm;
} moe_dispatch_t;

/* Outputs of the whole layer.  y [T, d] (dtype) is required; every other
 * pointer is nullable and, when NULL, the value lives in the workspace.
 * y_perm [T*K, d] (dtype): each kept row's expert output before its gate
 * (rows at and after offset[N] untouched); the backward pass reads it.
 * u, v [T*K + (F_shared > 0 ? T : 0), F] (dtype), nullable, given together:
 * the first expert GEMM's gate(x) = x W1^T and up(x) = x W3^T of every kept
 * row (the shared expert's T rows after the T*K routed rows), written only
 * where moe_layer_saves_uv(cfg) is 1.  Saved for the backward pass, which
 * then skips recomputing them.                                           */
typedef struct {
  void* y;
  int32_t* topk_idx;    /* [T, K] */
  float* topk_gate;     /* [T, K] */
  float* logits;        /* [T, N] */
  moe_stats_t stats;
  moe_dispatch_t dispatch;  /* x_perm is ignored (rows are gathered in place) */
  void* y_perm;
  void* u;
  void* v;
} moe_layer_out_t;

/* Optional timing hooks: hipEvent_t handles recorded on `stream` at stage
 * boundaries of moe_layer_forward (any may be NULL):
 *   ev[0] before the router, ev[1] after routing + statistics,
 *   ev[2] after dispatch, right before the first grouped GEMM (gate/up),
 *   ev[3] after it, ev[4] after the main launch of the second grouped GEMM
 *   (down), ev[5] after its tail launch, ev[6] after the combine.  With the
 *   largest tiles (more than 640 rows per expert on average) the main launch
 *   covers each expert's rows in whole 256-row tiles, the last at least half
 *   full, and the tail launch the remainder; otherwise there is no tail.  */
#define MOE_TRACE_EVENTS 7
typedef struct {
  void* ev[MOE_TRACE_EVENTS];
} moe_trace_t;

/* Human-readable name of a status code (static string).  Host only. */
const char* moe_status_string(moe_status_t s);

/* Capacity floor(K / N * cf * T) (mzlw.cn 2.3, S read as the tokens in the
 * batch), computed with the factor cf rounded to 1e-9 and exact integer
 * arithmetic afterwards.  cf < 0 means unlimited and returns T.  Returns -1
 * on invalid arguments (K < 1, N < 1, T < 0).  Host only.               */
int64_t moe_capacity(int32_t K, int32_t N, int64_t T, double cf);

/* Bytes of workspace moe_layer_forward needs for `cfg` (host only).     */
moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* bytes);

/* Bytes of workspace the staged entry points need (host only).          */
moe_status_t moe_router_workspace_size(const moe_config_t* cfg, size_t* bytes);
moe_status_t moe_dispatch_workspace_size(const moe_config_t* cfg, size_t* bytes);
moe_status_t moe_ffn_workspace_size(const moe_config_t* cfg, size_t* bytes);

/* Router: logits, selection, gates and statistics.
 * Pages: logits = x W_r^T, mzlw.cn 2.1 and section 三 (MoERouter); softmax
 * and top-K, learnagent.wiki 结构 2 and 运行示例; renormalised gates, wmrh.cn
 * 公式表达重点; selection-only bias, learnagent.wiki 结构 4; f, p and the
 * auxiliary loss, mzlw.cn 2.2; z-loss, wmrh.cn Router Z-Loss.
 *   x [T, d] (cfg->dtype), w->w_r, w->b_r, w->b_sel as above.
 *   topk_idx [T, K] int32, topk_gate [T, K] fp32 (required);
 *   logits [T, N] fp32 (nullable), stats (nullable, and each member).
 * Selection key s = logits + b_sel; gates use logits only (cfg->gate).  */
moe_status_t moe_router_topk(const moe_config_t* cfg, const moe_weights_t* w,
                             const void* x, int32_t* topk_idx, float* topk_gate,
                             float* logits, const moe_stats_t* stats,
                             void* ws, size_t ws_bytes, void* stream);

/* Dispatch: per-expert counts, capacity clamp in token order, layout of the
 * kept pairs in expert-contiguous rows, and (if out->x_perm) the gathered
 * rows.  Pages: capacity and token dropping, mzlw.cn 2.3; the per-expert
 * token lists cut to capacity and the gather x_flat[expert_tokens], mzlw.cn
 * section 三 (MoELayer.forward).  topk_idx [T, K] int32 on the device; ids outside [0, N) and ids
 * repeated within one token are counted in counters[2] and dropped.
 * out->kept, out->dropped, out->counters, out->x_perm are nullable; x may
 * be NULL when out->x_perm is NULL.                                      */
moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* topk_idx,
                          const void* x, const moe_dispatch_t* out,
                          void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs as grouped GEMMs over the expert-contiguous rows.  Pages:
 * SwiGLU expert, mzlw.cn section 三 (Expert); GELU expert, learnagent.wiki
 * 运行示例; grouped GEMM instead of the per-expert loop, the comment in
 * mzlw.cn section 三 (MoELayer.forward); shared expert, mstx.cn section 5.
 *   a      : x_perm [rows, d] when a_rows == NULL; otherwise x [T, d] and
 *            row r reads x[a_rows[r] / K] (a_rows = row_pair).
 *   offset : [N+1] device row offsets (from moe_dispatch).
 *   y_perm : [T*K, d] output rows (rows >= offset[N] untouched).
 *   x_shared / y_shared : [T, d] input / output of the shared expert (both
 *            required iff F_shared > 0; then every token goes through it). */
moe_status_t moe_expert_ffn(const moe_config_t* cfg, const moe_weights_t* w,
                            const void* a, const int32_t* a_rows,
                            const int32_t* offset, void* y_perm,
                            const void* x_shared, void* y_shared,
                            void* ws, size_t ws_bytes, void* stream);

/* Combine (wmrh.cn 公式表达重点; learnagent.wiki 结构 3; dropped pairs add
 * nothing, mzlw.cn 2.3):
 * y[t] = sum_{k=0}^{K-1} [pair_row[t,k] >= 0] gate[t,k] *
 * y_perm[pair_row[t,k]]  (+ y_shared[t] when y_shared != NULL), summed in
 * fp32 in that fixed order and rounded once to cfg->dtype.  Dropped pairs
 * add nothing; the remaining gates are not renormalised.                 */
moe_status_t moe_combine(const moe_config_t* cfg, const void* y_perm,
                         const int32_t* pair_row, const float* topk_gate,
                         const void* y_shared, void* y, void* stream);

/* The whole layer: router, statistics, dispatch, expert FFNs (+ shared
 * expert), combine, in the order of mzlw.cn section 三 (MoELayer.forward)
 * and learnagent.wiki 结构 3.  ws must hold moe_workspace_size(cfg) bytes.  trace
 * is nullable.                                                           */
moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w,
                               const void* x, const moe_layer_out_t* out,
                               void* ws, size_t ws_bytes, const moe_trace_t* trace,
                               void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_layer_forward with
 * no ws argument.  The workspace is a fixed device array inside the library,
 * MOE_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until the process
 * ends; layers whose moe_workspace_size exceeds it (e.g. more than about
 * 350 tokens of the DeepSeek-shaped decode layer) return MOE_ERR_WORKSPACE
 * before anything is enqueued.  Nothing is allocated.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, different host threads) race and must be ordered by the caller.
 * Outputs, errors and determinism are those of moe_layer_forward.          */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w,
                                       const void* x, const moe_layer_out_t* out,
                                       const moe_trace_t* trace, void* stream);

/* Weight-only INT8 quantization of a bf16 weight matrix w [rows, cols]
 * (linear-layer layout [out, in]): q [rows, cols] int8 and scale [rows] fp32
 * with s = absmax(row) / 127 and q = rint(w / s) (fp32, correctly rounded
 * division, ties to even), clamped to [-127, 127]; a zero row gets s = 0,
 * q = 0.  Symmetric per-row absmax quantization as published by Dettmers et
 * al., "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale"
 * (2022), section 2; the pages name no scheme.  Expert stacks [N, R, C] are
 * quantized as rows = N*R.  Errors: INVALID_ARG for null pointers, rows < 0
 * or cols <= 0; UNSUPPORTED for cols % 64 != 0 or rows*cols >= 2^40.
 * rows == 0 enqueues nothing.                                              */
moe_status_t moe_quantize_int8(const void* w, int64_t rows, int32_t cols, int8_t* q,
                               float* scale, void* stream);

/* Weight-only INT4 quantization of a bf16 weight matrix w [rows, cols]
 * (linear-layer layout [out, in]) for the decode layers (wmrh.cn section
 * 工程优化方案 names INT4/INT8 quantization of the experts; the pages give no
 * scheme): one fp32 scale per group of 128 consecutive columns of a row,
 * s = absmax(group) / 7 and q = rint(w / s) (fp32, correctly rounded
 * division, ties to even) clamped to [-7, 7]; an all-zero group gets s = 0.
 * This is the round-to-nearest quantizer that GPTQ (Frantar et al., ICLR
 * 2023) and AWQ (Lin et al., MLSys 2024) use as their baseline at group size
 * 128.  q [rows, cols / 2] bytes: each code as u = q + 8 in 4 bits, the codes
 * of columns 8j .. 8j+7 of a row in one little-endian 32-bit word, column
 * 8j + 2i in bits 4i .. 4i+3 and column 8j + 2i + 1 in bits 16+4i .. 19+4i.
 * scale [rows, cols / 128] fp32.  Errors: INVALID_ARG for null pointers,
 * rows < 0 or cols <= 0; UNSUPPORTED for cols % 128 != 0 or
 * rows*cols >= 2^40.  rows == 0 enqueues nothing.                        */
moe_status_t moe_quantize_int4(const void* w, int64_t rows, int32_t cols, uint8_t* q,
                               float* scale, void* stream);

/* ======================================================== backward ===
 * The backward pass: for upstream gradients dy [T, d] of y and
 * (aux, z, z_lse) of the three router losses, the gradient of
 *     L = sum_{t,j} dy[t,j] y[t,j] + aux_g * aux + z_g * z + zlse_g * z_lse
 * with respect to x, the router weights and every expert weight, i.e. what
 * automatic differentiation computes through the PyTorch modules of mzlw.cn
 * "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战" section 三 plus its
 * 2.2 loss and the z-loss of wmrh.cn/news/98181 (Router Z-Loss).  Top-K
 * selection, the capacity cut and the counts f are piecewise constant and
 * pass no gradient (mstx.cn "MoE 如何替代 FFN？…", challenges: routing is a
 * discrete choice); the selection-only bias gets none; the routing entropy is
 * a diagnostic without gradient.  Router noise is additive, so with
 * w->noise the gradient with respect to the logits equals that with respect
 * to the noisy logits.  Only cfg->weight_format MOE_WEIGHTS_DTYPE is
 * supported (UNSUPPORTED otherwise).  Expert weight gradients are in
 * cfg->dtype (fp32 accumulation, rounded once); router gradients in fp32.
 * Every pointer is a device pointer unless noted; the caller owns all
 * memory; nothing is allocated or synchronised.  T == 0 zero-fills every
 * gradient output and launches nothing else.                             */

/* Forward values the backward pass reads (all required): what
 * moe_layer_forward (or the staged entry points) wrote for the same x.   */
typedef struct {
  const float* logits;      /* [T, N] noise-free router logits              */
  const int32_t* topk_idx;  /* [T, K]                                       */
  const float* topk_gate;   /* [T, K]                                       */
  const int32_t* count;     /* [N] pairs per expert before capacity         */
  const int32_t* offset;    /* [N+1]                                        */
  const int32_t* pair_row;  /* [T*K]                                        */
  const int32_t* row_pair;  /* [T*K]                                        */
  const void* y_perm;       /* [T*K, d] dtype, expert output per kept row   */
  const void* u;            /* nullable: moe_layer_out_t.u / .v, used where */
  const void* v;            /* moe_layer_saves_uv(cfg) is 1                 */
} moe_saved_t;

/* Gradient outputs.  dx [T, d] dtype; dw_r [N, d] fp32; db_r [N] fp32
 * (nullable); dw1 [N, F, d], dw2 [N, d, F] and, SwiGLU, dw3 [N, F, d];
 * GELU: db1 [N, F], db2 [N, d] (nullable; meaningful for layers with the
 * biases); shared expert (F_shared > 0): dws1, dws3 [F, d], dws2 [d, F];
 * dlogits [T, N] fp32 (nullable).  Experts that keep no row get zeros.   */
typedef struct {
  void* dx;
  float* dw_r;
  float* db_r;
  void* dw1;
  void* dw3;
  void* dw2;
  void* db1;
  void* db2;
  void* dws1;
  void* dws3;
  void* dws2;
  float* dlogits;
} moe_grads_t;

/* Upstream gradients of the router losses (host values).                 */
typedef struct {
  float aux;
  float z;
  float z_lse;
} moe_loss_grad_t;

/* 1 if moe_layer_forward writes moe_layer_out_t.u / .v for this layer
 * (bf16 SwiGLU layers with more than 96 rows per expert on average, whose
 * first grouped GEMM runs the large-tile kernel), else 0 (host only).     */
int32_t moe_layer_saves_uv(const moe_config_t* cfg);

/* Bytes of workspace moe_layer_backward needs (host only); the staged
 * entry points need at most as much.                                     */
moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, size_t* bytes);

/* Combine backward (the transpose of moe_combine; the gate-weighted sum of
 * wmrh.cn 公式表达重点 and mzlw.cn section 三): for every kept pair
 * d_perm[pair_row[p]] = topk_gate[p] * dy[p / K] and
 * dgate[p] = dy[p / K] . y_perm[pair_row[p]] (fp32, a fixed-order wave
 * reduction); a dropped pair gets dgate = 0.  d_perm [T*K, d] dtype
 * (rows >= offset[N] untouched), dgate [T*K] fp32.                       */
moe_status_t moe_combine_backward(const moe_config_t* cfg, const void* dy, const void* y_perm,
                                  const float* topk_gate, const int32_t* pair_row,
                                  void* d_perm, float* dgate, void* stream);

/* Router backward (the router of mzlw.cn section 三 with the losses of
 * mzlw.cn 2.2 and wmrh.cn Router Z-Loss; top-K passes no gradient, mstx.cn
 * challenges): dlogits [T, N] from the gates (per cfg->gate, using only
 * the kept pairs' dgate), the aux loss through p (f = count / (T K) fixed),
 * z and z_lse, all on logits + noise_std * w->noise when w->noise is set;
 * then dw_r = dlogits^T x and db_r = the column sums of dlogits (nullable),
 * each reduced in a fixed order.  w->w_r is not read (x is).              */
moe_status_t moe_router_backward(const moe_config_t* cfg, const moe_weights_t* w,
                                 const void* x, const float* logits, const int32_t* topk_idx,
                                 const int32_t* pair_row, const float* dgate,
                                 const int32_t* count, moe_loss_grad_t loss_grad,
                                 float* dlogits, float* dw_r, float* db_r,
                                 void* ws, size_t ws_bytes, void* stream);

/* Expert FFN backward (the SwiGLU expert of mzlw.cn section 三, the GELU
 * expert of learnagent.wiki 运行示例, the shared expert of mstx.cn section 5)
 * over the expert-contiguous rows (the forward's
 * first GEMM is recomputed from x): given d_perm (gradient of each kept
 * row's expert output) and, with a shared expert, dy (its output's
 * gradient), writes dx_perm [T*K, d] (each kept row's input gradient),
 * dx_shared [T, d] (shared expert only, else NULL) and the weight members
 * of grads (dw1, dw3, dw2, db1, db2, dws1, dws3, dws2 as described above).  */
moe_status_t moe_expert_ffn_backward(const moe_config_t* cfg, const moe_weights_t* w,
                                     const void* x, const int32_t* row_pair,
                                     const int32_t* offset, const void* d_perm, const void* dy,
                                     void* dx_perm, void* dx_shared, const moe_grads_t* grads,
                                     void* ws, size_t ws_bytes, void* stream);

/* Dispatch backward (the transpose of the row gather x_flat[expert_tokens]
 * of mzlw.cn section 三): dx[t] = sum over
 * k of [pair_row[t,k] >= 0] dx_perm[pair_row[t,k]] (+ dx_shared[t]) (+ the
 * router term dlogits[t] . w_r), fp32 in that order, rounded once.
 * dx_shared, dlogits (with w_r) nullable.                               */
moe_status_t moe_dispatch_backward(const moe_config_t* cfg, const void* dx_perm,
                                   const int32_t* pair_row, const void* dx_shared,
                                   const float* dlogits, const float* w_r, void* dx,
                                   void* stream);

/* Optional timing hooks of moe_layer_backward: hipEvent_t handles recorded
 * on `stream` (any may be NULL): ev[0] before the combine backward, ev[1]
 * after it, ev[2] after the router backward (dlogits, db_r, dw_r), ev[3]
 * after the recompute of the first expert GEMM, ev[4] after the dh GEMM
 * (with the activation backward), ev[5] after dw2, ev[6] after dx_perm,
 * ev[7] after dw1 (and dw3), ev[8] after the bias gradients, ev[9] after
 * the dispatch backward (dx).                                            */
#define MOE_BWD_TRACE_EVENTS 10
typedef struct {
  void* ev[MOE_BWD_TRACE_EVENTS];
} moe_bwd_trace_t;

/* The whole backward pass (what automatic differentiation computes through
 * the modules of mzlw.cn section 三, as described above): combine, router,
 * expert FFN and dispatch backward in that order.  ws must hold moe_backward_workspace_size(cfg)
 * bytes.  trace is nullable.                                             */
moe_status_t moe_layer_backward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                const moe_saved_t* saved, const void* dy,
                                moe_loss_grad_t loss_grad, const moe_grads_t* grads,
                                void* ws, size_t ws_bytes, const moe_bwd_trace_t* trace,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
