"""CPU oracle for the forward pass of a token-choice Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It is plain NumPy in
float64, imports neither torch nor the GPU library, and shares no code with
the GPU path.  It takes exactly the bits the GPU takes (bf16 inputs widened
exactly to float64) and does not round intermediates.

The pages it follows (cited by title and section):
  [P1]  wmrh.cn/news/98181, the explainer that opens with "MoE 的核心思想":
        sections 公式表达重点 (gate scores, softmax, top-K with the other
        scores sent to minus infinity, renormalised gates), 具体数值示例
        (worked example), 专家容量限制 (capacity), Router Z-Loss.
  [P3]  mzlw.cn/news/6844 "MoE 混合专家模型稀疏激活的架构原理与负载均衡挑战":
        2.1 (h(x) equation and logits = x W_r), 2.2 (L_aux equation),
        2.3 (capacity equation, token dropping), 三 (the PyTorch MoELayer:
        SwiGLU Expert, MoERouter top-K then softmax of the top-K logits,
        load-balance loss from scatter-add counts, per-expert truncation of
        the ascending token list to capacity, gate-weighted accumulation).
  [P4]  learnagent.wiki "混合专家模型（Mixture of Experts, MoE）":
        结构 2 (G(x) = Softmax(W_r x)), 结构 3 (y = sum over top-K of
        G_i E_i), 结构 4 (selection-only per-expert bias; the auxiliary-loss-
        free method adjusts that bias by how often each expert is chosen),
        运行示例 (softmax, top-K on probabilities, renormalise, GELU experts,
        compute all experts then gather).
  [P5]  mstx.cn/posts/467.html "MoE 如何替代 FFN？它解决了什么问题？带来哪些新挑战？":
        section 1 (FFN(x) = W2 act(W1 x)), section 2 (MoE(x) formula),
        section 5 (DeepSeek-MoE: fine-grained experts plus a shared expert),
        the challenges list (expert usage and routing entropy are what a
        training run monitors).

Readings taken where the pages are silent or disagree are listed next to the
function that takes them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

GATE_MODES = ("renorm_all", "softmax_topk", "prob_no_renorm")


# ---------------------------------------------------------------- format ---

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 stored as uint16 bits -> float64 (exact): a bf16 is the upper half
    of an IEEE fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


class Bf16Stack:
    """A stack of bf16 matrices held as uint16 bits; indexing one entry
    returns it widened to float64, so large expert weights are converted one
    expert at a time."""

    def __init__(self, bits: np.ndarray):
        self.bits = np.asarray(bits, dtype=np.uint16)
        self.shape = self.bits.shape

    def __getitem__(self, e):
        return bf16_bits_to_f64(self.bits[e])

    def __len__(self):
        return self.shape[0]


# ---------------------------------------------------------------- router ---

# ------------------------------------------------- weight-only INT8 ---

def quantize_int8_rows(w):
    """Weight-only INT8 with one scale per output channel (row), symmetric
    absmax quantization as published by Dettmers et al., "LLM.int8(): 8-bit
    Matrix Multiplication for Transformers at Scale" (2022), section 2: the
    row's largest magnitude maps to 127.  The pages give no scheme.

    Both steps are defined in fp32 so that codes are decided identically
    everywhere: s = absmax(row) / 127 and q = rint(w / s) (round half to
    even), clamped to [-127, 127]; an all-zero row gets s = 0 and q = 0.
    w: float array [..., rows, cols] (bf16 values are exact in fp32).
    Returns (q int8, s float32 [..., rows])."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((w32 / safe[..., None]).astype(np.float32))
    q = np.where(scale[..., None] > 0, q, 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, scale


def dequantize_int8_rows(q, scale):
    """The weights an INT8 layer computes with: q * s, exact in float64."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


class Int8Stack:
    """Per-expert INT8 weights (q [E, rows, cols], s [E, rows]); indexing one
    expert returns its dequantized matrix in float64."""

    def __init__(self, q, scale):
        self.q = np.asarray(q, dtype=np.int8)
        self.scale = np.asarray(scale, dtype=np.float32)
        self.shape = self.q.shape

    def __getitem__(self, e):
        return dequantize_int8_rows(self.q[e], self.scale[e])

    def __len__(self):
        return self.shape[0]


# ------------------------------------------------- weight-only INT4 ---

INT4_GROUP = 128


def quantize_int4_groups(w, group=INT4_GROUP):
    """Weight-only INT4 with one scale per group of `group` consecutive input
    columns of each row: symmetric absmax round-to-nearest, the RTN
    quantizer that Frantar et al. ("GPTQ", ICLR 2023) and Lin et al. ("AWQ",
    MLSys 2024) use as their baseline at group size 128.  [P1] names INT4
    quantization of the expert weights but gives no scheme.

    In fp32, like quantize_int8_rows: s = absmax(group) / 7 and
    q = rint(w / s) (round half to even), clamped to [-7, 7]; an all-zero
    group gets s = 0 and q = 0.  w: float array [..., rows, cols] with cols a
    multiple of `group`.  Returns (q int8 in [-7, 7], s float32
    [..., rows, cols / group])."""
    w32 = np.asarray(w, dtype=np.float32)
    *lead, cols = w32.shape
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    g = w32.reshape(*lead, cols // group, group)
    amax = np.max(np.abs(g), axis=-1)
    scale = (amax / np.float32(7.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((g / safe[..., None]).astype(np.float32))
    q = np.where(scale[..., None] > 0, q, 0.0)
    q = np.clip(q, -7, 7).astype(np.int8).reshape(*lead, cols)
    return q, scale


def dequantize_int4_groups(q, scale, group=INT4_GROUP):
    """The weights an INT4 layer computes with: q * s of its group, exact in
    float64."""
    q = np.asarray(q, dtype=np.float64)
    *lead, cols = q.shape
    s = np.asarray(scale, dtype=np.float64)
    return (q.reshape(*lead, cols // group, group) * s[..., None]).reshape(*lead, cols)


def pack_int4(q):
    """The library's storage of INT4 codes (a layout of this library; the
    pages give none): each code as u = q + 8 in 4 bits; the 8 codes of
    columns 8j .. 8j+7 of a row fill one little-endian 32-bit word, the code
    of column 8j + 2i in bits 4i .. 4i+3 and that of column 8j + 2i + 1 in
    bits 16 + 4i .. 16 + 4i + 3 (i = 0 .. 3).  q int [..., rows, cols] with
    cols a multiple of 8 -> uint8 [..., rows, cols / 2]."""
    q = np.asarray(q, dtype=np.int64)
    *lead, cols = q.shape
    u = (q + 8).reshape(*lead, cols // 8, 8).astype(np.uint32)
    word = np.zeros((*lead, cols // 8), dtype=np.uint32)
    for i in range(4):
        word |= u[..., 2 * i] << np.uint32(4 * i)
        word |= u[..., 2 * i + 1] << np.uint32(16 + 4 * i)
    return word.view(np.uint8).reshape(*lead, cols // 2)


def unpack_int4(packed):
    """Inverse of pack_int4: uint8 [..., rows, cols / 2] -> int8 codes."""
    b = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    *lead, half = b.shape
    word = b.reshape(*lead, half // 4, 4).view(np.uint32)[..., 0]
    out = np.zeros((*lead, half // 4, 8), dtype=np.int64)
    for i in range(4):
        out[..., 2 * i] = (word >> np.uint32(4 * i)) & np.uint32(15)
        out[..., 2 * i + 1] = (word >> np.uint32(16 + 4 * i)) & np.uint32(15)
    return (out - 8).astype(np.int8).reshape(*lead, half * 2)


class Int4Stack:
    """Per-expert INT4 weights (packed codes [E, rows, cols / 2], group scales
    [E, rows, cols / 128]); indexing one expert returns its dequantized
    matrix in float64."""

    def __init__(self, packed, scale, group=INT4_GROUP):
        self.packed = np.asarray(packed, dtype=np.uint8)
        self.scale = np.asarray(scale, dtype=np.float32)
        self.group = group
        self.shape = self.packed.shape[:-1] + (self.packed.shape[-1] * 2,)

    def __getitem__(self, e):
        return dequantize_int4_groups(unpack_int4(self.packed[e]), self.scale[e], self.group)

    def __len__(self):
        return self.shape[0]


def router_logits(x: np.ndarray, w_r: np.ndarray, b_r: np.ndarray | None = None):
    """logits[t, e] = sum_j x[t, j] * w_r[e, j] (+ b_r[e]).

    [P3] 2.1 writes logits = x . W_r with W_r of shape d x N; the page's
    MoERouter stores the weight as [N, d] and multiplies by its transpose,
    which is the same map.  [P4] 结构 2 / 运行示例 uses a linear layer with a
    bias; the bias (and any fixed per-expert logit offset) is folded in here.
    """
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    out = x @ w_r.T
    if b_r is not None:
        out = out + np.asarray(b_r, dtype=np.float64)[None, :]
    return out


def softmax_rows(v: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted ([P4] 结构 2)."""
    m = v.max(axis=-1, keepdims=True)
    e = np.exp(v - m)
    return e / e.sum(axis=-1, keepdims=True)


def logsumexp_rows(v: np.ndarray) -> np.ndarray:
    m = v.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(v - m).sum(axis=-1, keepdims=True)))[:, 0]


def select_topk(scores: np.ndarray, K: int):
    """The K experts with the largest score for every token.

    Reading (pages silent): equal scores go to the LOWER expert index; the K
    chosen ids are listed in order of decreasing score.  Implemented as a
    full stable sort of every row by descending score ([P3] 三 calls topk on
    the logits, [P4] 运行示例 on the probabilities: softmax is monotone, so
    the chosen set is the same).

    Returns (idx[T, K] int64, margin[T]) where margin is the score gap
    between the K-th and (K+1)-th ranked experts (+inf when K == N).
    """
    s = np.asarray(scores, dtype=np.float64)
    if not np.all(np.isfinite(s)):
        raise ValueError("oracle: non-finite router scores")
    T, N = s.shape
    order = np.argsort(-s, axis=1, kind="stable")  # ties keep index order
    idx = order[:, :K].astype(np.int64)
    srt = np.take_along_axis(s, order, axis=1)
    if K < N:
        margin = srt[:, K - 1] - srt[:, K]
    else:
        margin = np.full(T, np.inf)
    return idx, margin


def gate_weights(logits: np.ndarray, idx: np.ndarray, mode: str) -> np.ndarray:
    """Gate of each chosen expert.

    renorm_all     : P = softmax over all N logits, g = P[idx] / sum P[idx]
                     ([P4] 运行示例 divides the top-K probabilities by their
                     sum; [P1] 公式表达重点 says the gates are renormalised).
    softmax_topk   : g = softmax of the K chosen logits ([P3] 三, MoERouter;
                     [P3] 2.1 diagram: top-K then softmax).  Equal to
                     renorm_all in exact arithmetic.
    prob_no_renorm : g = P[idx] ([P4] 结构 3 and [P3] 2.1 read literally).
    """
    if mode == "renorm_all":
        P = softmax_rows(logits)
        pk = np.take_along_axis(P, idx, axis=1)
        return pk / pk.sum(axis=1, keepdims=True)
    if mode == "softmax_topk":
        return softmax_rows(np.take_along_axis(logits, idx, axis=1))
    if mode == "prob_no_renorm":
        return np.take_along_axis(softmax_rows(logits), idx, axis=1)
    raise ValueError(mode)


# ----------------------------------------------------------------- stats ---

@dataclass
class RouterStats:
    count: np.ndarray   # [N] int64: pairs that chose e (before capacity)
    f: np.ndarray       # [N] count / (T*K)
    p: np.ndarray       # [N] mean router probability
    aux: float          # alpha * N * sum f*p
    z: float            # mean_t sum_e logits^2
    z_lse: float        # mean_t logsumexp(logits_t)^2  (not from the pages)
    entropy: float      # mean_t of the entropy of softmax(logits_t)


def router_stats(logits: np.ndarray, idx: np.ndarray, alpha: float) -> RouterStats:
    """Switch load-balance loss [P3] 2.2: L_aux = alpha * N * sum_i f_i p_i,
    f_i = share of routed slots that went to expert i, p_i = mean router
    probability of expert i.  [P3] 三 counts the top-K indices of all T
    tokens (before any capacity cut) and divides by T*K; that reading is
    taken, so sum_i f_i = 1.

    Router z-loss, [P1] Router Z-Loss: the page only says the sum of squares
    of the router logits is penalised.  Read literally as z = mean over
    tokens of sum_e logits^2, no coefficient.  z_lse (mean squared
    log-sum-exp) is an extra, common form that the pages do not give.
    """
    T, N = logits.shape
    K = idx.shape[1]
    count = np.zeros(N, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            count[idx[t, k]] += 1
    f = count / float(T * K)
    p = softmax_rows(logits).mean(axis=0)
    aux = float(alpha * N * np.sum(f * p))
    z = float(np.mean(np.sum(logits * logits, axis=1)))
    lse = logsumexp_rows(logits)
    z_lse = float(np.mean(lse * lse))
    entropy = routing_entropy(logits)
    return RouterStats(count=count, f=f, p=p, aux=aux, z=z, z_lse=z_lse, entropy=entropy)


def routing_entropy(logits: np.ndarray) -> float:
    """Mean over tokens of the entropy of the token's routing distribution,
    H_t = -sum_e P_te log P_te with P_t = softmax(logits_t).  [P5] lists
    routing entropy among what a training run monitors and gives no formula;
    this per-token mean is the plain reading (0 = every token certain of one
    expert, log N = uniform).  Terms with P = 0 contribute 0."""
    P = softmax_rows(np.asarray(logits, dtype=np.float64))
    T = P.shape[0]
    total = 0.0
    for t in range(T):
        row = P[t]
        nz = row[row > 0]
        total += float(-np.sum(nz * np.log(nz)))
    return total / T


def noisy_logits(logits: np.ndarray, noise: np.ndarray, noise_std: float) -> np.ndarray:
    """Training-time router noise, [P3] 三 (MoERouter.forward): a standard
    normal draw per (token, expert), scaled by noise_std, is added to the
    logits; top-K, the gates and the load-balance loss then all use the noisy
    logits.  The draws are an input here (the caller's generator), so both
    sides see the same numbers."""
    return np.asarray(logits, np.float64) + float(noise_std) * np.asarray(noise, np.float64)


def bias_update(b_sel, count: np.ndarray, T: int, K: int, rate: float) -> np.ndarray:
    """Auxiliary-loss-free balancing, [P4] 结构 4: the selection-only bias is
    not trained by gradients but moved after each step by how often its
    expert was chosen; an expert chosen too little gets a larger bias.

    Reading (the page gives neither the comparison nor the step): "too
    little" and "too much" are measured against the mean load T*K/N, and the
    bias moves by a fixed step `rate` up or down (the sign rule of the
    DeepSeek-V3 report the page cites); an expert exactly at the mean keeps
    its bias.  count = pairs that chose the expert, before capacity."""
    count = np.asarray(count, dtype=np.int64)
    N = count.shape[0]
    b = np.zeros(N) if b_sel is None else np.asarray(b_sel, np.float64).copy()
    for e in range(N):
        # compare count_e with T*K/N without rounding: count_e*N vs T*K
        diff = T * K - int(count[e]) * N
        step = 1.0 if diff > 0 else (-1.0 if diff < 0 else 0.0)
        b[e] = b[e] + rate * step
    return b


# -------------------------------------------------------------- capacity ---

def capacity(K: int, N: int, T: int, cf) -> int:
    """capacity = floor(K / N * CF * S)  [P3] 2.3, with S read as the number
    of tokens in the batch (the page's MoELayer uses B*S there).  Computed
    with exact rationals (CF taken from its decimal string), so it never
    suffers the floating truncation of int(K/N*CF*T).  cf=None: unlimited,
    returned as T (no expert can receive more than T tokens)."""
    if cf is None:
        return int(T)
    q = Fraction(K, N) * Fraction(str(cf)) * T
    return int(math.floor(q))


@dataclass
class Assignment:
    kept: np.ndarray      # [N] rows each expert keeps
    offset: np.ndarray    # [N+1] exclusive scan of kept
    pair_row: np.ndarray  # [T, K] row in the expert-contiguous buffer, -1 = dropped
    row_pair: np.ndarray  # [sum kept] t*K + k of each row
    dropped: np.ndarray   # [T, K] uint8
    n_dropped: int


def assign_capacity(idx: np.ndarray, N: int, cap: int) -> Assignment:
    """Token dropping [P3] 2.3 and 三: each expert takes the tokens that chose
    it in ascending token order and keeps the first `cap`; the rest are
    dropped (their contribution is 0; the residual outside the layer carries
    them).  Reading: the cap counts all K slots of an expert together (an
    expert appears at most once per token), whereas the page's loop caps
    each k slot separately; the two agree for K=1.

    Kept pairs are laid out expert-contiguously: expert e owns rows
    [offset[e], offset[e+1]) in ascending token order.
    """
    T, K = idx.shape
    rank = np.full((T, K), -1, dtype=np.int64)
    seen = np.zeros(N, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            rank[t, k] = seen[e]
            seen[e] += 1
    kept = np.minimum(seen, cap)
    offset = np.zeros(N + 1, dtype=np.int64)
    offset[1:] = np.cumsum(kept)
    pair_row = np.full((T, K), -1, dtype=np.int64)
    row_pair = np.full(int(offset[N]), -1, dtype=np.int64)
    dropped = np.zeros((T, K), dtype=np.uint8)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if rank[t, k] < cap:
                r = offset[e] + rank[t, k]
                pair_row[t, k] = r
                row_pair[r] = t * K + k
            else:
                dropped[t, k] = 1
    return Assignment(kept=kept, offset=offset, pair_row=pair_row,
                      row_pair=row_pair, dropped=dropped,
                      n_dropped=int(dropped.sum()))


# --------------------------------------------------------------- experts ---

def silu(u):
    """silu(u) = u * sigmoid(u) = u / (1 + exp(-u))."""
    return u / (1.0 + np.exp(-u))


def gelu_tanh(u):
    """Tanh approximation of GELU (Hendrycks & Gimpel):
    0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def expert_swiglu(xr, w1, w3, w2):
    """[P3] 三, Expert.forward: down( silu(gate(x)) * up(x) ).  Weights in
    linear-layer layout [out, in]: w1 (gate) [F, d], w3 (up) [F, d],
    w2 (down) [d, F].  No biases, dropout off (eval mode)."""
    g = xr @ np.asarray(w1, dtype=np.float64).T
    u = xr @ np.asarray(w3, dtype=np.float64).T
    return (silu(g) * u) @ np.asarray(w2, dtype=np.float64).T


def expert_gelu(xr, w1, w2, b1=None, b2=None):
    """[P4] 运行示例 expert: Linear(d, F) -> GELU -> Linear(F, d), biases
    optional; [P5] section 1 gives the same FFN(x) = W2 act(W1 x)."""
    h = xr @ np.asarray(w1, dtype=np.float64).T
    if b1 is not None:
        h = h + np.asarray(b1, dtype=np.float64)[None, :]
    o = gelu_tanh(h) @ np.asarray(w2, dtype=np.float64).T
    if b2 is not None:
        o = o + np.asarray(b2, dtype=np.float64)[None, :]
    return o


def run_expert(act, xr, e, W):
    if act == "swiglu":
        return expert_swiglu(xr, W["w1"][e], W["w3"][e], W["w2"][e])
    if act == "gelu_tanh":
        b1 = None if W.get("b1") is None else W["b1"][e]
        b2 = None if W.get("b2") is None else W["b2"][e]
        return expert_gelu(xr, W["w1"][e], W["w2"][e], b1, b2)
    raise ValueError(act)


def expert_outputs(act, x, asg: Assignment, W, N, K, experts=None):
    """y_perm[row] = E_e(x[t]) for every kept row, expert by expert, each as a
    dense matmul over that expert's rows (the page's per-expert loop, [P3]
    三).  `experts` limits the work to a subset (rows of others stay NaN)."""
    d = x.shape[1]
    y_perm = np.full((int(asg.offset[N]), d), np.nan)
    for e in range(N) if experts is None else experts:
        lo, hi = int(asg.offset[e]), int(asg.offset[e + 1])
        if hi == lo:
            continue
        toks = asg.row_pair[lo:hi] // K
        y_perm[lo:hi] = run_expert(act, x[toks], e, W)
    return y_perm


def combine(y_perm, pair_row, gates, T, d, y_shared=None):
    """y_t = sum_k [kept] g_tk * E_{idx_tk}(x_t) (+ shared expert), [P1]
    公式表达重点, [P3] 三 (gate-weighted accumulation), [P4] 结构 3.  A
    dropped pair adds nothing and the other gates are NOT renormalised."""
    y = np.zeros((T, d)) if y_shared is None else np.array(y_shared, dtype=np.float64)
    K = pair_row.shape[1]
    for t in range(T):
        for k in range(K):
            r = pair_row[t, k]
            if r >= 0:
                y[t] += gates[t, k] * y_perm[r]
    return y


# ----------------------------------------------------------------- layer ---

@dataclass
class LayerResult:
    logits: np.ndarray        # router output x W_r^T + b_r (before any noise)
    logits_used: np.ndarray   # what selection, gates and statistics see
    idx: np.ndarray
    margin: np.ndarray
    gates: np.ndarray
    stats: RouterStats
    cap: int
    asg: Assignment
    y_perm: np.ndarray | None
    y_shared: np.ndarray | None
    y: np.ndarray | None


def layer_forward(x, W, *, K, act, gate_mode, cf=None, alpha=1.0,
                  b_r=None, b_sel=None, shared=None, tokens=None,
                  experts_needed=True, noise=None, noise_std=0.0, idx=None):
    """Whole layer, in the order the pages give it: router logits, selection
    (scores + optional selection-only bias, [P4] 结构 4), gates (from the raw
    logits only), statistics, capacity and dispatch, per-expert FFN, shared
    expert ([P5] section 5), combine.

    W: dict of float64-able arrays w_r [N,d], w1 [N,F,d], w3 [N,F,d] (SwiGLU),
    w2 [N,d,F], optional b1 [N,F], b2 [N,d].  shared: None or dict
    (w1 [Fs,d], w3 [Fs,d], w2 [d,Fs]).
    tokens: optional list of token ids; routing/dispatch/stats are always
    computed for all T tokens, but the expert FFN and combine only for these
    tokens (y rows of other tokens are NaN).
    noise: optional [T, N] standard-normal draws; with it the router works on
    noisy_logits(logits, noise, noise_std) from selection on.
    idx: optional [T, K] chosen experts that replace this oracle's own top-K
    choice (another implementation's decisions on near-tie tokens, so that
    every later step can be compared from the same routing); the margin is
    still this oracle's.
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    N = W["w_r"].shape[0]
    logits = router_logits(x, W["w_r"], b_r)
    used = logits if noise is None else noisy_logits(logits, noise, noise_std)
    scores = used if b_sel is None else used + np.asarray(b_sel, np.float64)[None, :]
    own, margin = select_topk(scores, K)
    idx = own if idx is None else np.asarray(idx, dtype=np.int64)
    gates = gate_weights(used, idx, gate_mode)
    stats = router_stats(used, idx, alpha)
    cap = capacity(K, N, T, cf)
    asg = assign_capacity(idx, N, cap)
    if not experts_needed:
        return LayerResult(logits, used, idx, margin, gates, stats, cap, asg, None, None, None)
    if tokens is None:
        y_perm = expert_outputs(act, x, asg, W, N, K)
        y_shared = None if shared is None else expert_swiglu(
            x, shared["w1"], shared["w3"], shared["w2"])
        y = combine(y_perm, asg.pair_row, gates, T, d, y_shared)
    else:
        # only the listed tokens: each expert runs once over the listed
        # tokens it kept (so its weights are read once), then every token
        # sums its K terms in slot order
        tokens = np.asarray(tokens, dtype=np.int64)
        y_perm = None
        y = np.full((T, d), np.nan)
        y_shared = np.full((T, d), np.nan) if shared is not None else None
        if shared is not None:
            y_shared[tokens] = expert_swiglu(x[tokens], shared["w1"], shared["w3"], shared["w2"])
        term = {}
        for e in range(N):
            sel = [(int(t), k) for t in tokens for k in range(K)
                   if idx[t, k] == e and asg.pair_row[t, k] >= 0]
            if not sel:
                continue
            out = run_expert(act, x[[t for t, _ in sel]], e, W)
            for (t, k), o in zip(sel, out):
                term[(t, k)] = o
        for t in tokens:
            acc = np.zeros(d) if shared is None else y_shared[t].copy()
            for k in range(K):
                if (int(t), k) in term:
                    acc = acc + gates[t, k] * term[(int(t), k)]
            y[t] = acc
    return LayerResult(logits, used, idx, margin, gates, stats, cap, asg, y_perm, y_shared, y)


def brute_force_layer(x, W, *, K, act, gate_mode, cf=None, b_r=None,
                      b_sel=None, shared=None):
    """A second, independent route to the same output, following [P4]
    运行示例: run EVERY expert on EVERY token, then pick each token's chosen
    outputs and weight them.  Capacity (if any) is applied by listing, for
    each expert, the tokens that chose it and keeping the first `cap`.
    Used only on tiny inputs to cross-check layer_forward."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    N = W["w_r"].shape[0]
    logits = x @ np.asarray(W["w_r"], np.float64).T
    if b_r is not None:
        logits = logits + b_r
    scores = logits if b_sel is None else logits + b_sel
    # selection by exhaustive ranking: expert e outranks e' iff (s_e > s_e')
    # or (s_e == s_e' and e < e')
    idx = np.zeros((T, K), dtype=np.int64)
    for t in range(T):
        beaten_by = [sum(1 for j in range(N) if scores[t, j] > scores[t, e]
                         or (scores[t, j] == scores[t, e] and j < e)) for e in range(N)]
        for e in range(N):
            if beaten_by[e] < K:
                idx[t, beaten_by[e]] = e
    # gates via the masked-softmax form of [P1] 公式表达重点: scores of the
    # experts not chosen are set to -inf before the softmax
    masked = np.full_like(logits, -np.inf)
    np.put_along_axis(masked, idx, np.take_along_axis(logits, idx, axis=1), axis=1)
    if gate_mode == "prob_no_renorm":
        full = np.exp(logits - logits.max(axis=1, keepdims=True))
        full = full / full.sum(axis=1, keepdims=True)
        gates = np.take_along_axis(full, idx, axis=1)
    else:
        m = np.exp(masked - masked.max(axis=1, keepdims=True))
        gates = np.take_along_axis(m / m.sum(axis=1, keepdims=True), idx, axis=1)
    all_out = np.stack([run_expert(act, x, e, W) for e in range(N)], axis=1)  # [T,N,d]
    cap = capacity(K, N, T, cf)
    keep = np.zeros((T, K), dtype=bool)
    for e in range(N):
        chosen = [(t, k) for t in range(T) for k in range(K) if idx[t, k] == e]
        for (t, k) in chosen[:cap]:
            keep[t, k] = True
    y = np.zeros((T, d)) if shared is None else expert_swiglu(
        x, shared["w1"], shared["w3"], shared["w2"])
    for t in range(T):
        for k in range(K):
            if keep[t, k]:
                y[t] = y[t] + gates[t, k] * all_out[t, idx[t, k]]
    return idx, gates, keep, y
