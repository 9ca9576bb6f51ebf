"""CPU oracle for the backward pass of the token-choice Mixture-of-Experts FFN
layer: the vector-Jacobian product of the forward in oracle/moe_ref.py.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It is plain NumPy in
float64, imports neither torch nor the GPU library, and shares no code with
the GPU path (it builds on the forward oracle only).

What is differentiated.  The pages train the layer through the PyTorch
modules of [P3] section 三 (router, experts, MoELayer) plus the auxiliary
losses of [P3] 2.2 and the router z-loss of [P1] (Router Z-Loss); the
backward is what automatic differentiation computes through those modules.
For the scalar

    L = sum_{t,j} dy[t,j] * y[t,j] + c_aux * aux + c_z * z + c_zlse * z_lse

every function here returns dL/d(input).  Readings, where the pages leave
the step open:
  * Top-K selection, the capacity cut and the counts f are piecewise
    constant in the inputs, so their derivative is zero wherever it exists
    ([P5] lists the discrete routing choice among the training challenges;
    [P3] 三 builds the counts by scatter-adding constant ones).  Gradients
    reach the router only through the gate values and through p (aux loss),
    z and z_lse.
  * The selection-only bias ([P4] 结构 4) feeds selection alone: no gradient.
  * Router noise ([P3] 三) is added to the logits, so d/d(logits) equals
    d/d(noisy logits).
  * The routing entropy is a monitored quantity, not a loss: no gradient.
  * A dropped pair contributes nothing to y, so it passes no gradient to its
    expert and its gate receives none.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from oracle import moe_ref as ref


# ------------------------------------------------------------ activations ---

def silu_grad(u):
    """d/du [u * sigmoid(u)] = sigmoid(u) * (1 + u * (1 - sigmoid(u)))."""
    u = np.asarray(u, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def gelu_tanh_grad(u):
    """Derivative of 0.5 u (1 + tanh(a)), a = sqrt(2/pi) (u + 0.044715 u^3):
    0.5 (1 + tanh a) + 0.5 u (1 - tanh^2 a) sqrt(2/pi) (1 + 3 * 0.044715 u^2)."""
    u = np.asarray(u, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    th = np.tanh(c * (u + 0.044715 * u ** 3))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * c * (1.0 + 3.0 * 0.044715 * u * u)


# ---------------------------------------------------------------- experts ---

def expert_swiglu_backward(xr, w1, w3, w2, do):
    """Backward of o = (silu(xr w1^T) * (xr w3^T)) w2^T ([P3] 三, Expert).

    Returns (dxr [M,d], dw1 [F,d], dw3 [F,d], dw2 [d,F])."""
    xr = np.asarray(xr, np.float64)
    w1 = np.asarray(w1, np.float64)
    w3 = np.asarray(w3, np.float64)
    w2 = np.asarray(w2, np.float64)
    do = np.asarray(do, np.float64)
    u = xr @ w1.T
    v = xr @ w3.T
    s = ref.silu(u)
    h = s * v
    dw2 = do.T @ h
    dh = do @ w2
    du = dh * v * silu_grad(u)
    dv = dh * s
    dxr = du @ w1 + dv @ w3
    return dxr, du.T @ xr, dv.T @ xr, dw2


def expert_gelu_backward(xr, w1, w2, b1=None, b2=None, do=None):
    """Backward of o = gelu_tanh(xr w1^T + b1) w2^T + b2 ([P4] 运行示例).

    Returns (dxr, dw1 [F,d], dw2 [d,F], db1 [F] or None, db2 [d] or None)."""
    xr = np.asarray(xr, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    do = np.asarray(do, np.float64)
    u = xr @ w1.T
    if b1 is not None:
        u = u + np.asarray(b1, np.float64)[None, :]
    h = ref.gelu_tanh(u)
    dw2 = do.T @ h
    dh = do @ w2
    du = dh * gelu_tanh_grad(u)
    db1 = None if b1 is None else du.sum(axis=0)
    db2 = None if b2 is None else do.sum(axis=0)
    return du @ w1, du.T @ xr, dw2, db1, db2


# ---------------------------------------------------------------- combine ---

def combine_backward(dy, y_perm, pair_row, gates):
    """Backward of y_t = sum_k [kept] g_tk o_{row(t,k)} (+ shared):
    d o_row = g_tk dy_t for every kept pair, d g_tk = dy_t . o_row, and 0
    for a dropped pair.  Returns (d_perm [rows, d], dgate [T, K])."""
    dy = np.asarray(dy, np.float64)
    T, K = pair_row.shape
    d_perm = np.zeros((y_perm.shape[0], dy.shape[1]))
    dgate = np.zeros((T, K))
    for t in range(T):
        for k in range(K):
            r = int(pair_row[t, k])
            if r >= 0:
                d_perm[r] = gates[t, k] * dy[t]
                dgate[t, k] = float(np.dot(dy[t], y_perm[r]))
    return d_perm, dgate


# ----------------------------------------------------------------- router ---

def softmax_backward(P, dP):
    """dL/dl for P = softmax(l) given dL/dP: P * (dP - sum_e P_e dP_e)."""
    return P * (dP - np.sum(P * dP, axis=1, keepdims=True))


def gate_backward(used, idx, dgate, mode):
    """dL/d(logits) through the gates, following each mode's own definition
    (moe_ref.gate_weights) step by step.

    renorm_all     : g_k = P_{i_k} / S with S = sum_j P_{i_j} and
                     P = softmax(l): dP_{i_j} = (dg_j - sum_k dg_k g_k) / S,
                     then back through the softmax over all N.
    softmax_topk   : g = softmax(l[idx]): the softmax backward on the K
                     chosen logits, scattered back to their experts.
    prob_no_renorm : g_k = P_{i_k}: dP_{i_k} = dg_k, then the softmax
                     backward over all N."""
    used = np.asarray(used, np.float64)
    T, N = used.shape
    out = np.zeros((T, N))
    if mode == "softmax_topk":
        sel = np.take_along_axis(used, idx, axis=1)
        g = ref.softmax_rows(sel)
        dsel = softmax_backward(g, dgate)
        for t in range(T):
            for k in range(idx.shape[1]):
                out[t, idx[t, k]] += dsel[t, k]
        return out
    P = ref.softmax_rows(used)
    pk = np.take_along_axis(P, idx, axis=1)
    dP = np.zeros((T, N))
    if mode == "renorm_all":
        S = pk.sum(axis=1, keepdims=True)
        g = pk / S
        dpk = (dgate - np.sum(dgate * g, axis=1, keepdims=True)) / S
    elif mode == "prob_no_renorm":
        dpk = dgate
    else:
        raise ValueError(mode)
    for t in range(T):
        for k in range(idx.shape[1]):
            dP[t, idx[t, k]] += dpk[t, k]
    return softmax_backward(P, dP)


def stats_backward(used, count, K, alpha, c_aux=0.0, c_z=0.0, c_zlse=0.0, T=None):
    """dL/d(logits) through the losses of moe_ref.router_stats:
    aux = alpha N sum_e f_e p_e with p_e = mean_t P_te and f fixed
    ([P3] 2.2), z = mean_t sum_e l_te^2 ([P1] Router Z-Loss, literal
    reading) and z_lse = mean_t lse_t^2 (not from the pages).  Each token's
    row depends only on its own logits, so `used` may hold a subset of the
    rows; T is then the batch's token count (default: the rows given)."""
    used = np.asarray(used, np.float64)
    N = used.shape[1]
    T = used.shape[0] if T is None else T
    P = ref.softmax_rows(used)
    f = np.asarray(count, np.float64) / float(T * K)
    dP = np.broadcast_to(c_aux * alpha * N * f / T, used.shape)
    out = softmax_backward(P, dP)
    out = out + c_z * 2.0 * used / T
    lse = ref.logsumexp_rows(used)
    out = out + c_zlse * (2.0 * lse / T)[:, None] * P
    return out


# ------------------------------------------------------------------ layer ---

@dataclass
class LayerGrads:
    dx: np.ndarray
    dw_r: np.ndarray
    db_r: np.ndarray
    dw1: np.ndarray
    dw3: np.ndarray | None
    dw2: np.ndarray
    db1: np.ndarray | None
    db2: np.ndarray | None
    shared: dict | None       # dw1, dw3, dw2 of the shared expert
    dlogits: np.ndarray       # dL/d(router logits), [T, N]
    dgate: np.ndarray         # [T, K]
    d_perm: np.ndarray        # [rows, d] gradient of the expert outputs
    fwd: object               # the forward LayerResult


def layer_backward(x, W, dy, *, K, act, gate_mode, cf=None, alpha=1.0, b_r=None,
                   b_sel=None, shared=None, noise=None, noise_std=0.0,
                   c_aux=0.0, c_z=0.0, c_zlse=0.0, idx=None):
    """All gradients of L (module docstring) for the layer that
    moe_ref.layer_forward computes with the same arguments.

    Order: forward; combine backward (expert-output and gate gradients);
    each expert's FFN backward over its kept rows, scattered back to the
    tokens; the shared expert's backward (its output enters with weight 1,
    [P5] section 5); the gate and loss gradients on the logits; the router
    linear layer.  idx: optional routing to use instead of this oracle's own
    top-K choice (moe_ref.layer_forward)."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    N = W["w_r"].shape[0]
    dy = np.asarray(dy, np.float64)
    fwd = ref.layer_forward(x, W, K=K, act=act, gate_mode=gate_mode, cf=cf, alpha=alpha,
                            b_r=b_r, b_sel=b_sel, shared=shared, noise=noise,
                            noise_std=noise_std, idx=idx)
    asg = fwd.asg
    d_perm, dgate = combine_backward(dy, fwd.y_perm, asg.pair_row, fwd.gates)

    dx = np.zeros((T, d))
    dw1 = np.zeros(W["w1"].shape)   # arrays, or stacks widened one expert at a time
    dw2 = np.zeros(W["w2"].shape)
    dw3 = np.zeros(W["w3"].shape) if act == "swiglu" else None
    has_b = act == "gelu_tanh" and W.get("b1") is not None
    db1 = np.zeros(np.shape(W["b1"])) if has_b else None
    db2 = np.zeros(np.shape(W["b2"])) if act == "gelu_tanh" and W.get("b2") is not None else None
    for e in range(N):
        lo, hi = int(asg.offset[e]), int(asg.offset[e + 1])
        if hi == lo:
            continue
        toks = asg.row_pair[lo:hi] // K
        xr = x[toks]
        if act == "swiglu":
            dxr, dw1[e], dw3[e], dw2[e] = expert_swiglu_backward(
                xr, W["w1"][e], W["w3"][e], W["w2"][e], d_perm[lo:hi])
        else:
            b1 = None if W.get("b1") is None else W["b1"][e]
            b2 = None if W.get("b2") is None else W["b2"][e]
            dxr, dw1[e], dw2[e], g1, g2 = expert_gelu_backward(
                xr, W["w1"][e], W["w2"][e], b1, b2, d_perm[lo:hi])
            if g1 is not None:
                db1[e] = g1
            if g2 is not None:
                db2[e] = g2
        for i, t in enumerate(toks):
            dx[t] += dxr[i]

    gshared = None
    if shared is not None:
        dxs, s1, s3, s2 = expert_swiglu_backward(x, shared["w1"], shared["w3"], shared["w2"], dy)
        dx += dxs
        gshared = {"w1": s1, "w3": s3, "w2": s2}

    dl = gate_backward(fwd.logits_used, fwd.idx, dgate, gate_mode)
    dl = dl + stats_backward(fwd.logits_used, fwd.stats.count, K, alpha, c_aux, c_z, c_zlse)
    w_r = np.asarray(W["w_r"], np.float64)
    dx += dl @ w_r
    return LayerGrads(dx=dx, dw_r=dl.T @ x, db_r=dl.sum(axis=0), dw1=dw1, dw3=dw3, dw2=dw2,
                      db1=db1, db2=db2, shared=gshared, dlogits=dl, dgate=dgate,
                      d_perm=d_perm, fwd=fwd)


def layer_loss(x, W, dy, *, K, act, gate_mode, cf=None, alpha=1.0, b_r=None, b_sel=None,
               shared=None, noise=None, noise_std=0.0, c_aux=0.0, c_z=0.0, c_zlse=0.0):
    """The scalar L of the module docstring, from the forward oracle alone
    (what finite differences of the backward are taken against)."""
    r = ref.layer_forward(x, W, K=K, act=act, gate_mode=gate_mode, cf=cf, alpha=alpha,
                          b_r=b_r, b_sel=b_sel, shared=shared, noise=noise, noise_std=noise_std)
    s = r.stats
    return (float(np.sum(np.asarray(dy, np.float64) * r.y)) + c_aux * s.aux + c_z * s.z
            + c_zlse * s.z_lse), r


# ------------------------------------------------------- sampled entries ---

def _row(stack, e, f):
    """Row f of expert e's matrix, widened alone when the stack keeps bits."""
    if hasattr(stack, "bits"):
        return ref.bf16_bits_to_f64(stack.bits[e, f])
    return np.asarray(stack[e][f], np.float64)


def _col(stack, e, f):
    if hasattr(stack, "bits"):
        return ref.bf16_bits_to_f64(stack.bits[e][:, f])
    return np.asarray(stack[e][:, f], np.float64)


def layer_backward_sampled(x, W, dy, *, K, act, gate_mode, cf=None, alpha=1.0, b_r=None,
                           b_sel=None, shared=None, noise=None, noise_std=0.0, c_aux=0.0,
                           c_z=0.0, c_zlse=0.0, idx=None, tokens=(), wcols=()):
    """Selected entries of layer_backward's result, for sizes where the whole
    backward is too slow.  The definitions are the same, restricted to what
    the entries depend on: a token's rows (dx, dlogits, dgate) need only its
    own K expert rows and the shared expert; row f of dw1 / dw3 and column f
    of dw2 of expert e need only column f of the first expert GEMM over that
    expert's rows.

    tokens: token ids -> dict t -> {"dx", "dlogits", "dgate"}.
    wcols: (e, f) pairs, e == N meaning the shared expert ->
      dict (e, f) -> {"dw1": [d], "dw3": [d] (SwiGLU), "dw2": [d] (column f),
      "db1": float and "db2": [d] (GELU layers with biases)}.
    Returns (fwd, tok, wts) with fwd the routing-only forward result."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, d = x.shape
    N = W["w_r"].shape[0]
    fwd = ref.layer_forward(x, W, K=K, act=act, gate_mode=gate_mode, cf=cf, alpha=alpha, b_r=b_r,
                            b_sel=b_sel, shared=shared, noise=noise, noise_std=noise_std,
                            experts_needed=False, idx=idx)
    asg, gates = fwd.asg, fwd.gates
    tokens = [int(t) for t in tokens]
    # ---- token rows: each expert's sampled rows through that expert's FFN
    dxr = {t: np.zeros(d) for t in tokens}
    dg = {t: np.zeros(K) for t in tokens}
    for e in range(N):
        pairs = [(t, k) for t in tokens for k in range(K)
                 if fwd.idx[t, k] == e and asg.pair_row[t, k] >= 0]
        if not pairs:
            continue
        ts = [t for t, _ in pairs]
        X = x[ts]
        o = ref.run_expert(act, X, e, W)
        g = np.array([gates[t, k] for t, k in pairs])
        do = g[:, None] * dy[ts]
        if act == "swiglu":
            dX = expert_swiglu_backward(X, W["w1"][e], W["w3"][e], W["w2"][e], do)[0]
        else:
            b1 = None if W.get("b1") is None else W["b1"][e]
            dX = expert_gelu_backward(X, W["w1"][e], W["w2"][e], b1, None, do)[0]
        for i, (t, k) in enumerate(pairs):
            dg[t][k] = float(np.dot(dy[t], o[i]))
            dxr[t] = dxr[t] + dX[i]
    if shared is not None and tokens:
        dxs = expert_swiglu_backward(x[tokens], shared["w1"], shared["w3"], shared["w2"],
                                     dy[tokens])[0]
        for i, t in enumerate(tokens):
            dxr[t] = dxr[t] + dxs[i]
    tok = {}
    if tokens:
        used = fwd.logits_used[tokens]
        dgm = np.stack([dg[t] for t in tokens])
        dl = gate_backward(used, fwd.idx[tokens], dgm, gate_mode)
        dl = dl + stats_backward(used, fwd.stats.count, K, alpha, c_aux, c_z, c_zlse, T=T)
        w_r = np.asarray(W["w_r"], np.float64)
        for i, t in enumerate(tokens):
            tok[t] = {"dx": dxr[t] + dl[i] @ w_r, "dlogits": dl[i], "dgate": dg[t]}
    # ---- weight rows / columns
    wts = {}
    for e, f in wcols:
        e, f = int(e), int(f)
        if e < N:
            lo, hi = int(asg.offset[e]), int(asg.offset[e + 1])
            pr = asg.row_pair[lo:hi]
            toks, ks = pr // K, pr % K
            g = gates[toks, ks]
            src = {k: W.get(k) for k in ("w1", "w3", "w2")}
        else:
            toks = np.arange(T)
            g = np.ones(T)
            src = {k: (None if shared is None else shared[k][None]) for k in ("w1", "w3", "w2")}
        X = x[toks]
        ee = e if e < N else 0
        u = X @ _row(src["w1"], ee, f)
        if act == "gelu_tanh" and e < N and W.get("b1") is not None:
            u = u + float(np.asarray(W["b1"][e], np.float64)[f])
        dog = g[:, None] * dy[toks]                       # d(expert output) rows
        dh = dog @ _col(src["w2"], ee, f)                 # column f of dh
        rec = {}
        if act == "swiglu":
            v = X @ _row(src["w3"], ee, f)
            sg = ref.silu(u)
            du = dh * v * silu_grad(u)
            rec["dw3"] = (dh * sg) @ X
            h = sg * v
        else:
            du = dh * gelu_tanh_grad(u)
            h = ref.gelu_tanh(u)
            if e < N and W.get("b1") is not None:
                rec["db1"] = float(du.sum())
            if e < N and W.get("b2") is not None:
                rec["db2"] = dog.sum(axis=0)
        rec["dw1"] = du @ X
        rec["dw2"] = dog.T @ h                            # column f of dw2
        wts[(e, f)] = rec
    return fwd, tok, wts


def router_backward_full(x, W, dy, *, K, act, gate_mode, cf=None, alpha=1.0, b_r=None,
                         b_sel=None, shared=None, noise=None, noise_std=0.0, c_aux=0.0,
                         c_z=0.0, c_zlse=0.0, idx=None):
    """The router's gradients over every token, without the expert weight
    gradients (which at full size would not fit in memory as float64): the
    same steps as layer_backward up to the router linear layer, i.e. the
    forward, the combine backward's gate gradients, the gate and loss
    gradients on the logits, then dW_r = dlogits^T x and db_r = the column
    sums of dlogits.  Returns (fwd, dlogits [T, N], dgate [T, K], dw_r [N, d],
    db_r [N])."""
    x = np.asarray(x, np.float64)
    fwd = ref.layer_forward(x, W, K=K, act=act, gate_mode=gate_mode, cf=cf, alpha=alpha,
                            b_r=b_r, b_sel=b_sel, shared=shared, noise=noise,
                            noise_std=noise_std, idx=idx)
    _, dgate = combine_backward(dy, fwd.y_perm, fwd.asg.pair_row, fwd.gates)
    dl = gate_backward(fwd.logits_used, fwd.idx, dgate, gate_mode)
    dl = dl + stats_backward(fwd.logits_used, fwd.stats.count, K, alpha, c_aux, c_z, c_zlse)
    return fwd, dl, dgate, dl.T @ x, dl.sum(axis=0)
