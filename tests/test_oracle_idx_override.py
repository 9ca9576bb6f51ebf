"""Pins of the oracle's routing override (CPU only).

moe_ref.layer_forward and moe_bwd.layer_backward accept ``idx=``: a [T, K]
routing that replaces the oracle's own top-K choice.  The GPU parity tests
use it when a near-tie token's choice differs between the fp32 kernel and the
fp64 oracle, so that gates, statistics, the capacity cut, the combine and
every gradient are compared from one and the same routing.  These tests pin
that every later step really follows the injected routing, against routes
that do not go through the override:

  * the oracle's own choice injected back changes nothing, bit for bit;
  * a routing forced by a selection-only bias ([P4] 结构 4: it enters the
    choice, never the gates) equals the same routing injected with no bias,
    and the brute-force layer (compute every expert, then gather) agrees;
  * an arbitrary per-token routing (not the top-K) against values built
    here from library routines: scipy's softmax for the gates, numpy's
    bincount for the counts, a first-C list per expert for the capacity cut
    ([P3] 2.3), torch's CPU float64 FFN for the expert outputs;
  * the backward with an injected routing against central finite
    differences of the forward with the same injected routing.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_bwd as bwd
from oracle import moe_ref as ref


def rng(seed):
    return np.random.default_rng(seed)


def weights(r, N, d, F, act, Fs=0, bias=False):
    W = {"w_r": r.normal(size=(N, d)) / math.sqrt(d),
         "w1": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w2": r.normal(size=(N, d, F)) / math.sqrt(F)}
    if act == "swiglu":
        W["w3"] = r.normal(size=(N, F, d)) / math.sqrt(d)
    if bias:
        W["b1"] = r.normal(size=(N, F)) * 0.2
        W["b2"] = r.normal(size=(N, d)) * 0.2
    shared = None
    if Fs:
        shared = {"w1": r.normal(size=(Fs, d)) / math.sqrt(d),
                  "w3": r.normal(size=(Fs, d)) / math.sqrt(d),
                  "w2": r.normal(size=(d, Fs)) / math.sqrt(Fs)}
    return W, shared


def random_routing(r, T, N, K):
    """K distinct experts per token, uniformly at random (not the top-K)."""
    return np.stack([r.permutation(N)[:K] for _ in range(T)]).astype(np.int64)


def same_result(a, b):
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.gates, b.gates)
    assert np.array_equal(a.stats.count, b.stats.count)
    for k in ("f", "p"):
        assert np.array_equal(getattr(a.stats, k), getattr(b.stats, k))
    for k in ("aux", "z", "z_lse", "entropy"):
        assert getattr(a.stats, k) == getattr(b.stats, k), k
    for k in ("kept", "offset", "pair_row", "row_pair", "dropped"):
        assert np.array_equal(getattr(a.asg, k), getattr(b.asg, k)), k
    assert np.array_equal(a.y, b.y)


CASES = [
    # T, N, K, F, d, act, gate mode, capacity factor, shared width, biases
    (40, 8, 2, 6, 5, "swiglu", "softmax_topk", None, 0, False),
    (57, 6, 3, 5, 4, "gelu_tanh", "renorm_all", 1.0, 0, True),
    (33, 5, 2, 4, 6, "swiglu", "prob_no_renorm", 0.8, 4, False),
    (64, 16, 1, 4, 4, "gelu_tanh", "softmax_topk", 1.25, 0, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[0]}_N{c[1]}_K{c[2]}_{c[6]}")
def test_own_choice_injected_changes_nothing(case):
    T, N, K, F, d, act, mode, cf, Fs, bias = case
    r = rng(T + N)
    W, shared = weights(r, N, d, F, act, Fs, bias)
    x = r.normal(size=(T, d))
    b_sel = r.uniform(-0.5, 0.5, size=N)
    args = dict(K=K, act=act, gate_mode=mode, cf=cf, alpha=0.01, b_sel=b_sel, shared=shared)
    own = ref.layer_forward(x, W, **args)
    inj = ref.layer_forward(x, W, idx=own.idx.copy(), **args)
    same_result(own, inj)


@pytest.mark.parametrize("mode", ["softmax_topk", "renorm_all", "prob_no_renorm"])
def test_bias_forced_choice_equals_injected_choice(mode):
    """A huge selection-only bias on K experts makes them every token's
    choice.  Injecting that routing without the bias must give the same
    gates, statistics, capacity cut and output, and so must the brute-force
    layer with the bias."""
    T, N, K, F, d = 30, 6, 2, 5, 4
    r = rng(7)
    W, shared = weights(r, N, d, F, "swiglu", Fs=3)
    x = r.normal(size=(T, d))
    b_big = np.zeros(N)
    b_big[[4, 1]] = [1e3, 2e3]
    args = dict(K=K, act="swiglu", gate_mode=mode, cf=1.0, alpha=0.3, shared=shared)
    forced = ref.layer_forward(x, W, b_sel=b_big, **args)
    assert np.all(forced.idx == np.array([1, 4])[None, :])
    inj = ref.layer_forward(x, W, idx=forced.idx.copy(), **args)
    same_result(forced, inj)
    bidx, bg, keep, by = ref.brute_force_layer(x, W, K=K, act="swiglu", gate_mode=mode, cf=1.0,
                                               b_sel=b_big, shared=shared)
    assert np.array_equal(bidx, inj.idx)
    assert np.allclose(bg, inj.gates, rtol=0, atol=1e-15)
    assert np.array_equal(keep, inj.asg.pair_row >= 0)
    assert np.allclose(by, inj.y, rtol=0, atol=1e-12)
    # capacity 1.0 * K * T / N = 10 of 30 tokens per chosen expert: 20 dropped each
    assert inj.asg.n_dropped == 2 * (T - 10)


def torch_expert(X, e, W, act):
    t = lambda a: torch.tensor(np.asarray(a, np.float64))  # noqa: E731
    Xt = t(X)
    if act == "swiglu":
        h = torch.nn.functional.silu(Xt @ t(W["w1"][e]).T) * (Xt @ t(W["w3"][e]).T)
        return (h @ t(W["w2"][e]).T).numpy()
    u = Xt @ t(W["w1"][e]).T + (t(W["b1"][e]) if "b1" in W else 0.0)
    o = torch.nn.functional.gelu(u, approximate="tanh") @ t(W["w2"][e]).T
    return (o + (t(W["b2"][e]) if "b2" in W else 0.0)).numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"T{c[0]}_N{c[1]}_K{c[2]}_{c[6]}")
def test_arbitrary_routing_flows_into_every_step(case):
    T, N, K, F, d, act, mode, cf, Fs, bias = case
    r = rng(100 + T)
    W, shared = weights(r, N, d, F, act, Fs, bias)
    x = r.normal(size=(T, d))
    X = random_routing(r, T, N, K)
    alpha = 0.02
    res = ref.layer_forward(x, W, K=K, act=act, gate_mode=mode, cf=cf, alpha=alpha,
                            shared=shared, idx=X)
    own = ref.layer_forward(x, W, K=K, act=act, gate_mode=mode, cf=cf, alpha=alpha,
                            shared=shared)
    assert not np.array_equal(own.idx, X)  # the override is really a different routing
    assert np.array_equal(res.idx, X)
    # gates, from scipy's softmax
    lg = x @ W["w_r"].T
    P = scipy.special.softmax(lg, axis=1)
    pk = np.take_along_axis(P, X, axis=1)
    if mode == "softmax_topk":
        g = scipy.special.softmax(np.take_along_axis(lg, X, axis=1), axis=1)
    elif mode == "renorm_all":
        g = pk / pk.sum(axis=1, keepdims=True)
    else:
        g = pk
    assert np.allclose(res.gates, g, rtol=0, atol=1e-14)
    # statistics: counts of the injected routing; p does not depend on it
    cnt = np.bincount(X.ravel(), minlength=N)
    assert np.array_equal(res.stats.count, cnt)
    assert np.allclose(res.stats.f, cnt / (T * K), rtol=0, atol=1e-16)
    assert np.allclose(res.stats.p, P.mean(axis=0), rtol=0, atol=1e-15)
    assert abs(res.stats.aux - alpha * N * np.sum(cnt / (T * K) * P.mean(axis=0))) < 1e-15
    # capacity cut: each expert keeps the first C tokens (ascending) that chose it
    C = ref.capacity(K, N, T, cf)
    keep = np.zeros((T, K), dtype=bool)
    for e in range(N):
        chosen = [(t, k) for t in range(T) for k in range(K) if X[t, k] == e]
        for t, k in chosen[:C]:
            keep[t, k] = True
    assert np.array_equal(res.asg.pair_row >= 0, keep)
    assert np.array_equal(res.asg.kept, np.minimum(cnt, C))
    # output: every expert on every token (torch), then gather and weight
    allo = np.stack([torch_expert(x, e, W, act) for e in range(N)], axis=1)
    y = np.zeros((T, d))
    if shared is not None:
        Wsh = {"w1": shared["w1"][None], "w3": shared["w3"][None], "w2": shared["w2"][None]}
        y += torch_expert(x, 0, Wsh, "swiglu")
    for t in range(T):
        for k in range(K):
            if keep[t, k]:
                y[t] += g[t, k] * allo[t, X[t, k]]
    assert np.allclose(res.y, y, rtol=0, atol=1e-12)
    # the token-subset path follows the override too
    sub = [0, 3, T - 1]
    part = ref.layer_forward(x, W, K=K, act=act, gate_mode=mode, cf=cf, alpha=alpha,
                             shared=shared, idx=X, tokens=sub)
    assert np.allclose(part.y[sub], y[sub], rtol=0, atol=1e-12)


EPS = 1e-6


def fd(arr, f):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + EPS
        fp = f()
        arr[i] = old - EPS
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * EPS)
    return g


@pytest.mark.parametrize("act,mode,cf,Fs", [("swiglu", "softmax_topk", None, 3),
                                            ("gelu_tanh", "renorm_all", 1.0, 0),
                                            ("swiglu", "prob_no_renorm", 0.75, 0)])
def test_backward_follows_injected_routing(act, mode, cf, Fs):
    """With the routing held fixed the loss is smooth in every input, so the
    backward with an injected routing must equal central differences of the
    forward with the same routing (no margin condition is needed)."""
    T, N, K, F, d = 9, 5, 2, 4, 4
    r = rng(hash((act, mode)) % 1000)
    W, shared = weights(r, N, d, F, act, Fs, bias=(act == "gelu_tanh"))
    x = r.normal(size=(T, d))
    dy = r.normal(size=(T, d))
    X = random_routing(r, T, N, K)
    coef = dict(c_aux=0.6, c_z=0.2, c_zlse=0.1)
    args = dict(K=K, act=act, gate_mode=mode, cf=cf, alpha=0.05, shared=shared)

    def loss():
        o = ref.layer_forward(x, W, idx=X, **args)
        return (float(np.sum(dy * o.y)) + coef["c_aux"] * o.stats.aux + coef["c_z"] * o.stats.z
                + coef["c_zlse"] * o.stats.z_lse)

    G = bwd.layer_backward(x, W, dy, idx=X, **args, **coef)
    own = bwd.layer_backward(x, W, dy, **args, **coef)
    assert not np.array_equal(own.fwd.idx, X)

    def close(a, b, what):
        tol = 2e-7 * (1.0 + np.abs(b).max())
        assert np.abs(np.asarray(a) - b).max() <= tol, what

    close(G.dx, fd(x, loss), "dx")
    close(G.dw_r, fd(W["w_r"], loss), "dw_r")
    close(G.dw1, fd(W["w1"], loss), "dw1")
    close(G.dw2, fd(W["w2"], loss), "dw2")
    if act == "swiglu":
        close(G.dw3, fd(W["w3"], loss), "dw3")
    else:
        close(G.db1, fd(W["b1"], loss), "db1")
    if shared is not None:
        close(G.shared["w1"], fd(shared["w1"], loss), "shared w1")
    # the sampled entries follow the injected routing as well
    toks = [0, 4, 8]
    wcols = [(e, f) for e in range(N) for f in (0, F - 1)]
    _, tok, wts = bwd.layer_backward_sampled(x, W, dy, idx=X, tokens=toks, wcols=wcols,
                                             **args, **coef)
    for t in toks:
        assert np.allclose(tok[t]["dx"], G.dx[t], rtol=0, atol=1e-12)
        assert np.allclose(tok[t]["dlogits"], G.dlogits[t], rtol=0, atol=1e-12)
    for (e, f), rec in wts.items():
        assert np.allclose(rec["dw1"], G.dw1[e][f], rtol=0, atol=1e-12)
        assert np.allclose(rec["dw2"], G.dw2[e][:, f], rtol=0, atol=1e-12)
