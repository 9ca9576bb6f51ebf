"""Pins of the backward oracle (oracle/moe_bwd.py) to facts outside itself
(CPU only).

The main pin is the forward oracle: every gradient is compared, entry by
entry, with central finite differences of the scalar loss computed by
moe_ref.layer_forward (which has its own pins).  Selection and the capacity
cut are piecewise constant, so each case checks first that its top-K margin
is far wider than the step.  Independent routes add: torch's CPU autograd in
float64 for the expert FFNs (a library routine), closed forms for the z-loss
and for the aux loss at uniform load, and the invariants of the gate
Jacobians.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_bwd as bwd
from oracle import moe_ref as ref

EPS = 1e-6


def rng(seed):
    return np.random.default_rng(seed)


def make_case(seed, *, T, d, N, K, F, act, bias=False, Fs=0, sel_bias=False, router_bias=False,
              noise=False):
    r = rng(seed)
    x = r.normal(size=(T, d))
    W = {"w_r": r.normal(size=(N, d)) * 0.8,
         "w1": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w2": r.normal(size=(N, d, F)) / math.sqrt(F)}
    if act == "swiglu":
        W["w3"] = r.normal(size=(N, F, d)) / math.sqrt(d)
    if bias:
        W["b1"] = r.normal(size=(N, F)) * 0.3
        W["b2"] = r.normal(size=(N, d)) * 0.3
    shared = None
    if Fs:
        shared = {"w1": r.normal(size=(Fs, d)) / math.sqrt(d),
                  "w3": r.normal(size=(Fs, d)) / math.sqrt(d),
                  "w2": r.normal(size=(d, Fs)) / math.sqrt(Fs)}
    extra = {"b_r": r.normal(size=N) * 0.5 if router_bias else None,
             "b_sel": r.uniform(-0.5, 0.5, size=N) if sel_bias else None,
             "noise": r.normal(size=(T, N)) if noise else None,
             "noise_std": 0.3 if noise else 0.0}
    dy = r.normal(size=(T, d))
    return x, W, shared, extra, dy


CASES = [
    # id, shape, act, gate mode, capacity factor, flags, loss coefficients
    ("swiglu_softmax_topk", dict(T=7, d=5, N=4, K=2, F=6), "swiglu", "softmax_topk", None,
     dict(), (0.0, 0.0, 0.0)),
    ("swiglu_renorm_cap_aux", dict(T=9, d=4, N=4, K=2, F=5), "swiglu", "renorm_all", 1.0,
     dict(), (0.7, 0.0, 0.0)),
    ("gelu_bias_renorm_z", dict(T=6, d=5, N=3, K=2, F=4), "gelu_tanh", "renorm_all", None,
     dict(bias=True, router_bias=True), (0.0, 0.4, 0.0)),
    ("gelu_noren_zlse_cap", dict(T=8, d=4, N=5, K=2, F=3), "gelu_tanh", "prob_no_renorm", 1.0,
     dict(), (0.5, 0.2, 0.3)),
    ("swiglu_shared_selbias", dict(T=6, d=4, N=6, K=3, F=4), "swiglu", "softmax_topk", None,
     dict(Fs=4, sel_bias=True), (1.0, 0.1, 0.0)),
    ("swiglu_k1_cap_noise", dict(T=8, d=4, N=4, K=1, F=3), "swiglu", "renorm_all", 1.0,
     dict(noise=True, router_bias=True), (0.9, 0.0, 0.2)),
    ("gelu_k_eq_n", dict(T=5, d=3, N=3, K=3, F=4), "gelu_tanh", "prob_no_renorm", None,
     dict(bias=True), (0.3, 0.0, 0.0)),
]


def loss_fn(x, W, shared, extra, dy, shape, act, mode, cf, coef):
    return bwd.layer_loss(x, W, dy, K=shape["K"], act=act, gate_mode=mode, cf=cf, alpha=0.01 * 37,
                          b_r=extra["b_r"], b_sel=extra["b_sel"], shared=shared,
                          noise=extra["noise"], noise_std=extra["noise_std"],
                          c_aux=coef[0], c_z=coef[1], c_zlse=coef[2])[0]


def fd(arr, f):
    """Central differences of f() with respect to every entry of arr (in place)."""
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


def close(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    tol = 2e-7 * (1.0 + np.abs(b).max())
    assert a.shape == b.shape, what
    err = np.abs(a - b).max()
    assert err <= tol, (what, err, tol)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gradients_match_finite_differences(case):
    name, shape, act, mode, cf, flags, coef = case
    x, W, shared, extra, dy = make_case(len(name) * 13 + shape["T"], act=act, **shape, **flags)
    args = dict(K=shape["K"], act=act, gate_mode=mode, cf=cf, alpha=0.01 * 37, b_r=extra["b_r"],
                b_sel=extra["b_sel"], shared=shared, noise=extra["noise"],
                noise_std=extra["noise_std"], c_aux=coef[0], c_z=coef[1], c_zlse=coef[2])
    G = bwd.layer_backward(x, W, dy, **args)
    # finite differences are valid only if no selection flips within the step
    assert G.fwd.margin.min() > 1e-4, G.fwd.margin.min()
    if cf is not None:
        assert G.fwd.asg.n_dropped > 0 or name == "swiglu_k1_cap_noise"
    f = lambda: loss_fn(x, W, shared, extra, dy, shape, act, mode, cf, coef)  # noqa: E731
    close(G.dx, fd(x, f), "dx")
    close(G.dw_r, fd(W["w_r"], f), "dw_r")
    close(G.dw1, fd(W["w1"], f), "dw1")
    close(G.dw2, fd(W["w2"], f), "dw2")
    if act == "swiglu":
        close(G.dw3, fd(W["w3"], f), "dw3")
    if flags.get("bias"):
        close(G.db1, fd(W["b1"], f), "db1")
        close(G.db2, fd(W["b2"], f), "db2")
    if extra["b_r"] is not None:
        close(G.db_r, fd(extra["b_r"], f), "db_r")
    if extra["b_sel"] is not None:
        # selection-only bias: the loss does not move with it
        close(np.zeros_like(extra["b_sel"]), fd(extra["b_sel"], f), "db_sel")
    if shared is not None:
        for k in ("w1", "w3", "w2"):
            close(G.shared[k], fd(shared[k], f), "shared " + k)


def test_dropped_pairs_pass_no_gradient():
    """With capacity 1 per expert most pairs drop; their gates get 0 and
    their tokens get no expert gradient from that slot."""
    x, W, _, _, dy = make_case(5, T=8, d=4, N=2, K=1, F=3, act="swiglu")
    G = bwd.layer_backward(x, W, dy, K=1, act="swiglu", gate_mode="softmax_topk", cf=0.25)
    drop = G.fwd.asg.pair_row < 0
    assert drop.sum() == 6
    assert np.all(G.dgate[drop] == 0.0)
    # a token all of whose pairs dropped gets only the router's gradient
    t = int(np.nonzero(drop[:, 0])[0][0])
    assert np.allclose(G.dx[t], G.dlogits[t] @ W["w_r"], rtol=0, atol=1e-14)


# ------------------------------------------------ library-routine routes ---

def torch_expert(xr, w1, w3, w2, do, act, b1=None, b2=None):
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    X, A, C, B = t(xr), t(w1), t(w2), (t(w3) if w3 is not None else None)
    P1 = t(b1) if b1 is not None else None
    P2 = t(b2) if b2 is not None else None
    if act == "swiglu":
        o = (torch.nn.functional.silu(X @ A.T) * (X @ B.T)) @ C.T
        ins = [X, A, B, C]
    else:
        u = X @ A.T + (P1 if P1 is not None else 0.0)
        o = torch.nn.functional.gelu(u, approximate="tanh") @ C.T + (P2 if P2 is not None else 0.0)
        ins = [X, A, C] + [p for p in (P1, P2) if p is not None]
    grads = torch.autograd.grad(o, ins, torch.tensor(do, dtype=torch.float64))
    return [g.numpy() for g in grads]


def test_swiglu_expert_backward_matches_torch_autograd():
    r = rng(11)
    M, d, F = 9, 7, 5
    xr, w1, w3, w2 = r.normal(size=(M, d)), r.normal(size=(F, d)), r.normal(size=(F, d)), \
        r.normal(size=(d, F))
    do = r.normal(size=(M, d))
    ours = bwd.expert_swiglu_backward(xr, w1, w3, w2, do)
    theirs = torch_expert(xr, w1, w3, w2, do, "swiglu")  # dX, dW1, dW3, dW2
    for a, b in zip(ours, theirs):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_gelu_expert_backward_matches_torch_autograd():
    r = rng(12)
    M, d, F = 8, 6, 4
    xr, w1, w2 = r.normal(size=(M, d)), r.normal(size=(F, d)), r.normal(size=(d, F))
    b1, b2, do = r.normal(size=F), r.normal(size=d), r.normal(size=(M, d))
    dxr, dw1, dw2, db1, db2 = bwd.expert_gelu_backward(xr, w1, w2, b1, b2, do)
    tx, tw1, tw2, tb1, tb2 = torch_expert(xr, w1, None, w2, do, "gelu", b1, b2)
    for a, b in [(dxr, tx), (dw1, tw1), (dw2, tw2), (db1, tb1), (db2, tb2)]:
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_activation_derivatives():
    u = np.linspace(-9.0, 9.0, 181)
    h = 1e-6
    assert np.allclose(bwd.silu_grad(u), (ref.silu(u + h) - ref.silu(u - h)) / (2 * h), atol=1e-9)
    assert np.allclose(bwd.gelu_tanh_grad(u), (ref.gelu_tanh(u + h) - ref.gelu_tanh(u - h)) / (2 * h),
                       atol=1e-9)
    # special values: silu'(0) = 1/2, gelu'(0) = 1/2; both tend to 1 and 0
    assert bwd.silu_grad(0.0) == 0.5 and bwd.gelu_tanh_grad(0.0) == 0.5
    assert abs(bwd.silu_grad(40.0) - 1.0) < 1e-15 and abs(bwd.silu_grad(-40.0)) < 1e-15


# ------------------------------------------------------------ closed forms ---

def test_zloss_gradient_closed_form():
    """z = mean_t sum_e l^2 gives dL/dl = 2 c_z l / T, so dW_r = (2 c_z / T) l^T x."""
    x, W, _, _, _ = make_case(21, T=6, d=5, N=4, K=2, F=3, act="swiglu")
    dy = np.zeros((6, 5))
    G = bwd.layer_backward(x, W, dy, K=2, act="swiglu", gate_mode="softmax_topk", c_z=1.5)
    lg = x @ W["w_r"].T
    assert np.allclose(G.dlogits, 3.0 * lg / 6, rtol=0, atol=1e-14)
    assert np.allclose(G.dw_r, (3.0 / 6) * lg.T @ x, rtol=0, atol=1e-13)


def test_aux_gradient_vanishes_at_uniform_load():
    """With every expert chosen equally often (f = 1/N) the aux gradient on
    each token's logits is P * (f - sum f P) = 0 ([P3] 2.2 balance point)."""
    N, K, m = 4, 2, 2
    v = np.array([0.9, 0.2, -0.4, -1.1])
    T = N * m
    x = np.stack([np.roll(v, t % N) for t in range(T)])
    W = {"w_r": np.eye(N), "w1": np.ones((N, 2, N)), "w3": np.ones((N, 2, N)),
         "w2": np.ones((N, N, 2))}
    G = bwd.layer_backward(x, W, np.zeros((T, N)), K=K, act="swiglu", gate_mode="softmax_topk",
                           alpha=0.01, c_aux=1.0)
    assert np.all(G.fwd.stats.count == T * K // N)
    assert np.abs(G.dlogits).max() < 1e-16


def test_aux_gradient_closed_form_single_token():
    """T = 1, K = 1: aux = alpha N P_{i}, so dL/dl = alpha N P_i (onehot_i - P)."""
    l = np.array([[0.3, -0.2, 1.1, 0.0]])
    P = ref.softmax_rows(l)[0]
    g = bwd.stats_backward(l, np.array([0, 0, 1, 0]), 1, 0.5, c_aux=1.0)[0]
    assert np.allclose(g, 0.5 * 4 * P[2] * (np.eye(4)[2] - P), rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode", ["renorm_all", "softmax_topk", "prob_no_renorm"])
def test_gate_jacobian_invariants(mode):
    """Renormalised gates sum to 1, so their logit gradient sums to 0 over the
    chosen experts and is 0 elsewhere; the raw probabilities sum to less than
    one, so prob_no_renorm spreads gradient to every expert and sums to 0 over
    all N (softmax is shift-invariant)."""
    r = rng(31)
    l = r.normal(size=(5, 6))
    idx, _ = ref.select_topk(l, 3)
    dg = r.normal(size=(5, 3))
    dl = bwd.gate_backward(l, idx, dg, mode)
    assert np.abs(dl.sum(axis=1)).max() < 1e-15
    mask = np.zeros_like(l, dtype=bool)
    np.put_along_axis(mask, idx, True, axis=1)
    if mode == "prob_no_renorm":
        assert np.all(dl[~mask] != 0.0)
    elif mode == "softmax_topk":
        assert np.all(dl[~mask] == 0.0)
    else:  # through the full softmax: zero up to rounding
        assert np.abs(dl[~mask]).max() < 1e-15
    # K = 1 renormalised: the gate is 1 whatever the logits, so no gradient
    idx1, _ = ref.select_topk(l, 1)
    if mode != "prob_no_renorm":
        assert np.abs(bwd.gate_backward(l, idx1, dg[:, :1], mode)).max() < 1e-16


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sampled_entries_equal_the_full_backward(case):
    """layer_backward_sampled (what the full-size GPU tests compare against)
    gives exactly the entries of layer_backward."""
    name, shape, act, mode, cf, flags, coef = case
    x, W, shared, extra, dy = make_case(len(name) * 13 + shape["T"], act=act, **shape, **flags)
    args = dict(K=shape["K"], act=act, gate_mode=mode, cf=cf, alpha=0.37, b_r=extra["b_r"],
                b_sel=extra["b_sel"], shared=shared, noise=extra["noise"],
                noise_std=extra["noise_std"], c_aux=coef[0], c_z=coef[1], c_zlse=coef[2])
    G = bwd.layer_backward(x, W, dy, **args)
    N, F = shape["N"], shape["F"]
    tokens = list(range(0, shape["T"], 2))
    wcols = [(e, f) for e in range(N) for f in (0, F - 1)]
    if shared is not None:
        wcols += [(N, 0), (N, shared["w1"].shape[0] - 1)]
    fwd, tok, wts = bwd.layer_backward_sampled(x, W, dy, tokens=tokens, wcols=wcols, **args)
    for t in tokens:
        assert np.allclose(tok[t]["dx"], G.dx[t], rtol=0, atol=1e-12)
        assert np.allclose(tok[t]["dlogits"], G.dlogits[t], rtol=0, atol=1e-12)
        assert np.allclose(tok[t]["dgate"], G.dgate[t], rtol=0, atol=1e-12)
    for (e, f), rec in wts.items():
        if e < N:
            w1, w2, w3 = G.dw1[e], G.dw2[e], (G.dw3[e] if act == "swiglu" else None)
        else:
            w1, w2, w3 = G.shared["w1"], G.shared["w2"], G.shared["w3"]
        assert np.allclose(rec["dw1"], w1[f], rtol=0, atol=1e-12)
        assert np.allclose(rec["dw2"], w2[:, f], rtol=0, atol=1e-12)
        if act == "swiglu":
            assert np.allclose(rec["dw3"], w3[f], rtol=0, atol=1e-12)
        if "db1" in rec:
            assert abs(rec["db1"] - G.db1[e, f]) < 1e-12
            assert np.allclose(rec["db2"], G.db2[e], rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_router_backward_full_equals_the_full_backward(case):
    """router_backward_full (what the full-size GPU tests compare the router
    gradients with) gives exactly layer_backward's router gradients."""
    name, shape, act, mode, cf, flags, coef = case
    x, W, shared, extra, dy = make_case(len(name) * 13 + shape["T"], act=act, **shape, **flags)
    args = dict(K=shape["K"], act=act, gate_mode=mode, cf=cf, alpha=0.37, b_r=extra["b_r"],
                b_sel=extra["b_sel"], shared=shared, noise=extra["noise"],
                noise_std=extra["noise_std"], c_aux=coef[0], c_z=coef[1], c_zlse=coef[2])
    G = bwd.layer_backward(x, W, dy, **args)
    _, dl, dg, dw_r, db_r = bwd.router_backward_full(x, W, dy, **args)
    for a, b in [(dl, G.dlogits), (dg, G.dgate), (dw_r, G.dw_r), (db_r, G.db_r)]:
        assert np.allclose(a, b, rtol=0, atol=1e-12)
