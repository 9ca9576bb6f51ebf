"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties an oracle function to something the pages print, to a closed
form, to an independent brute-force route, or to a library routine, chosen
so that a plausible slip (dropped term, wrong sign or index, transposed
operand, missing renormalisation, wrong normaliser) fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rand_weights(r, N, d, F, act, bias=False, Fs=0):
    W = {"w_r": r.normal(size=(N, d)) / math.sqrt(d),
         "w1": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w2": r.normal(size=(N, d, F)) / math.sqrt(F)}
    if act == "swiglu":
        W["w3"] = r.normal(size=(N, F, d)) / math.sqrt(d)
    if bias:
        W["b1"] = r.normal(size=(N, F)) * 0.1
        W["b2"] = r.normal(size=(N, d)) * 0.1
    shared = None
    if Fs:
        shared = {"w1": r.normal(size=(Fs, d)) / math.sqrt(d),
                  "w3": r.normal(size=(Fs, d)) / math.sqrt(d),
                  "w2": r.normal(size=(d, Fs)) / math.sqrt(Fs)}
    return W, shared


# ------------------------------------------------------- page worked example

def test_worked_example_8_experts_top2():
    """wmrh.cn 具体数值示例: 8 experts, top-2 -> expert 6 (0.67), expert 2 (0.33)."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_8x2.json")))
    N, K = g["N"], g["K"]
    # logits that realise the example: l6 - l2 = ln 2, the other six lower
    logits = np.full(N, -1.5)
    logits[2] = 0.3
    logits[6] = 0.3 + math.log(2.0)
    logits[[0, 1, 3, 4, 5, 7]] = [-1.0, -0.2, -2.0, 0.1, -0.7, -3.0]
    x = logits[None, :]
    W = {"w_r": np.eye(N)}  # router output equals x
    lg = ref.router_logits(x, W["w_r"])
    idx, margin = ref.select_topk(lg, K)
    assert list(idx[0]) == g["experts"]
    for mode in ("renorm_all", "softmax_topk"):
        gates = ref.gate_weights(lg, idx, mode)[0]
        assert [round(v, 2) for v in gates] == g["gates_2dp"]
        assert abs(gates.sum() - 1.0) < 1e-15
        assert abs(gates[0] - 2.0 / 3.0) < 1e-15
    # without renormalisation the printed weights are NOT reproduced
    raw = ref.gate_weights(lg, idx, "prob_no_renorm")[0]
    assert [round(v, 2) for v in raw] != g["gates_2dp"]
    # only the two chosen experts get rows
    asg = ref.assign_capacity(idx, N, ref.capacity(K, N, 1, None))
    assert list(asg.kept) == [1 if e in (6, 2) else 0 for e in range(N)]


# ------------------------------------------------------------ aux loss pins

@pytest.mark.parametrize("N,K", [(4, 1), (4, 2), (8, 2), (64, 1), (64, 8), (256, 8)])
@pytest.mark.parametrize("alpha", [0.01, 1.0])
def test_aux_equals_alpha_when_uniform(N, K, alpha):
    """mzlw.cn 2.2: when f_i = p_i = 1/N the loss equals alpha."""
    v = rng(N * 10 + K).permutation(N).astype(np.float64) * 0.37  # distinct entries
    m = 3
    T = N * m
    x = np.stack([np.roll(v, t % N) for t in range(T)])  # each value visits each expert m times
    lg = ref.router_logits(x, np.eye(N))
    idx, _ = ref.select_topk(lg, K)
    st = ref.router_stats(lg, idx, alpha)
    assert np.allclose(st.f, 1.0 / N, rtol=0, atol=1e-15)
    assert np.allclose(st.p, 1.0 / N, rtol=0, atol=1e-15)
    assert abs(st.aux - alpha) < 1e-14


def test_aux_closed_form_nonuniform():
    """Hand-worked: one token, logits ln(1..4), top-2 -> experts 3,2;
    p = (.1,.2,.3,.4), f = (0,0,.5,.5); aux = alpha*4*(.5*.3+.5*.4) = 1.4 alpha."""
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    idx, _ = ref.select_topk(lg, 2)
    assert list(idx[0]) == [3, 2]
    st = ref.router_stats(lg, idx, 0.01)
    assert np.allclose(st.p, [0.1, 0.2, 0.3, 0.4], atol=1e-15)
    assert np.allclose(st.f, [0, 0, 0.5, 0.5], atol=0)
    assert abs(st.aux - 0.014) < 1e-15


def test_counts_match_bincount():
    r = rng(5)
    T, N, K = 300, 16, 3
    lg = r.normal(size=(T, N))
    idx, _ = ref.select_topk(lg, K)
    st = ref.router_stats(lg, idx, 1.0)
    assert np.array_equal(st.count, np.bincount(idx.ravel(), minlength=N))
    assert abs(st.f.sum() - 1.0) < 1e-14
    assert abs(st.p.sum() - 1.0) < 1e-12


def test_zloss_closed_forms():
    """All logits equal to c: z = N c^2, logsumexp = c + ln N."""
    for N, c in [(4, 0.5), (64, -1.25), (256, 2.0)]:
        lg = np.full((5, N), c)
        idx = np.tile(np.arange(2), (5, 1))
        st = ref.router_stats(lg, idx, 1.0)
        assert abs(st.z - N * c * c) < 1e-12
        assert abs(st.z_lse - (c + math.log(N)) ** 2) < 1e-12


# ------------------------------------------------------------ capacity pins

def test_capacity_golden_cases():
    g = json.load(open(os.path.join(GOLDEN, "capacity_cases.json")))
    for c in g["cases"]:
        assert ref.capacity(c["K"], c["N"], c["T"], c["cf"]) == c["capacity"], c


@pytest.mark.parametrize("cf", [1.0, 1.1, 1.25, 1.5, 2.0, 0.3])
def test_capacity_is_largest_integer_within_budget(cf):
    """Characterisation independent of the floor formula: the capacity c is
    the largest integer with c * N <= K * CF * T (checked by search, with CF
    as an exact decimal ratio)."""
    num, den = {1.0: (10, 10), 1.1: (11, 10), 1.25: (125, 100), 1.5: (15, 10),
                2.0: (2, 1), 0.3: (3, 10)}[cf]
    for K, N in [(1, 64), (2, 8), (8, 256), (1, 3), (3, 7)]:
        for T in [0, 1, 5, 16, 128, 1000, 8192]:
            c = 0
            while (c + 1) * N * den <= K * num * T:
                c += 1
            assert ref.capacity(K, N, T, cf) == c
    assert ref.capacity(2, 8, 77, None) == 77


# ------------------------------------------------------------ top-K pins

def test_topk_matches_subset_enumeration():
    r = rng(11)
    for N, K in [(4, 1), (5, 2), (6, 3), (7, 7), (8, 2)]:
        s = r.normal(size=(20, N))
        idx, margin = ref.select_topk(s, K)
        for t in range(20):
            best = max(itertools.combinations(range(N), K), key=lambda c: sum(s[t, list(c)]))
            assert set(idx[t]) == set(best)
            assert all(s[t, idx[t, i]] >= s[t, idx[t, i + 1]] for i in range(K - 1))
            if K < N:
                rest = sorted(set(range(N)) - set(idx[t]), key=lambda e: -s[t, e])
                assert abs(margin[t] - (s[t, idx[t, K - 1]] - s[t, rest[0]])) < 1e-15


def test_exact_ties_go_to_lower_index():
    """Duplicate router rows give bit-identical logits: lower id must win."""
    r = rng(3)
    N, d = 8, 16
    w = r.normal(size=(N, d))
    w[5] = w[2]
    w[7] = w[2]
    x = r.normal(size=(50, d))
    x[:, :] = x * np.sign(x @ w[2])[:, None]  # make the tied experts score high
    lg = ref.router_logits(x, w)
    hits = 0
    for K in (1, 2, 3):
        idx, margin = ref.select_topk(lg, K)
        for t in range(50):
            top = int(np.argmax(lg[t]))
            if lg[t, top] == lg[t, 2]:
                hits += 1
                tied = [e for e in range(N) if lg[t, e] == lg[t, 2]]
                assert tied == [2, 5, 7]
                assert tied[:K] == list(idx[t, :K])
                assert margin[t] == (0.0 if K < 3 else margin[t])
    assert hits > 10


# ------------------------------------------------------------ gate forms

def test_three_gate_forms_agree():
    """wmrh.cn: mask the rest to -inf then softmax; mzlw.cn: softmax of the
    top-K logits; learnagent.wiki: softmax over all then divide by the top-K
    sum.  Equal in exact arithmetic."""
    r = rng(7)
    lg = r.normal(size=(64, 16)) * 3
    for K in (1, 2, 8, 16):
        idx, _ = ref.select_topk(lg, K)
        a = ref.gate_weights(lg, idx, "renorm_all")
        b = ref.gate_weights(lg, idx, "softmax_topk")
        masked = np.full_like(lg, -np.inf)
        np.put_along_axis(masked, idx, np.take_along_axis(lg, idx, 1), 1)
        e = np.exp(masked - masked.max(1, keepdims=True))
        c = np.take_along_axis(e / e.sum(1, keepdims=True), idx, 1)
        assert np.max(np.abs(a - b)) < 1e-15
        assert np.max(np.abs(a - c)) < 1e-15
        if K == 1:
            assert np.all(a == 1.0)


# ------------------------------------------------- activations vs library

def test_activations_match_torch():
    torch = pytest.importorskip("torch")
    u = np.linspace(-12, 12, 2001)
    tu = torch.tensor(u, dtype=torch.float64)
    assert np.max(np.abs(ref.silu(u) - torch.nn.functional.silu(tu).numpy())) < 1e-14
    gt = torch.nn.functional.gelu(tu, approximate="tanh").numpy()
    assert np.max(np.abs(ref.gelu_tanh(u) - gt)) < 1e-14
    # the tanh form stays within 1e-3 of the erf form (published bound ~5e-4)
    ge = torch.nn.functional.gelu(tu).numpy()
    assert np.max(np.abs(ref.gelu_tanh(u) - ge)) < 1e-3


def test_softmax_matches_scipy():
    sp = pytest.importorskip("scipy.special")
    v = rng(1).normal(size=(10, 33)) * 5
    assert np.max(np.abs(ref.softmax_rows(v) - sp.softmax(v, axis=1))) < 1e-15
    assert np.max(np.abs(ref.logsumexp_rows(v) - sp.logsumexp(v, axis=1))) < 1e-13


# ------------------------------------------- special cases vs library FFNs

def _torch_ffn(x, w1, w3, w2, act, b1=None, b2=None):
    """Expert FFN built from torch.nn.Linear (the page's module structure)."""
    import torch
    F, d = w1.shape
    with torch.no_grad():
        l1 = torch.nn.Linear(d, F, bias=b1 is not None).double()
        l1.weight.copy_(torch.tensor(w1))
        if b1 is not None:
            l1.bias.copy_(torch.tensor(b1))
        l2 = torch.nn.Linear(F, d, bias=b2 is not None).double()
        l2.weight.copy_(torch.tensor(w2))
        if b2 is not None:
            l2.bias.copy_(torch.tensor(b2))
        tx = torch.tensor(x)
        if act == "swiglu":
            l3 = torch.nn.Linear(d, F, bias=False).double()
            l3.weight.copy_(torch.tensor(w3))
            h = torch.nn.functional.silu(l1(tx)) * l3(tx)
        else:
            h = torch.nn.functional.gelu(l1(tx), approximate="tanh")
        return l2(h).numpy()


@pytest.mark.parametrize("act", ["swiglu", "gelu_tanh"])
def test_single_expert_is_plain_ffn(act):
    """N = K = 1: the layer reduces to one FFN (mstx.cn section 1)."""
    pytest.importorskip("torch")
    r = rng(21)
    T, d, F = 9, 12, 20  # non-square so a transposed operand fails
    W, _ = rand_weights(r, 1, d, F, act, bias=(act == "gelu_tanh"))
    x = r.normal(size=(T, d))
    res = ref.layer_forward(x, W, K=1, act=act, gate_mode="softmax_topk")
    want = _torch_ffn(x, W["w1"][0], W.get("w3", [None])[0], W["w2"][0], act,
                      W.get("b1", [None])[0], W.get("b2", [None])[0])
    assert np.max(np.abs(res.y - want)) < 1e-12
    assert np.all(res.gates == 1.0)


def test_k_equals_n_is_dense_soft_mixture():
    """K = N, no capacity, renormalised gates: y = sum_e softmax(l)_e E_e(x)."""
    torch = pytest.importorskip("torch")
    r = rng(22)
    T, d, F, N = 6, 10, 14, 4
    W, _ = rand_weights(r, N, d, F, "swiglu")
    x = r.normal(size=(T, d))
    res = ref.layer_forward(x, W, K=N, act="swiglu", gate_mode="renorm_all")
    P = torch.softmax(torch.tensor(x) @ torch.tensor(W["w_r"]).T, dim=1).numpy()
    want = sum(P[:, e:e + 1] * _torch_ffn(x, W["w1"][e], W["w3"][e], W["w2"][e], "swiglu")
               for e in range(N))
    assert np.max(np.abs(res.y - want)) < 1e-12


def test_shared_expert_adds_plain_ffn():
    torch = pytest.importorskip("torch")
    r = rng(23)
    T, d, F, N, K, Fs = 10, 8, 12, 5, 2, 6
    W, shared = rand_weights(r, N, d, F, "swiglu", Fs=Fs)
    x = r.normal(size=(T, d))
    a = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="softmax_topk", shared=shared)
    b = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="softmax_topk")
    want = _torch_ffn(x, shared["w1"], shared["w3"], shared["w2"], "swiglu")
    assert np.max(np.abs((a.y - b.y) - want)) < 1e-12


# ------------------------------------------------ sparse vs brute force

CASES = [
    # T, N, K, d, F, act, cf, bias, sel, Fs, mode
    (7, 4, 2, 6, 10, "gelu_tanh", None, True, False, 0, "renorm_all"),
    (12, 4, 1, 8, 6, "swiglu", 1.0, False, False, 0, "softmax_topk"),
    (20, 6, 2, 8, 12, "swiglu", 1.25, False, True, 0, "softmax_topk"),
    (16, 5, 3, 7, 9, "swiglu", 0.5, False, True, 4, "softmax_topk"),
    (15, 8, 2, 5, 6, "gelu_tanh", 0.3, True, False, 0, "prob_no_renorm"),
    (9, 3, 3, 4, 5, "swiglu", None, False, False, 3, "renorm_all"),
]


@pytest.mark.parametrize("case", CASES)
def test_sparse_matches_brute_force(case):
    """learnagent.wiki 运行示例 computes every expert on every token and then
    gathers; that route must agree with the sparse per-expert dispatch."""
    T, N, K, d, F, act, cf, bias, sel, Fs, mode = case
    r = rng(hash(case) % 2**32)
    W, shared = rand_weights(r, N, d, F, act, bias=bias, Fs=Fs)
    x = r.normal(size=(T, d))
    b_r = r.normal(size=N) * 0.5 if bias else None
    b_sel = r.uniform(-0.5, 0.5, size=N) if sel else None
    res = ref.layer_forward(x, W, K=K, act=act, gate_mode=mode, cf=cf, b_r=b_r,
                            b_sel=b_sel, shared=shared)
    idx, gates, keep, y = ref.brute_force_layer(x, W, K=K, act=act, gate_mode=mode,
                                                cf=cf, b_r=b_r, b_sel=b_sel, shared=shared)
    assert np.array_equal(res.idx, idx)
    assert np.max(np.abs(res.gates - gates)) < 1e-15
    assert np.array_equal(res.asg.dropped == 0, keep)
    assert np.max(np.abs(res.y - y)) < 1e-12
    # token-subset evaluation gives the same rows
    sub = [0, T // 2, T - 1]
    res2 = ref.layer_forward(x, W, K=K, act=act, gate_mode=mode, cf=cf, b_r=b_r,
                             b_sel=b_sel, shared=shared, tokens=sub)
    assert np.max(np.abs(res2.y[sub] - y[sub])) < 1e-12


def test_selection_bias_does_not_enter_gates():
    """learnagent.wiki 结构 4: the per-expert bias only steers the choice."""
    r = rng(31)
    T, N, K, d = 40, 8, 2, 8
    W, _ = rand_weights(r, N, d, 4, "swiglu")
    x = r.normal(size=(T, d))
    b_sel = np.zeros(N)
    b_sel[3] = 100.0  # forces expert 3 into every token's set
    res = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="softmax_topk",
                            b_sel=b_sel, experts_needed=False)
    assert np.all(res.idx[:, 0] == 3)
    lg = x @ W["w_r"].T
    want = ref.softmax_rows(np.take_along_axis(lg, res.idx, 1))
    assert np.max(np.abs(res.gates - want)) < 1e-15


# ------------------------------------------------ dispatch invariants

@pytest.mark.parametrize("T,N,K,cf", [(200, 8, 2, 1.0), (333, 16, 3, 0.7),
                                      (64, 4, 4, None), (1, 4, 2, 1.0), (0, 4, 2, 1.0),
                                      (500, 64, 1, 1.25)])
def test_dispatch_invariants(T, N, K, cf):
    r = rng(T + N)
    skew = np.exp(2.0 * r.normal(size=N))
    idx = np.array([r.choice(N, size=K, replace=False, p=skew / skew.sum())
                    for _ in range(T)], dtype=np.int64).reshape(T, K)
    cap = ref.capacity(K, N, T, cf)
    a = ref.assign_capacity(idx, N, cap)
    cnt = np.bincount(idx.ravel(), minlength=N)
    assert np.array_equal(a.kept, np.minimum(cnt, cap))
    assert a.kept.sum() + a.n_dropped == T * K
    assert a.offset[0] == 0 and np.all(np.diff(a.offset) == a.kept)
    for e in range(N):
        rows = a.row_pair[a.offset[e]:a.offset[e + 1]]
        toks = rows // K
        assert np.all(np.diff(toks) > 0)                  # ascending token order
        assert np.all(idx[toks, rows % K] == e)
        # the kept tokens are exactly the first `cap` tokens that chose e
        chose = [t for t in range(T) if e in idx[t]]
        assert list(toks) == chose[:cap]
    for t in range(T):
        for k in range(K):
            rr = a.pair_row[t, k]
            assert (rr < 0) == bool(a.dropped[t, k])
            if rr >= 0:
                assert a.row_pair[rr] == t * K + k


def test_bf16_decoding():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    v = ref.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[3] == 0.0
    assert abs(v[2] - 3.140625) == 0.0
    assert v[5] == float.fromhex("0x1.fep127")
    assert v[6] == 2.0 ** -133


# ------------------------------------------- router training variants pins

def test_entropy_closed_forms():
    """Uniform logits: H = ln N.  Two experts with P = (1/4, 3/4):
    H = -(1/4 ln 1/4 + 3/4 ln 3/4).  One dominant expert: H -> 0."""
    for N in (2, 8, 256):
        lg = np.full((3, N), 0.7)
        assert abs(ref.routing_entropy(lg) - math.log(N)) < 1e-13
    lg = np.array([[0.2, 0.2 + math.log(3.0)]])
    want = -(0.25 * math.log(0.25) + 0.75 * math.log(0.75))
    assert abs(ref.routing_entropy(lg) - want) < 1e-15
    lg = np.array([[0.0, -60.0, -60.0, -60.0]])
    assert ref.routing_entropy(lg) < 1e-23


def test_entropy_matches_scipy():
    """Against scipy.stats.entropy of scipy.special.softmax rows (an
    independent library route: different softmax, different entropy sum)."""
    import scipy.special
    import scipy.stats
    r = rng(41)
    lg = r.normal(size=(50, 37)) * 3.0
    want = float(np.mean(scipy.stats.entropy(scipy.special.softmax(lg, axis=1), axis=1)))
    assert abs(ref.routing_entropy(lg) - want) < 1e-12
    st = ref.router_stats(lg, ref.select_topk(lg, 4)[0], 1.0)
    assert st.entropy == ref.routing_entropy(lg)


def test_noise_zero_is_the_clean_router():
    r = rng(42)
    T, N, d, K = 40, 16, 32, 3
    x = r.normal(size=(T, d))
    W, _ = rand_weights(r, N, d, 64, "swiglu")
    clean = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="softmax_topk",
                              experts_needed=False)
    for noise, std in [(np.zeros((T, N)), 0.1), (r.normal(size=(T, N)), 0.0)]:
        res = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="softmax_topk",
                                experts_needed=False, noise=noise, noise_std=std)
        assert np.array_equal(res.idx, clean.idx)
        assert np.array_equal(res.gates, clean.gates)
        assert np.array_equal(res.logits, clean.logits)
        assert res.stats.z == clean.stats.z and res.stats.entropy == clean.stats.entropy


def test_noise_constant_per_token_closed_forms():
    """Noise c_t shared by every expert of a token shifts the token's logits:
    softmax, top-K and gates do not change (shift invariance), and the
    z-loss gains exactly 2 s mean_t(c_t sum_e l_te) + N s^2 mean_t(c_t^2)."""
    r = rng(43)
    T, N, d, K, s = 30, 12, 16, 2, 0.25
    x = r.normal(size=(T, d))
    W, _ = rand_weights(r, N, d, 64, "swiglu")
    c = r.normal(size=T)
    noise = np.repeat(c[:, None], N, axis=1)
    clean = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="renorm_all",
                              experts_needed=False)
    res = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="renorm_all",
                            experts_needed=False, noise=noise, noise_std=s)
    assert np.array_equal(res.idx, clean.idx)
    assert np.allclose(res.gates, clean.gates, rtol=0, atol=1e-14)
    assert np.allclose(res.stats.p, clean.stats.p, rtol=0, atol=1e-14)
    assert abs(res.stats.entropy - clean.stats.entropy) < 1e-12
    lg = clean.logits
    dz = 2 * s * np.mean(c * lg.sum(axis=1)) + N * s * s * np.mean(c * c)
    assert abs(res.stats.z - (clean.stats.z + dz)) < 1e-10
    assert np.array_equal(res.logits, clean.logits)  # the router output itself is clean


def test_noise_spike_forces_the_choice():
    """A noise spike on one expert of each token puts it first, and the
    statistics follow the noisy logits (p_e is the mean noisy probability)."""
    r = rng(44)
    T, N, d, K = 25, 10, 16, 2
    x = r.normal(size=(T, d))
    W, _ = rand_weights(r, N, d, 64, "swiglu")
    forced = r.integers(0, N, size=T)
    noise = np.zeros((T, N))
    noise[np.arange(T), forced] = 1000.0
    res = ref.layer_forward(x, W, K=K, act="swiglu", gate_mode="softmax_topk",
                            experts_needed=False, noise=noise, noise_std=0.1)
    assert np.array_equal(res.idx[:, 0], forced)
    assert np.allclose(res.gates[:, 0], 1.0, atol=1e-12)
    want_p = np.bincount(forced, minlength=N) / T
    assert np.allclose(res.stats.p, want_p, atol=1e-12)


def test_bias_update_rules():
    """Hand-worked: N=4, K=1, T=8, counts (4,2,2,0): mean load 2, so the
    over-loaded expert 0 loses `rate`, expert 3 gains it, 1 and 2 keep theirs.
    Balanced counts leave the bias alone; a missing bias counts as zero."""
    b = np.array([0.5, -0.25, 0.0, 1.0])
    out = ref.bias_update(b, np.array([4, 2, 2, 0]), T=8, K=1, rate=0.125)
    assert np.array_equal(out, [0.375, -0.25, 0.0, 1.125])
    assert np.array_equal(b, [0.5, -0.25, 0.0, 1.0])  # input untouched
    assert np.array_equal(ref.bias_update(b, np.array([3, 3, 3, 3]), T=6, K=2, rate=1.0), b)
    assert np.array_equal(ref.bias_update(None, np.array([5, 1, 0]), T=3, K=2, rate=0.5),
                          [-0.5, 0.5, 0.5])  # mean load 2: 5 above it, 1 and 0 below


def test_bias_update_uses_exact_mean():
    """T*K/N = 7/3 is not an integer: counts 2 (below) and 3 (above) move
    in opposite directions; no rounding of the mean may merge them."""
    out = ref.bias_update(None, np.array([2, 3, 2]), T=7, K=1, rate=1.0)
    assert np.array_equal(out, [1.0, -1.0, 1.0])


# ------------------------------------------------ weight-only INT8 pins

def test_int8_hand_worked_row():
    """Row (2, -1.5, 0.3, 0): absmax 2, s = 2/127; codes 127, -95 (-95.25),
    19 (19.05), 0.  A second row scaled by -1 gives the negated codes."""
    w = np.array([[2.0, -1.5, 0.3, 0.0], [-2.0, 1.5, -0.3, 0.0]])
    q, s = ref.quantize_int8_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert q[0].tolist() == [127, -95, 19, 0]
    assert q[1].tolist() == [-127, 95, -19, 0]
    assert s[0] == np.float32(2.0) / np.float32(127.0) and s[1] == s[0]


def test_int8_error_bound_and_extremes():
    """|w - q s| <= s/2 (plus fp32 slack), the absmax entry codes to +-127,
    a zero row stays zero, and the codes are odd-symmetric."""
    r = rng(61)
    w = (r.normal(size=(40, 96)) * r.uniform(0.01, 3.0, size=(40, 1))).astype(np.float32)
    w[7] = 0.0
    q, s = ref.quantize_int8_rows(w)
    deq = ref.dequantize_int8_rows(q, s)
    err = np.abs(deq - w.astype(np.float64))
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 1e-6) + 1e-30)
    amax_col = np.argmax(np.abs(w), axis=1)
    for i in range(40):
        if i == 7:
            continue
        assert abs(int(q[i, amax_col[i]])) == 127
    assert np.all(q[7] == 0) and s[7] == 0 and np.all(deq[7] == 0)
    qn, sn = ref.quantize_int8_rows(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    assert np.abs(q.astype(int)).max() <= 127


def test_int8_stack_feeds_the_expert_ffn():
    """An expert FFN on Int8Stack weights equals the same FFN on the dense
    dequantized matrices, and differs from the unquantized FFN by no more
    than the weight error allows (a first-order bound on the output)."""
    r = rng(62)
    N, F, d, M = 3, 64, 32, 5
    W = {"w1": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w3": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w2": r.normal(size=(N, d, F)) / math.sqrt(F)}
    Wq = {k: ref.Int8Stack(*ref.quantize_int8_rows(v)) for k, v in W.items()}
    xr = r.normal(size=(M, d))
    for e in range(N):
        dense = {k: ref.dequantize_int8_rows(*ref.quantize_int8_rows(W[k][e])) for k in W}
        a = ref.run_expert("swiglu", xr, e, Wq)
        b = ref.expert_swiglu(xr, dense["w1"], dense["w3"], dense["w2"])
        assert np.array_equal(a, b)
        full = ref.run_expert("swiglu", xr, e, W)
        assert np.max(np.abs(a - full)) < 0.05 * np.max(np.abs(full))


# ------------------------------------------------ weight-only INT4 pins

def test_int4_hand_worked_group():
    """Group (2, -1.5, 0.3, 0, 0 ...): absmax 2, s = 2/7; codes 7, -5
    (-5.25), 1 (1.05), 0.  The negated group gives the negated codes; a
    second group of the same row is quantized on its own."""
    w = np.zeros((2, 256))
    w[0, :4] = [2.0, -1.5, 0.3, 0.0]
    w[1, :4] = [-2.0, 1.5, -0.3, 0.0]
    w[0, 128] = 0.7
    q, s = ref.quantize_int4_groups(w)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (2, 2)
    assert q[0, :4].tolist() == [7, -5, 1, 0] and q[1, :4].tolist() == [-7, 5, -1, 0]
    assert s[0, 0] == np.float32(2.0) / np.float32(7.0) and s[1, 0] == s[0, 0]
    assert q[0, 128] == 7 and s[0, 1] == np.float32(0.7) / np.float32(7.0)
    assert s[1, 1] == 0 and np.all(q[1, 128:] == 0)  # an all-zero group


def test_int4_round_half_to_even():
    """With absmax 7 the scale is 1, so w / s = w exactly: 2.5 -> 2, 3.5 -> 4,
    -0.5 -> 0, -1.5 -> -2 (ties to even)."""
    w = np.zeros((1, 128))
    w[0, :5] = [7.0, 2.5, 3.5, -0.5, -1.5]
    q, s = ref.quantize_int4_groups(w)
    assert s[0, 0] == 1.0
    assert q[0, :5].tolist() == [7, 2, 4, 0, -2]


def test_int4_error_bound_and_extremes():
    """|w - q s| <= s/2 (plus fp32 slack) per group, every group's absmax
    entry codes to +-7, codes stay in [-7, 7], a group's codes do not move
    when another group of the row changes, and the codes are
    odd-symmetric."""
    r = rng(63)
    w = (r.normal(size=(24, 384)) * r.uniform(0.01, 3.0, size=(24, 1))).astype(np.float32)
    w[5, 128:256] = 0.0
    q, s = ref.quantize_int4_groups(w)
    deq = ref.dequantize_int4_groups(q, s)
    err = np.abs(deq - w.astype(np.float64))
    assert np.all(err <= np.repeat(s.astype(np.float64), 128, axis=1) * (0.5 + 1e-6) + 1e-30)
    assert np.abs(q.astype(int)).max() <= 7
    g = w.reshape(24, 3, 128)
    am = np.argmax(np.abs(g), axis=2)
    for i in range(24):
        for j in range(3):
            if i == 5 and j == 1:
                continue
            assert abs(int(q[i, 128 * j + am[i, j]])) == 7
    assert np.all(q[5, 128:256] == 0) and s[5, 1] == 0
    w2 = w.copy()
    w2[:, 256:] *= 3.0
    q2, s2 = ref.quantize_int4_groups(w2)
    assert np.array_equal(q2[:, :256], q[:, :256]) and np.array_equal(s2[:, :2], s[:, :2])
    qn, sn = ref.quantize_int4_groups(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def test_int4_packing_layout():
    """Hand-worked word: codes (7, -5, 1, 0, 0, 0, 0, 0) of columns 0..7 are
    stored as u = q + 8 = (15, 3, 9, 8, 8, 8, 8, 8); even columns fill the
    low half-word's nibbles 0..3, odd columns the high half-word's, so the
    word is 0x8883889F (bytes 9F 88 83 88).  Packing round-trips."""
    q = np.zeros((1, 8), dtype=np.int8)
    q[0, :3] = [7, -5, 1]
    p = ref.pack_int4(q)
    assert p.dtype == np.uint8 and p.shape == (1, 4)
    assert p[0].tolist() == [0x9F, 0x88, 0x83, 0x88]
    r = rng(64)
    qq = r.integers(-7, 8, size=(3, 5, 256)).astype(np.int8)
    assert np.array_equal(ref.unpack_int4(ref.pack_int4(qq)), qq)


def test_int4_stack_feeds_the_expert_ffn():
    """An expert FFN on Int4Stack weights equals the same FFN on the dense
    dequantized matrices, and stays near the unquantized FFN (a loose bound:
    7 levels per side)."""
    r = rng(65)
    N, F, d, M = 2, 128, 256, 4
    W = {"w1": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w3": r.normal(size=(N, F, d)) / math.sqrt(d),
         "w2": r.normal(size=(N, d, F)) / math.sqrt(F)}
    Wq = {}
    for k, v in W.items():
        q, s = ref.quantize_int4_groups(v)
        Wq[k] = ref.Int4Stack(ref.pack_int4(q), s)
    xr = r.normal(size=(M, d))
    for e in range(N):
        dense = {k: ref.dequantize_int4_groups(*ref.quantize_int4_groups(W[k][e])) for k in W}
        a = ref.run_expert("swiglu", xr, e, Wq)
        b = ref.expert_swiglu(xr, dense["w1"], dense["w3"], dense["w2"])
        assert np.array_equal(a, b)
        full = ref.run_expert("swiglu", xr, e, W)
        assert np.max(np.abs(a - full)) < 0.3 * np.max(np.abs(full))
