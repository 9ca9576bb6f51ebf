"""Glue between seeded torch inputs and the NumPy oracle (test-only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_ref as ref


def f64(t):
    """Exact widening of a bf16/fp32 torch tensor to float64 numpy (host)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_bits(t):
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_weights(inp: dict, bf16: bool):
    """Weights in the oracle's form: expert stacks stay bf16 bits and are
    widened one expert at a time."""
    stack = (lambda t: ref.Bf16Stack(bf16_bits(t))) if bf16 else f64
    W = {"w_r": f64(inp["w_r"]), "w1": stack(inp["w1"]), "w2": stack(inp["w2"])}
    if inp.get("w3") is not None:
        W["w3"] = stack(inp["w3"])
    if inp.get("b1") is not None:
        W["b1"] = f64(inp["b1"])
        W["b2"] = f64(inp["b2"])
    shared = None
    if inp.get("ws1") is not None:
        shared = {"w1": f64(inp["ws1"]), "w3": f64(inp["ws3"]), "w2": f64(inp["ws2"])}
    return W, shared


def run_oracle(w, inp, tokens=None, experts_needed=True, idx=None, weights=None):
    """The forward oracle on the inputs of workload w (idx: a routing to use
    instead of the oracle's own top-K choice; weights: oracle_weights(inp)
    when already built)."""
    W, shared = weights if weights is not None else oracle_weights(inp, w.dtype == "bf16")
    return ref.layer_forward(f64(inp["x"]), W, K=w.K, act=w.act, gate_mode=w.gate, cf=w.cf,
                             alpha=w.aux_alpha, b_r=f64(inp["b_r"]), b_sel=f64(inp["b_sel"]),
                             shared=shared, tokens=tokens, experts_needed=experts_needed,
                             idx=idx)


def rel_err(got, want) -> float:
    """max |got - want| / max |want| (the tolerance rule for float outputs)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.max(np.abs(want))
    if den == 0:
        return float(np.max(np.abs(got - want))) if got.size else 0.0
    return float(np.max(np.abs(got - want)) / den)


TOL_BF16 = 2e-2
TOL_F32 = 1e-5
NEAR_TIE = 1e-3

# one line per routing comparison: label, tokens in the near-tie band, and
# how many of them the GPU chose differently (printed at the end of the run)
NEAR_TIE_REPORT: list = []


def report_near_ties(label, n_band, n_diff, T):
    NEAR_TIE_REPORT.append(f"{label}: {n_band} of {T} tokens within {NEAR_TIE} of a tie, "
                           f"{n_diff} chosen differently")
