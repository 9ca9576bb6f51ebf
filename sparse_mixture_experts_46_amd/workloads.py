"""The six layer shapes this library is measured and checked on.

Every shape is a token-choice MoE FFN layer forward on one GPU.  The model
families they imitate are the ones the pages name (Mixtral 8 experts top-2,
Switch top-1, DeepSeek-V3 256 experts top-8 with a shared expert:
learnagent.wiki "混合专家模型（Mixture of Experts, MoE）", 结构 3; mstx.cn
"MoE 如何替代 FFN？…", section 5).  The sizes themselves are this library's
choice of test points; no page prints them.

This module holds only shape bookkeeping (no arithmetic of the method), so
both the GPU path's tests and the oracle's tests may import it.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                    # tokens (batch * sequence)
    d: int                    # model width
    N: int                    # routed experts
    K: int                    # experts chosen per token
    F: int                    # routed expert intermediate width
    F_shared: int = 0         # shared (always-on) expert width; 0 = none
    act: str = "swiglu"       # "swiglu" | "gelu_tanh"
    dtype: str = "bf16"       # activations + expert weights: "bf16" | "f32"
    gate: str = "softmax_topk"  # "renorm_all" | "softmax_topk" | "prob_no_renorm"
    cf: float | None = None   # capacity factor; None = unlimited
    router_bias: str = "none"  # "none" | "uniform" | "offset2z"
    sel_bias: bool = False    # selection-only per-expert bias b ~ U(-1/2, 1/2)
    expert_bias: bool = False  # biases on the expert linears
    aux_alpha: float = 1.0
    seed: int = 0
    init: str = "normal"      # "normal": W ~ N(0, 1/fan_in); "uniform": U(+-1/sqrt(fan_in))
    desc: str = field(default="", compare=False)

    @property
    def pairs(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny_f32", T=8, d=64, N=4, K=2, F=128, act="gelu_tanh", dtype="f32",
    gate="renorm_all", router_bias="uniform", expert_bias=True, seed=0,
    init="uniform",
    desc="T=8 d=64 N=4 top-2, GELU(tanh) experts 64->128->64 with biases, fp32")

MIXTRAL_PREFILL = Workload(
    name="mixtral_prefill", T=4096, d=4096, N=8, K=2, F=14336, act="swiglu",
    gate="softmax_topk", seed=2,
    desc="T=4096 (2x2048) d=4096 N=8 top-2 SwiGLU F=14336, bf16, fp32 router")

SWITCH_TOP1 = Workload(
    name="switch_top1_cap", T=8192, d=1024, N=64, K=1, F=4096, act="gelu_tanh",
    gate="softmax_topk", cf=1.25, router_bias="offset2z", aux_alpha=0.01, seed=3,
    desc="T=8192 d=1024 N=64 top-1 GELU F=4096, capacity floor(1/64*1.25*T)=160")

DEEPSEEK_PREFILL = Workload(
    name="deepseek_prefill", T=8192, d=7168, N=256, K=8, F=2048, F_shared=2048,
    act="swiglu", gate="softmax_topk", sel_bias=True, seed=4,
    desc="T=8192 d=7168 N=256 top-8 SwiGLU F=2048 + shared expert, selection bias")

# Decode: the routing should touch about every expert (256 (1 - (1 - 8/256)^128)
# ~ 251.6 on average for independent choices); a selection bias of +-1/2 on
# logits of unit scale skews the choice towards ~235, so this shape has none.
DEEPSEEK_DECODE = DEEPSEEK_PREFILL.with_(
    name="deepseek_decode", T=128, sel_bias=False,
    desc="T=128 decode, DeepSeek-V3 shape (d=7168 N=256 top-8 F=2048 + shared), no selection bias")

MIXTRAL_DECODE = MIXTRAL_PREFILL.with_(
    name="mixtral_decode", T=16,
    desc="T=16 decode, Mixtral shape (d=4096 N=8 top-2 F=14336)")

ALL = {w.name: w for w in (TINY, MIXTRAL_PREFILL, SWITCH_TOP1, DEEPSEEK_PREFILL,
                           DEEPSEEK_DECODE, MIXTRAL_DECODE)}


def scaled(w: Workload, T: int | None = None, d: int | None = None,
           F: int | None = None, N: int | None = None, K: int | None = None,
           F_shared: int | None = None, name: str | None = None) -> Workload:
    """A smaller copy of a workload with the same structure (for parity tests
    the oracle finishes in seconds)."""
    kw = {}
    for k, v in dict(T=T, d=d, F=F, N=N, K=K, F_shared=F_shared).items():
        if v is not None:
            kw[k] = v
    return w.with_(name=name or (w.name + "_small"), **kw)
