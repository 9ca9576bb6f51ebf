"""Seeded synthetic inputs for a MoE layer forward.

This module only draws random numbers: it holds none of the layer's
arithmetic.  It is the one piece shared between the GPU path's tests/bench
and the CPU oracle's tests, so both consume the very same bits.

Recipe (one torch.Generator per tensor role, seeded with seed*1000+role, on
the device the tensors are made on; draws are fp32 and rounded to bf16 with
round-to-nearest-even where the layer runs in bf16):
  x        [T, d]     N(0, 1)
  w_r      [N, d]     fp32 router weight, N(0, 1/d)  (uniform init: U(+-1/sqrt(d)))
  b_r      [N]        router bias: "uniform" -> U(+-1/sqrt(d)); "offset2z" -> 2.0*z, z~N(0,1)
  b_sel    [N]        selection-only bias, U(-1/2, 1/2)
  w1       [N, F, d]  first projection (SwiGLU gate / GELU input), N(0, 1/d)
  w3       [N, F, d]  SwiGLU up projection, N(0, 1/d)
  w2       [N, d, F]  down projection, N(0, 1/F)
  b1, b2   [N, F], [N, d]  expert biases (uniform init only)
  ws1/ws3  [Fs, d], ws2 [d, Fs]  the shared expert
  dy       [T, d]     upstream gradient of the layer output (backward), N(0, 1)
Large weight tensors are drawn one expert slab at a time, so the fp32
temporaries stay small.
"""
from __future__ import annotations

import math

import torch

from .workloads import Workload

ROLE = dict(x=1, w_r=2, b_r=3, b_sel=4, w1=5, w3=6, w2=7, b1=8, b2=9,
            ws1=10, ws3=11, ws2=12, dy=13)


def _gen(w: Workload, role: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + ROLE[role])
    return g


def _draw(shape, kind: str, scale: float, g, device, out_dtype):
    if kind == "normal":
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(scale)
    else:  # uniform in [-scale, scale)
        t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(2.0 * scale).sub_(scale)
    return t.to(out_dtype)


def _draw_slabs(n: int, shape, kind, scale, g, device, out_dtype):
    out = torch.empty((n,) + tuple(shape), dtype=out_dtype, device=device)
    for e in range(n):
        out[e].copy_(_draw(shape, kind, scale, g, device, out_dtype))
    return out


def make_inputs(w: Workload, device="cpu") -> dict:
    """Draw every tensor of workload ``w`` on ``device``; returns a dict of
    torch tensors (missing roles are None)."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kind = "uniform" if w.init == "uniform" else "normal"

    def sc(fan_in):
        return 1.0 / math.sqrt(fan_in)

    t = {}
    t["x"] = _draw((w.T, w.d), "normal", 1.0, _gen(w, "x", device), device, dt)
    t["w_r"] = _draw((w.N, w.d), kind, sc(w.d), _gen(w, "w_r", device), device,
                     torch.float32)
    if w.router_bias == "uniform":
        t["b_r"] = _draw((w.N,), "uniform", sc(w.d), _gen(w, "b_r", device),
                         device, torch.float32)
    elif w.router_bias == "offset2z":
        t["b_r"] = 2.0 * _draw((w.N,), "normal", 1.0, _gen(w, "b_r", device),
                               device, torch.float32)
    else:
        t["b_r"] = None
    t["b_sel"] = (_draw((w.N,), "uniform", 0.5, _gen(w, "b_sel", device),
                        device, torch.float32) if w.sel_bias else None)
    t["w1"] = _draw_slabs(w.N, (w.F, w.d), kind, sc(w.d), _gen(w, "w1", device),
                          device, dt)
    t["w3"] = (_draw_slabs(w.N, (w.F, w.d), kind, sc(w.d), _gen(w, "w3", device),
                           device, dt) if w.act == "swiglu" else None)
    t["w2"] = _draw_slabs(w.N, (w.d, w.F), kind, sc(w.F), _gen(w, "w2", device),
                          device, dt)
    if w.expert_bias:
        t["b1"] = _draw((w.N, w.F), "uniform", sc(w.d), _gen(w, "b1", device),
                        device, dt)
        t["b2"] = _draw((w.N, w.d), "uniform", sc(w.F), _gen(w, "b2", device),
                        device, dt)
    else:
        t["b1"] = t["b2"] = None
    if w.F_shared:
        Fs = w.F_shared
        t["ws1"] = _draw((Fs, w.d), kind, sc(w.d), _gen(w, "ws1", device), device, dt)
        t["ws3"] = _draw((Fs, w.d), kind, sc(w.d), _gen(w, "ws3", device), device, dt)
        t["ws2"] = _draw((w.d, Fs), kind, sc(Fs), _gen(w, "ws2", device), device, dt)
    else:
        t["ws1"] = t["ws3"] = t["ws2"] = None
    return t


def make_dy(w: Workload, device="cpu") -> torch.Tensor:
    """The upstream gradient of the layer output for a backward pass of
    workload ``w``: [T, d] N(0, 1) in the layer dtype."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return _draw((w.T, w.d), "normal", 1.0, _gen(w, "dy", device), device, dt)


def random_topk_indices(T: int, N: int, K: int, seed: int, skew: float = 0.0,
                        device="cpu") -> torch.Tensor:
    """Seeded synthetic routing decisions [T, K] int32: K distinct experts per
    token, drawn without replacement with weights exp(skew * z_e)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    z = torch.randn(N, generator=g, dtype=torch.float64)
    wts = torch.exp(skew * z).expand(T, N).contiguous()
    idx = torch.multinomial(wts, K, replacement=False, generator=g)
    return idx.to(torch.int32).to(device)


def bf16_to_f64_numpy(t: torch.Tensor):
    """Exact widening of a (bf16 or fp32) torch tensor to a float64 numpy array
    on the host (every bf16/fp32 value is representable in fp64)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
