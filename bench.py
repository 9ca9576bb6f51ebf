#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_layer_forward (router, statistics, dispatch, both grouped
GEMMs with the shared expert when present, combine) over one batch of seeded
synthetic input already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-decode]

Default workload: Mixtral-shaped prefill (T=4096, d=4096, N=8, top-2, SwiGLU
F=14336, bf16).  Unless --no-decode, the line also carries the decode-shaped
DeepSeek-V3 layer (T=128, d=7168, N=256, top-8, F=2048 + shared expert)
measured the same way, as HBM GB/s on the expert weights it touches, and
again with weight-only INT8 and INT4 expert weights ("int8", "int4"; the
same for every decode-sized workload).  For each workload the router entry point is
also timed alone, plain and with the training-time variants (noise,
entropy, bias update): "router_train".  Unless --no-backward, "backward"
times moe_layer_backward on the main workload (gradients of every input and
weight for an upstream dy and the aux loss), with its stages.  Unless
--no-extra, "workloads" holds the other layer shapes measured the same way
(the Switch-style top-1 layer with capacity, the DeepSeek-shaped prefill,
the Mixtral-shaped decode, the tiny fp32 layer), each with its step's
position against both rooflines, its dominant kernel's roofline and its
own CPU baseline (the oracle on a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s + active TFLOP/s (prefill); HBM GB/s (decode T=128)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other layer shapes (the \"workloads\" records)")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens the oracle runs for the CPU baseline (0: all T tokens)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run one elementwise fp32 kernel that reads and "
                         "writes this many MiB (reference for the HBM byte counters)")
    return ap.parse_args()


def copy_probe(mib):
    """One plain streaming kernel of known size: dst = -src over `mib` MiB of
    fp32, i.e. mib MiB read and mib MiB written."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.h = C.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventSynchronize.argtypes = [C.c_void_p]
        self.h.hipEventDestroy.argtypes = [C.c_void_p]
        self.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def create(self):
        e = C.c_void_p()
        if self.h.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed(self, a, b):
        ms = C.c_float()
        if self.h.hipEventElapsedTime(C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


STAGES = ["router+stats", "dispatch", "gemm1", "gemm2_main", "gemm2_tail", "combine"]


def active_work(w, kept_rows):
    """Algorithmic flops of the two grouped GEMMs (kept pairs + shared
    expert) and of the first one alone (gate/up, one launch)."""
    mats = 3 if w.act == "swiglu" else 2
    flops_routed = 2.0 * kept_rows * w.d * w.F * mats
    flops_shared = 2.0 * w.T * w.d * w.F_shared * 3 if w.F_shared else 0.0
    g1_flops = 2.0 * kept_rows * w.d * w.F * (mats - 1) + (
        2.0 * w.T * w.d * w.F_shared * 2 if w.F_shared else 0.0)
    return flops_routed + flops_shared, g1_flops


def stage_work(w, kept_rows, touched, quant=None):
    """Algorithmic flops and HBM bytes of each grouped-GEMM launch and of the
    whole step.  Bytes: every touched expert's weights once (bf16; INT8: one
    byte per code plus a 4-byte scale per output row; INT4: half a byte per
    code plus a 4-byte scale per 128 inputs of a row), each kept row's
    input read once and its output written once; for the step, the touched
    weights plus x read and y written once (intermediates are not counted)."""
    eb = 2 if w.dtype == "bf16" else 4
    wb = {"int8": 1.0, "int4": 0.5}.get(quant, eb)
    m1 = 2 if w.act == "swiglu" else 1
    rows, Fs, T, d, F = kept_rows, w.F_shared, w.T, w.d, w.F

    def scales(out, inp):  # scale bytes of one [out, inp] matrix
        return {"int8": 4.0 * out, "int4": 4.0 * out * inp / 128}.get(quant, 0.0)

    g1_f = 2.0 * rows * d * F * m1 + (2.0 * T * d * Fs * 2 if Fs else 0.0)
    g1_b = (touched * m1 * (F * d * wb + scales(F, d)) + rows * d * eb + rows * F * eb +
            ((2 * (Fs * d * wb + scales(Fs, d)) + T * d * eb + T * Fs * eb) if Fs else 0.0))
    g2_f = 2.0 * rows * d * F + (2.0 * T * d * Fs if Fs else 0.0)
    g2_b = (touched * (d * F * wb + scales(d, F)) + rows * F * eb + rows * d * eb +
            ((d * Fs * wb + scales(d, Fs) + T * Fs * eb + T * d * eb) if Fs else 0.0))
    step_f = g1_f + g2_f + 2.0 * T * d * w.N   # + the router's fp32 logits
    wts = touched * ((m1 + 1) * F * d * wb + m1 * scales(F, d) + scales(d, F)) + (
        (3 * Fs * d * wb + 2 * scales(Fs, d) + scales(d, Fs)) if Fs else 0.0)
    step_b = wts + 2.0 * T * d * eb + 4.0 * w.N * d
    return {"gemm1": (g1_f, g1_b), "gemm2": (g2_f, g2_b), "step": (step_f, step_b),
            "weight_bytes": wts}


def roofline_of(flops, nbytes, ms, peak_tflops=PEAK_BF16_TFLOPS):
    """Position of a launch (or step) of `flops` and `nbytes` that took `ms`:
    its bound is whichever of the two peaks allows less (MFMA time
    flops / peak, 2.5 PF/s for bf16, against HBM time bytes / 8 TB/s); frac
    is that time over the measured one.  Both fractions are given."""
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    s = ms * 1e-3
    if t_mfma >= t_hbm:
        rec = {"bound": "mfma", "achieved": flops / s / 1e12, "peak": peak_tflops,
               "unit": "TFLOP/s"}
    else:
        rec = {"bound": "hbm", "achieved": nbytes / s / 1e9, "peak": PEAK_HBM_GBS,
               "unit": "GB/s"}
    rec["frac"] = rec["achieved"] / rec["peak"]
    rec.update(frac_mfma=t_mfma / s, frac_hbm=t_hbm / s, flops=flops, bytes=nbytes, ms=ms)
    return rec


def run_workload(w, steps, warmup, ev, quant=None):
    import numpy as np
    import torch

    from sparse_mixture_experts_46_amd import _lib as L
    from sparse_mixture_experts_46_amd import api
    from sparse_mixture_experts_46_amd.inputs import make_inputs

    inp = make_inputs(w, device="cuda")
    cfg = api.config_for(w)
    if quant:
        # weight-only INT8 / INT4 expert weights (quantized once, outside the timing)
        inp = api.quantize_expert_weights(inp, quant)
        cfg.weight_format = quant
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    bufs = api.LayerBuffers(cfg, torch.device("cuda"))
    wst = api.weights_struct(inp)
    traces = []
    for _ in range(steps):
        t = L.MoeTrace()
        for i in range(L.MOE_TRACE_EVENTS):
            t.ev[i] = ev.create()
        traces.append(t)
    for _ in range(warmup):
        api.moe_layer_forward(cfg, inp, inp["x"], bufs=bufs, wstruct=wst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        api.moe_layer_forward(cfg, inp, inp["x"], bufs=bufs, wstruct=wst, trace=traces[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.zeros(len(STAGES))
    for t in traces:
        for j in range(len(STAGES)):
            stage[j] += ev.elapsed(t.ev[j], t.ev[j + 1])
    stage /= steps
    for t in traces:
        for i in range(L.MOE_TRACE_EVENTS):
            ev.destroy(t.ev[i])
    # the same step captured once into a HIP graph and replayed: the way a
    # serving loop launches the layer (one launch instead of one per kernel)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        api.moe_layer_forward(cfg, inp, inp["x"], bufs=bufs, wstruct=wst)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.moe_layer_forward(cfg, inp, inp["x"], bufs=bufs, wstruct=wst)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t0
    del graph
    cnt = bufs.counters.cpu().numpy()
    kept_rows, touched = int(cnt[0]), int(cnt[3])
    total_flops, g1_flops = active_work(w, kept_rows)
    wbytes = stage_work(w, kept_rows, touched, quant)["weight_bytes"]
    res = dict(inp=inp, bufs=bufs, wall=wall, wall_graph=wall_graph, stage_ms=stage, kept_rows=kept_rows,
               touched=touched, total_flops=total_flops, g1_flops=g1_flops, wbytes=wbytes)
    return res


def kernel_rooflines(w, rd, quant=None):
    """Each grouped GEMM's roofline from a run_workload result (the tail
    launch, when there is one, counted with the second GEMM; an fp32 layer's
    one FFN kernel covers both GEMMs), with its counter-measured traffic
    where profiles/ holds it, and the dominant one's name."""
    sw = stage_work(w, rd["kept_rows"], rd["touched"], quant)
    st = {k: float(v) for k, v in zip(STAGES, rd["stage_ms"])}
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    if w.dtype == "bf16":
        kernels = {"gemm1": roofline_of(*sw["gemm1"], st["gemm1"], peak),
                   "gemm2": roofline_of(*sw["gemm2"], st["gemm2_main"] + st["gemm2_tail"], peak)}
    else:
        f = sw["gemm1"][0] + sw["gemm2"][0]
        b = sw["gemm1"][1] + sw["gemm2"][1]
        kernels = {"ffn_f32": roofline_of(f, b, st["gemm1"], peak)}
    for k in kernels:
        kernels[k]["traffic"] = traffic_of(w.name, quant or "bf16", k)
    return kernels, max(kernels, key=lambda k: kernels[k]["ms"]), sw, st, peak


def layer_record(w, steps, warmup, ev, quant=None, cpu=None):
    """One layer shape: graph-replayed step time, per-stage times, the step's
    position against both rooflines, each grouped GEMM's roofline (the
    dominant one as "roofline") and, with cpu (cpu_baseline's keyword
    arguments), the oracle's rate on a bounded sample of the same inputs."""
    rd = run_workload(w, steps, warmup, ev, quant=quant)
    ms = rd["wall_graph"] * 1e3 / steps
    kernels, dom, sw, st, peak = kernel_rooflines(w, rd, quant)
    rec = {"workload": w.name, "desc": w.desc, "T": w.T, "dtype": w.dtype,
           "weights": {"int8": "int8 + fp32 row scales",
                       "int4": "int4 + fp32 scales per 128 inputs"}.get(quant, w.dtype),
           "ms_per_step": ms, "us_per_step": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3),
           "eager_ms_per_step": rd["wall"] * 1e3 / steps,
           "kept_rows": rd["kept_rows"], "touched_experts": rd["touched"],
           "weight_bytes": sw["weight_bytes"],
           "weight_gbs": sw["weight_bytes"] / (ms * 1e-3) / 1e9,
           "active_tflops": (sw["gemm1"][0] + sw["gemm2"][0]) / (ms * 1e-3) / 1e12,
           "step_roofline": roofline_of(*sw["step"], ms, peak),
           "roofline": dict(kernels[dom], kernel=dom), "kernels": kernels, "stage_ms": st}
    if cpu is not None:
        rec["cpu_baseline"] = cpu_baseline(w, rd["inp"], **cpu)
    return rec, rd


def decode_record(w, steps, warmup, ev, quant=None, cpu=None):
    """A decode-sized layer: as layer_record, plus the HBM GB/s of the whole
    step on the expert weights it touches (bf16 weights, or INT8 / INT4
    codes plus scales) against the HBM peak; "roofline" stays the dominant
    kernel's."""
    rec, rd = layer_record(w, steps, warmup, ev, quant=quant, cpu=cpu)
    rec["hbm_gbs"] = rec["weight_gbs"]
    rec["hbm_frac"] = rec["weight_gbs"] / PEAK_HBM_GBS
    return rec, rd


BWD_STAGES = ["combine_bwd", "router_bwd", "recompute_gemm1", "dh_gemm", "dw2_gemm",
              "dx_perm_gemm", "dw1_dw3_gemm", "bias_grads", "dx"]


def backward_work(w, kept_rows):
    """Algorithmic flops of the backward's expert GEMMs (dgrad + wgrad: twice
    the forward's), and the flops of each GEMM stage as launched (the
    recompute of the first GEMM is extra work, not part of the algorithm)."""
    rows, rs = kept_rows, (w.T if w.F_shared else 0)
    dF = 2.0 * w.d * w.F
    m = 2 if w.act == "swiglu" else 1  # first-GEMM weight matrices
    stage = {"recompute_gemm1": dF * m * (rows + rs), "dh_gemm": dF * (rows + rs),
             "dw2_gemm": dF * (rows + rs), "dx_perm_gemm": dF * m * (rows + rs),
             "dw1_dw3_gemm": dF * m * (rows + rs)}
    algo = stage["dh_gemm"] + stage["dw2_gemm"] + stage["dx_perm_gemm"] + stage["dw1_dw3_gemm"]
    return algo, stage


def backward_record(w, steps, warmup, ev):
    """moe_layer_backward on the workload (aux-loss gradient 1, as in
    training): graph-replayed step time, per-stage times from HIP events on
    the library's stream, and the dominant GEMM's roofline."""
    import numpy as np
    import torch

    from sparse_mixture_experts_46_amd import _lib as L
    from sparse_mixture_experts_46_amd import api
    from sparse_mixture_experts_46_amd.inputs import make_dy, make_inputs

    inp = make_inputs(w, device="cuda")
    dy = make_dy(w, device="cuda")
    cfg = api.config_for(w)
    fwd = api.moe_layer_forward(cfg, inp, inp["x"], save_for_backward=True)
    wst0 = api.weights_struct(inp)

    def graph_ms(fn):
        # one call captured into a HIP graph, replayed `steps` times
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        del graph
        return (time.perf_counter() - t0) * 1e3 / steps

    # the forward a training step runs: it also keeps what the backward reads
    # (logits, y_perm and, where stored, gate(x) / up(x))
    fwd_save_ms = graph_ms(lambda: api.moe_layer_forward(cfg, inp, inp["x"], bufs=fwd,
                                                         wstruct=wst0))
    bufs = api.BackwardBuffers(cfg, torch.device("cuda"))
    wst = api.weights_struct(inp)
    saved = api.saved_struct(fwd)
    lg = (1.0, 0.0, 0.0)

    def step(trace=None):
        api.moe_layer_backward(cfg, inp, inp["x"], fwd, dy, lg, bufs=bufs, wstruct=wst,
                               saved=saved, trace=trace)

    traces = []
    for _ in range(steps):
        t = L.MoeBwdTrace()
        for i in range(L.MOE_BWD_TRACE_EVENTS):
            t.ev[i] = ev.create()
        traces.append(t)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(traces[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.zeros(len(BWD_STAGES))
    for t in traces:
        for j in range(len(BWD_STAGES)):
            stage[j] += ev.elapsed(t.ev[j], t.ev[j + 1])
        for i in range(L.MOE_BWD_TRACE_EVENTS):
            ev.destroy(t.ev[i])
    stage /= steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del graph
    kept = int(fwd.counters.cpu()[0])
    algo, sflops = backward_work(w, kept)
    st = {k: float(v) for k, v in zip(BWD_STAGES, stage)}
    gemm = {k: sflops[k] / (st[k] * 1e-3) / 1e12 for k in sflops if st[k] > 0}
    dom = max(sflops, key=lambda k: st[k])
    tf = gemm[dom]
    # the dW1 + dW3 stage is two launches of one kernel (SwiGLU)
    launches = 2 if (dom == "dw1_dw3_gemm" and w.act == "swiglu") else 1
    return {"workload": w.name, "ms_per_step": ms, "eager_ms_per_step": wall * 1e3 / steps,
            "forward_saving_ms": fwd_save_ms, "saves_gate_up": fwd.u is not None,
            "tokens_per_s": w.T / (ms * 1e-3), "loss_grad": {"aux": lg[0], "z": lg[1], "z_lse": lg[2]},
            "algorithmic_tflop": algo / 1e12,
            "active_tflops": algo / (ms * 1e-3) / 1e12,
            "active_frac_of_bf16_peak": algo / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "stage_ms": st, "gemm_tflops": gemm,
            "roofline": {"bound": "mfma", "kernel": dom, "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS, "traffic": None,
                         "launches": launches, "avg_ms": st[dom] / launches,
                         "flops_per_launch": sflops[dom] / launches}}


def router_train_timing(w, inp, steps, warmup, noise_std=0.1, bias_rate=1e-3):
    """moe_router_topk alone on the workload's inputs, plain and with the
    training variants on (router noise, routing entropy, a bias-update step
    written to a separate buffer).  Torch events on torch's current stream
    around graph replays of one captured call."""
    import torch

    from sparse_mixture_experts_46_amd import api

    cfg = api.config_for(w)
    cfg_t = api.config_for(w)
    cfg_t.noise_std, cfg_t.bias_rate = noise_std, bias_rate
    g = torch.Generator(device="cuda").manual_seed(1234)
    winp = dict(inp)
    winp["noise"] = torch.randn((w.T, w.N), generator=g, device="cuda", dtype=torch.float32)
    b_out = torch.empty(w.N, dtype=torch.float32, device="cuda")

    def timed(c, wd, bo):
        # one call captured into a HIP graph and replayed, so the host-side
        # marshalling of the Python binding is not timed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            api.moe_router_topk(c, wd, inp["x"], b_sel_out=bo)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            api.moe_router_topk(c, wd, inp["x"], b_sel_out=bo)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / steps

    plain = timed(cfg, inp, None)
    train = timed(cfg_t, winp, b_out)
    return {"entry_point": "moe_router_topk (logits, selection, gates, statistics)",
            "plain_ms": plain, "train_ms": train, "noise_std": noise_std, "bias_rate": bias_rate,
            "noise_bytes": 4.0 * w.T * w.N}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, sample, seeded=False, repeats=1, single_core=False):
    """The oracle, as it stands, on `sample` tokens of the same workload with
    the same weights (the first ones, or a seeded random set): routing over
    those tokens, capacity, experts, combine.  Median of `repeats` runs; with
    single_core, the same again with the BLAS library held to one thread."""
    import numpy as np
    import torch

    from oracle import moe_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def f64(t):
        return None if t is None else t.detach().cpu().double().numpy()

    bf = w.dtype == "bf16"
    stack = (lambda t: ref.Bf16Stack(bits(t))) if bf else f64
    W = {"w_r": f64(inp["w_r"]), "w1": stack(inp["w1"]), "w2": stack(inp["w2"])}
    if inp.get("w3") is not None:
        W["w3"] = stack(inp["w3"])
    if inp.get("b1") is not None:
        W["b1"], W["b2"] = f64(inp["b1"]), f64(inp["b2"])
    shared = None
    if inp.get("ws1") is not None:
        shared = {"w1": f64(inp["ws1"]), "w3": f64(inp["ws3"]), "w2": f64(inp["ws2"])}
    if seeded:
        rows = np.sort(np.random.default_rng(0).choice(w.T, size=sample, replace=False))
        x = f64(inp["x"])[rows]
        which = f"{sample} of {w.T} tokens drawn with numpy default_rng(0)"
    else:
        x = f64(inp["x"][:sample])
        which = f"first {sample} of {w.T} tokens"
    def timed():
        times = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            ref.layer_forward(x, W, K=w.K, act=w.act, gate_mode=w.gate, cf=w.cf,
                              alpha=w.aux_alpha, b_r=f64(inp["b_r"]), b_sel=f64(inp["b_sel"]),
                              shared=shared)
            times.append(time.perf_counter() - t0)
        return float(np.median(times))

    dt = timed()
    med = f", median of {repeats} runs" if repeats > 1 else ""
    rec = {"value": sample / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "cpu": cpu_model(), "seconds": dt,
           "sample": f"{which} of {w.name} (same weights), full layer in NumPy float64 "
                     f"incl. per-expert bf16->fp64 weight widening{med}; {dt:.3g} s"}
    if single_core:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1, user_api="blas"):
                dt1 = timed()
            rec["single_core"] = {"value": sample / dt1, "unit": "tokens/s", "cores": 1,
                                  "seconds": dt1}
        except Exception as e:  # threadpoolctl missing or unable to limit
            rec["single_core"] = {"error": repr(e)}
    return rec


def counter_record(name, weights, stage):
    """The committed rocprofv3 counter summary of one grouped-GEMM stage
    ("gemm1" / "gemm2") of a workload with bf16, INT8 or INT4 weights, or
    None when there is none or its kernel's sources changed since it was
    taken."""
    p = os.path.join(ROOT, "profiles", f"counters_{name}.json")
    if not os.path.exists(p):
        return None
    st = json.load(open(p))["stages"].get(f"{weights}:{stage}")
    from sparse_mixture_experts_46_amd.profsum import family_of, source_sha256
    if not st or st.get("source_sha256") != source_sha256(family_of(st["kernel"])):
        return None
    return st


def traffic_of(name, weights, stage):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, probe-scaled) or None."""
    c = counter_record(name, weights, stage)
    if not c or c.get("fetch_bytes") is None or c.get("write_bytes") is None:
        return None
    return c["fetch_bytes"] + c["write_bytes"]


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the layer runs on one GPU (asked for --gpus {a.gpus}); the "
              "multi-GPU expert-parallel path is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_mixture_experts_46_amd import _lib as L
    from sparse_mixture_experts_46_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.load()
    ev = HipEvents()
    if a.copy_probe_mib:
        copy_probe(a.copy_probe_mib)
    w = WL.ALL[a.workload]
    r = run_workload(w, a.steps, a.warmup, ev)
    ms = r["wall_graph"] * 1e3 / a.steps  # graph-launched steps
    ms_eager = r["wall"] * 1e3 / a.steps
    tok_s = w.T / (ms / 1e3)
    kernels, dom, _sw, _st, _peak = kernel_rooflines(w, r)
    names = {"gemm1": "grouped GEMM 1 (gate/up + SiLU*mul)" if w.act == "swiglu"
             else "grouped GEMM 1 (+ GELU)", "gemm2": "grouped GEMM 2 (down projection)",
             "ffn_f32": "fp32 expert FFN (both GEMMs)"}
    rf = dict(kernels[dom], kernel=names[dom], avg_ms=kernels[dom]["ms"],
              flops_per_launch=kernels[dom]["flops"], bytes_per_launch=kernels[dom]["bytes"])
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "launch": "HIP graph: one moe_layer_forward captured, replayed per step",
        "eager_ms_per_step": ms_eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights, random init)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "N": w.N, "K": w.K, "F": w.F,
                   "F_shared": w.F_shared, "act": w.act, "capacity_factor": w.cf,
                   "router": "fp32", "desc": w.desc},
        "roofline": rf,
        "kernels": kernels,
        "active_tflops": r["total_flops"] / (ms * 1e-3) / 1e12,
        "active_frac_of_bf16_peak": r["total_flops"] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "weight_gbs": r["wbytes"] / (ms * 1e-3) / 1e9,
        "stage_ms": {k: float(v) for k, v in zip(STAGES, r["stage_ms"])},
        "kept_rows": r["kept_rows"],
    }
    line["router_train"] = router_train_timing(w, r["inp"], a.steps, a.warmup)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["inp"], min(a.cpu_sample or w.T, w.T))
    del r
    torch.cuda.empty_cache()
    if not a.no_backward:
        if a.copy_probe_mib:  # a second probe marks where the backward's launches begin
            copy_probe(a.copy_probe_mib)
        line["backward"] = backward_record(w, a.steps, a.warmup, ev)
        torch.cuda.empty_cache()
    if w.T * w.K <= 24 * w.N and w.act == "swiglu" and w.dtype == "bf16":
        # a decode-sized main workload: also its INT8-weight variant
        for q in ("int8", "int4"):
            if q == "int4" and (w.d % 128 or w.F % 128):
                continue
            line[q], _ = decode_record(w, a.steps, a.warmup, ev, quant=q)
            torch.cuda.empty_cache()
        torch.cuda.empty_cache()
    if not a.no_decode:
        wd = WL.DEEPSEEK_DECODE
        cpu = None if a.no_cpu_baseline else {"sample": wd.T}
        rec, rd = decode_record(wd, a.steps, a.warmup, ev, cpu=cpu)
        rec["router_train"] = router_train_timing(wd, rd["inp"], a.steps, a.warmup)
        del rd
        torch.cuda.empty_cache()
        rec["int8"], _ = decode_record(wd, a.steps, a.warmup, ev, quant="int8")
        torch.cuda.empty_cache()
        rec["int4"], _ = decode_record(wd, a.steps, a.warmup, ev, quant="int4")
        line["decode"] = rec
        torch.cuda.empty_cache()
    if not a.no_extra:
        # the other layer shapes; the oracle's sample for each: every token
        # where that is seconds of CPU work, else a seeded 512-token set
        extra = [(WL.SWITCH_TOP1, {"sample": WL.SWITCH_TOP1.T, "single_core": True}),
                 (WL.DEEPSEEK_PREFILL, {"sample": 512, "seeded": True}),
                 (WL.MIXTRAL_DECODE, {"sample": WL.MIXTRAL_DECODE.T}),
                 (WL.TINY, {"sample": WL.TINY.T, "repeats": 10, "single_core": True})]
        line["workloads"] = {}
        for we, cpu in extra:
            if we.name == w.name:
                continue
            rec, rd = layer_record(we, a.steps, a.warmup, ev,
                                   cpu=None if a.no_cpu_baseline else cpu)
            del rd
            torch.cuda.empty_cache()
            if we.T * we.K <= 24 * we.N and we.act == "swiglu" and we.dtype == "bf16":
                # decode-sized: also with weight-only INT8 and INT4 expert weights
                for q in ("int8", "int4"):
                    rec[q], _ = decode_record(we, a.steps, a.warmup, ev, quant=q)
                    torch.cuda.empty_cache()
            line["workloads"][we.name] = rec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
