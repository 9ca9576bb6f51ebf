"""Python binding of libmoe with the C entry points' names.

Torch tensors supply device memory and the current HIP stream; every step
of the layer runs in libmoe's HIP kernels.  There is no CPU fallback: the
functions raise if the library is missing or a tensor is not on the GPU.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib as L
from .workloads import Workload

_ACT = {"swiglu": L.MOE_ACT_SWIGLU, "gelu_tanh": L.MOE_ACT_GELU_TANH}
_GATE = {"renorm_all": L.MOE_GATE_RENORM_ALL, "softmax_topk": L.MOE_GATE_SOFTMAX_TOPK,
         "prob_no_renorm": L.MOE_GATE_PROB_NO_RENORM}


@dataclass
class Config:
    T: int
    d: int
    N: int
    K: int
    F: int
    F_shared: int = 0
    dtype: str = "bf16"
    act: str = "swiglu"
    gate: str = "softmax_topk"
    capacity: int = -1
    aux_alpha: float = 1.0
    # scale of the router noise, used only when noise is on (w["noise"] or
    # noise_seed); 0.1 is the value of the page's router
    noise_std: float = 0.1
    bias_rate: float = 0.0   # step of the selection-bias update (used with b_sel_out)
    weight_format: str = "dtype"  # "dtype", "int8" or "int4" (moe_quantize_int8 / _int4)
    # router noise drawn in the kernels (Philox-4x32-10 + Box-Muller): the
    # generator key, or None for no in-kernel noise; noise_offset selects the
    # stream of a call (e.g. the training step)
    noise_seed: int | None = None
    noise_offset: int = 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def c(self) -> L.MoeConfig:
        return L.MoeConfig(T=self.T, d=self.d, N=self.N, K=self.K, F=self.F,
                           F_shared=self.F_shared,
                           dtype=L.MOE_BF16 if self.dtype == "bf16" else L.MOE_F32,
                           act=_ACT[self.act], gate=_GATE[self.gate], capacity=self.capacity,
                           aux_alpha=self.aux_alpha,
                           flags=0 if self.noise_seed is None else L.MOE_FLAG_NOISE_PHILOX,
                           noise_std=self.noise_std, bias_rate=self.bias_rate,
                           weight_format={"int8": L.MOE_WEIGHTS_INT8,
                                          "int4": L.MOE_WEIGHTS_INT4}.get(self.weight_format,
                                                                          L.MOE_WEIGHTS_DTYPE),
                           noise_seed=0 if self.noise_seed is None else self.noise_seed,
                           noise_offset=self.noise_offset)


def config_for(w: Workload) -> Config:
    cap = -1 if w.cf is None else moe_capacity(w.K, w.N, w.T, w.cf)
    return Config(T=w.T, d=w.d, N=w.N, K=w.K, F=w.F, F_shared=w.F_shared, dtype=w.dtype,
                  act=w.act, gate=w.gate, capacity=cap, aux_alpha=w.aux_alpha)


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _size(fn, cfg: Config) -> int:
    n = C.c_size_t(0)
    L.check(fn(C.byref(cfg.c()), C.byref(n)), fn.__name__)
    return n.value


def moe_capacity(K: int, N: int, T: int, cf) -> int:
    """floor(K/N * cf * T); cf None/negative = unlimited (returns T)."""
    return int(L.load().moe_capacity(K, N, T, -1.0 if cf is None else float(cf)))


def moe_layer_saves_uv(cfg: Config) -> bool:
    return bool(L.load().moe_layer_saves_uv(C.byref(cfg.c())))


def moe_workspace_size(cfg: Config) -> int:
    return _size(L.load().moe_workspace_size, cfg)


def weights_struct(t: dict) -> L.MoeWeights:
    w = L.MoeWeights()
    for k in ("w_r", "b_r", "b_sel", "w1", "w3", "w2", "b1", "b2", "ws1", "ws3", "ws2", "noise",
              "w1_scale", "w3_scale", "w2_scale", "ws1_scale", "ws3_scale", "ws2_scale"):
        v = t.get(k)
        setattr(w, k, None if v is None else _p(v).value)
    return w


def moe_quantize_int8(w: torch.Tensor):
    """bf16 weights [..., rows, cols] -> (int8 codes of the same shape, fp32
    per-row scales [..., rows])."""
    if w.dtype != torch.bfloat16:
        raise ValueError("moe_quantize_int8 takes bf16 weights")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    s = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    L.check(L.load().moe_quantize_int8(_p(w), rows, cols, _p(q), _p(s), _stream()),
            "moe_quantize_int8")
    return q, s


def moe_quantize_int4(w: torch.Tensor):
    """bf16 weights [..., rows, cols] -> (packed INT4 codes uint8
    [..., rows, cols / 2], fp32 scales [..., rows, cols / 128])."""
    if w.dtype != torch.bfloat16:
        raise ValueError("moe_quantize_int4 takes bf16 weights")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    q = torch.empty(w.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=w.device)
    s = torch.empty(w.shape[:-1] + (max(cols // 128, 1),), dtype=torch.float32, device=w.device)
    L.check(L.load().moe_quantize_int4(_p(w), rows, cols, _p(q), _p(s), _stream()),
            "moe_quantize_int4")
    return q, s


def quantize_expert_weights(w: dict, fmt: str = "int8") -> dict:
    """A copy of the weight dict with every expert matrix (w1, w3, w2 and the
    shared ws1, ws3, ws2) replaced by its codes ("int8" or "int4") plus its
    *_scale."""
    quant = {"int8": moe_quantize_int8, "int4": moe_quantize_int4}[fmt]
    out = dict(w)
    for k in ("w1", "w3", "w2", "ws1", "ws3", "ws2"):
        if w.get(k) is not None:
            out[k], out[k + "_scale"] = quant(w[k])
    return out


def moe_router_topk(cfg: Config, w: dict, x: torch.Tensor, want_logits=False,
                    want_stats=True, b_sel_out: torch.Tensor | None = None) -> dict:
    """Router entry point.  Router noise (scale cfg.noise_std): w["noise"]
    [T, N] fp32 draws, or cfg.noise_seed for draws made in the kernels;
    b_sel_out [N] fp32 receives one bias-update step (with cfg.bias_rate)
    and may be w["b_sel"] itself."""
    lib = L.load()
    dev = x.device
    T, N, K = cfg.T, cfg.N, cfg.K
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    logits = torch.empty((T, N), dtype=torch.float32, device=dev) if want_logits else None
    out = {"idx": idx, "gate": gate, "logits": logits}
    st = None
    if want_stats or b_sel_out is not None:
        out["count"] = torch.empty(N, dtype=torch.int32, device=dev)
        out["f"] = torch.empty(N, dtype=torch.float32, device=dev)
        out["p"] = torch.empty(N, dtype=torch.float32, device=dev)
        out["loss"] = torch.empty(3, dtype=torch.float32, device=dev)
        out["entropy"] = torch.empty(1, dtype=torch.float32, device=dev)
        out["b_sel_out"] = b_sel_out
        st = L.MoeStats(count=_p(out["count"]).value, f=_p(out["f"]).value,
                        p=_p(out["p"]).value, loss=_p(out["loss"]).value,
                        entropy=_p(out["entropy"]).value,
                        b_sel_out=None if b_sel_out is None else _p(b_sel_out).value)
    ws = _ws(_size(lib.moe_router_workspace_size, cfg), dev)
    L.check(lib.moe_router_topk(C.byref(cfg.c()), C.byref(weights_struct(w)), _p(x), _p(idx),
                                _p(gate), _p(logits), C.byref(st) if st else None, _p(ws),
                                ws.numel(), _stream()), "moe_router_topk")
    out["_ws"] = ws
    return out


def moe_dispatch(cfg: Config, idx: torch.Tensor, x: torch.Tensor | None = None,
                 want_x_perm=False) -> dict:
    lib = L.load()
    dev = idx.device
    T, N, K = cfg.T, cfg.N, cfg.K
    o = {"kept": torch.empty(N, dtype=torch.int32, device=dev),
         "offset": torch.empty(N + 1, dtype=torch.int32, device=dev),
         "pair_row": torch.empty(T * K, dtype=torch.int32, device=dev),
         "row_pair": torch.full((T * K,), -1, dtype=torch.int32, device=dev),
         "dropped": torch.empty(T * K, dtype=torch.uint8, device=dev),
         "counters": torch.empty(4, dtype=torch.int32, device=dev),
         "x_perm": (torch.empty((T * K, cfg.d), dtype=cfg.torch_dtype, device=dev)
                    if want_x_perm else None)}
    d = L.MoeDispatch(**{k: (None if o[k] is None else _p(o[k]).value)
                         for k in ("kept", "offset", "pair_row", "row_pair", "dropped",
                                   "counters", "x_perm")})
    ws = _ws(_size(lib.moe_dispatch_workspace_size, cfg), dev)
    L.check(lib.moe_dispatch(C.byref(cfg.c()), _p(idx), _p(x), C.byref(d), _p(ws), ws.numel(),
                             _stream()), "moe_dispatch")
    o["_ws"] = ws
    return o


def moe_expert_ffn(cfg: Config, w: dict, a: torch.Tensor, offset: torch.Tensor,
                   a_rows: torch.Tensor | None = None, x_shared: torch.Tensor | None = None,
                   y_perm: torch.Tensor | None = None) -> dict:
    lib = L.load()
    dev = a.device
    if y_perm is None:
        y_perm = torch.empty((cfg.T * cfg.K, cfg.d), dtype=cfg.torch_dtype, device=dev)
    y_shared = (torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=dev)
                if cfg.F_shared else None)
    ws = _ws(_size(lib.moe_ffn_workspace_size, cfg), dev)
    L.check(lib.moe_expert_ffn(C.byref(cfg.c()), C.byref(weights_struct(w)), _p(a), _p(a_rows),
                               _p(offset), _p(y_perm), _p(x_shared), _p(y_shared), _p(ws),
                               ws.numel(), _stream()), "moe_expert_ffn")
    return {"y_perm": y_perm, "y_shared": y_shared, "_ws": ws}


def moe_combine(cfg: Config, y_perm: torch.Tensor, pair_row: torch.Tensor, gate: torch.Tensor,
                y_shared: torch.Tensor | None = None) -> torch.Tensor:
    lib = L.load()
    y = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=y_perm.device)
    L.check(lib.moe_combine(C.byref(cfg.c()), _p(y_perm), _p(pair_row), _p(gate), _p(y_shared),
                            _p(y), _stream()), "moe_combine")
    return y


class LayerBuffers:
    """Preallocated outputs and workspace for repeated moe_layer_forward calls."""

    def __init__(self, cfg: Config, device, want_logits=False, save_for_backward=False):
        T, N, K = cfg.T, cfg.N, cfg.K
        self.cfg = cfg
        want_logits = want_logits or save_for_backward
        self.y = torch.empty((T, cfg.d), dtype=cfg.torch_dtype, device=device)
        self.idx = torch.empty((T, K), dtype=torch.int32, device=device)
        self.gate = torch.empty((T, K), dtype=torch.float32, device=device)
        self.logits = (torch.empty((T, N), dtype=torch.float32, device=device)
                       if want_logits else None)
        self.count = torch.empty(N, dtype=torch.int32, device=device)
        self.f = torch.empty(N, dtype=torch.float32, device=device)
        self.p = torch.empty(N, dtype=torch.float32, device=device)
        self.loss = torch.empty(3, dtype=torch.float32, device=device)
        self.entropy = torch.empty(1, dtype=torch.float32, device=device)
        self.kept = torch.empty(N, dtype=torch.int32, device=device)
        self.offset = torch.empty(N + 1, dtype=torch.int32, device=device)
        self.pair_row = torch.empty(T * K, dtype=torch.int32, device=device)
        self.row_pair = torch.empty(T * K, dtype=torch.int32, device=device)
        self.dropped = torch.empty(T * K, dtype=torch.uint8, device=device)
        self.counters = torch.empty(4, dtype=torch.int32, device=device)
        self.y_perm = (torch.empty((T * K, cfg.d), dtype=cfg.torch_dtype, device=device)
                       if save_for_backward else None)
        # gate(x) and up(x) of the first GEMM, where the forward stores them
        uv_rows = T * K + (T if cfg.F_shared else 0)
        keep_uv = save_for_backward and moe_layer_saves_uv(cfg)
        self.u = (torch.empty((uv_rows, cfg.F), dtype=cfg.torch_dtype, device=device)
                  if keep_uv else None)
        self.v = (torch.empty((uv_rows, cfg.F), dtype=cfg.torch_dtype, device=device)
                  if keep_uv else None)
        self.ws = _ws(moe_workspace_size(cfg), device)
        self.out = L.MoeLayerOut()
        self.out.y = _p(self.y).value
        self.out.topk_idx = _p(self.idx).value
        self.out.topk_gate = _p(self.gate).value
        self.out.logits = None if self.logits is None else _p(self.logits).value
        self.out.stats = L.MoeStats(count=_p(self.count).value, f=_p(self.f).value,
                                    p=_p(self.p).value, loss=_p(self.loss).value,
                                    entropy=_p(self.entropy).value, b_sel_out=None)
        self.out.dispatch = L.MoeDispatch(
            kept=_p(self.kept).value, offset=_p(self.offset).value,
            pair_row=_p(self.pair_row).value, row_pair=_p(self.row_pair).value,
            dropped=_p(self.dropped).value, counters=_p(self.counters).value, x_perm=None)
        self.out.y_perm = None if self.y_perm is None else _p(self.y_perm).value
        self.out.u = None if self.u is None else _p(self.u).value
        self.out.v = None if self.v is None else _p(self.v).value
        self.ccfg = cfg.c()

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k in ("y", "idx", "gate", "logits", "count", "f", "p",
                                               "loss", "entropy", "kept", "offset", "pair_row",
                                               "row_pair", "dropped", "counters")}


def moe_layer_forward(cfg: Config, w: dict, x: torch.Tensor, bufs: LayerBuffers | None = None,
                      wstruct: L.MoeWeights | None = None, trace: L.MoeTrace | None = None,
                      want_logits=False, save_for_backward=False) -> LayerBuffers:
    lib = L.load()
    if bufs is None:
        bufs = LayerBuffers(cfg, x.device, want_logits=want_logits,
                            save_for_backward=save_for_backward)
    if wstruct is None:
        wstruct = weights_struct(w)
    L.check(lib.moe_layer_forward(C.byref(bufs.ccfg), C.byref(wstruct), _p(x), C.byref(bufs.out),
                                  _p(bufs.ws), bufs.ws.numel(),
                                  C.byref(trace) if trace is not None else None, _stream()),
            "moe_layer_forward")
    return bufs


def moe_layer_forward_noalloc(cfg: Config, w: dict, x: torch.Tensor, bufs: LayerBuffers,
                              wstruct: L.MoeWeights | None = None,
                              trace: L.MoeTrace | None = None) -> LayerBuffers:
    """moe_layer_forward with the library's fixed device scratch as the
    workspace: allocates nothing (bufs supplies the outputs; bufs.ws is not
    used)."""
    lib = L.load()
    if wstruct is None:
        wstruct = weights_struct(w)
    L.check(lib.moe_layer_forward_noalloc(C.byref(bufs.ccfg), C.byref(wstruct), _p(x),
                                          C.byref(bufs.out),
                                          C.byref(trace) if trace is not None else None,
                                          _stream()), "moe_layer_forward_noalloc")
    return bufs


# ------------------------------------------------------------- backward ---

def moe_backward_workspace_size(cfg: Config) -> int:
    return _size(L.load().moe_backward_workspace_size, cfg)


def _loss_grad(loss_grad) -> L.MoeLossGrad:
    a, z, zl = loss_grad
    return L.MoeLossGrad(aux=float(a), z=float(z), z_lse=float(zl))


class BackwardBuffers:
    """Gradient outputs and workspace for repeated moe_layer_backward calls."""

    def __init__(self, cfg: Config, device):
        T, d, N, F, Fs = cfg.T, cfg.d, cfg.N, cfg.F, cfg.F_shared
        dt, f32 = cfg.torch_dtype, torch.float32
        e = lambda *shape, dtype=dt: torch.empty(shape, dtype=dtype, device=device)  # noqa: E731
        swiglu = cfg.act == "swiglu"
        self.dx = e(T, d)
        self.dw_r = e(N, d, dtype=f32)
        self.db_r = e(N, dtype=f32)
        self.dw1 = e(N, F, d)
        self.dw3 = e(N, F, d) if swiglu else None
        self.dw2 = e(N, d, F)
        self.db1 = None if swiglu else e(N, F)
        self.db2 = None if swiglu else e(N, d)
        self.dws1 = e(Fs, d) if Fs else None
        self.dws3 = e(Fs, d) if Fs else None
        self.dws2 = e(d, Fs) if Fs else None
        self.dlogits = e(T, N, dtype=f32)
        self.ws = _ws(moe_backward_workspace_size(cfg), device)
        self.grads = L.MoeGrads(**{k: (None if getattr(self, k) is None
                                       else _p(getattr(self, k)).value)
                                   for k in ("dx", "dw_r", "db_r", "dw1", "dw3", "dw2", "db1",
                                             "db2", "dws1", "dws3", "dws2", "dlogits")})
        self.ccfg = cfg.c()

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k in ("dx", "dw_r", "db_r", "dw1", "dw3", "dw2", "db1",
                                               "db2", "dws1", "dws3", "dws2", "dlogits")}


def saved_struct(fwd: LayerBuffers) -> L.MoeSaved:
    if fwd.y_perm is None or fwd.logits is None:
        raise ValueError("run moe_layer_forward with save_for_backward=True first")
    return L.MoeSaved(logits=_p(fwd.logits).value, topk_idx=_p(fwd.idx).value,
                      topk_gate=_p(fwd.gate).value, count=_p(fwd.count).value,
                      offset=_p(fwd.offset).value, pair_row=_p(fwd.pair_row).value,
                      row_pair=_p(fwd.row_pair).value, y_perm=_p(fwd.y_perm).value,
                      u=None if fwd.u is None else _p(fwd.u).value,
                      v=None if fwd.v is None else _p(fwd.v).value)


def moe_layer_backward(cfg: Config, w: dict, x: torch.Tensor, fwd: LayerBuffers,
                       dy: torch.Tensor, loss_grad=(0.0, 0.0, 0.0),
                       bufs: BackwardBuffers | None = None,
                       wstruct: L.MoeWeights | None = None,
                       saved: L.MoeSaved | None = None,
                       trace: L.MoeBwdTrace | None = None) -> BackwardBuffers:
    """Gradients of sum(dy * y) + aux_g * aux + z_g * z + zlse_g * z_lse for
    the forward recorded in ``fwd`` (loss_grad = (aux_g, z_g, zlse_g))."""
    lib = L.load()
    if bufs is None:
        bufs = BackwardBuffers(cfg, x.device)
    if wstruct is None:
        wstruct = weights_struct(w)
    if saved is None:
        saved = saved_struct(fwd)
    L.check(lib.moe_layer_backward(C.byref(bufs.ccfg), C.byref(wstruct), _p(x), C.byref(saved),
                                   _p(dy), _loss_grad(loss_grad), C.byref(bufs.grads),
                                   _p(bufs.ws), bufs.ws.numel(),
                                   C.byref(trace) if trace is not None else None, _stream()),
            "moe_layer_backward")
    return bufs


def moe_combine_backward(cfg: Config, dy: torch.Tensor, y_perm: torch.Tensor,
                         gate: torch.Tensor, pair_row: torch.Tensor):
    """-> (d_perm [T*K, d], dgate [T, K] fp32)."""
    lib = L.load()
    d_perm = torch.zeros((cfg.T * cfg.K, cfg.d), dtype=cfg.torch_dtype, device=dy.device)
    dgate = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device=dy.device)
    L.check(lib.moe_combine_backward(C.byref(cfg.c()), _p(dy), _p(y_perm), _p(gate),
                                     _p(pair_row), _p(d_perm), _p(dgate), _stream()),
            "moe_combine_backward")
    return d_perm, dgate


def moe_router_backward(cfg: Config, w: dict, x: torch.Tensor, logits: torch.Tensor,
                        idx: torch.Tensor, pair_row: torch.Tensor, dgate: torch.Tensor,
                        count: torch.Tensor, loss_grad=(0.0, 0.0, 0.0)):
    """-> (dlogits [T, N], dw_r [N, d], db_r [N]), all fp32."""
    lib = L.load()
    dev = x.device
    dl = torch.empty((cfg.T, cfg.N), dtype=torch.float32, device=dev)
    dw_r = torch.empty((cfg.N, cfg.d), dtype=torch.float32, device=dev)
    db_r = torch.empty(cfg.N, dtype=torch.float32, device=dev)
    ws = _ws(moe_backward_workspace_size(cfg), dev)
    L.check(lib.moe_router_backward(C.byref(cfg.c()), C.byref(weights_struct(w)), _p(x),
                                    _p(logits), _p(idx), _p(pair_row), _p(dgate), _p(count),
                                    _loss_grad(loss_grad), _p(dl), _p(dw_r), _p(db_r), _p(ws),
                                    ws.numel(), _stream()), "moe_router_backward")
    return dl, dw_r, db_r


def moe_expert_ffn_backward(cfg: Config, w: dict, x: torch.Tensor, row_pair: torch.Tensor,
                            offset: torch.Tensor, d_perm: torch.Tensor,
                            dy: torch.Tensor | None = None) -> dict:
    """-> dict of dx_perm [T*K, d], dx_shared [T, d] (shared expert) and the
    weight gradients dw1, dw3, dw2, db1, db2, dws1, dws3, dws2."""
    lib = L.load()
    dev = x.device
    g = BackwardBuffers(cfg, dev)
    dx_perm = torch.zeros((cfg.T * cfg.K, cfg.d), dtype=cfg.torch_dtype, device=dev)
    dx_shared = (torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=dev)
                 if cfg.F_shared else None)
    L.check(lib.moe_expert_ffn_backward(C.byref(cfg.c()), C.byref(weights_struct(w)), _p(x),
                                        _p(row_pair), _p(offset), _p(d_perm), _p(dy),
                                        _p(dx_perm), _p(dx_shared), C.byref(g.grads), _p(g.ws),
                                        g.ws.numel(), _stream()), "moe_expert_ffn_backward")
    out = {k: getattr(g, k) for k in ("dw1", "dw3", "dw2", "db1", "db2", "dws1", "dws3", "dws2")}
    out.update(dx_perm=dx_perm, dx_shared=dx_shared, _ws=g.ws)
    return out


def moe_dispatch_backward(cfg: Config, dx_perm: torch.Tensor, pair_row: torch.Tensor,
                          dx_shared: torch.Tensor | None = None,
                          dlogits: torch.Tensor | None = None,
                          w_r: torch.Tensor | None = None) -> torch.Tensor:
    lib = L.load()
    dx = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=dx_perm.device)
    L.check(lib.moe_dispatch_backward(C.byref(cfg.c()), _p(dx_perm), _p(pair_row), _p(dx_shared),
                                      _p(dlogits), _p(w_r), _p(dx), _stream()),
            "moe_dispatch_backward")
    return dx
