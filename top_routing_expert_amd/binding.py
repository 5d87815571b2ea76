"""Thin Python binding of ``libmoe.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: torch tensors provide device memory (``data_ptr``)
and the current HIP stream; every step of the layer runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .presets import Preset

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

# moe_status: 0 on success, negative on failure
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
SCORE = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2}
ACT = {"swiglu": 0, "gelu": 1}
DTYPE = {"f32": 0, "bf16": 1}
ROUTING = {"topk": 0, "uniform": 1, "noisy_topk": 2, "gshard": 3, "hash": 4}
PRIORITY = {"token": 0, "slot": 1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class Dims(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("T", "d", "E", "k", "F", "F_shared")]


class Opts(C.Structure):
    _fields_ = [("score", C.c_int32), ("act", C.c_int32), ("dtype", C.c_int32),
                ("renorm", C.c_int32), ("gate_scale", C.c_float),
                ("capacity_factor", C.c_float), ("aux_coef", C.c_float), ("z_coef", C.c_float),
                ("routing", C.c_int32), ("priority", C.c_int32), ("act_pair", C.c_int32)]


class RouterInputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("W_noise", "noise", "uniform", "token_ids")]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("Wg", "logit_offset", "sel_bias", "W13", "W2",
                                          "Ws13", "Ws2")]


class Saved(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_idx", "topk_gate", "logits", "counts", "offsets",
                                          "row_of_slot", "token_of_row", "x_perm", "h", "a", "o",
                                          "h_shared", "a_shared", "losses", "noise_logits")]


class Grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dWg", "dW13", "dW2", "dWs13", "dWs2", "dW_noise", "dH",
                                          "dH_shared")]


class Stats(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("counts", "n_dropped", "losses", "n_nonfinite")]


ABI_FUNCTIONS = ("moe_capacity", "moe_workspace_size", "moe_route", "moe_permute",
                 "moe_permute_noalloc",
                 "moe_expert_ffn", "moe_combine", "moe_layer_fwd", "moe_layer_bwd",
                 "moe_bias_update", "moe_score_histogram", "moe_bias_from_histogram",
                 "moe_router_report", "moe_mx_quantize_weights", "moe_mx_quantize_act",
                 "moe_expert_ffn_mx", "moe_router_draws", "moe_strerror")

_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """Load libmoe.so once; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m top_routing_expert_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, I64, VP, F32 = C.POINTER, C.c_int64, C.c_void_p, C.c_float
    D, O = P(Dims), P(Opts)
    L.moe_capacity.argtypes = [D, O, P(I64)]
    L.moe_workspace_size.argtypes = [D, O, C.c_int, P(C.c_size_t)]
    L.moe_route.argtypes = [D, O, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, P(RouterInputs), VP,
                            C.c_size_t, VP]
    L.moe_permute.argtypes = [D, O, VP, VP, VP, VP, VP, VP, VP, VP, C.c_size_t, VP]
    L.moe_permute_noalloc.argtypes = [D, O, VP, VP, VP, VP, VP, VP, VP, VP]
    L.moe_expert_ffn.argtypes = [D, O, I64, I64, I64, VP, VP, VP, VP, VP, VP, VP, VP, C.c_size_t, VP]
    L.moe_combine.argtypes = [D, VP, VP, VP, VP, VP, VP]
    L.moe_layer_fwd.argtypes = [D, O, P(Weights), P(RouterInputs), VP, VP, P(Saved), P(Stats), VP,
                                C.c_size_t, VP]
    L.moe_layer_bwd.argtypes = [D, O, P(Weights), P(RouterInputs), VP, P(Saved), VP, VP, P(Grads),
                                VP, C.c_size_t, VP]
    L.moe_bias_update.argtypes = [VP, VP, I64, F32, F32, VP]
    L.moe_score_histogram.argtypes = [VP, I64, I64, F32, F32, C.c_int32, VP, VP]
    L.moe_bias_from_histogram.argtypes = [VP, I64, C.c_int32, F32, F32, F32, VP, VP]
    L.moe_router_report.argtypes = [I64, I64, VP, VP, VP, VP, VP, VP, VP]
    L.moe_mx_quantize_weights.argtypes = [O, VP, I64, I64, I64, VP, VP, VP]
    L.moe_mx_quantize_act.argtypes = [O, VP, I64, I64, I64, VP, VP, VP]
    L.moe_expert_ffn_mx.argtypes = [D, O, I64, I64, I64, VP, VP, I64, VP, VP, VP, VP, VP, VP, VP,
                                    I64, VP, VP]
    L.moe_router_draws.argtypes = [D, C.c_uint64, C.c_uint64, VP, VP, VP]
    L.moe_strerror.argtypes = [C.c_int]
    L.moe_strerror.restype = C.c_char_p
    for f in ABI_FUNCTIONS[:-1]:
        getattr(L, f).restype = C.c_int
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_strerror(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def dims_of(p: Preset, T: Optional[int] = None) -> Dims:
    return Dims(p.T if T is None else T, p.d, p.E, p.k, p.F, p.F_shared)


def opts_of(p: Preset) -> Opts:
    return Opts(SCORE[p.score], ACT[p.act], DTYPE[p.dtype], int(p.renorm), p.gate_scale,
                p.capacity_factor, p.aux_coef, p.z_coef, ROUTING[p.routing], PRIORITY[p.priority],
                int(p.act_pair))


def act_cols(p: Preset, F: Optional[int] = None) -> int:
    """Columns of the saved routed activation: F, or 2F for bf16 (hi, lo) pairs."""
    F = p.F if F is None else F
    return 2 * F if (p.act_pair and p.dtype == "bf16") else F


def capacity(p: Preset, T: Optional[int] = None) -> int:
    c = C.c_int64()
    _check("moe_capacity", lib().moe_capacity(C.byref(dims_of(p, T)), C.byref(opts_of(p)), C.byref(c)))
    return c.value


def workspace_size(p: Preset, with_bwd: bool = False, T: Optional[int] = None) -> int:
    n = C.c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(
        C.byref(dims_of(p, T)), C.byref(opts_of(p)), int(with_bwd), C.byref(n)))
    return n.value


def _need(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


class Workspace:
    """Caller-owned device scratch for the library (grown on demand)."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = torch.empty(0, dtype=torch.uint8, device=self.device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


# --------------------------------------------------------------------------- steps
def route(p: Preset, x, Wg, offset=None, sel_bias=None, *, want_scores=False, want_logits=False,
          ri: Optional["LayerRouterInputs"] = None, ws: Optional[Workspace] = None):
    """moe_route: returns dict(idx [T,k] i32, gate [T,k] f32, counts [E], losses [2], ...)."""
    dev = x.device
    T = x.shape[0]
    _need(x, "x", (T, p.d), TORCH_DTYPE[p.dtype], dev)
    _need(Wg, "Wg", (p.d, p.E), torch.float32, dev)
    out = dict(idx=torch.empty(T, p.k, dtype=torch.int32, device=dev),
               gate=torch.empty(T, p.k, dtype=torch.float32, device=dev),
               counts=torch.empty(p.E, dtype=torch.int32, device=dev),
               losses=torch.empty(2, dtype=torch.float32, device=dev))
    out["scores"] = torch.empty(T, p.E, dtype=torch.float32, device=dev) if want_scores else None
    out["logits"] = torch.empty(T, p.E, dtype=torch.float32, device=dev) if want_logits else None
    ws = ws or Workspace(dev)
    nb = workspace_size(p, T=T)
    buf = ws.get(nb)
    _check("moe_route", lib().moe_route(
        C.byref(dims_of(p, T)), C.byref(opts_of(p)), _ptr(x), _ptr(Wg), _ptr(offset), _ptr(sel_bias),
        _ptr(out["idx"]), _ptr(out["gate"]), _ptr(out["scores"]), _ptr(out["logits"]),
        _ptr(out["counts"]), _ptr(out["losses"]), _ri_c(ri), _ptr(buf), nb, _stream()))
    return out


def router_draws(T: int, E: int, seed: int, offset: int, device, *, noise: bool = True,
                 uniform: bool = True, out: Optional[dict] = None):
    """moe_router_draws: the stochastic routers' draws for one call, generated on
    the device.  Returns dict(noise [T, E] f32 or None, uniform [T] f32 or None);
    `out` may hold preallocated tensors of those shapes (e.g. a LayerRouterInputs'
    buffers, refilled each step with a new offset)."""
    dev = torch.device(device)
    out = dict(out or {})
    if noise and out.get("noise") is None:
        out["noise"] = torch.empty(T, E, dtype=torch.float32, device=dev)
    if uniform and out.get("uniform") is None:
        out["uniform"] = torch.empty(T, dtype=torch.float32, device=dev)
    nz, un = (out.get("noise") if noise else None), (out.get("uniform") if uniform else None)
    if nz is not None:
        _need(nz, "noise", (T, E), torch.float32, dev)
    if un is not None:
        _need(un, "uniform", (T,), torch.float32, dev)
    d = Dims(T, 0, E, 0, 0, 0)
    _check("moe_router_draws", lib().moe_router_draws(
        C.byref(d), C.c_uint64(seed), C.c_uint64(offset), _ptr(nz), _ptr(un), _stream()))
    return dict(noise=nz, uniform=un)


def permute(p: Preset, x, idx, ws: Optional[Workspace] = None):
    """moe_permute: returns dict(counts, offsets, row_of_slot, token_of_row, x_perm)."""
    dev = x.device
    T = x.shape[0]
    _need(x, "x", (T, p.d), TORCH_DTYPE[p.dtype], dev)
    _need(idx, "idx", (T, p.k), torch.int32, dev)
    out = dict(counts=torch.empty(p.E, dtype=torch.int32, device=dev),
               offsets=torch.empty(p.E + 1, dtype=torch.int32, device=dev),
               row_of_slot=torch.empty(T, p.k, dtype=torch.int32, device=dev),
               token_of_row=torch.empty(max(T * p.k, 1), dtype=torch.int32, device=dev),
               x_perm=torch.empty(max(T * p.k, 1), p.d, dtype=x.dtype, device=dev))
    ws = ws or Workspace(dev)
    nb = workspace_size(p, T=T)
    buf = ws.get(nb)
    _check("moe_permute", lib().moe_permute(
        C.byref(dims_of(p, T)), C.byref(opts_of(p)), _ptr(x), _ptr(idx), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(out["row_of_slot"]), _ptr(out["token_of_row"]),
        _ptr(out["x_perm"]), _ptr(buf), nb, _stream()))
    return out


def permute_noalloc(p: Preset, x, idx, out: Optional[dict] = None):
    """moe_permute_noalloc (no workspace): the same outputs as permute(); `out`
    may hold preallocated output tensors (the call itself allocates nothing)."""
    dev = x.device
    T = x.shape[0]
    _need(x, "x", (T, p.d), TORCH_DTYPE[p.dtype], dev)
    _need(idx, "idx", (T, p.k), torch.int32, dev)
    if out is None:
        out = dict(counts=torch.empty(p.E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(p.E + 1, dtype=torch.int32, device=dev),
                   row_of_slot=torch.empty(T, p.k, dtype=torch.int32, device=dev),
                   token_of_row=torch.empty(max(T * p.k, 1), dtype=torch.int32, device=dev),
                   x_perm=torch.empty(max(T * p.k, 1), p.d, dtype=x.dtype, device=dev))
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        C.byref(dims_of(p, T)), C.byref(opts_of(p)), _ptr(x), _ptr(idx), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(out["row_of_slot"]), _ptr(out["token_of_row"]),
        _ptr(out["x_perm"]), _stream()))
    return out


def expert_ffn(p: Preset, x_perm, offsets, W13, W2, *, max_rows=None, F=None, act=None,
               save_hidden=False, ws: Optional[Workspace] = None):
    """moe_expert_ffn over len(offsets)-1 groups; returns dict(out [rows,d] f32, h, a)."""
    dev = x_perm.device
    G = offsets.numel() - 1
    F = p.F if F is None else F
    act = p.act if act is None else act
    rows = x_perm.shape[0] if max_rows is None else max_rows
    q = p.with_(act=act, F=F)
    nu = 2 * F if act == "swiglu" else F
    _need(W13, "W13", (G, nu, p.d), TORCH_DTYPE[p.dtype], dev)
    _need(W2, "W2", (G, p.d, F), TORCH_DTYPE[p.dtype], dev)
    out = torch.empty(max(rows, 1), p.d, dtype=torch.float32, device=dev)
    h = torch.empty(max(rows, 1), nu, dtype=x_perm.dtype, device=dev) if save_hidden else None
    a = torch.empty(max(rows, 1), act_cols(q, F), dtype=x_perm.dtype, device=dev) if save_hidden else None
    ws = ws or Workspace(dev)
    nb = workspace_size(q) + rows * act_cols(q, F) * (2 if p.dtype == "bf16" else 4) + 4096
    buf = ws.get(nb)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        C.byref(dims_of(q)), C.byref(opts_of(q)), G, rows, F, _ptr(x_perm), _ptr(offsets),
        _ptr(W13), _ptr(W2), _ptr(h), _ptr(a), _ptr(out), _ptr(buf), nb, _stream()))
    return dict(out=out, h=h, a=a)


def combine(p: Preset, out_perm, row_of_slot, gate, shared=None):
    T = row_of_slot.shape[0]
    y = torch.empty(T, p.d, dtype=torch.float32, device=row_of_slot.device)
    _check("moe_combine", lib().moe_combine(
        C.byref(dims_of(p, T)), _ptr(out_perm), _ptr(row_of_slot), _ptr(gate), _ptr(shared),
        _ptr(y), _stream()))
    return y


def bias_update(counts, bias, target: float, gamma: float):
    _check("moe_bias_update", lib().moe_bias_update(_ptr(counts), _ptr(bias), counts.numel(),
                                                    target, gamma, _stream()))


# --------------------------------------------------------------------------- layer
@dataclass
class LayerWeights:
    Wg: torch.Tensor
    W13: torch.Tensor
    W2: torch.Tensor
    offset: Optional[torch.Tensor] = None
    sel_bias: Optional[torch.Tensor] = None
    Ws13: Optional[torch.Tensor] = None
    Ws2: Optional[torch.Tensor] = None

    def c(self) -> Weights:
        return Weights(*(None if t is None else t.data_ptr() for t in
                         (self.Wg, self.offset, self.sel_bias, self.W13, self.W2, self.Ws13,
                          self.Ws2)))


@dataclass
class LayerRouterInputs:
    """The variant routers' per-call inputs on the device (see moe_router_inputs)."""
    W_noise: Optional[torch.Tensor] = None
    noise: Optional[torch.Tensor] = None
    uniform: Optional[torch.Tensor] = None
    token_ids: Optional[torch.Tensor] = None

    def c(self) -> RouterInputs:
        return RouterInputs(*(None if t is None else t.data_ptr() for t in
                              (self.W_noise, self.noise, self.uniform, self.token_ids)))


def _ri_c(ri: Optional[LayerRouterInputs]):
    return None if ri is None else C.byref(ri.c())


def router_inputs_to_device(inp: dict, device) -> LayerRouterInputs:
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return LayerRouterInputs(W_noise=t(inp.get("W_noise")), noise=t(inp.get("noise")),
                             uniform=t(inp.get("uniform")), token_ids=t(inp.get("token_ids")))


def weights_to_device(p: Preset, inp: dict, device) -> LayerWeights:
    wd = TORCH_DTYPE[p.dtype]
    # upload fp32 and convert on the device (values are already representable in dt)
    t = lambda a, dt: None if a is None else torch.from_numpy(a).to(device).to(dt).contiguous()
    return LayerWeights(Wg=t(inp["Wg"], torch.float32), W13=t(inp["W13"], wd), W2=t(inp["W2"], wd),
                        offset=t(inp.get("offset"), torch.float32),
                        sel_bias=t(inp.get("sel_bias"), torch.float32),
                        Ws13=t(inp.get("Ws13"), wd), Ws2=t(inp.get("Ws2"), wd))


def alloc_saved(p: Preset, device, T: Optional[int] = None) -> dict:
    T = p.T if T is None else T
    Tk = max(T * p.k, 1)
    xd = TORCH_DTYPE[p.dtype]
    nu = 2 * p.F if p.act == "swiglu" else p.F
    e = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=device)
    s = dict(topk_idx=e(T, p.k, dt=torch.int32), topk_gate=e(T, p.k), logits=e(T, p.E),
             counts=e(p.E, dt=torch.int32), offsets=e(p.E + 1, dt=torch.int32),
             row_of_slot=e(T, p.k, dt=torch.int32), token_of_row=e(Tk, dt=torch.int32),
             x_perm=e(Tk, p.d, dt=xd), h=e(Tk, nu, dt=xd), a=e(Tk, act_cols(p), dt=xd), o=e(Tk, p.d),
             h_shared=e(T, 2 * p.F_shared, dt=xd) if p.F_shared else None,
             a_shared=e(T, p.F_shared, dt=xd) if p.F_shared else None, losses=e(2),
             noise_logits=e(T, p.E) if p.routing == "noisy_topk" else None)
    return s


def _saved_c(s: Optional[dict]):
    if s is None:
        return None
    return C.byref(Saved(*(None if s[n] is None else s[n].data_ptr() for n, _ in Saved._fields_)))


def layer_fwd(p: Preset, w: LayerWeights, x, *, saved: Optional[dict] = None, stats: bool = False,
              ri: Optional[LayerRouterInputs] = None, ws: Optional[Workspace] = None,
              y: Optional[torch.Tensor] = None):
    """moe_layer_fwd; returns y (and the stats dict when asked)."""
    dev = x.device
    T = x.shape[0]
    _need(x, "x", (T, p.d), TORCH_DTYPE[p.dtype], dev)
    if y is None:
        y = torch.empty(T, p.d, dtype=torch.float32, device=dev)
    st = None
    st_c = None
    if stats:
        st = dict(counts=torch.empty(p.E, dtype=torch.int32, device=dev),
                  n_dropped=torch.empty(1, dtype=torch.int32, device=dev),
                  losses=torch.empty(2, dtype=torch.float32, device=dev),
                  n_nonfinite=torch.empty(1, dtype=torch.int32, device=dev))
        st_c = C.byref(Stats(*(st[n].data_ptr() for n, _ in Stats._fields_)))
    ws = ws or Workspace(dev)
    nb = workspace_size(p, with_bwd=saved is not None, T=T)
    buf = ws.get(nb)
    _check("moe_layer_fwd", lib().moe_layer_fwd(
        C.byref(dims_of(p, T)), C.byref(opts_of(p)), C.byref(w.c()), _ri_c(ri), _ptr(x), _ptr(y),
        _saved_c(saved), st_c, _ptr(buf), nb, _stream()))
    return (y, st) if stats else y


def layer_bwd(p: Preset, w: LayerWeights, x, saved: dict, dy, *,
              ri: Optional[LayerRouterInputs] = None, ws: Optional[Workspace] = None,
              want_dH: bool = False):
    """moe_layer_bwd; returns dict(dx, dWg, dW13, dW2, dWs13, dWs2, dW_noise, dH, dH_shared)
    (dH and dH_shared, the gradients of the saved pre-activations, only when asked)."""
    dev = x.device
    T = x.shape[0]
    e = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)
    nu = 2 * p.F if p.act == "swiglu" else p.F
    xd = TORCH_DTYPE[p.dtype]
    g = dict(dx=e(T, p.d), dWg=e(p.d, p.E), dW13=e(p.E, nu, p.d), dW2=e(p.E, p.d, p.F),
             dWs13=e(2 * p.F_shared, p.d) if p.F_shared else None,
             dWs2=e(p.d, p.F_shared) if p.F_shared else None,
             dW_noise=e(p.d, p.E) if p.routing == "noisy_topk" else None,
             dH=torch.empty(max(T * p.k, 1), nu, dtype=xd, device=dev) if want_dH else None,
             dH_shared=(torch.empty(T, 2 * p.F_shared, dtype=xd, device=dev)
                        if want_dH and p.F_shared else None))
    gc = Grads(*(None if g[n] is None else g[n].data_ptr() for n, _ in Grads._fields_))
    ws = ws or Workspace(dev)
    nb = workspace_size(p, with_bwd=True, T=T)
    buf = ws.get(nb)
    _check("moe_layer_bwd", lib().moe_layer_bwd(
        C.byref(dims_of(p, T)), C.byref(opts_of(p)), C.byref(w.c()), _ri_c(ri), _ptr(x),
        _saved_c(saved), _ptr(dy), _ptr(g["dx"]), C.byref(gc), _ptr(buf), nb, _stream()))
    return g


class Layer:
    """One MoE layer bound to device weights, with its workspace, saved state and
    output buffers allocated once, and the ctypes arguments built once, so a
    forward or backward call is a single C call that only enqueues kernels."""

    def __init__(self, p: Preset, w: LayerWeights, device, T: Optional[int] = None,
                 train: bool = False, ri: Optional[LayerRouterInputs] = None):
        self.p, self.w, self.T = p, w, p.T if T is None else T
        self.ri = ri
        self._ri = ri.c() if ri is not None else None
        self.device = torch.device(device)
        self.train = train
        self._dims, self._opts, self._w = dims_of(p, self.T), opts_of(p), w.c()
        self.ws_bytes = workspace_size(p, with_bwd=train, T=self.T)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.y = torch.empty(self.T, p.d, dtype=torch.float32, device=self.device)
        self.saved = alloc_saved(p, self.device, self.T) if train else None
        self._saved_c = (Saved(*(None if self.saved[n] is None else self.saved[n].data_ptr()
                                 for n, _ in Saved._fields_)) if train else None)
        self.grads = None
        self.dx = None
        self._grads_c = None

    def fwd(self, x: torch.Tensor) -> torch.Tensor:
        _check("moe_layer_fwd", lib().moe_layer_fwd(
            C.byref(self._dims), C.byref(self._opts), C.byref(self._w),
            C.byref(self._ri) if self._ri is not None else None, C.c_void_p(x.data_ptr()),
            C.c_void_p(self.y.data_ptr()), C.byref(self._saved_c) if self.train else None, None,
            C.c_void_p(self.ws.data_ptr()), self.ws_bytes, _stream()))
        return self.y

    def draw(self, seed: int, offset: int) -> None:
        """Refill the bound router inputs' noise / uniform buffers (whichever
        the routing uses) with moe_router_draws(seed, offset), in place; call
        once per step with a new offset, before fwd (bwd reads the same draws)."""
        if self.ri is None:
            raise ValueError("no router inputs bound to this layer")
        p = self.p
        router_draws(self.T, p.E, seed, offset, self.device,
                     noise=self.ri.noise is not None, uniform=self.ri.uniform is not None,
                     out=dict(noise=self.ri.noise, uniform=self.ri.uniform))

    def bwd(self, x: torch.Tensor, dy: torch.Tensor) -> dict:
        p = self.p
        if self.grads is None:
            e = lambda *s: torch.empty(*s, dtype=torch.float32, device=self.device)
            nu = 2 * p.F if p.act == "swiglu" else p.F
            self.grads = dict(dWg=e(p.d, p.E), dW13=e(p.E, nu, p.d), dW2=e(p.E, p.d, p.F),
                              dWs13=e(2 * p.F_shared, p.d) if p.F_shared else None,
                              dWs2=e(p.d, p.F_shared) if p.F_shared else None,
                              dW_noise=e(p.d, p.E) if p.routing == "noisy_topk" else None)
            self.dx = e(self.T, p.d)
            self._grads_c = Grads(*(None if self.grads.get(n) is None else self.grads[n].data_ptr()
                                    for n, _ in Grads._fields_))
        _check("moe_layer_bwd", lib().moe_layer_bwd(
            C.byref(self._dims), C.byref(self._opts), C.byref(self._w),
            C.byref(self._ri) if self._ri is not None else None, C.c_void_p(x.data_ptr()),
            C.byref(self._saved_c), C.c_void_p(dy.data_ptr()), C.c_void_p(self.dx.data_ptr()),
            C.byref(self._grads_c), C.c_void_p(self.ws.data_ptr()), self.ws_bytes, _stream()))
        return dict(self.grads, dx=self.dx)


# --------------------------------------------------------------------------- balance / monitoring
def score_histogram(scores, lo: float, hi: float, nbins: int):
    """moe_score_histogram: hist [E, nbins] int32 of the scores [T, E]."""
    T, E = scores.shape
    _need(scores, "scores", (T, E), torch.float32, scores.device)
    hist = torch.empty(E, nbins, dtype=torch.int32, device=scores.device)
    _check("moe_score_histogram", lib().moe_score_histogram(
        _ptr(scores), T, E, lo, hi, nbins, _ptr(hist), _stream()))
    return hist


def bias_from_histogram(hist, lo: float, hi: float, target: float):
    """moe_bias_from_histogram: the quantile-balancing selection bias [E]."""
    E, nbins = hist.shape
    bias = torch.empty(E, dtype=torch.float32, device=hist.device)
    _check("moe_bias_from_histogram", lib().moe_bias_from_histogram(
        _ptr(hist), E, nbins, lo, hi, target, _ptr(bias), _stream()))
    return bias


def router_report(counts, n_dropped=None, out_perm=None, offsets=None, d: int = 0):
    """moe_router_report: dict(report [5] f32, expert_norm [E] or None)."""
    E = counts.numel()
    dev = counts.device
    norm = torch.empty(E, dtype=torch.float32, device=dev) if out_perm is not None else None
    rep = torch.empty(5, dtype=torch.float32, device=dev)
    _check("moe_router_report", lib().moe_router_report(
        E, d if out_perm is None else out_perm.shape[1], _ptr(counts), _ptr(n_dropped),
        _ptr(out_perm), _ptr(offsets), _ptr(norm), _ptr(rep), _stream()))
    return dict(report=rep, expert_norm=norm)


# --------------------------------------------------------------------------- MXFP4 experts
def mx_quantize_weights(p: Preset, w):
    """moe_mx_quantize_weights: w [G, N, K] -> codes [G, K/64, N, 32] u8, scales [G, K/32, N] u8."""
    G, N, K = w.shape
    _need(w, "w", (G, N, K), TORCH_DTYPE[p.dtype], w.device)
    codes = torch.empty(G, K // 64, N, 32, dtype=torch.uint8, device=w.device)
    scales = torch.empty(G, K // 32, N, dtype=torch.uint8, device=w.device)
    _check("moe_mx_quantize_weights", lib().moe_mx_quantize_weights(
        C.byref(opts_of(p)), _ptr(w), G, N, K, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def mx_stride(rows: int) -> int:
    """Row stride of an activation scale array usable by moe_expert_ffn_mx."""
    return (rows + 4 + 3) // 4 * 4


def mx_quantize_act(p: Preset, x, stride: Optional[int] = None):
    """moe_mx_quantize_act: x [rows, K] -> FP8 codes [K/64, stride, 64] u8, scales [K/64, stride] u8."""
    rows, K = x.shape
    stride = rows if stride is None else stride
    _need(x, "x", (rows, K), TORCH_DTYPE[p.dtype], x.device)
    codes = torch.empty(K // 64, max(stride, 1), 64, dtype=torch.uint8, device=x.device)
    scales = torch.empty(K // 64, max(stride, 1), dtype=torch.uint8, device=x.device)
    _check("moe_mx_quantize_act", lib().moe_mx_quantize_act(
        C.byref(opts_of(p)), _ptr(x), rows, K, stride, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def expert_ffn_mx(p: Preset, xq, xs, offsets, W13q, W13s, W2q, W2s, *, max_rows: int,
                  F: Optional[int] = None, act: Optional[str] = None):
    """moe_expert_ffn_mx: returns dict(out [rows, d] f32, aq [F/64, a_stride, 64] u8,
    aqs [F/64, a_stride] u8)."""
    dev = xq.device
    G = offsets.numel() - 1
    F = p.F if F is None else F
    q = p.with_(act=p.act if act is None else act, F=F)
    rows = max(max_rows, 1)
    a_stride = mx_stride(rows)
    out = torch.empty(rows, p.d, dtype=torch.float32, device=dev)
    aq = torch.empty(F // 64, a_stride, 64, dtype=torch.uint8, device=dev)
    aqs = torch.empty(F // 64, a_stride, dtype=torch.uint8, device=dev)
    _check("moe_expert_ffn_mx", lib().moe_expert_ffn_mx(
        C.byref(dims_of(q)), C.byref(opts_of(q)), G, max_rows, F, _ptr(xq), _ptr(xs), xs.shape[1],
        _ptr(offsets), _ptr(W13q), _ptr(W13s), _ptr(W2q), _ptr(W2s), _ptr(aq), _ptr(aqs), a_stride,
        _ptr(out), _stream()))
    return dict(out=out, aq=aq, aqs=aqs)
