"""Python binding of libmoe.so (ctypes).  Argument marshalling only: every
step of routing, forward and backward runs in the library's HIP kernels;
torch provides device memory and the stream.

If the library is missing this module raises instead of computing anything
another way.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# In-tree build; MOE_LIBRARY may name another build of the same library.
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")

MOE_BF16, MOE_F32 = 0, 1
MOE_ROUTE_TC, MOE_ROUTE_TR, MOE_ROUTE_TR_UP, MOE_ROUTE_TR_DOWN, MOE_ROUTE_TR_STOCHASTIC = range(5)
ROUTE_MODES = {"tc": MOE_ROUTE_TC, "tr": MOE_ROUTE_TR, "tr_up": MOE_ROUTE_TR_UP,
               "tr_down": MOE_ROUTE_TR_DOWN, "tr_stochastic": MOE_ROUTE_TR_STOCHASTIC}
TILE_M = 128

ROUTE_KERNELS = ("route_topk", "route_count", "route_select", "route_tslots")
FWD_KERNELS = ("up_swiglu", "down", "aggregate_O")
ROUTER_FWD_KERNELS = ("router_logits",)
ROUTER_BWD_KERNELS = ("router_dlogits", "router_dx", "router_dw", "router_dw_reduce")
BWD_KERNELS = ("dw_plan", "dh", "dxt", "aggregate_dX", "dw1", "dw2")


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("n", ctypes.c_int64),
                ("E", ctypes.c_int64), ("K", ctypes.c_int64), ("M_tile", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32)]


class Sizes(ctypes.Structure):
    _fields_ = [("slot_cap", ctypes.c_int64), ("tile_cap", ctypes.c_int64),
                ("ws_route", ctypes.c_size_t), ("ws_fwd", ctypes.c_size_t),
                ("ws_bwd", ctypes.c_size_t), ("ws_router", ctypes.c_size_t)]


ROUTING_FIELDS = ("tc_counts", "counts", "expert_offsets", "expert_order", "topk_ids",
                  "slot_token", "slot_weight", "token_offsets", "token_slots", "tile_expert",
                  "tile_row", "totals")


class RoutingStruct(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ROUTING_FIELDS]


class Trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("count", ctypes.c_int32)]


class MoEError(RuntimeError):
    pass


_lib = None


def lib():
    """Loads libmoe.so (built in-tree by fine_grained_mixture_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoEError(f"{LIB_PATH} is missing; build it with "
                       "`python -m fine_grained_mixture_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, V, S = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
    L.moe_sizes.argtypes = [P(Problem), P(Sizes)]
    L.moe_route.argtypes = [P(Problem), V, V, P(RoutingStruct), V, S, V, P(Trace)]
    L.moe_fwd.argtypes = [P(Problem), V, V, V, P(RoutingStruct), V, V, V, S, V, P(Trace)]
    L.moe_bwd.argtypes = [P(Problem), V, V, V, V, V, P(RoutingStruct), V, V, V, V, V, S, V,
                          P(Trace)]
    L.moe_gate_bwd.argtypes = [P(Problem), V, V, P(RoutingStruct), V, V, P(Trace)]
    L.moe_router_fwd.argtypes = [P(Problem), V, V, V, V, P(Trace)]
    L.moe_router_bwd.argtypes = [P(Problem), V, V, V, V, P(RoutingStruct), V, V, V, V, S, V,
                                 P(Trace)]
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    for f in ("moe_sizes", "moe_route", "moe_fwd", "moe_bwd", "moe_gate_bwd", "moe_router_fwd",
              "moe_router_bwd", "moe_abi_version"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(status):
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoEError(f"libmoe returned {status}: {msg}")


def problem(T, d, n, E, K, M_tile, dtype=torch.bfloat16, mode="tr") -> Problem:
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[dtype]
    md = ROUTE_MODES[mode]
    return Problem(T, d, n, E, K, M_tile, dt, md)


def torch_dtype(p: Problem):
    return torch.float32 if p.dtype == MOE_F32 else torch.bfloat16


def sizes(p: Problem) -> Sizes:
    s = Sizes()
    _check(lib().moe_sizes(ctypes.byref(p), ctypes.byref(s)))
    return s


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _trace(events):
    if not events:
        return None
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    return Trace(arr, len(events))


def _dev(t: torch.Tensor, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoEError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MoEError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoEError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoEError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class Routing:
    """Device-resident routing metadata (see moe_routing in include/moe.h)."""
    problem: Problem
    tensors: dict
    struct: RoutingStruct = field(repr=False)

    def __getattr__(self, k):
        t = self.__dict__.get("tensors")
        if t is not None and k in t:
            return t[k]
        raise AttributeError(k)

    @property
    def S(self) -> int:
        """Slot count.  The first read after moe_route copies one int from the
        device (waiting for the routing); later reads reuse it."""
        if self.__dict__.get("_S") is None:
            self.__dict__["_S"] = int(self.tensors["totals"][0].item())
        return self.__dict__["_S"]


def alloc_routing(p: Problem, device="cuda") -> Routing:
    s = sizes(p)
    i32 = dict(dtype=torch.int32, device=device)
    T, E, K = p.T, p.E, p.K
    t = {
        "tc_counts": torch.empty(E, **i32),
        "counts": torch.empty(E, **i32),
        "expert_offsets": torch.empty(E + 1, **i32),
        "expert_order": torch.empty(E, **i32),
        "topk_ids": torch.empty(T * K, **i32),
        "slot_token": torch.empty(s.slot_cap, **i32),
        "slot_weight": torch.empty(s.slot_cap, dtype=torch.float32, device=device),
        "token_offsets": torch.empty(T + 1, **i32),
        "token_slots": torch.empty(s.slot_cap, **i32),
        "tile_expert": torch.empty(s.tile_cap, **i32),
        "tile_row": torch.empty(s.tile_cap, **i32),
        "totals": torch.empty(2, **i32),
    }
    st = RoutingStruct(*[t[f].data_ptr() for f in ROUTING_FIELDS])
    return Routing(p, t, st)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def route(p: Problem, logits: torch.Tensor, rt: Routing | None = None, ws=None, stream=None,
          events=None, round_rand: torch.Tensor | None = None) -> Routing:
    """moe_route: top-K token choice, optionally token rounding.  `round_rand`
    ([E] int32 on the device, read as uint32 draws) is needed by the
    stochastic rounding mode and ignored by the others."""
    lg = _dev(logits, "logits", torch.float32, (p.T, p.E))
    rr = None
    if p.mode == MOE_ROUTE_TR_STOCHASTIC:
        if round_rand is None:
            raise MoEError("stochastic token rounding needs round_rand ([E] draws)")
        rr = _dev(round_rand, "round_rand", torch.int32, (p.E,))
    rt = rt if rt is not None else alloc_routing(p, logits.device)
    rt.__dict__["_S"] = None  # refilled below
    ws = ws if ws is not None else workspace(sizes(p).ws_route, logits.device)
    tr = _trace(events)
    _check(lib().moe_route(ctypes.byref(p), lg, rr, ctypes.byref(rt.struct),
                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
                           ctypes.byref(tr) if tr else None))
    return rt


def _h_arg(H, p: Problem, s: Sizes, rt: Routing, dt):
    """H may have slot_cap rows, or fewer but at least S (checked against S
    read back from the device, so that the kernels never write past it)."""
    if not isinstance(H, torch.Tensor) or H.dim() != 2 or H.shape[1] != 2 * p.n:
        raise MoEError(f"H must be [rows, {2 * p.n}]")
    rows = H.shape[0]
    if not 1 <= rows <= s.slot_cap:
        raise MoEError(f"H must have between 1 and {s.slot_cap} rows, got {rows}")
    if rows < s.slot_cap and rows < rt.S:
        raise MoEError(f"H has {rows} rows, fewer than the {rt.S} slots of this routing")
    return _dev(H, "H", dt)


def forward(p: Problem, X, W1, W2, rt: Routing, out=None, ws=None, stream=None, events=None):
    """moe_fwd: returns O [T, d] and H [slot_cap, 2n] (rows [0, S) valid).
    `out` = (O, H) may pass an H of fewer rows, down to S."""
    dt = torch_dtype(p)
    s = sizes(p)
    dev = X.device
    x = _dev(X, "X", dt, (p.T, p.d))
    w1 = _dev(W1, "W1", dt, (p.E, p.d, 2 * p.n))
    w2 = _dev(W2, "W2", dt, (p.E, p.n, p.d))
    O, H = out if out is not None else (torch.empty(p.T, p.d, dtype=dt, device=dev),
                                        torch.empty(s.slot_cap, 2 * p.n, dtype=dt, device=dev))
    ws = ws if ws is not None else workspace(s.ws_fwd, dev)
    tr = _trace(events)
    _check(lib().moe_fwd(ctypes.byref(p), x, w1, w2, ctypes.byref(rt.struct),
                         _dev(O, "O", dt, (p.T, p.d)), _h_arg(H, p, s, rt, dt),
                         ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
                         ctypes.byref(tr) if tr else None))
    return O, H


def backward(p: Problem, dO, X, H, W1, W2, rt: Routing, out=None, ws=None, stream=None,
             events=None):
    """moe_bwd: returns dX [T, d], dW1 [E, d, 2n], dW2 [E, n, d], dS [slot_cap]."""
    dt = torch_dtype(p)
    s = sizes(p)
    dev = X.device
    if out is None:
        out = (torch.empty(p.T, p.d, dtype=dt, device=dev),
               torch.empty(p.E, p.d, 2 * p.n, dtype=dt, device=dev),
               torch.empty(p.E, p.n, p.d, dtype=dt, device=dev),
               torch.empty(s.slot_cap, dtype=torch.float32, device=dev))
    dX, dW1, dW2, dS = out
    ws = ws if ws is not None else workspace(s.ws_bwd, dev)
    tr = _trace(events)
    _check(lib().moe_bwd(ctypes.byref(p), _dev(dO, "dO", dt, (p.T, p.d)),
                         _dev(X, "X", dt, (p.T, p.d)), _h_arg(H, p, s, rt, dt),
                         _dev(W1, "W1", dt, (p.E, p.d, 2 * p.n)),
                         _dev(W2, "W2", dt, (p.E, p.n, p.d)), ctypes.byref(rt.struct),
                         _dev(dX, "dX", dt, (p.T, p.d)),
                         _dev(dW1, "dW1", dt, (p.E, p.d, 2 * p.n)),
                         _dev(dW2, "dW2", dt, (p.E, p.n, p.d)),
                         _dev(dS, "dS", torch.float32, (s.slot_cap,)),
                         ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
                         ctypes.byref(tr) if tr else None))
    return dX, dW1, dW2, dS



def gate_backward(p: Problem, logits, dS, rt: Routing, out=None, stream=None,
                  events=None) -> torch.Tensor:
    """moe_gate_bwd: dlogits [T, E] fp32 from the slot gradients dS."""
    s = sizes(p)
    dl = out if out is not None else torch.empty(p.T, p.E, dtype=torch.float32,
                                                 device=logits.device)
    tr = _trace(events)
    _check(lib().moe_gate_bwd(ctypes.byref(p), _dev(logits, "logits", torch.float32, (p.T, p.E)),
                              _dev(dS, "dS", torch.float32, (s.slot_cap,)),
                              ctypes.byref(rt.struct),
                              _dev(dl, "dlogits", torch.float32, (p.T, p.E)), _stream(stream),
                              ctypes.byref(tr) if tr else None))
    return dl


def router_forward(p: Problem, X, Wr, out=None, stream=None, events=None) -> torch.Tensor:
    """moe_router_fwd: logits = X Wr^T in fp32, [T, E]."""
    dt = torch_dtype(p)
    lg = out if out is not None else torch.empty(p.T, p.E, dtype=torch.float32, device=X.device)
    tr = _trace(events)
    _check(lib().moe_router_fwd(ctypes.byref(p), _dev(X, "X", dt, (p.T, p.d)),
                                _dev(Wr, "Wr", dt, (p.E, p.d)),
                                _dev(lg, "logits", torch.float32, (p.T, p.E)), _stream(stream),
                                ctypes.byref(tr) if tr else None))
    return lg


def router_backward(p: Problem, X, Wr, logits, dS, rt: Routing, dX, out=None, ws=None,
                    stream=None, events=None):
    """moe_router_bwd: returns dlogits [T, E] fp32 and dWr [E, d]; adds the
    router's share of the input gradient to dX in place."""
    dt = torch_dtype(p)
    s = sizes(p)
    dev = X.device
    dl, dWr = out if out is not None else (
        torch.empty(p.T, p.E, dtype=torch.float32, device=dev),
        torch.empty(p.E, p.d, dtype=dt, device=dev))
    ws = ws if ws is not None else workspace(s.ws_router, dev)
    tr = _trace(events)
    _check(lib().moe_router_bwd(ctypes.byref(p), _dev(X, "X", dt, (p.T, p.d)),
                                _dev(Wr, "Wr", dt, (p.E, p.d)),
                                _dev(logits, "logits", torch.float32, (p.T, p.E)),
                                _dev(dS, "dS", torch.float32, (s.slot_cap,)),
                                ctypes.byref(rt.struct),
                                _dev(dl, "dlogits", torch.float32, (p.T, p.E)),
                                _dev(dWr, "dWr", dt, (p.E, p.d)), _dev(dX, "dX", dt, (p.T, p.d)),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
                                ctypes.byref(tr) if tr else None))
    return dl, dWr


class MoELayerFunction(torch.autograd.Function):
    """Autograd op of the layer: X, W1, W2 and the router logits -> O.

    It keeps for the backward exactly what the notes' key design 3 keeps: X,
    H and the routing metadata (plus references to the weights, and to the
    logits when they require a gradient).  H is allocated with exactly S
    rows: after routing, the slot count is read back from the device (one
    4-byte copy, which waits for the routing kernels).  The backward returns
    dX, dW1, dW2 and, when the logits require a gradient, dlogits through
    the gate's softmax backward (moe_gate_bwd).  The draws of stochastic
    rounding (``round_rand``) are an input."""

    @staticmethod
    def forward(ctx, X, W1, W2, logits, K, M_tile, mode, round_rand):
        T, d = X.shape
        E, _, n2 = W1.shape
        p = problem(T, d, n2 // 2, E, K, M_tile, X.dtype, mode)
        rt = route(p, logits, round_rand=round_rand)
        H = torch.empty(max(rt.S, 1), n2, dtype=X.dtype, device=X.device)
        O, H = forward(p, X, W1, W2, rt, out=(torch.empty_like(X), H))
        need_dl = ctx.needs_input_grad[3]
        ctx.save_for_backward(X, H, W1, W2, logits if need_dl else None)
        ctx.moe = (p, rt)
        return O

    @staticmethod
    def backward(ctx, dO):
        X, H, W1, W2, logits = ctx.saved_tensors
        p, rt = ctx.moe
        dX, dW1, dW2, dS = backward(p, dO.contiguous(), X, H, W1, W2, rt)
        dl = gate_backward(p, logits, dS, rt) if ctx.needs_input_grad[3] else None
        return dX, dW1, dW2, dl, None, None, None, None


def moe_layer(X, W1, W2, logits, K, M_tile, mode="tr", round_rand=None):
    return MoELayerFunction.apply(X, W1, W2, logits, K, M_tile, mode, round_rand)


class MoERouterLayerFunction(torch.autograd.Function):
    """The whole layer with its router: logits = X Wr^T are computed by the
    library, and the backward returns dX (experts' and router's shares), dWr,
    dW1 and dW2.  Saves X, H (exactly S rows, as MoELayerFunction), Wr, W1,
    W2, the logits and the routing; the draws of stochastic rounding
    (``round_rand``) are an input."""

    @staticmethod
    def forward(ctx, X, Wr, W1, W2, K, M_tile, mode, round_rand):
        T, d = X.shape
        E, _, n2 = W1.shape
        p = problem(T, d, n2 // 2, E, K, M_tile, X.dtype, mode)
        logits = router_forward(p, X, Wr)
        rt = route(p, logits, round_rand=round_rand)
        H = torch.empty(max(rt.S, 1), n2, dtype=X.dtype, device=X.device)
        O, H = forward(p, X, W1, W2, rt, out=(torch.empty_like(X), H))
        ctx.save_for_backward(X, H, Wr, W1, W2, logits)
        ctx.moe = (p, rt)
        return O

    @staticmethod
    def backward(ctx, dO):
        X, H, Wr, W1, W2, logits = ctx.saved_tensors
        p, rt = ctx.moe
        dX, dW1, dW2, dS = backward(p, dO.contiguous(), X, H, W1, W2, rt)
        _, dWr = router_backward(p, X, Wr, logits, dS, rt, dX)
        return dX, dWr, dW1, dW2, None, None, None, None


def moe_router_layer(X, Wr, W1, W2, K, M_tile, mode="tr", round_rand=None):
    return MoERouterLayerFunction.apply(X, Wr, W1, W2, K, M_tile, mode, round_rand)
