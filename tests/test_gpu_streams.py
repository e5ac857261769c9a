"""GPU: the backward's two-stream schedule.

Untraced, moe_bwd runs dW1 and dW2 on the library's own stream of the device,
forked from the caller's stream after dH and joined back before it returns;
traced, it runs every kernel in order on the caller's stream.  Both orders run the same kernels on
the same inputs, so they must give the same bytes, also when the untraced
call is captured into a HIP graph and replayed (the join makes the capture
take in both branches).  Outputs start as NaN, so an element that no kernel
writes shows.
"""
import sys

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import moe
from fine_grained_mixture_amd.inputs import SHAPES, LayerShape, make_layer_inputs

pytestmark = pytest.mark.gpu

NAMES = ("dX", "dW1", "dW2", "dS")
# skewed load under token rounding: many experts end with no slots, whose
# dW1 / dW2 tiles the weight-gradient kernels fill with zeros
SKEWED = LayerShape("skewed", 2048, 512, 128, 64, 4, 128, "fan_in", "zipf_bias")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def nan_outputs(p, dev):
    s = moe.sizes(p)
    return (torch.full((p.T, p.d), float("nan"), dtype=torch.bfloat16, device=dev),
            torch.full((p.E, p.d, 2 * p.n), float("nan"), dtype=torch.bfloat16, device=dev),
            torch.full((p.E, p.n, p.d), float("nan"), dtype=torch.bfloat16, device=dev),
            torch.full((s.slot_cap,), float("nan"), dtype=torch.float32, device=dev))


def bwd_events():
    events = [torch.cuda.Event(enable_timing=True) for _ in range(len(moe.BWD_KERNELS) + 1)]
    for e in events:
        e.record()  # torch creates the HIP event on its first record
    return events


def layer(name):
    shape = SKEWED if name == "skewed" else SHAPES[name]
    log(f"[streams] {name}: T={shape.T} d={shape.d} n={shape.n} E={shape.E} K={shape.K}")
    inp = make_layer_inputs(shape, dtype=torch.bfloat16, seed=0)
    dev = torch.device("cuda", 0)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, torch.bfloat16, "tr")
    X, W1, W2, lg, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "logits", "dO"))
    rt = moe.route(p, lg)
    _, H = moe.forward(p, X, W1, W2, rt)
    return p, (dO, X, H, W1, W2, rt)


def same(a, b, S):
    for x, y, name in zip(a, b, NAMES):
        if name == "dS":
            x, y = x[:S], y[:S]
        assert torch.equal(x, y), f"{name} differs"


@pytest.mark.parametrize("name", ["small", "7b", "skewed"])
def test_bwd_traced_and_forked_agree(name):
    p, args = layer(name)
    dev = args[0].device
    forked = moe.backward(p, *args, out=nan_outputs(p, dev))
    traced = moe.backward(p, *args, out=nan_outputs(p, dev), events=bwd_events())
    torch.cuda.synchronize()
    same(forked, traced, int(args[-1].totals[0]))


def test_experts_without_slots_get_zero_gradients():
    p, args = layer("skewed")
    dev = args[0].device
    counts = args[-1].counts.cpu().numpy()
    empty, busy = np.flatnonzero(counts == 0), np.flatnonzero(counts > 0)
    log(f"[streams] skewed: {len(empty)} of {p.E} experts without slots")
    assert len(empty) >= 8 and len(busy) >= 8
    for traced in (False, True):
        dX, dW1, dW2, _ = moe.backward(p, *args, out=nan_outputs(p, dev),
                                       events=bwd_events() if traced else None)
        torch.cuda.synchronize()
        e0 = torch.from_numpy(empty).to(dev)
        e1 = torch.from_numpy(busy).to(dev)
        assert torch.count_nonzero(dW1[e0].float()) == 0 and torch.count_nonzero(dW2[e0].float()) == 0
        assert bool(torch.isfinite(dW1[e1].float()).all()) and bool(torch.isfinite(dW2[e1].float()).all())
        assert bool(torch.isfinite(dX.float()).all())


@pytest.mark.parametrize("name", ["small", "skewed"])
def test_bwd_graph_replays_match_eager(name):
    p, args = layer(name)
    dev = args[0].device
    s = moe.sizes(p)
    ws = moe.workspace(s.ws_bwd, dev)
    out = (torch.empty(p.T, p.d, dtype=torch.bfloat16, device=dev),
           torch.empty(p.E, p.d, 2 * p.n, dtype=torch.bfloat16, device=dev),
           torch.empty(p.E, p.n, p.d, dtype=torch.bfloat16, device=dev),
           torch.empty(s.slot_cap, dtype=torch.float32, device=dev))
    # eager first: it also creates the library's stream for this device
    ref = [t.clone() for t in moe.backward(p, *args, out=out, ws=ws)]
    torch.cuda.synchronize()
    S = int(args[-1].totals[0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.backward(p, *args, out=out, ws=ws)
    torch.cuda.synchronize()
    for i in range(3):
        for t in out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[streams] replay {i}")
        same(out, ref, S)


def test_step_graph_replays_match_eager():
    """The whole step (route, forward, backward) captured once and replayed,
    as the benchmark times it, reproduces the eager step's bytes."""
    shape = SHAPES["small"]
    log(f"[streams] step graph: small T={shape.T}")
    inp = make_layer_inputs(shape, dtype=torch.bfloat16, seed=0)
    dev = torch.device("cuda", 0)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, torch.bfloat16, "tr")
    X, W1, W2, lg, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "logits", "dO"))
    s = moe.sizes(p)
    rt = moe.alloc_routing(p, dev)
    ws_r, ws_f, ws_b = (moe.workspace(n, dev) for n in (s.ws_route, s.ws_fwd, s.ws_bwd))
    O = torch.empty(p.T, p.d, dtype=torch.bfloat16, device=dev)
    H = torch.empty(s.slot_cap, 2 * p.n, dtype=torch.bfloat16, device=dev)
    grads = (torch.empty(p.T, p.d, dtype=torch.bfloat16, device=dev),
             torch.empty(p.E, p.d, 2 * p.n, dtype=torch.bfloat16, device=dev),
             torch.empty(p.E, p.n, p.d, dtype=torch.bfloat16, device=dev),
             torch.empty(s.slot_cap, dtype=torch.float32, device=dev))

    def step():
        moe.route(p, lg, rt=rt, ws=ws_r)
        moe.forward(p, X, W1, W2, rt, out=(O, H), ws=ws_f)
        moe.backward(p, dO, X, H, W1, W2, rt, out=grads, ws=ws_b)

    def outputs():
        S = int(rt.totals[0])
        return [t.clone() for t in (rt.totals, rt.slot_token[:S], rt.token_slots[:S], O, H[:S],
                                    grads[0], grads[1], grads[2], grads[3][:S])]

    step()  # eager first: it also creates the library's stream for this device
    torch.cuda.synchronize()
    want = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (O, H, *grads):
            t.fill_(float("nan"))
        for t in (rt.slot_token, rt.token_slots):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[streams] step replay {i}")
        for a, b in zip(outputs(), want):
            assert torch.equal(a, b)
