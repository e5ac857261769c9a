"""moe_route_noalloc (the routing entry point that allocates nothing, for
callers that cannot allocate) against moe_route, through the C ABI: the same
routing arrays bit for bit, on two calls in a row, the second with a smaller
problem (the fixed scratch keeps the first call's contents)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import moe
from fine_grained_mixture_amd.inputs import SHAPES, make_layer_inputs, make_round_rand, round_rand_tensor

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def route_noalloc(p, logits, rr):
    L = moe.lib()
    L.moe_route_noalloc.argtypes = [ctypes.POINTER(moe.Problem), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.POINTER(moe.RoutingStruct),
                                    ctypes.c_void_p, ctypes.c_void_p]
    L.moe_route_noalloc.restype = ctypes.c_int
    rt = moe.alloc_routing(p, logits.device)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    status = L.moe_route_noalloc(ctypes.byref(p), ctypes.c_void_p(logits.data_ptr()),
                                 ctypes.c_void_p(rr.data_ptr()) if rr is not None else None,
                                 ctypes.byref(rt.struct), st, None)
    assert status == 0, moe.lib().moe_status_string(status)
    return rt


def same_routing(a, b):
    S = int(b.totals[0])
    assert int(a.totals[0]) == S
    for k in ("tc_counts", "counts", "expert_offsets", "expert_order", "topk_ids",
              "token_offsets", "totals"):
        assert torch.equal(a.tensors[k], b.tensors[k]), k
    for k in ("slot_token", "slot_weight", "token_slots"):
        assert torch.equal(a.tensors[k][:S], b.tensors[k][:S]), k
    nt = int(b.totals[1])
    for k in ("tile_expert", "tile_row"):
        assert torch.equal(a.tensors[k][:nt], b.tensors[k][:nt]), k


@pytest.mark.parametrize("mode", ["tr", "tr_stochastic", "tc"])
def test_route_noalloc_matches_route(mode):
    dev = torch.device("cuda", 0)
    # first the 7B layer, then the small one: the scratch still holds the
    # first call's keys and bitmaps when the second, smaller call runs
    for name in ("7b", "small"):
        sh = SHAPES[name]
        log(f"[noalloc] {name} {mode}")
        lg = make_layer_inputs(sh, dtype=torch.bfloat16, seed=4)["logits"].to(dev)
        rr = round_rand_tensor(make_round_rand(sh.E, 4)).to(dev)
        p = moe.problem(sh.T, sh.d, sh.n, sh.E, sh.K, sh.M, torch.bfloat16, mode)
        got = route_noalloc(p, lg, rr if mode == "tr_stochastic" else None)
        want = moe.route(p, lg, round_rand=rr)
        torch.cuda.synchronize()
        same_routing(got, want)


def test_route_noalloc_allocates_nothing():
    # no device memory is allocated by the call itself (the routing arrays
    # are the caller's, made before)
    dev = torch.device("cuda", 0)
    sh = SHAPES["7b"]
    lg = make_layer_inputs(sh, dtype=torch.bfloat16, seed=5)["logits"].to(dev)
    p = moe.problem(sh.T, sh.d, sh.n, sh.E, sh.K, sh.M, torch.bfloat16, "tr")
    rt = moe.alloc_routing(p, dev)
    L = moe.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # one call first: the library's code object (and with it the scratch
    # array) is loaded on its first use in the process
    assert L.moe_route_noalloc(ctypes.byref(p), ctypes.c_void_p(lg.data_ptr()), None,
                               ctypes.byref(rt.struct), st, None) == 0
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info(dev)
    before = torch.cuda.memory_stats(dev)["requested_bytes.all.current"]
    for _ in range(3):
        assert L.moe_route_noalloc(ctypes.byref(p), ctypes.c_void_p(lg.data_ptr()), None,
                                   ctypes.byref(rt.struct), st, None) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(dev)
    assert torch.cuda.memory_stats(dev)["requested_bytes.all.current"] == before
    assert free1 == free0
    want = moe.route(p, lg)
    torch.cuda.synchronize()
    same_routing(rt, want)
