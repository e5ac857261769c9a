"""CPU checks of the C ABI: the library loads, exports every function that
include/moe.h declares, sizes its buffers, and rejects bad arguments on the
host before anything is enqueued (no GPU needed: no call here reaches a
launch)."""
import ctypes
import os
import re

import pytest

from fine_grained_mixture_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                                reason="libmoe.so not built (run __graft_entry__.build())")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert names == ["moe_abi_version", "moe_bwd", "moe_fwd", "moe_gate_bwd", "moe_route",
                     "moe_route_noalloc", "moe_router_bwd", "moe_router_fwd", "moe_sizes",
                     "moe_status_string"]
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == 4


def test_status_strings():
    L = moe.lib()
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert L.moe_status_string(st)
    assert L.moe_status_string(7) == b"unknown status"


def test_sizes_7b_layer():
    p = moe.problem(16384, 1536, 256, 128, 8, 128)
    s = moe.sizes(p)
    assert s.slot_cap == 16384 * 8 + 128 * 63
    assert s.tile_cap == -(-s.slot_cap // 128) + 128
    esz = 2
    assert s.ws_fwd >= s.slot_cap * (256 + 1536) * esz
    assert s.ws_bwd >= s.slot_cap * (512 + 256 + 1536) * esz
    assert s.ws_route >= 16384 * 128 * 8


@pytest.mark.parametrize("mode,pad", [("tc", 0), ("tr_down", 0), ("tr", 63), ("tr_up", 127),
                                      ("tr_stochastic", 127)])
def test_slot_cap_per_mode(mode, pad):
    # token choice keeps T K pairs; nearest rounding pads an expert only when
    # the upward gap is below M/2 (at most floor((M-1)/2) = 63 slots for
    # M = 128), up and stochastic rounding by at most M - 1, down never
    for T, d, n, E, K in ((16384, 1536, 256, 128, 8), (8192, 2048, 384, 512, 8)):
        s = moe.sizes(moe.problem(T, d, n, E, K, 128, mode=mode))
        assert s.slot_cap == T * K + E * pad
    # odd M: nearest pads by at most (M - 1) / 2
    s = moe.sizes(moe.problem(900, 256, 128, 12, 3, 49, mode="tr"))
    assert s.slot_cap == 900 * 3 + 12 * 24
    # no expert can hold more than T tokens: the bound is capped at T E
    s = moe.sizes(moe.problem(1, 128, 64, 4, 2, 16, mode="tr_up"))
    assert s.slot_cap == 4


def test_slot_cap_bounds_every_rounding():
    # brute force over every token-choice count vector of a small problem:
    # the rounded total never exceeds the mode's slot_cap
    import itertools

    from oracle import moe_oracle as orc
    T, E, K, M = 7, 3, 2, 4
    u = [0, 1 << 31, (1 << 32) - 1]
    for mode, cm in (("tc", orc.TC), ("tr", orc.TR), ("tr_up", orc.TR_UP),
                     ("tr_down", orc.TR_DOWN), ("tr_stochastic", orc.TR_STOCHASTIC)):
        cap = moe.sizes(moe.problem(T, 128, 64, E, K, M, mode=mode)).slot_cap
        worst = 0
        for f in itertools.product(range(T + 1), repeat=E):
            if sum(f) != T * K:
                continue
            worst = max(worst, int(orc.round_counts(f, M, T, cm, u).sum()))
        assert worst <= cap, (mode, worst, cap)


def test_sizes_fp32_doubles_transients():
    b = moe.sizes(moe.problem(256, 128, 64, 8, 2, 16, dtype=moe.torch.bfloat16))
    f = moe.sizes(moe.problem(256, 128, 64, 8, 2, 16, dtype=moe.torch.float32))
    assert f.ws_fwd >= 2 * b.ws_fwd - 512 and f.ws_route == b.ws_route


@pytest.mark.parametrize("field,value,status", [
    ("T", 0, INVALID), ("d", -128, INVALID), ("K", 9, INVALID), ("M_tile", 0, INVALID),
    ("dtype", 5, INVALID), ("mode", 5, INVALID), ("mode", -1, INVALID), ("K", 33, UNSUPPORTED),
    ("d", 192, UNSUPPORTED), ("n", 96, UNSUPPORTED), ("n", 640, UNSUPPORTED),
    ("E", 2048, UNSUPPORTED), ("M_tile", 4096, UNSUPPORTED), ("T", 1 << 26, UNSUPPORTED),
])
def test_invalid_problems(field, value, status):
    p = moe.problem(256, 128, 64, 8, 2, 16)
    if field == "K" and value == 33:
        p.E = 64
    setattr(p, field, value)
    s = moe.Sizes()
    assert moe.lib().moe_sizes(ctypes.byref(p), ctypes.byref(s)) == status


@pytest.mark.parametrize("dims,what", [
    # one expert of W1 (d x 2n bf16) past 4 GiB: d = 2^22, n = 512
    ((2, 1 << 22, 512, 2, 1, 16), "W1 expert"),
    # the router's padded dlogits copy (T x ceil(E/128)*128 bf16) past 4 GiB,
    # with every activation array below it: T = 2.2M, d = 128, n = 64,
    # E = 1024, K = 1
    ((2_200_000, 128, 64, 1024, 1, 16), "router dl copy"),
    # logits (T x E fp32) past 4 GiB
    ((1_100_000, 128, 64, 1024, 1, 16), "logits"),
])
def test_byte_extent_limits(dims, what):
    p = moe.problem(*dims, mode="tc")
    s = moe.Sizes()
    assert moe.lib().moe_sizes(ctypes.byref(p), ctypes.byref(s)) == UNSUPPORTED, what


def test_extent_limit_is_tight():
    # just below the logits limit (T E 4 bytes <= 4 GiB - 1) the problem is
    # accepted
    T = (1 << 32) // (4 * 1024) - 1
    p = moe.problem(T, 128, 64, 1024, 1, 16, mode="tc")
    s = moe.Sizes()
    assert moe.lib().moe_sizes(ctypes.byref(p), ctypes.byref(s)) == OK


def _routing(ptr=FAKE):
    return moe.RoutingStruct(*([ptr] * len(moe.ROUTING_FIELDS)))


def test_route_validation_before_launch():
    L = moe.lib()
    p = moe.problem(256, 128, 64, 8, 2, 16)
    need = moe.sizes(p).ws_route
    r = _routing()
    rr = ctypes.byref(r)
    assert L.moe_route(ctypes.byref(p), None, None, rr, FAKE, need, None, None) == INVALID
    assert L.moe_route(ctypes.byref(p), FAKE + 4, None, rr, FAKE, need, None, None) == INVALID
    assert L.moe_route(ctypes.byref(p), FAKE, None, ctypes.byref(_routing(0)), FAKE, need, None,
                       None) == INVALID
    assert L.moe_route(ctypes.byref(p), FAKE, None, rr, FAKE, need - 1, None,
                       None) == WORKSPACE
    assert L.moe_route(None, FAKE, None, rr, FAKE, need, None, None) == INVALID


def test_stochastic_rounding_needs_draws():
    L = moe.lib()
    p = moe.problem(256, 128, 64, 8, 2, 16, mode="tr_stochastic")
    need = moe.sizes(p).ws_route
    rr = ctypes.byref(_routing())
    assert L.moe_route(ctypes.byref(p), FAKE, None, rr, FAKE, need, None, None) == INVALID
    assert L.moe_route(ctypes.byref(p), FAKE, FAKE + 2, rr, FAKE, need, None, None) == INVALID
    # with valid draws the next check is the workspace size (nothing is
    # launched); the other modes never look at the draws
    assert L.moe_route(ctypes.byref(p), FAKE, FAKE, rr, FAKE, need - 1, None, None) == WORKSPACE
    for mode in ("tr_up", "tr_down"):
        q = moe.problem(256, 128, 64, 8, 2, 16, mode=mode)
        assert L.moe_route(ctypes.byref(q), FAKE, None, rr, FAKE, need - 1, None,
                           None) == WORKSPACE


def test_fwd_bwd_validation_before_launch():
    L = moe.lib()
    p = moe.problem(256, 128, 64, 8, 2, 16)
    s = moe.sizes(p)
    r = _routing()
    args = [FAKE] * 3
    assert L.moe_fwd(ctypes.byref(p), *args, ctypes.byref(r), FAKE, FAKE, FAKE, s.ws_fwd - 1,
                     None, None) == WORKSPACE
    assert L.moe_fwd(ctypes.byref(p), None, FAKE, FAKE, ctypes.byref(r), FAKE, FAKE, FAKE,
                     s.ws_fwd, None, None) == INVALID
    assert L.moe_bwd(ctypes.byref(p), *([FAKE] * 5), ctypes.byref(r), FAKE, FAKE, FAKE, FAKE,
                     FAKE, s.ws_bwd - 1, None, None) == WORKSPACE
    assert L.moe_bwd(ctypes.byref(p), *([FAKE] * 5), ctypes.byref(r), FAKE, FAKE, FAKE, FAKE + 8,
                     FAKE, s.ws_bwd, None, None) == INVALID
    bad = moe.problem(256, 128, 64, 8, 2, 16)
    bad.n = 100
    assert L.moe_bwd(ctypes.byref(bad), *([FAKE] * 5), ctypes.byref(r), FAKE, FAKE, FAKE, FAKE,
                     FAKE, s.ws_bwd, None, None) == UNSUPPORTED


def test_null_trace_event_rejected():
    L = moe.lib()
    p = moe.problem(256, 128, 64, 8, 2, 16)
    need = moe.sizes(p).ws_route
    ev = (ctypes.c_void_p * 7)(*([FAKE] * 6 + [None]))
    tr = moe.Trace(ev, 7)
    assert L.moe_route(ctypes.byref(p), FAKE, None, ctypes.byref(_routing()), FAKE, need, None,
                       ctypes.byref(tr)) == INVALID


def test_gate_bwd_validation_before_launch():
    L = moe.lib()
    p = moe.problem(256, 128, 64, 8, 2, 16)
    rr = ctypes.byref(_routing())
    assert L.moe_gate_bwd(ctypes.byref(p), None, FAKE, rr, FAKE, None, None) == INVALID
    assert L.moe_gate_bwd(ctypes.byref(p), FAKE, FAKE + 4, rr, FAKE, None, None) == INVALID
    assert L.moe_gate_bwd(ctypes.byref(p), FAKE, FAKE, ctypes.byref(_routing(0)), FAKE, None,
                          None) == INVALID
    assert L.moe_gate_bwd(ctypes.byref(p), FAKE, FAKE, rr, None, None, None) == INVALID
    bad = moe.problem(256, 128, 64, 8, 2, 16)
    bad.K = 9
    assert L.moe_gate_bwd(ctypes.byref(bad), FAKE, FAKE, rr, FAKE, None, None) == INVALID


def test_router_validation_before_launch():
    L = moe.lib()
    p = moe.problem(256, 128, 64, 8, 2, 16)
    s = moe.sizes(p)
    assert s.ws_router > 0
    assert L.moe_router_fwd(ctypes.byref(p), None, FAKE, FAKE, None, None) == INVALID
    assert L.moe_router_fwd(ctypes.byref(p), FAKE, FAKE, FAKE + 4, None, None) == INVALID
    rr = ctypes.byref(_routing())
    args = [FAKE] * 4
    assert L.moe_router_bwd(ctypes.byref(p), *args, rr, FAKE, FAKE, FAKE, FAKE,
                            s.ws_router - 1, None, None) == WORKSPACE
    assert L.moe_router_bwd(ctypes.byref(p), *args, ctypes.byref(_routing(0)), FAKE, FAKE,
                            FAKE, FAKE, s.ws_router, None, None) == INVALID
    assert L.moe_router_bwd(ctypes.byref(p), *args, rr, None, FAKE, FAKE, FAKE, s.ws_router,
                            None, None) == INVALID


def test_route_noalloc_rejects_before_any_hip_call():
    # the fixed scratch holds 48 MiB: a routing workspace beyond it is refused
    # with MOE_ERR_WORKSPACE, and bad arguments as moe_route refuses them,
    # all before the library touches the device
    L = moe.lib()
    L.moe_route_noalloc.argtypes = [ctypes.POINTER(moe.Problem), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.POINTER(moe.RoutingStruct),
                                    ctypes.c_void_p, ctypes.c_void_p]
    rr = ctypes.byref(_routing())
    big = moe.problem(16384, 128, 64, 512, 2, 16)  # keys alone: 512 * 16384 * 8 = 64 MiB
    assert moe.sizes(big).ws_route > 48 << 20
    assert L.moe_route_noalloc(ctypes.byref(big), FAKE, None, rr, None, None) == WORKSPACE
    p = moe.problem(16384, 1536, 256, 128, 8, 128)
    assert moe.sizes(p).ws_route <= 48 << 20
    assert L.moe_route_noalloc(ctypes.byref(p), None, None, rr, None, None) == INVALID
    assert L.moe_route_noalloc(ctypes.byref(p), FAKE, None, ctypes.byref(_routing(0)), None,
                               None) == INVALID
    st = moe.problem(256, 128, 64, 8, 2, 16, mode="tr_stochastic")
    assert L.moe_route_noalloc(ctypes.byref(st), FAKE, None, rr, None, None) == INVALID
    bad = moe.problem(256, 128, 64, 8, 2, 16)
    bad.K = 9
    assert L.moe_route_noalloc(ctypes.byref(bad), FAKE, None, rr, None, None) == INVALID
