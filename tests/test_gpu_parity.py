"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Routing metadata must match bit for bit.  O, H, dX, dW1, dW2 and dS are
compared element by element in full, each against two bounds
(tests/parity_checks.py): a relative Frobenius error of 1e-2 for bf16 inputs
(1e-5 for fp32: the layer's arithmetic is fp32 with fp32 accumulation, whose
rounding error at these sizes is ~1e-6), and a per-row bound that a single
wrong slot cannot pass.

Shapes: the tiny and small layers, extra ragged / edge shapes (T past 32768
tokens, K = 32, M_tile = 1024, E = 1024, non-finite logits, ...), and the
three large layers at full size in the launch configuration the benchmark
uses (7B under token choice, nearest and stochastic rounding; high
granularity and high sparsity under token choice and nearest rounding).
"""
import sys

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import moe
from fine_grained_mixture_amd.inputs import (SHAPES, LayerShape, make_layer_inputs,
                                             make_round_rand, round_rand_tensor)
from oracle import moe_oracle as orc
from tests.parity_checks import check

pytestmark = pytest.mark.gpu

EXTRA = {
    # T not a multiple of 32, d not a multiple of 256, n = 128
    "ragged": LayerShape("ragged", 1000, 384, 128, 24, 3, 32, "fan_in", "normal_bias"),
    # n = 384 (the 64-row dH tile), skewed load, empty experts under TR
    "wide_n": LayerShape("wide_n", 2048, 512, 384, 32, 4, 64, "fan_in", "zipf_bias"),
    # K = E: every expert holds every token
    "all_experts": LayerShape("all_experts", 300, 128, 64, 4, 4, 16, "fan_in", "iid"),
    # fewer tokens than one bitmap word, K = 1
    "few_tokens": LayerShape("few_tokens", 20, 128, 64, 8, 1, 16, "tiny", "router"),
    # M_tile = 1: token rounding is token choice
    "m1": LayerShape("m1", 512, 256, 64, 16, 2, 1, "fan_in", "iid"),
    # n = 512 (granularity d/n = 2 at d = 1024): the 64 x 512 dH tile
    "n512": LayerShape("n512", 1024, 1024, 512, 16, 2, 64, "fan_in", "normal_bias"),
    # a single token
    "one_token": LayerShape("one_token", 1, 128, 64, 4, 2, 16, "fan_in", "iid"),
    # one expert holding every token (E = K = 1: a dense SwiGLU MLP)
    "one_expert": LayerShape("one_expert", 200, 256, 128, 1, 1, 32, "fan_in", "iid"),
    # an M_tile that is not a power of two
    "tile48": LayerShape("tile48", 900, 256, 128, 12, 3, 48, "fan_in", "normal_bias"),
    # the largest expert count (E = 1024), few tokens per expert
    "e1024": LayerShape("e1024", 512, 128, 64, 1024, 4, 16, "fan_in", "zipf_bias"),
    # E = 1024 with many tokens: the select grid's extra scan workgroup and
    # every expert's own offset sum run over the full 1024 counts
    "big_bitmap": LayerShape("big_bitmap", 8192, 128, 64, 1024, 4, 16, "fan_in", "iid"),
    # more tokens than the selection keeps in registers (T > 32768): the
    # selection reads its keys from memory in every radix pass
    "long_t": LayerShape("long_t", 40000, 128, 64, 64, 2, 16, "fan_in", "normal_bias"),
    # the largest K and the largest M_tile the library takes
    "k32": LayerShape("k32", 512, 128, 64, 64, 32, 16, "fan_in", "iid"),
    "m1024": LayerShape("m1024", 2048, 128, 64, 8, 4, 1024, "fan_in", "iid"),
    # launch boundaries of the persistent kernels: dX-tilde persistent with its
    # fewest slabs (2n / 64 = 2) at the widest d it takes (2048) while the
    # down-projection, with one slab, runs the per-tile kernel ...
    "d2048_n64": LayerShape("d2048_n64", 700, 2048, 64, 16, 2, 64, "fan_in", "normal_bias"),
    # ... and d past 2048: dX-tilde per tile, the down-projection persistent
    "d2304": LayerShape("d2304", 640, 2304, 128, 8, 2, 32, "fan_in", "iid"),
    # the persistent weight-gradient kernels with more output tiles per item
    # than workgroups per XCD (48 for dW1 on 256 x 256 tiles, 48 for dW2 on
    # 128 x 256), so one workgroup gets several tiles of an item
    "d4096_n384": LayerShape("d4096_n384", 400, 4096, 384, 6, 2, 32, "fan_in", "normal_bias"),
}
KIND = {torch.bfloat16: "bf16", torch.float32: "f32"}
ORC_MODE = {"tc": orc.TC, "tr": orc.TR, "tr_up": orc.TR_UP, "tr_down": orc.TR_DOWN,
            "tr_stochastic": orc.TR_STOCHASTIC}


def oracle_route(logits, shape, mode):
    return orc.route(logits, shape.K, shape.M, ORC_MODE[mode], make_round_rand(shape.E, 0))
INT_FIELDS = ("tc_counts", "counts", "expert_offsets")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def shape_of(name):
    return SHAPES[name] if name in SHAPES else EXTRA[name]


def run_gpu(shape, dtype, mode, inp):
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, dtype, mode)
    dev = torch.device("cuda", 0)
    X, W1, W2, lg, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "logits", "dO"))
    rr = round_rand_tensor(make_round_rand(shape.E, 0)).to(dev)
    rt = moe.route(p, lg, round_rand=rr)
    O, H = moe.forward(p, X, W1, W2, rt)
    dX, dW1, dW2, dS = moe.backward(p, dO, X, H, W1, W2, rt)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in rt.tensors.items()}
    out.update(O=O.float().cpu(), H=H.float().cpu(), dX=dX.float().cpu(), dW1=dW1.float().cpu(),
               dW2=dW2.float().cpu(), dS=dS.cpu())
    return out


def check_routing(g, ref: orc.Routing, shape):
    T, E, K = shape.T, shape.E, shape.K
    S = ref.S
    assert int(g["totals"][0]) == S
    for f in INT_FIELDS:
        np.testing.assert_array_equal(g[f].numpy(), getattr(ref, f), err_msg=f)
    np.testing.assert_array_equal(g["topk_ids"].numpy().reshape(T, K), ref.topk_ids)
    np.testing.assert_array_equal(g["slot_token"].numpy()[:S], ref.slot_token)
    np.testing.assert_array_equal(g["token_offsets"].numpy(), ref.token_offsets)
    np.testing.assert_array_equal(g["token_slots"].numpy()[:S], ref.token_slots)
    # gate weights: fp32 rounding of the same fp64 probability
    np.testing.assert_allclose(g["slot_weight"].numpy()[:S], ref.slot_weight.astype(np.float32),
                               rtol=2.5e-7, atol=0)
    order = np.lexsort((np.arange(E), -ref.counts))
    np.testing.assert_array_equal(g["expert_order"].numpy(), order)
    ntiles = -(-ref.counts // moe.TILE_M)
    assert int(g["totals"][1]) == int(ntiles.sum())
    te = np.repeat(np.arange(E), ntiles)
    tr = np.concatenate([ref.expert_offsets[e] + moe.TILE_M * np.arange(ntiles[e])
                         for e in range(E)] + [np.zeros(0, np.int64)])
    np.testing.assert_array_equal(g["tile_expert"].numpy()[:len(te)], te)
    np.testing.assert_array_equal(g["tile_row"].numpy()[:len(tr)], tr)


def np_inputs(inp):
    return {k: v.float().numpy() for k, v in inp.items()}


SMALL_CASES = [
    ("tiny", torch.float32, "tc"), ("tiny", torch.float32, "tr"),
    ("tiny", torch.bfloat16, "tc"), ("tiny", torch.bfloat16, "tr"),
    ("small", torch.bfloat16, "tc"), ("small", torch.bfloat16, "tr"),
    ("ragged", torch.bfloat16, "tc"), ("ragged", torch.bfloat16, "tr"),
    ("ragged", torch.float32, "tr"),
    ("wide_n", torch.bfloat16, "tr"), ("wide_n", torch.bfloat16, "tc"),
    ("all_experts", torch.bfloat16, "tr"), ("few_tokens", torch.bfloat16, "tr"),
    ("few_tokens", torch.float32, "tc"), ("m1", torch.bfloat16, "tr"),
    # the other token-rounding subroutines
    ("small", torch.bfloat16, "tr_up"), ("small", torch.bfloat16, "tr_down"),
    ("small", torch.bfloat16, "tr_stochastic"), ("tiny", torch.float32, "tr_stochastic"),
    ("wide_n", torch.bfloat16, "tr_up"), ("ragged", torch.bfloat16, "tr_down"),
    ("n512", torch.bfloat16, "tr"), ("n512", torch.float32, "tc"),
    # edge shapes
    ("one_token", torch.bfloat16, "tr"), ("one_token", torch.float32, "tc"),
    ("one_expert", torch.bfloat16, "tr"), ("one_expert", torch.bfloat16, "tc"),
    ("tile48", torch.bfloat16, "tr"), ("tile48", torch.bfloat16, "tr_stochastic"),
    ("e1024", torch.bfloat16, "tr"), ("e1024", torch.bfloat16, "tc"),
    ("big_bitmap", torch.bfloat16, "tr"),
]


def check_layer(g, ref, O, H, grads, kind, tag):
    """Every element of O, H, dX, dW1, dW2 and dS against the oracle, plus
    exact zeros where the layer defines them."""
    S = ref.S
    dX, dW1, dW2, dS = grads
    n2 = H.shape[1]
    out = {}
    for name, got, want in (("O", g["O"], O), ("H", g["H"][:S], H), ("dX", g["dX"], dX),
                            ("dW1", g["dW1"], dW1), ("dW2", g["dW2"], dW2),
                            ("dS", g["dS"][:S], dS)):
        out[name] = check(name, np.asarray(got), want, kind)
    log(f"[parity] {tag}: " + " ".join(f"{k}={v[0]:.2e}/{v[1]:.2e}" for k, v in out.items())
        + " (Frobenius/worst row)")
    # tokens that lost every expert under rounding get exact zeros
    empty = np.nonzero(np.diff(ref.token_offsets) == 0)[0]
    assert np.all(g["O"].numpy()[empty] == 0) and np.all(g["dX"].numpy()[empty] == 0)
    # experts that hold no token get exact zero weight gradients
    idle = np.nonzero(ref.counts == 0)[0]
    assert np.all(g["dW1"].numpy()[idle] == 0) and np.all(g["dW2"].numpy()[idle] == 0)
    assert n2 == g["H"].shape[1]


def nonfinite_logits(logits, seed=7):
    """Logits with NaN, +inf and -inf planted: about 2% of the entries, a
    few whole rows of NaN, and rows where several experts tie at +inf."""
    lg = logits.clone()
    rng = np.random.default_rng(seed)
    T, E = lg.shape
    mask = rng.random((T, E)) < 0.02
    vals = rng.choice(np.array([np.nan, np.inf, -np.inf], np.float32), size=(T, E))
    a = lg.numpy()
    a[mask] = vals[mask]
    a[rng.choice(T, 5, replace=False)] = np.nan
    for t in rng.choice(T, 5, replace=False):
        a[t, rng.choice(E, 3, replace=False)] = np.inf
    return lg


SMALL_CASES = SMALL_CASES + [
    ("d2048_n64", torch.bfloat16, "tr"), ("d2304", torch.bfloat16, "tc"),
    ("d4096_n384", torch.bfloat16, "tr"),
    ("long_t", torch.bfloat16, "tr"), ("long_t", torch.bfloat16, "tc"),
    ("long_t", torch.bfloat16, "tr_stochastic"),
    ("k32", torch.bfloat16, "tr"), ("k32", torch.float32, "tc"),
    ("m1024", torch.bfloat16, "tr"), ("m1024", torch.bfloat16, "tr_up"),
]


@pytest.mark.parametrize("name,dtype,mode", SMALL_CASES)
def test_parity_full_oracle(name, dtype, mode):
    shape = shape_of(name)
    log(f"[parity] {name} {dtype} {mode}: T={shape.T} d={shape.d} n={shape.n} "
        f"E={shape.E} K={shape.K} M={shape.M}")
    inp = make_layer_inputs(shape, dtype=dtype, seed=0)
    g = run_gpu(shape, dtype, mode, inp)
    a = np_inputs(inp)
    ref = oracle_route(a["logits"], shape, mode)
    check_routing(g, ref, shape)
    O, c = orc.forward(a["X"], a["W1"], a["W2"], ref)
    grads = orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], ref)
    check_layer(g, ref, O, c["H"], grads, KIND[dtype], f"{name} {dtype} {mode}")


@pytest.mark.parametrize("mode", ["tr", "tc", "tr_stochastic"])
def test_parity_nonfinite_logits(mode):
    # NaN / +inf / -inf logits: routing and gates follow the stated rule on
    # both sides (non-finite values replaced by -FLT_MAX / +FLT_MAX first)
    shape = EXTRA["ragged"]
    log(f"[parity] nonfinite logits {mode}: T={shape.T} E={shape.E} K={shape.K}")
    inp = make_layer_inputs(shape, dtype=torch.bfloat16, seed=0)
    inp["logits"] = nonfinite_logits(inp["logits"])
    assert not np.isfinite(inp["logits"].numpy()).all()
    g = run_gpu(shape, torch.bfloat16, mode, inp)
    a = np_inputs(inp)
    ref = oracle_route(a["logits"], shape, mode)
    check_routing(g, ref, shape)
    O, c = orc.forward(a["X"], a["W1"], a["W2"], ref)
    grads = orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], ref)
    check_layer(g, ref, O, c["H"], grads, "bf16", f"nonfinite {mode}")


def test_layer_autograd_matches_explicit_calls():
    # moe_layer wires route -> fwd and bwd through autograd; with stochastic
    # rounding (draws as an input) it must reproduce the explicit C-ABI calls
    # bit for bit.
    shape = SHAPES["small"]
    dt = torch.bfloat16
    inp = make_layer_inputs(shape, dtype=dt, seed=3)
    dev = torch.device("cuda", 0)
    X, W1, W2, lg, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "logits", "dO"))
    rr = round_rand_tensor(make_round_rand(shape.E, 3)).to(dev)
    Xa, W1a, W2a = (t.clone().requires_grad_(True) for t in (X, W1, W2))
    O = moe.moe_layer(Xa, W1a, W2a, lg, shape.K, shape.M, "tr_stochastic", round_rand=rr)
    O.backward(dO)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, dt, "tr_stochastic")
    rt = moe.route(p, lg, round_rand=rr)
    O2, H = moe.forward(p, X, W1, W2, rt)
    dX, dW1, dW2, dS = moe.backward(p, dO, X, H, W1, W2, rt)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    for got, want in ((Xa.grad, dX), (W1a.grad, dW1), (W2a.grad, dW2)):
        assert torch.equal(got, want)


def test_deterministic():
    shape = SHAPES["small"]
    inp = make_layer_inputs(shape, dtype=torch.bfloat16, seed=1)
    a = run_gpu(shape, torch.bfloat16, "tr", inp)
    b = run_gpu(shape, torch.bfloat16, "tr", inp)
    S = int(a["totals"][0])
    assert int(b["totals"][0]) == S
    for k in ("O", "dX", "dW1", "dW2"):
        assert torch.equal(a[k], b[k]), k
    # slot-indexed outputs are defined on rows [0, S) only
    for k in ("slot_token", "token_slots", "dS"):
        assert torch.equal(a[k][:S], b[k][:S]), k


LARGE_CASES = [("7b", "tr"), ("7b", "tc"), ("7b", "tr_stochastic"), ("high_g", "tr"),
               ("high_g", "tc"), ("high_sparsity", "tr"), ("high_sparsity", "tc")]


@pytest.fixture(scope="module")
def large_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()  # one full-size layer at a time in host memory
            inp = make_layer_inputs(SHAPES[name], dtype=torch.bfloat16, seed=0)
            cache[name] = (inp, np_inputs(inp))
        return cache[name]
    return get


@pytest.mark.parametrize("name,mode", LARGE_CASES)
def test_parity_full_size(name, mode, large_inputs):
    # the full-size layers, in the benchmark's launch configuration, against
    # the whole fp64 oracle: every element of every output
    shape = SHAPES[name]
    log(f"[parity-full] {name} {mode}: T={shape.T} d={shape.d} n={shape.n} E={shape.E} "
        f"K={shape.K} M={shape.M}")
    inp, a = large_inputs(name)
    g = run_gpu(shape, torch.bfloat16, mode, inp)
    ref = oracle_route(a["logits"], shape, mode)
    check_routing(g, ref, shape)
    O, c = orc.forward(a["X"], a["W1"], a["W2"], ref)
    H = c.pop("H")
    del c  # A and Y are not compared; free them before the backward
    grads = orc.backward_minimal(a["dO"], a["X"], H, a["W1"], a["W2"], ref)
    check_layer(g, ref, O, H, grads, "bf16", f"{name} {mode}")


def test_layer_autograd_logits_grad():
    # logits that require a gradient get dlogits from the gate's softmax
    # backward (moe_gate_bwd), against the oracle's chain route -> forward ->
    # minimal backward -> gate backward on the same logits
    shape = SHAPES["small"]
    dt = torch.bfloat16
    inp = make_layer_inputs(shape, dtype=dt, seed=2)
    dev = torch.device("cuda", 0)
    X, W1, W2, dO = (inp[k].to(dev).requires_grad_(k != "dO") for k in ("X", "W1", "W2", "dO"))
    lg = inp["logits"].to(dev).requires_grad_(True)
    O = moe.moe_layer(X, W1, W2, lg, shape.K, shape.M, "tr")
    O.backward(dO)
    torch.cuda.synchronize()
    a = np_inputs(inp)
    ref = oracle_route(a["logits"], shape, "tr")
    _, c = orc.forward(a["X"], a["W1"], a["W2"], ref)
    dS = orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], ref)[3]
    dl, _, _ = orc.router_backward(dS, ref, a["X"], np.zeros((shape.E, shape.d)), a["logits"])
    fro, mx, _ = check("dlogits", lg.grad.cpu().numpy(), dl, "bf16")
    log(f"[parity] autograd dlogits: {fro:.2e}/{mx:.2e}")
    # without requires_grad the logits get no gradient and nothing extra is kept
    lg2 = inp["logits"].to(dev)
    O2 = moe.moe_layer(X, W1, W2, lg2, shape.K, shape.M, "tr")
    assert O2.grad_fn.saved_tensors[4] is None
