"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Routing metadata must match bit for bit; O, dX, dW1, dW2 and dS must agree
within a relative Frobenius error of 1e-2 for bf16 inputs and 1e-5 for fp32
inputs (the fp32 bound is a reading: the layer's arithmetic is fp32 with fp32
accumulation, whose rounding error at these sizes is ~1e-6).

Shapes: the tiny and small layers (and a few extra ragged / edge shapes) are
checked element by element against the full oracle; the three large layers
are run at full size in the launch configuration the benchmark uses, with
routing compared in full and the other outputs on sampled tokens, slots and
experts that the oracle evaluates one by one.
"""
import sys

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import moe
from fine_grained_mixture_amd.inputs import (SHAPES, LayerShape, make_layer_inputs,
                                             make_round_rand, round_rand_tensor)
from oracle import moe_oracle as orc

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
}
TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-5}
ORC_MODE = {"tc": orc.TC, "tr": orc.TR, "tr_up": orc.TR_UP, "tr_down": orc.TR_DOWN,
            "tr_stochastic": orc.TR_STOCHASTIC}


def oracle_route(logits, shape, mode):
    return orc.route(logits, shape.K, shape.M, ORC_MODE[mode], make_round_rand(shape.E, 0))
INT_FIELDS = ("tc_counts", "counts", "expert_offsets")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def shape_of(name):
    return SHAPES[name] if name in SHAPES else EXTRA[name]


def rel_fro(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return np.linalg.norm(got - want) / (den if den > 0 else 1.0)


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
    S = ref.S
    O, c = orc.forward(a["X"], a["W1"], a["W2"], ref)
    dX, dW1, dW2, dS = orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], ref)
    tol = TOL[dtype]
    errs = {
        "H": rel_fro(g["H"][:S], c["H"]), "O": rel_fro(g["O"], O), "dX": rel_fro(g["dX"], dX),
        "dW1": rel_fro(g["dW1"], dW1), "dW2": rel_fro(g["dW2"], dW2),
        "dS": rel_fro(g["dS"][:S], dS),
    }
    log(f"[parity] {name} {dtype} {mode}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)
    # tokens that lost every expert under rounding get exact zeros
    empty = np.nonzero(np.diff(ref.token_offsets) == 0)[0]
    assert np.all(g["O"].numpy()[empty] == 0) and np.all(g["dX"].numpy()[empty] == 0)
    # experts that hold no token get exact zero weight gradients
    idle = np.nonzero(ref.counts == 0)[0]
    assert np.all(g["dW1"].numpy()[idle] == 0) and np.all(g["dW2"].numpy()[idle] == 0)


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
               ("high_sparsity", "tr"), ("high_sparsity", "tc")]


@pytest.mark.parametrize("name,mode", LARGE_CASES)
def test_parity_full_size_sampled(name, mode):
    shape = SHAPES[name]
    log(f"[parity-full] {name} {mode}: T={shape.T} d={shape.d} n={shape.n} E={shape.E} "
        f"K={shape.K} M={shape.M}")
    inp = make_layer_inputs(shape, dtype=torch.bfloat16, seed=0)
    g = run_gpu(shape, torch.bfloat16, mode, inp)
    logits = inp["logits"].numpy()
    ref = oracle_route(logits, shape, mode)
    check_routing(g, ref, shape)
    a = np_inputs(inp)
    rng = np.random.default_rng(123)
    cnt = np.diff(ref.token_offsets)
    toks = set(rng.choice(shape.T, 48, replace=False).tolist())
    toks |= {0, shape.T - 1, int(np.argmax(cnt))}
    toks |= set(np.nonzero(cnt == 0)[0][:4].tolist())
    toks = sorted(toks)
    errs = {
        "O": rel_fro(g["O"].numpy()[toks], orc.forward_tokens(toks, a["X"], a["W1"], a["W2"], ref)),
        "dX": rel_fro(g["dX"].numpy()[toks],
                      orc.dx_tokens(toks, a["X"], a["W1"], a["W2"], a["dO"], ref)),
    }
    slots = np.unique(np.concatenate([rng.choice(ref.S, 256, replace=False), [0, ref.S - 1]]))
    errs["dS"] = rel_fro(g["dS"].numpy()[slots],
                         orc.slot_grads(slots, a["X"], a["W1"], a["W2"], a["dO"], ref)[0])
    live = np.nonzero(ref.counts > 0)[0]
    experts = {int(np.argmax(ref.counts)), int(live[np.argmin(ref.counts[live])]),
               int(rng.choice(live))}
    w1g, w1r, w2g, w2r = [], [], [], []
    for e in sorted(experts):
        r1, r2 = orc.expert_weight_grads(e, a["X"], a["W1"], a["W2"], a["dO"], ref)
        w1g.append(g["dW1"][e].numpy()); w1r.append(r1)
        w2g.append(g["dW2"][e].numpy()); w2r.append(r2)
    errs["dW1"] = rel_fro(np.stack(w1g), np.stack(w1r))
    errs["dW2"] = rel_fro(np.stack(w2g), np.stack(w2r))
    log(f"[parity-full] {name} {mode}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[torch.bfloat16], (k, v)
    idle = np.nonzero(ref.counts == 0)[0]
    assert np.all(g["dW1"].numpy()[idle] == 0) and np.all(g["dW2"].numpy()[idle] == 0)
    empty = np.nonzero(cnt == 0)[0]
    assert np.all(g["O"].numpy()[empty] == 0) and np.all(g["dX"].numpy()[empty] == 0)
