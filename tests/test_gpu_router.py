"""GPU parity of the router (moe_router_fwd / moe_router_bwd) against the
fp64 oracle, through the C ABI.

Forward: logits = X Wr^T within a relative Frobenius error of 1e-5 (fp32
accumulation of products that are exact in fp32).  Backward: the whole chain
route -> fwd -> bwd -> router bwd on the GPU against the same chain in the
oracle, on the same logits (the oracle's fp64 X Wr^T rounded to fp32, so that
both sides route identically): dlogits, dWr and the total dX (experts' share
plus the router's) within the layer's tolerances (1e-2 bf16, 1e-5 fp32).
"""
import sys

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import moe
from fine_grained_mixture_amd.inputs import SHAPES, make_layer_inputs, make_router_weight
from oracle import moe_oracle as orc
from tests.parity_checks import check
from tests.test_gpu_parity import KIND, nonfinite_logits, shape_of

pytestmark = pytest.mark.gpu
ORC_MODE = {"tc": orc.TC, "tr": orc.TR}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


FWD_CASES = [("tiny", torch.float32), ("tiny", torch.bfloat16), ("small", torch.bfloat16),
             ("ragged", torch.bfloat16), ("all_experts", torch.bfloat16),
             ("7b", torch.bfloat16), ("high_sparsity", torch.bfloat16)]


@pytest.mark.parametrize("name,dtype", FWD_CASES)
def test_router_fwd_parity(name, dtype):
    shape = shape_of(name)
    log(f"[router-fwd] {name} {dtype}: T={shape.T} d={shape.d} E={shape.E}")
    inp = make_layer_inputs(shape, dtype=dtype, seed=0)
    Wr = make_router_weight(shape, dtype, seed=0)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, dtype, "tr")
    dev = torch.device("cuda", 0)
    lg = moe.router_forward(p, inp["X"].to(dev), Wr.to(dev))
    torch.cuda.synchronize()
    ref = orc.router_logits(inp["X"].double().numpy(), Wr.double().numpy())
    # fp32 result of fp32 accumulation over exact products
    check("logits", lg.cpu().numpy(), ref, "f32")


BWD_CASES = [("tiny", torch.float32, "tr"), ("tiny", torch.bfloat16, "tr"),
             ("small", torch.bfloat16, "tr"), ("small", torch.bfloat16, "tc"),
             ("ragged", torch.bfloat16, "tr"), ("all_experts", torch.bfloat16, "tr"),
             ("7b", torch.bfloat16, "tr")]


@pytest.mark.parametrize("name,dtype,mode", BWD_CASES)
def test_router_bwd_parity(name, dtype, mode):
    shape = shape_of(name)
    log(f"[router-bwd] {name} {dtype} {mode}: T={shape.T} d={shape.d} n={shape.n} "
        f"E={shape.E} K={shape.K} M={shape.M}")
    inp = make_layer_inputs(shape, dtype=dtype, seed=0)
    Wr = make_router_weight(shape, dtype, seed=0)
    a = {k: v.double().numpy() for k, v in inp.items() if k != "logits"}
    Wr64 = Wr.double().numpy()
    logits = orc.router_logits(a["X"], Wr64).astype(np.float32)
    # GPU chain
    dev = torch.device("cuda", 0)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, dtype, mode)
    X, W1, W2, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "dO"))
    lg, Wrd = torch.from_numpy(logits).to(dev), Wr.to(dev)
    rt = moe.route(p, lg)
    O, H = moe.forward(p, X, W1, W2, rt)
    dX, dW1, dW2, dS = moe.backward(p, dO, X, H, W1, W2, rt)
    dl, dWr = moe.router_backward(p, X, Wrd, lg, dS, rt, dX)
    torch.cuda.synchronize()
    # oracle chain
    ref = orc.route(logits, shape.K, shape.M, ORC_MODE[mode])
    _, cache = orc.forward(a["X"], a["W1"], a["W2"], ref)
    dX_ref, _, _, dS_ref = orc.backward_minimal(a["dO"], a["X"], cache["H"], a["W1"], a["W2"],
                                                ref)
    dl_ref, dWr_ref, dXr_ref = orc.router_backward(dS_ref, ref, a["X"], Wr64, logits)
    kind = KIND[dtype]
    dl_g = dl.cpu().numpy()
    check("dlogits", dl_g, dl_ref, kind)
    check("dWr", dWr.float().cpu().numpy(), dWr_ref, kind)
    check("dX", dX.float().cpu().numpy(), dX_ref + dXr_ref, kind)
    # the softmax Jacobian's rows sum to zero
    assert np.abs(dl_g.sum(axis=1)).max() <= 1e-5 * max(1.0, np.abs(dl_g).max())


def test_router_layer_autograd_matches_explicit_calls():
    # The autograd op wires router fwd -> route -> fwd and bwd -> router bwd;
    # it must reproduce the explicit sequence of C-ABI calls bit for bit.
    shape = SHAPES["small"]
    dt = torch.bfloat16
    inp = make_layer_inputs(shape, dtype=dt, seed=2)
    dev = torch.device("cuda", 0)
    X, W1, W2, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "dO"))
    Wr = make_router_weight(shape, dt, seed=2).to(dev)
    Xa, Wra, W1a, W2a = (t.clone().requires_grad_(True) for t in (X, Wr, W1, W2))
    O = moe.moe_router_layer(Xa, Wra, W1a, W2a, shape.K, shape.M, "tr")
    O.backward(dO)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, dt, "tr")
    lg = moe.router_forward(p, X, Wr)
    rt = moe.route(p, lg)
    O2, H = moe.forward(p, X, W1, W2, rt)
    dX, dW1, dW2, dS = moe.backward(p, dO, X, H, W1, W2, rt)
    _, dWr = moe.router_backward(p, X, Wr, lg, dS, rt, dX)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    for got, want in ((Xa.grad, dX), (Wra.grad, dWr), (W1a.grad, dW1), (W2a.grad, dW2)):
        assert torch.equal(got, want)


@pytest.mark.parametrize("name,mode,nonfinite", [("small", "tr", False), ("7b", "tc", False),
                                                 ("ragged", "tr", True)])
def test_gate_bwd_parity(name, mode, nonfinite):
    # moe_gate_bwd alone: dlogits from the slot gradients, on the oracle's own
    # dS (so only the gate's softmax backward is under test)
    shape = shape_of(name)
    log(f"[gate-bwd] {name} {mode} nonfinite={nonfinite}: T={shape.T} E={shape.E}")
    inp = make_layer_inputs(shape, dtype=torch.bfloat16, seed=0)
    if nonfinite:
        inp["logits"] = nonfinite_logits(inp["logits"])
    logits = inp["logits"].numpy()
    ref = orc.route(logits, shape.K, shape.M, ORC_MODE[mode])
    rng = np.random.default_rng(11)
    dS = rng.standard_normal(ref.S).astype(np.float32)
    dl_ref = orc.router_backward(dS, ref, np.zeros((shape.T, 1)), np.zeros((shape.E, 1)),
                                 logits)[0]
    dev = torch.device("cuda", 0)
    p = moe.problem(shape.T, shape.d, shape.n, shape.E, shape.K, shape.M, torch.bfloat16, mode)
    lg = inp["logits"].to(dev)
    rt = moe.route(p, lg)
    dSd = torch.zeros(moe.sizes(p).slot_cap, dtype=torch.float32, device=dev)
    dSd[:ref.S] = torch.from_numpy(dS).to(dev)
    dl = moe.gate_backward(p, lg, dSd, rt)
    torch.cuda.synchronize()
    assert int(rt.totals[0]) == ref.S
    assert np.array_equal(rt.slot_token[:ref.S].cpu().numpy(), ref.slot_token)
    # fp32 softmax and products against fp64: about 1e-6 relative
    fro, mx, _ = check("dlogits", dl.cpu().numpy(), dl_ref, "f32")
    log(f"[gate-bwd] {name}: {fro:.2e}/{mx:.2e}")
