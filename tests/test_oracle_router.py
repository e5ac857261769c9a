"""Pins for the oracle's router: logits = X Wr^T and its backward.

Independent checks: a pure-Python dot product for the logits; torch autograd
(fp64, CPU) and central finite differences for the backward with the routing
held fixed; the softmax-Jacobian identity (each row of dlogits sums to zero);
and an end-to-end check that the router backward of the layer's own dS is the
derivative of L = <dO, O> with respect to the logits.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc


def _problem(seed, T=40, d=16, n=8, E=6, K=2, M=4, mode=orc.TR):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) / np.sqrt(d)
    W1 = rng.standard_normal((E, d, 2 * n)) / np.sqrt(d)
    W2 = rng.standard_normal((E, n, d)) / np.sqrt(n)
    dO = rng.standard_normal((T, d))
    logits = orc.router_logits(X, Wr).astype(np.float32)
    rt = orc.route(logits, K, M, mode)
    return X, Wr, W1, W2, dO, logits, rt


def test_router_logits_brute_force():
    rng = np.random.default_rng(0)
    X, Wr = rng.standard_normal((5, 7)), rng.standard_normal((3, 7))
    got = orc.router_logits(X, Wr)
    for t in range(5):
        for e in range(3):
            assert got[t, e] == pytest.approx(sum(X[t, i] * Wr[e, i] for i in range(7)),
                                              rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("mode", [orc.TC, orc.TR])
def test_router_backward_matches_autograd(mode):
    X, Wr, W1, W2, dO, logits, rt = _problem(1, mode=mode)
    dS = np.random.default_rng(2).standard_normal(rt.S)
    dl, dWr, dXr = orc.router_backward(dS, rt, X, Wr, logits)
    # autograd through l -> softmax -> s[kept], routing fixed; logits
    # recomputed in fp64 from X and Wr
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(Wr, requires_grad=True)
    lt = Xt @ Wt.T
    p = torch.softmax(lt, dim=1)
    s = p[torch.tensor(rt.slot_token), torch.tensor(rt.slot_expert)]
    L = (torch.tensor(dS) * s).sum()
    gl, gW, gX = torch.autograd.grad(L, (lt, Wt, Xt))
    # the oracle evaluates p from the fp32 logits; compare at that precision
    np.testing.assert_allclose(dl, gl.numpy(), rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(dWr, gW.numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dXr, gX.numpy(), rtol=1e-5, atol=1e-6)


def test_router_backward_rows_sum_to_zero_and_empty_tokens():
    X, Wr, W1, W2, dO, logits, rt = _problem(3, M=8)
    dS = np.random.default_rng(4).standard_normal(rt.S)
    dl, _, _ = orc.router_backward(dS, rt, X, Wr, logits)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    empty = np.nonzero(np.diff(rt.token_offsets) == 0)[0]
    assert np.all(dl[empty] == 0.0)


def test_router_backward_finite_differences():
    X, Wr, W1, W2, dO, logits, rt = _problem(5, T=12, d=6, E=4)
    dS = np.random.default_rng(6).standard_normal(rt.S)
    _, dWr, _ = orc.router_backward(dS, rt, X, Wr, orc.router_logits(X, Wr))

    def loss(W):
        p = orc.softmax_probs(orc.router_logits(X, W))
        return float((dS * p[rt.slot_token, rt.slot_expert]).sum())

    h = 1e-6
    for e in range(4):
        for i in range(6):
            Wp, Wm = Wr.copy(), Wr.copy()
            Wp[e, i] += h
            Wm[e, i] -= h
            fd = (loss(Wp) - loss(Wm)) / (2 * h)
            assert dWr[e, i] == pytest.approx(fd, rel=1e-6, abs=1e-8)


def test_layer_dS_drives_router_gradient():
    # d<dO, O>/dlogits (routing fixed) equals the router backward of the
    # layer's own dS: central differences of the full forward in the logits.
    X, Wr, W1, W2, dO, logits, rt = _problem(7, T=16, d=8, n=4, E=4, K=2, M=2)
    logits64 = orc.router_logits(X, Wr)
    # the gate weights of the routing are those of the fp64 logits, so that
    # the same function is differentiated below
    p64 = orc.softmax_probs(logits64)
    rt = orc.Routing(rt.topk_ids, rt.tc_counts, rt.counts, rt.expert_offsets, rt.slot_token,
                     rt.slot_expert, p64[rt.slot_token, rt.slot_expert], rt.token_offsets,
                     rt.token_slots, p64)
    _, cache = orc.forward(X, W1, W2, rt)
    _, _, _, dS = orc.backward_minimal(dO, X, cache["H"], W1, W2, rt)
    dl, _, _ = orc.router_backward(dS, rt, X, Wr, logits64)

    def loss(lg):
        r2 = orc.Routing(rt.topk_ids, rt.tc_counts, rt.counts, rt.expert_offsets,
                         rt.slot_token, rt.slot_expert,
                         orc.softmax_probs(lg)[rt.slot_token, rt.slot_expert],
                         rt.token_offsets, rt.token_slots, orc.softmax_probs(lg))
        return float((dO * orc.forward(X, W1, W2, r2)[0]).sum())

    h = 1e-6
    for t in range(0, 16, 3):
        for e in range(4):
            lp, lm = logits64.copy(), logits64.copy()
            lp[t, e] += h
            lm[t, e] -= h
            assert dl[t, e] == pytest.approx((loss(lp) - loss(lm)) / (2 * h), rel=1e-5, abs=1e-8)
