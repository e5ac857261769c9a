"""Pins for the oracle's forward, backward and cost models.

Independent checks: special cases that reduce to a dense SwiGLU MLP or a dense
softmax mixture computed with torch (a different library), central finite
differences, torch.autograd in fp64 on the CPU, the inner-product identities
behind dS (SonicMoE ICLR-2026 notes, key design 2: dS = <dA, A'> in the dH
epilogue), the FLOP count (key design 3: (6 + 12) TnKd) and the arithmetic-
intensity model (background: byte counting of the forward's tensors).
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc


def rand_layer(seed, T, d, n, E, scale=0.5):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d))
    W1 = rng.standard_normal((E, d, 2 * n)) * scale
    W2 = rng.standard_normal((E, n, d)) * scale
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dO = rng.standard_normal((T, d))
    return X, W1, W2, logits, dO


def torch_swiglu_mlp(X, W1, W2):
    h = torch.from_numpy(X) @ torch.from_numpy(W1)
    n = W1.shape[1] // 2
    a = torch.nn.functional.silu(h[:, :n]) * h[:, n:]
    return (a @ torch.from_numpy(W2)).numpy()


def test_single_expert_is_dense_swiglu_mlp():
    X, W1, W2, logits, _ = rand_layer(0, 20, 6, 5, 1)
    rt = orc.route(logits, 1, 4, orc.TC)
    assert np.all(rt.slot_weight == 1.0)
    O, _ = orc.forward(X, W1, W2, rt)
    np.testing.assert_allclose(O, torch_swiglu_mlp(X, W1[0], W2[0]), rtol=1e-12, atol=1e-12)


def test_all_experts_is_dense_softmax_mixture():
    X, W1, W2, logits, _ = rand_layer(1, 15, 6, 4, 3)
    rt = orc.route(logits, 3, 4, orc.TC)
    O, _ = orc.forward(X, W1, W2, rt)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    want = sum(p[:, e:e + 1] * torch_swiglu_mlp(X, W1[e], W2[e]) for e in range(3))
    np.testing.assert_allclose(O, want, rtol=1e-12, atol=1e-12)


def test_token_without_expert_gets_zero():
    from tests.golden_io import worked_example
    g = worked_example()
    rng = np.random.default_rng(2)
    X = rng.standard_normal((8, 4))
    W1 = rng.standard_normal((3, 4, 6))
    W2 = rng.standard_normal((3, 3, 4))
    dO = rng.standard_normal((8, 4))
    rt = orc.route(g["logits"], 1, 4, orc.TR)
    O, c = orc.forward(X, W1, W2, rt)
    dX, _, _, _ = orc.backward_minimal(dO, X, c["H"], W1, W2, rt)
    assert np.all(O[3] == 0) and np.all(dX[3] == 0)
    assert np.any(O[6] != 0)


def torch_layer_grads(X, W1, W2, rt, dO):
    """Autograd of the layer written directly in torch with routing held
    fixed: O = sum over slots of s * SwiGLU(X_t W1_e) W2_e."""
    Xt = torch.tensor(X, requires_grad=True)
    W1t = torch.tensor(W1, requires_grad=True)
    W2t = torch.tensor(W2, requires_grad=True)
    st = torch.tensor(rt.slot_weight, requires_grad=True)
    n = W1.shape[2] // 2
    tok = torch.from_numpy(rt.slot_token)
    ex = torch.from_numpy(rt.slot_expert)
    h = torch.einsum("sd,sdk->sk", Xt[tok], W1t[ex])
    a = torch.nn.functional.silu(h[:, :n]) * h[:, n:]
    y = torch.einsum("sn,snd->sd", a, W2t[ex])
    O = torch.zeros(X.shape, dtype=torch.float64).index_add(0, tok, st[:, None] * y)
    (O * torch.from_numpy(dO)).sum().backward()
    return Xt.grad.numpy(), W1t.grad.numpy(), W2t.grad.numpy(), st.grad.numpy(), O.detach().numpy()


@pytest.mark.parametrize("mode", [orc.TC, orc.TR])
def test_backward_matches_torch_autograd(mode):
    X, W1, W2, logits, dO = rand_layer(3, 40, 8, 6, 5)
    rt = orc.route(logits, 2, 4, mode)
    O, c = orc.forward(X, W1, W2, rt)
    got = orc.backward_minimal(dO, X, c["H"], W1, W2, rt)
    want = torch_layer_grads(X, W1, W2, rt, dO)
    np.testing.assert_allclose(O, want[4], rtol=1e-12, atol=1e-12)
    for g, w in zip(got, want[:4]):
        np.testing.assert_allclose(g, w, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mode", [orc.TC, orc.TR])
def test_minimal_equals_naive(mode):
    X, W1, W2, logits, dO = rand_layer(4, 64, 12, 8, 6)
    rt = orc.route(logits, 2, 8, mode)
    _, c = orc.forward(X, W1, W2, rt)
    a = orc.backward_minimal(dO, X, c["H"], W1, W2, rt)
    b = orc.backward_naive(dO, X, W1, W2, rt, c)
    for x, y in zip(a, b):
        assert np.linalg.norm(x - y) <= 1e-12 * max(np.linalg.norm(y), 1e-300)


def test_finite_differences():
    X, W1, W2, logits, dO = rand_layer(5, 7, 4, 3, 3)
    rt = orc.route(logits, 2, 2, orc.TR)
    _, c = orc.forward(X, W1, W2, rt)
    dX, dW1, dW2, dS = orc.backward_minimal(dO, X, c["H"], W1, W2, rt)
    h = 1e-6

    def loss(X_, W1_, W2_, s_):
        rt.slot_weight = s_
        O, _ = orc.forward(X_, W1_, W2_, rt)
        return float((O * dO).sum())

    s0 = rt.slot_weight.copy()
    for arr, grad, name in [(X, dX, "X"), (W1, dW1, "W1"), (W2, dW2, "W2"), (s0, dS, "s")]:
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = arr[i]
            arr[i] = old + h
            args = [X, W1, W2, s0.copy()]
            lp = loss(*args)
            arr[i] = old - h
            args = [X, W1, W2, s0.copy()]
            lm = loss(*args)
            arr[i] = old
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)
    rt.slot_weight = s0


def test_ds_identities():
    X, W1, W2, logits, dO = rand_layer(6, 30, 8, 5, 4)
    rt = orc.route(logits, 3, 4, orc.TR)
    O, c = orc.forward(X, W1, W2, rt)
    _, _, _, dS = orc.backward_minimal(dO, X, c["H"], W1, W2, rt)
    # per slot: <dO_t W2^T, SwiGLU(H)> = <dO_t, Y>
    want = np.einsum("sd,sd->s", dO[rt.slot_token], c["Y"])
    np.testing.assert_allclose(dS, want, rtol=1e-12, atol=1e-13)
    # per token: sum_e s * dS = <dO_t, O_t>
    per_tok = np.zeros(X.shape[0])
    np.add.at(per_tok, rt.slot_token, rt.slot_weight * dS)
    np.testing.assert_allclose(per_tok, np.einsum("td,td->t", dO, O), rtol=1e-12, atol=1e-13)


def test_sampled_helpers_match_full():
    X, W1, W2, logits, dO = rand_layer(7, 50, 8, 4, 5)
    rt = orc.route(logits, 2, 4, orc.TR)
    O, c = orc.forward(X, W1, W2, rt)
    dX, dW1, dW2, dS = orc.backward_minimal(dO, X, c["H"], W1, W2, rt)
    toks = [0, 3, 17, 49]
    np.testing.assert_allclose(orc.forward_tokens(toks, X, W1, W2, rt), O[toks], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(orc.dx_tokens(toks, X, W1, W2, dO, rt), dX[toks], rtol=1e-13, atol=1e-14)
    slots = [0, 5, rt.S - 1]
    np.testing.assert_allclose(orc.slot_grads(slots, X, W1, W2, dO, rt)[0], dS[slots], rtol=1e-13, atol=1e-14)
    for e in range(5):
        g1, g2 = orc.expert_weight_grads(e, X, W1, W2, dO, rt)
        np.testing.assert_allclose(g1, dW1[e], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(g2, dW2[e], rtol=1e-13, atol=1e-14)


class FlopCounter(np.ndarray):
    """ndarray that counts the multiply-adds of every matmul it takes part in."""
    flops = 0

    def __array_ufunc__(self, ufunc, method, *inputs, **kw):
        args = [np.asarray(x) if isinstance(x, FlopCounter) else x for x in inputs]
        if ufunc is np.matmul:
            a, b = args
            FlopCounter.flops += 2 * a.shape[0] * a.shape[1] * b.shape[1]
        out = getattr(ufunc, method)(*args, **kw)
        return out.view(FlopCounter) if isinstance(out, np.ndarray) else out


@pytest.mark.parametrize("mode", [orc.TC, orc.TR])
def test_flop_count(mode):
    T, d, n, E, K = 48, 16, 8, 6, 2
    X, W1, W2, logits, dO = rand_layer(8, T, d, n, E)
    rt = orc.route(logits, K, 4, mode)
    wrap = lambda a: np.asarray(a).view(FlopCounter)
    FlopCounter.flops = 0
    _, c = orc.forward(wrap(X), wrap(W1), wrap(W2), rt)
    fwd = FlopCounter.flops
    FlopCounter.flops = 0
    orc.backward_minimal(wrap(dO), wrap(X), wrap(c["H"]), wrap(W1), wrap(W2), rt)
    bwd = FlopCounter.flops
    S = rt.S
    f6, f12 = orc.layer_flops(T, n, K, d)
    assert fwd == 6 * S * n * d and bwd == 12 * S * n * d
    if mode == orc.TC:
        assert (fwd, bwd) == (f6, f12)


@pytest.mark.parametrize("T,d,n,E,K", [(4096, 768, 256, 64, 8), (16384, 1536, 256, 128, 8),
                                       (16384, 4096, 256, 256, 16), (8192, 2048, 384, 512, 8)])
def test_arithmetic_intensity_equals_byte_count(T, d, n, E, K):
    Te = T * K / E                       # tokens per expert on average
    flops = 2 * Te * d * 2 * n + 2 * Te * n * d
    elems = (Te * d            # gathered X_e read
             + d * 2 * n       # W1_e
             + 2 * Te * n      # A written, then read back
             + n * d           # W2_e
             + Te * d)         # Y written
    assert orc.arithmetic_intensity(T, d, n, K, E) == pytest.approx(flops / (2 * elems), rel=1e-12)


def test_cached_bytes_are_x_and_h():
    T, d, n, K = 256, 128, 64, 2
    X = np.zeros((T, d), dtype=np.float16)        # 2-byte stand-in for bf16
    H = np.zeros((T * K, 2 * n), dtype=np.float16)
    assert orc.cached_activation_bytes(T, d, K, n) == X.nbytes + H.nbytes
