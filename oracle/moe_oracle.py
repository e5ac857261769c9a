"""Plain fp64 CPU oracle of one fine-grained MoE layer: routing, forward, backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or constants); both sides only
receive the same seeded input tensors.

The method is the one described in "SonicMoE: Accelerating MoE with IO and
Tile-aware Optimizations" (ICLR 2026 notes on papernotes.org, and the arXiv
abstract on mlsanity.com).  Those pages state that the SonicMoE layer is
mathematically equivalent to the textbook MoE layer (notes, "loss function /
training strategy" and key design 3), so the forward and both backward variants
here are that plain definition written out in fp64 numpy, one expert at a
time.  The one step that is an algorithm rather than a closed form, token
rounding, follows the notes' key design 1 step by step.

Readings where the pages are silent:
  * gate = softmax over all E experts of the fp32 logits, computed in fp64;
    the top-K gate weights are NOT renormalised (s = p);
  * top-K ties go to the lower expert index (decided on the fp32 logits);
  * non-finite logits are brought into the finite fp32 range before routing:
    NaN and -inf become -FLT_MAX, +inf becomes +FLT_MAX (so a NaN ranks
    below every number and gets probability 0 next to any larger logit);
  * token-rounding sort key = (chosen by token-choice?, p) descending, ties to
    the lower token index; the rounding tie (equal gaps) rounds DOWN, and a
    round-up that would need more than T tokens rounds down;
  * SwiGLU halves: W1 columns [0, n) are the gate (SiLU), [n, 2n) the up
    projection;
  * dS is the gradient of the loss with respect to the gate weight s of a
    slot, i.e. <dO_t, Y_{t,e}>, not scaled by s.

Every function is pinned by ``tests/test_oracle_*.py`` against something
other than itself (brute force, closed forms, finite differences, an
independent autograd library, invariants stated on the pages).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TC = 0             # vanilla top-K token choice
TR = 1             # token rounding, nearest multiple of M_tile (the default)
TR_UP = 2          # token rounding, always to the multiple above
TR_DOWN = 3        # token rounding, always to the multiple below
TR_STOCHASTIC = 4  # token rounding, up with probability (f - lo) / M_tile
TR_MODES = (TR, TR_UP, TR_DOWN, TR_STOCHASTIC)


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

FLT_MAX = float(np.finfo(np.float32).max)


def finite_logits(logits):
    """The logits with non-finite entries replaced: NaN and -inf by -FLT_MAX,
    +inf by +FLT_MAX (fp64 input keeps its precision, anything else is taken
    as fp32).  Router scores are real numbers on the pages (notes, key design
    1); this fixes one ranking and one gate for inputs outside that domain, so
    that both routing sides agree on them."""
    a = np.asarray(logits)
    a = a if a.dtype == np.float64 else a.astype(np.float32)
    return np.nan_to_num(a, nan=-FLT_MAX, posinf=FLT_MAX, neginf=-FLT_MAX)


def softmax_probs(logits):
    """Router probabilities p[t, e] = softmax over experts of the logits, fp64.

    The abstract and the notes' framework section route every token by router
    scores; the gate is a softmax over all E experts (the plainest reading;
    the pages do not print the gate formula).  Non-finite logits are first
    replaced as `finite_logits` states.
    """
    z = np.asarray(finite_logits(logits), dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def topk_token_choice(logits, K):
    """Vanilla top-K token choice (TC): for every token the K experts with the
    largest logit, best first; equal logits go to the lower expert index.

    Softmax is monotone per row, so ranking the fp32 logits ranks p.
    Non-finite logits are first replaced as `finite_logits` states.
    Returns int64 [T, K].
    """
    l32 = finite_logits(np.asarray(logits, dtype=np.float32))
    T, E = l32.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    # A stable sort of the negated logits keeps equal values in expert order.
    order = np.argsort(-l32, axis=1, kind="stable")
    return order[:, :K].astype(np.int64)


def round_counts(f, M, T, mode, rand_u32=None):
    """Per-expert token counts after the rounding subroutine of token rounding.

    Notes, key design 1: with lo = the largest multiple of M not above f_e
    and hi = the smallest multiple not below it, the default subroutine pads
    the expert up to hi when (hi - f_e) < (f_e - lo) and otherwise drops it to
    lo, so an equal gap rounds down.  The notes' loss function / training
    strategy section reports that the choice of subroutine matters little, and
    key design 1 that the expected total stays that of token choice; the other
    subroutines built here are the plain readings of those remarks:
      * TR_UP:   always hi;
      * TR_DOWN: always lo;
      * TR_STOCHASTIC: hi with probability (f_e - lo) / M, so E[r_e] = f_e.
        The draw is an input, one uint32 u_e per expert, and the decision is
        taken in integers: hi iff u_e * M < (f_e - lo) * 2**32.
    A pad needs hi distinct tokens, so hi is only taken when hi <= T.  Under
    TC the counts are left as they are.
    """
    f = np.asarray(f, dtype=np.int64)
    if mode == TC:
        return f.copy()
    lo = (f // M) * M
    hi = np.where(f % M == 0, f, lo + M)
    if mode == TR:
        up = (hi - f) < (f - lo)
    elif mode == TR_UP:
        up = hi > f
    elif mode == TR_DOWN:
        up = np.zeros(f.shape, dtype=bool)
    elif mode == TR_STOCHASTIC:
        if rand_u32 is None:
            raise ValueError("stochastic rounding needs one uint32 draw per expert")
        u = np.asarray(rand_u32, dtype=np.uint64)
        up = u * np.uint64(M) < (f - lo).astype(np.uint64) << np.uint64(32)
    else:
        raise ValueError(f"unknown routing mode {mode}")
    up = up & (hi <= T)
    return np.where(up, hi, lo)


def token_rounding_select(p, is_tc, r):
    """Per-expert token sets under token rounding (notes, key design 1).

    For each expert the T tokens are sorted by router score p in descending
    order, after the score matrix is adjusted so that every token the expert
    got under TC ranks ahead of every expert-choice candidate; the first r_e
    tokens are kept.  Equal scores go to the lower token index.  Returns a
    list of E sorted int64 arrays of token ids.
    """
    T, E = p.shape
    tok = np.arange(T)
    out = []
    for e in range(E):
        # lexsort: the last key is the primary one.
        order = np.lexsort((tok, -p[:, e], ~is_tc[:, e]))
        out.append(np.sort(order[: r[e]]).astype(np.int64))
    return out


@dataclass
class Routing:
    """Routing metadata in canonical slot order: experts ascending, tokens
    ascending inside an expert; a token's slots listed by ascending expert."""

    topk_ids: np.ndarray        # [T, K] int64, TC choice, best first
    tc_counts: np.ndarray       # [E]    f_e
    counts: np.ndarray          # [E]    r_e
    expert_offsets: np.ndarray  # [E+1]
    slot_token: np.ndarray      # [S]
    slot_expert: np.ndarray     # [S]
    slot_weight: np.ndarray     # [S] fp64 gate weight s = p[t, e]
    token_offsets: np.ndarray   # [T+1]
    token_slots: np.ndarray     # [S]
    probs: np.ndarray           # [T, E] fp64

    @property
    def S(self):
        return int(self.expert_offsets[-1])


def route(logits, K, M, mode, rand_u32=None):
    """Top-K token choice, optionally followed by token rounding (notes,
    key design 1; abstract).  Gate weights are the softmax probabilities of
    the kept (token, expert) pairs, not renormalised.  `rand_u32` holds the
    per-expert draws of stochastic rounding (ignored by the other modes)."""
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    p = softmax_probs(l32)
    topk = topk_token_choice(l32, K)
    is_tc = np.zeros((T, E), dtype=bool)
    is_tc[np.arange(T)[:, None], topk] = True
    f = is_tc.sum(axis=0).astype(np.int64)
    r = round_counts(f, M, T, mode, rand_u32)
    if mode == TC:
        sel = [np.nonzero(is_tc[:, e])[0].astype(np.int64) for e in range(E)]
    else:
        sel = token_rounding_select(p, is_tc, r)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(s) for s in sel])
    slot_token = np.concatenate(sel) if E else np.zeros(0, np.int64)
    slot_expert = np.repeat(np.arange(E), [len(s) for s in sel])
    slot_weight = p[slot_token, slot_expert]
    # Token CSR: slots grouped by token; a stable sort keeps ascending expert.
    order = np.argsort(slot_token, kind="stable")
    c = np.bincount(slot_token, minlength=T)
    token_offsets = np.zeros(T + 1, dtype=np.int64)
    token_offsets[1:] = np.cumsum(c)
    return Routing(topk, f, r, offsets, slot_token, slot_expert, slot_weight,
                   token_offsets, order.astype(np.int64), p)


# --------------------------------------------------------------------------
# Layer
# --------------------------------------------------------------------------

def silu(g):
    return g / (1.0 + np.exp(-g))


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def swiglu(H, n):
    """A = SiLU(gate) * up with gate = H[:, :n], up = H[:, n:]."""
    return silu(H[:, :n]) * H[:, n:]


def _f64(a):
    return np.asanyarray(a, dtype=np.float64)


def forward(X, W1, W2, rt: Routing):
    """Forward of the layer (notes, method > overall framework: up-proj,
    SwiGLU, down-proj, expert aggregation).

    For every expert e with token rows I_e:  H_e = X[I_e] W1_e,
    A_e = SiLU(H_e[:, :n]) * H_e[:, n:],  Y_e = A_e W2_e,  and
    O[t] = sum over t's slots of s * Y.  A token with no slot gets O = 0.
    Returns O [T, d] and a cache dict with H [S, 2n], A [S, n], Y [S, d].
    """
    X, W1, W2 = _f64(X), _f64(W1), _f64(W2)
    T, d = X.shape
    E, _, n2 = W1.shape
    n = n2 // 2
    S = rt.S
    H = np.zeros((S, n2))
    A = np.zeros((S, n))
    Y = np.zeros((S, d))
    O = np.zeros((T, d))
    for e in range(E):
        a, b = rt.expert_offsets[e], rt.expert_offsets[e + 1]
        if a == b:
            continue
        tok = rt.slot_token[a:b]
        H[a:b] = X[tok] @ W1[e]
        A[a:b] = swiglu(H[a:b], n)
        Y[a:b] = A[a:b] @ W2[e]
        O[tok] += rt.slot_weight[a:b, None] * Y[a:b]  # tokens distinct in e
    return O, {"H": H, "A": A, "Y": Y}


def backward_minimal(dO, X, H, W1, W2, rt: Routing):
    """Minimal-activation backward (notes, key designs 2 and 3).

    Uses only X, H and the routing metadata; Y and the gathered X_e are never
    read.  Per expert: dA' = dO[I_e] W2_e^T; A is recomputed from H;
    dS = rowsum(dA' * A) (the inner product taken in the dH epilogue instead
    of <dO, Y>); dA = s * dA'; dH = dSwiGLU(H; dA); then the varlen-K weight
    gradients dW2_e = (s*A)^T dO[I_e], dW1_e = X[I_e]^T dH, and
    dX[I_e] += dH W1_e^T.
    Returns dX [T, d], dW1 [E, d, 2n], dW2 [E, n, d], dS [S].
    """
    dO, X, H, W1, W2 = _f64(dO), _f64(X), _f64(H), _f64(W1), _f64(W2)
    T, d = X.shape
    E, _, n2 = W1.shape
    n = n2 // 2
    dX = np.zeros((T, d))
    dW1 = np.zeros_like(W1)
    dW2 = np.zeros_like(W2)
    dS = np.zeros(rt.S)
    for e in range(E):
        a, b = rt.expert_offsets[e], rt.expert_offsets[e + 1]
        if a == b:
            continue
        tok = rt.slot_token[a:b]
        s = rt.slot_weight[a:b, None]
        dOe = dO[tok]
        dAp = dOe @ W2[e].T
        g, u = H[a:b, :n], H[a:b, n:]
        Ae = silu(g) * u
        dS[a:b] = (dAp * Ae).sum(axis=1)
        dA = s * dAp
        sg = sigmoid(g)
        dg = dA * u * sg * (1.0 + g * (1.0 - sg))
        du = dA * silu(g)
        dH = np.concatenate([dg, du], axis=1)
        dW2[e] = (s * Ae).T @ dOe
        dW1[e] = X[tok].T @ dH
        dX[tok] += dH @ W1[e].T
    return dX, dW1, dW2, dS


def backward_naive(dO, X, W1, W2, rt: Routing, cache):
    """The textbook backward that caches Y and the gathered X_e.

    dY = s * dO[I_e], dS = rowsum(dO[I_e] * Y), dW2 = A^T dY, dA = dY W2^T,
    then dSwiGLU, dW1 = X_e^T dH and a scatter-add of dH W1^T into dX.
    It is a second, independent route to the same gradients.
    """
    dO, X, W1, W2 = _f64(dO), _f64(X), _f64(W1), _f64(W2)
    T, d = X.shape
    E, _, n2 = W1.shape
    n = n2 // 2
    Xe_cache = [X[rt.slot_token[rt.expert_offsets[e]:rt.expert_offsets[e + 1]]]
                for e in range(E)]
    H, A, Y = cache["H"], cache["A"], cache["Y"]
    dX = np.zeros((T, d))
    dW1 = np.zeros_like(W1)
    dW2 = np.zeros_like(W2)
    dS = np.zeros(rt.S)
    for e in range(E):
        a, b = rt.expert_offsets[e], rt.expert_offsets[e + 1]
        if a == b:
            continue
        tok = rt.slot_token[a:b]
        dY = rt.slot_weight[a:b, None] * dO[tok]
        dS[a:b] = np.einsum("ij,ij->i", dO[tok], Y[a:b])
        dW2[e] = A[a:b].T @ dY
        dA = dY @ W2[e].T
        g, u = H[a:b, :n], H[a:b, n:]
        sg = sigmoid(g)
        dH = np.concatenate([dA * u * (sg + g * sg * (1.0 - sg)),
                             dA * g * sg], axis=1)
        dW1[e] = Xe_cache[e].T @ dH
        np.add.at(dX, tok, dH @ W1[e].T)
    return dX, dW1, dW2, dS


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------

def router_logits(X, Wr):
    """Router scores l = X Wr^T in fp64 (Wr: [E, d], one row per expert).

    The notes (method > overall framework; key design 1) route every token by
    its router scores; the router itself is a linear map of the token.
    """
    return _f64(X) @ _f64(Wr).T


def router_backward(dS, rt: Routing, X, Wr, logits):
    """Gradients of the router from the gate-weight gradients dS.

    The gate weight of a kept (token, expert) pair is s = p[t, e], the softmax
    probability (no renormalisation), and the loss sees the router only
    through those weights (routing decisions are piecewise constant and carry
    no gradient).  So with g[t, e] = dS of the slot of (t, e), zero for pairs
    not kept, the softmax Jacobian gives
        dlogits[t] = p[t] * (g[t] - <p[t], g[t]>),
    and the linear map gives dWr = dlogits^T X ([E, d]) and the router's share
    of the input gradient dX_router = dlogits Wr ([T, d]).
    """
    p = softmax_probs(logits)
    T, E = p.shape
    g = np.zeros((T, E), dtype=np.float64)
    g[rt.slot_token, rt.slot_expert] = _f64(dS)[: rt.S]
    dlogits = p * (g - (p * g).sum(axis=1, keepdims=True))
    return dlogits, dlogits.T @ _f64(X), dlogits @ _f64(Wr)


# --------------------------------------------------------------------------
# Sampled evaluation for full-size shapes (same arithmetic, restricted rows).
# These recompute H from X and W1 themselves and convert only the rows and
# experts they touch to fp64, so they also serve shapes whose full fp64 copy
# would not fit in memory.
# --------------------------------------------------------------------------

def _slot_terms(slots, X, W1, W2, dO, rt: Routing):
    """For a batch of slots of ONE expert: H, A, dA', dS and dH."""
    e = int(rt.slot_expert[slots[0]])
    tok = rt.slot_token[slots]
    W1e, W2e = _f64(W1[e]), _f64(W2[e])
    n = W2e.shape[0]
    H = _f64(X[tok]) @ W1e
    A = swiglu(H, n)
    dAp = _f64(dO[tok]) @ W2e.T
    g, u = H[:, :n], H[:, n:]
    s = rt.slot_weight[slots, None]
    dA = s * dAp
    sg = sigmoid(g)
    dH = np.concatenate([dA * u * sg * (1.0 + g * (1.0 - sg)), dA * silu(g)], axis=1)
    return H, A, (dAp * A).sum(axis=1), dH


def _by_expert(slots, rt: Routing):
    slots = np.asarray(slots, dtype=np.int64)
    ex = rt.slot_expert[slots]
    for e in np.unique(ex):
        idx = np.nonzero(ex == e)[0]
        yield idx, slots[idx]


def forward_tokens(tokens, X, W1, W2, rt: Routing):
    """O[t] for selected tokens only, from each token's own slots."""
    out = np.zeros((len(tokens), X.shape[1]))
    pos = {int(t): i for i, t in enumerate(tokens)}
    slots = np.concatenate([rt.token_slots[rt.token_offsets[t]:rt.token_offsets[t + 1]]
                            for t in tokens] + [np.zeros(0, np.int64)])
    for _, sl in _by_expert(slots, rt):
        e = int(rt.slot_expert[sl[0]])
        A = swiglu(_f64(X[rt.slot_token[sl]]) @ _f64(W1[e]), W2.shape[1])
        Y = A @ _f64(W2[e])
        for k, p in enumerate(sl):
            out[pos[int(rt.slot_token[p])]] += rt.slot_weight[p] * Y[k]
    return out


def slot_grads(slots, X, W1, W2, dO, rt: Routing):
    """dS and dH for selected slots (the formulas of backward_minimal)."""
    slots = np.asarray(slots, dtype=np.int64)
    n = W2.shape[1]
    dS = np.zeros(len(slots))
    dH = np.zeros((len(slots), 2 * n))
    for idx, sl in _by_expert(slots, rt):
        _, _, dS[idx], dH[idx] = _slot_terms(sl, X, W1, W2, dO, rt)
    return dS, dH


def dx_tokens(tokens, X, W1, W2, dO, rt: Routing):
    """dX[t] for selected tokens: sum over t's slots of dH W1_e^T."""
    out = np.zeros((len(tokens), X.shape[1]))
    pos = {int(t): i for i, t in enumerate(tokens)}
    slots = np.concatenate([rt.token_slots[rt.token_offsets[t]:rt.token_offsets[t + 1]]
                            for t in tokens] + [np.zeros(0, np.int64)])
    for _, sl in _by_expert(slots, rt):
        e = int(rt.slot_expert[sl[0]])
        _, _, _, dH = _slot_terms(sl, X, W1, W2, dO, rt)
        dXt = dH @ _f64(W1[e]).T
        for k, p in enumerate(sl):
            out[pos[int(rt.slot_token[p])]] += dXt[k]
    return out


def expert_weight_grads(e, X, W1, W2, dO, rt: Routing):
    """dW1_e and dW2_e for one expert (varlen-K contraction over its slots)."""
    a, b = rt.expert_offsets[e], rt.expert_offsets[e + 1]
    d, n = X.shape[1], W2.shape[1]
    if a == b:
        return np.zeros((d, 2 * n)), np.zeros((n, d))
    sl = np.arange(a, b)
    tok = rt.slot_token[a:b]
    _, A, _, dH = _slot_terms(sl, X, W1, W2, dO, rt)
    s = rt.slot_weight[a:b, None]
    return _f64(X[tok]).T @ dH, (s * A).T @ _f64(dO[tok])


# --------------------------------------------------------------------------
# Cost models stated on the pages
# --------------------------------------------------------------------------

def layer_flops(T, n, K, d):
    """(6 + 12) T n K d: forward 6TnKd, backward 12TnKd (notes, key design 3)."""
    return 6 * T * n * K * d, 12 * T * n * K * d


def cached_activation_bytes(T, d, K, n, elem=2):
    """Bytes the minimal backward keeps from the forward: X [T, d] and
    H [TK, 2n] in bf16, i.e. 2Td + 4TKn (notes, key design 3); routing
    metadata comes on top."""
    return elem * T * d + elem * T * K * 2 * n


def arithmetic_intensity(T, d, n, K, E):
    """Forward arithmetic intensity of an expert's up+down projection
    (notes, background and insights): 3 / ((2 + 2G)/d + 3/(T rho)) with
    G = d/n and rho = K/E, ignoring the write-back of H.  The notes print the
    first term as 2 + 2G/d, which is not dimensionless; the form used here is
    the one that equals a byte count of the same kernels."""
    G = d / n
    rho = K / E
    return 3.0 / ((2.0 + 2.0 * G) / d + 3.0 / (T * rho))
