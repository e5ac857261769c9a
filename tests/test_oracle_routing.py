"""Pins for the oracle's routing: top-K token choice and token rounding.

Each check is independent of the oracle's own code: pure-Python brute force,
hand-worked fixtures (tests/golden/, derived from the rule in the SonicMoE
ICLR-2026 notes, key design 1), special cases with known answers, and the
invariants the notes state for token rounding.
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as orc
from fine_grained_mixture_amd.inputs import SHAPES, make_layer_inputs
from tests.golden_io import rounding_cases, rounding_variant_cases, worked_example


def brute_topk(row, K):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:K]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, E, K = 40, 9, 3
    # small integer-valued logits force many exact ties
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    got = orc.topk_token_choice(logits, K)
    for t in range(T):
        assert list(got[t]) == brute_topk(logits[t], K)


def test_topk_all_experts():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((17, 5)).astype(np.float32)
    rt = orc.route(logits, K=5, M=4, mode=orc.TC)
    assert np.all(rt.tc_counts == 17)
    for e in range(5):
        a, b = rt.expert_offsets[e], rt.expert_offsets[e + 1]
        assert list(rt.slot_token[a:b]) == list(range(17))


def test_softmax_closed_form():
    logits = np.array([[0.0, math.log(2.0), math.log(5.0)]], dtype=np.float32)
    p = orc.softmax_probs(logits)
    # exp of the fp32-rounded logs
    ex = [math.exp(float(np.float32(v))) for v in logits[0]]
    np.testing.assert_allclose(p[0], np.array(ex) / sum(ex), rtol=1e-15)


@pytest.mark.parametrize("f,M,T,expected", rounding_cases())
def test_rounding_rule_golden(f, M, T, expected):
    assert int(orc.round_counts([f], M, T, orc.TR)[0]) == expected
    assert int(orc.round_counts([f], M, T, orc.TC)[0]) == f


def test_worked_example_golden():
    g = worked_example()
    tr = orc.route(g["logits"], K=1, M=4, mode=orc.TR)
    assert list(tr.tc_counts) == list(g["tc_counts"])
    assert list(tr.counts) == list(g["tr_counts"])
    assert list(tr.slot_token) == list(g["tr_slot_token"])
    assert list(tr.token_offsets) == list(g["tr_token_offsets"])
    assert list(tr.token_slots) == list(g["tr_token_slots"])
    # padded pair (t6, e0) carries its own softmax probability
    e = math.e
    want = math.sqrt(e) / (math.sqrt(e) + 1.0 + e)
    assert tr.slot_weight[3] == pytest.approx(want, rel=1e-7)
    tc = orc.route(g["logits"], K=1, M=4, mode=orc.TC)
    assert list(tc.slot_token) == list(g["tc_slot_token"])
    assert list(tc.counts) == list(g["tc_counts"])


def _tr_reference_sets(p, is_tc, r):
    """Set-based restatement: all TC tokens plus the best EC candidates when
    padding, or the best TC tokens when dropping."""
    T, E = p.shape
    sets = []
    for e in range(E):
        tc = [t for t in range(T) if is_tc[t, e]]
        ec = [t for t in range(T) if not is_tc[t, e]]
        best = lambda ts: sorted(ts, key=lambda t: (-p[t, e], t))
        if r[e] >= len(tc):
            chosen = tc + best(ec)[: r[e] - len(tc)]
        else:
            chosen = best(tc)[: r[e]]
        sets.append(sorted(chosen))
    return sets


def check_tr_invariants(logits, K, M, mode=orc.TR, rand=None):
    T, E = logits.shape
    tc = orc.route(logits, K, M, orc.TC)
    tr = orc.route(logits, K, M, mode, rand)
    f, r = tr.tc_counts, tr.counts
    assert np.array_equal(f, tc.counts)
    assert np.all(r % M == 0)                       # multiples of the tile
    assert np.all(np.abs(r - f) < M)                # within one tile of TC
    lo = (f // M) * M
    hi = np.where(f % M == 0, f, lo + M)
    assert np.all((r == lo) | (r == hi))            # one of the two neighbours
    if mode == orc.TR:
        assert np.all(2 * np.abs(r - f) <= M)       # nearest rounding
        assert abs(int(r.sum()) - int(f.sum())) <= E * M // 2
    elif mode == orc.TR_UP:
        assert np.all((r >= f) | (hi > T))
    elif mode == orc.TR_DOWN:
        assert np.all(r <= f)
    p = tr.probs
    is_tc = np.zeros((T, E), bool)
    is_tc[np.arange(T)[:, None], tr.topk_ids] = True
    for e in range(E):
        a, b = tr.expert_offsets[e], tr.expert_offsets[e + 1]
        kept = set(tr.slot_token[a:b].tolist())
        tcs = set(np.nonzero(is_tc[:, e])[0].tolist())
        assert len(kept) == r[e]
        if r[e] >= f[e]:
            assert tcs <= kept                      # TC kept before EC
        else:
            assert kept < tcs                       # only TC tokens dropped
        dropped = [t for t in range(T) if t not in kept]
        if kept and dropped:
            key = lambda t: (is_tc[t, e], p[t, e], -t)
            assert min(key(t) for t in kept) > max(key(t) for t in dropped)
        # slots of an expert ascend by token
        assert np.all(np.diff(tr.slot_token[a:b]) > 0)
        assert np.all(tr.slot_weight[a:b] == p[tr.slot_token[a:b], e])
    ref = _tr_reference_sets(p, is_tc, r)
    for e in range(E):
        a, b = tr.expert_offsets[e], tr.expert_offsets[e + 1]
        assert tr.slot_token[a:b].tolist() == ref[e]
    # token CSR lists every slot once, by ascending expert
    assert tr.token_offsets[-1] == tr.S
    assert sorted(tr.token_slots.tolist()) == list(range(tr.S))
    for t in range(T):
        sl = tr.token_slots[tr.token_offsets[t]:tr.token_offsets[t + 1]]
        assert np.all(tr.slot_token[sl] == t)
        assert np.all(np.diff(tr.slot_expert[sl]) > 0)
    return tc, tr


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("T,E,K,M", [(64, 6, 2, 8), (50, 7, 3, 4), (33, 4, 1, 16),
                                     (128, 16, 4, 16)])
def test_tr_invariants_random(seed, T, E, K, M):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((T, E)) + rng.standard_normal(E)).astype(np.float32)
    check_tr_invariants(logits, K, M)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tr_invariants_tiny_shape(seed):
    import torch
    inp = make_layer_inputs("tiny", dtype=torch.bfloat16, seed=seed)
    s = SHAPES["tiny"]
    check_tr_invariants(inp["logits"].numpy(), s.K, s.M)


def test_tr_m1_equals_tc():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((70, 9)).astype(np.float32)
    tc = orc.route(logits, 3, 1, orc.TC)
    tr = orc.route(logits, 3, 1, orc.TR)
    assert np.array_equal(tc.slot_token, tr.slot_token)
    assert np.array_equal(tc.expert_offsets, tr.expert_offsets)


def test_tr_multiples_equal_tc():
    # 4 experts, K=1, tokens split 8/8/4/12 by a fixed argmax: every f_e is a
    # multiple of M=4, so rounding changes nothing.
    owners = [0] * 8 + [1] * 8 + [2] * 4 + [3] * 12
    rng = np.random.default_rng(6)
    logits = rng.uniform(-1, 0, size=(len(owners), 4)).astype(np.float32)
    for t, e in enumerate(owners):
        logits[t, e] = 2.0
    tc = orc.route(logits, 1, 4, orc.TC)
    tr = orc.route(logits, 1, 4, orc.TR)
    assert list(tc.counts) == [8, 8, 4, 12]
    assert np.array_equal(tc.slot_token, tr.slot_token)


def test_tr_drops_leave_tokens_without_expert():
    g = worked_example()
    tr = orc.route(g["logits"], K=1, M=4, mode=orc.TR)
    assert tr.token_offsets[4] - tr.token_offsets[3] == 0


def test_tr_equal_scores_go_to_lower_token():
    # Pad case: t0..t2 pick e0 (f=3, M=4 -> r=4); t3..t7 have identical rows,
    # so their p[t, 0] tie exactly and the pad must take the lowest token, t3.
    rows = [[2.0, 0.0]] * 3 + [[0.0, 1.0]] * 5
    tr = orc.route(np.array(rows, np.float32), K=1, M=4, mode=orc.TR)
    assert list(tr.counts) == [4, 4]
    assert tr.slot_token[:4].tolist() == [0, 1, 2, 3]
    # Drop case: t0..t4 pick e0 with equal rows (f=5 -> r=4): the highest
    # token, t4, is the one dropped.
    rows = [[2.0, 0.0]] * 5 + [[0.0, 1.0]] * 3
    tr = orc.route(np.array(rows, np.float32), K=1, M=4, mode=orc.TR)
    assert list(tr.counts) == [4, 4]
    assert tr.slot_token[:4].tolist() == [0, 1, 2, 3]


# ---- rounding subroutines other than the nearest one -----------------------

@pytest.mark.parametrize("section,row", rounding_variant_cases())
def test_rounding_variants_golden(section, row):
    if section == "updown":
        f, M, T, up, down = row
        assert int(orc.round_counts([f], M, T, orc.TR_UP)[0]) == up
        assert int(orc.round_counts([f], M, T, orc.TR_DOWN)[0]) == down
    else:
        f, M, T, u, expected = row
        assert int(orc.round_counts([f], M, T, orc.TR_STOCHASTIC, [u])[0]) == expected


@pytest.mark.parametrize("M", [1, 4, 16, 128])
def test_stochastic_rounding_expectation_is_exact(M):
    # Over the M evenly spaced draws u_j = floor(j 2^32 / M), exactly f - lo
    # of them round up, so the mean count is f itself (key design 1: the
    # expected total count is that of token choice).
    T = 1 << 20
    u = np.array([(j << 32) // M for j in range(M)], dtype=np.uint64)
    for f in list(range(0, 3 * M + 1)) + [5513, 1000]:
        r = np.array([int(orc.round_counts([f], M, T, orc.TR_STOCHASTIC, [x])[0]) for x in u])
        lo = (f // M) * M
        assert np.all((r == lo) | (r == lo + M))
        assert int((r > lo).sum()) == f - lo
        assert r.sum() == f * M


def test_rounding_modes_need_their_draws():
    with pytest.raises(ValueError):
        orc.round_counts([5], 4, 100, orc.TR_STOCHASTIC)
    with pytest.raises(ValueError):
        orc.round_counts([5], 4, 100, 99)


@pytest.mark.parametrize("mode", [orc.TR_UP, orc.TR_DOWN, orc.TR_STOCHASTIC])
@pytest.mark.parametrize("seed", [0, 1])
def test_variant_invariants_random(mode, seed):
    rng = np.random.default_rng(100 + seed)
    T, E, K, M = 300, 12, 3, 16
    logits = (rng.standard_normal((T, E)) + rng.standard_normal(E)).astype(np.float32)
    rand = rng.integers(0, 1 << 32, size=E, dtype=np.uint64)
    check_tr_invariants(logits, K, M, mode, rand)


@pytest.mark.parametrize("mode", [orc.TR_UP, orc.TR_DOWN, orc.TR_STOCHASTIC])
def test_variants_with_m1_equal_tc(mode):
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((70, 9)).astype(np.float32)
    tc = orc.route(logits, 3, 1, orc.TC)
    tr = orc.route(logits, 3, 1, mode, np.zeros(9, np.uint64))
    assert np.array_equal(tc.slot_token, tr.slot_token)
    assert np.array_equal(tc.expert_offsets, tr.expert_offsets)


def test_nonfinite_logits_rule_hand_worked():
    # Hand-worked rows under the rule stated in the oracle (NaN and -inf rank
    # as -FLT_MAX, +inf as +FLT_MAX; equal values to the lower expert):
    #   row 0  [nan, 1, -inf, +inf, 0]  -> ranks e3 (+inf), e1 (1), e4 (0), ...
    #          softmax: e3 holds all the mass, every other entry is exactly 0
    #   row 1  [nan, nan, -inf, 0, 0]   -> e3, e4 (equal, lower first); the
    #          three saturated entries underflow: p = (0, 0, 0, 1/2, 1/2)
    #   row 2  [nan] * 5                -> all equal: e0, e1; p = 1/5 each
    #   row 3  [-inf, +inf, +inf, 2, nan] -> e1, e2 (equal, lower first);
    #          p = (0, 1/2, 1/2, 0, 0)
    nan, inf = float("nan"), float("inf")
    logits = np.array([[nan, 1.0, -inf, inf, 0.0],
                       [nan, nan, -inf, 0.0, 0.0],
                       [nan] * 5,
                       [-inf, inf, inf, 2.0, nan]], dtype=np.float32)
    top = orc.topk_token_choice(logits, 2)
    assert top.tolist() == [[3, 1], [3, 4], [0, 1], [1, 2]]
    p = orc.softmax_probs(logits)
    want = np.array([[0, 0, 0, 1, 0], [0, 0, 0, 0.5, 0.5], [0.2] * 5, [0, 0.5, 0.5, 0, 0]])
    assert np.array_equal(p, want)
    # routing (TC, K = 2) keeps exactly those pairs with those gate weights
    rt = orc.route(logits, K=2, M=2, mode=orc.TC)
    pairs = sorted(zip(rt.slot_token.tolist(), rt.slot_expert.tolist(), rt.slot_weight.tolist()))
    assert pairs == [(0, 1, 0.0), (0, 3, 1.0), (1, 3, 0.5), (1, 4, 0.5), (2, 0, 0.2), (2, 1, 0.2),
                     (3, 1, 0.5), (3, 2, 0.5)]


def test_nonfinite_logits_finite_rows_unchanged():
    # the replacement leaves every finite value alone, so finite inputs route
    # exactly as before
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((64, 8)).astype(np.float32)
    logits[0, 0] = np.finfo(np.float32).max
    logits[1, 1] = -np.finfo(np.float32).max
    assert np.array_equal(orc.finite_logits(logits), logits)
    for t in range(64):
        assert list(orc.topk_token_choice(logits, 3)[t]) == brute_topk(logits[t], 3)
