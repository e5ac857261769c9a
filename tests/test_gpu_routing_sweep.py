"""GPU: routing alone over a seeded sweep of problem sizes, modes and logit
distributions, bit for bit against the oracle.

The layer tests route on Gaussian logits of the benchmark shapes.  This sweep
adds shapes in between (T from 1 to 40 000, past the 32 768 tokens the
selection keeps in registers; E from 1 to 1024, K up to 32, M_tile from 1 to
1024) and logits that force the tie rules: quantised logits
(equal logits inside a row go to the lower expert; equal probabilities across
tokens go to the lower token), rows of equal logits, duplicated tokens, and a
Zipf-skewed load that leaves experts empty or rounds them up past their
token-choice count.  Every routing array must match exactly.
"""
import sys
import types

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd import moe
from fine_grained_mixture_amd.inputs import (ROUTING_LOGIT_KINDS, make_round_rand,
                                             make_routing_logits, round_rand_tensor)
from oracle import moe_oracle as orc
from tests.test_gpu_parity import ORC_MODE, check_routing

pytestmark = pytest.mark.gpu

MODES = ("tc", "tr", "tr_up", "tr_down", "tr_stochastic")


def _cases(n=160, seed=20260):
    rng = np.random.default_rng(seed)
    Ts = (1, 31, 33, 500, 1000, 2047, 4096, 8191, 40000)
    Es = (1, 2, 7, 16, 64, 129, 300, 512, 1024)
    Ms = (1, 16, 48, 128, 256, 1024)
    out = []
    for i in range(n):
        T, E = int(rng.choice(Ts)), int(rng.choice(Es))
        if T * E > 4_200_000:  # keeps the oracle's per-expert sorts to seconds
            E = max(1, 4_200_000 // T)
        K = int(rng.integers(1, min(E, 32) + 1))
        M = int(rng.choice(Ms))
        mode = MODES[i % len(MODES)]
        kind = ROUTING_LOGIT_KINDS[(i // len(MODES)) % len(ROUTING_LOGIT_KINDS)]
        out.append((T, E, K, M, mode, kind, int(rng.integers(0, 1 << 16))))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-E{c[1]}-K{c[2]}-M{c[3]}-{c[4]}-{c[5]}"
                                             for c in CASES])
def test_routing_sweep(case):
    T, E, K, M, mode, kind, seed = case
    print(f"[sweep] T={T} E={E} K={K} M={M} {mode} {kind} seed={seed}", file=sys.stderr,
          flush=True)
    logits = make_routing_logits(T, E, kind, seed)
    rand = make_round_rand(E, seed)
    ref = orc.route(logits, K, M, ORC_MODE[mode], rand)
    dev = torch.device("cuda", 0)
    p = moe.problem(T, 128, 64, E, K, M, torch.bfloat16, mode)
    rt = moe.route(p, torch.from_numpy(logits).to(dev),
                   round_rand=round_rand_tensor(rand).to(dev))
    torch.cuda.synchronize()
    g = {k: v.cpu() for k, v in rt.tensors.items()}
    check_routing(g, ref, types.SimpleNamespace(T=T, E=E, K=K))
    # the invariants the rounding promises, on the device's own counts
    f, r = g["tc_counts"].numpy(), g["counts"].numpy()
    if mode != "tc" and M > 1:
        assert np.all(r % M == 0) and np.all(np.abs(r - f) < M)
