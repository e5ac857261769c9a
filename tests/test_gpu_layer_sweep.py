"""GPU: the whole layer (route, forward, backward) over a seeded sweep of
small problems, every element against the oracle.

The fixed cases of test_gpu_parity.py pick their shapes by hand.  This sweep
draws d (every column-tile class: multiples of 512, of 256, of 128), n (each
of the five supported widths), the element type, E, K, M_tile, the rounding
mode and the logit recipe from a seeded generator, so that every tile
configuration of every GEMM runs in both element types, including the fp32
dH tiles of n = 256 and n = 384.
"""
import numpy as np
import pytest
import torch

from fine_grained_mixture_amd.inputs import LayerShape, make_layer_inputs
from tests.test_gpu_parity import (KIND, check_layer, check_routing, log, np_inputs,
                                   oracle_route, run_gpu)
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu

MODES = ("tc", "tr", "tr_up", "tr_down", "tr_stochastic")
NS = (64, 128, 256, 384, 512)
DS = (128, 256, 384, 512, 640, 768, 1024, 1536)
LOGITS = ("iid", "normal_bias", "zipf_bias")


def _cases(seed=7):
    rng = np.random.default_rng(seed)
    out = []
    i = 0
    for n in NS:
        for dt in (torch.bfloat16, torch.float32):
            for _ in range(4):
                d = int(rng.choice(DS))
                E = int(rng.choice((4, 16, 33, 64)))
                K = int(rng.integers(1, min(E, 8) + 1))
                T = int(rng.integers(60, 1600))
                M = int(rng.choice((16, 32, 64, 128)))
                mode = MODES[i % len(MODES)]
                logits = LOGITS[i % len(LOGITS)]
                out.append((LayerShape(f"sweep{i}", T, d, n, E, K, M, "fan_in", logits), dt, mode,
                            int(rng.integers(0, 1 << 16))))
                i += 1
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0].name}-T{c[0].T}-d{c[0].d}-n{c[0].n}-E{c[0].E}-K{c[0].K}-M{c[0].M}-"
    f"{KIND[c[1]]}-{c[2]}" for c in CASES])
def test_layer_sweep(case):
    shape, dtype, mode, seed = case
    tag = (f"{shape.name} T={shape.T} d={shape.d} n={shape.n} E={shape.E} K={shape.K} "
           f"M={shape.M} {KIND[dtype]} {mode} seed={seed}")
    log(f"[layer-sweep] {tag}")
    inp = make_layer_inputs(shape, dtype=dtype, seed=seed)
    g = run_gpu(shape, dtype, mode, inp)
    a = np_inputs(inp)
    ref = oracle_route(a["logits"], shape, mode)
    check_routing(g, ref, shape)
    O, c = orc.forward(a["X"], a["W1"], a["W2"], ref)
    grads = orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], ref)
    check_layer(g, ref, O, c["H"], grads, KIND[dtype], tag)
