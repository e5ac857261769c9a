"""CPU checks of the acceptance bounds themselves (tests/parity_checks.py):
outputs that differ from the fp64 oracle only by bf16 output rounding pass,
and one wrong slot planted in the oracle, which the whole-tensor Frobenius
bound alone lets through at the small layer (S = 32768 slots), fails the
per-row bound."""
import dataclasses

import numpy as np
import pytest
import torch

from fine_grained_mixture_amd.inputs import SHAPES, make_layer_inputs
from oracle import moe_oracle as orc
from tests.parity_checks import TOL_FRO, TOL_ROW, check, rel_fro, row_errors


def bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.fixture(scope="module")
def small_layer():
    sh = SHAPES["small"]
    inp = make_layer_inputs(sh, dtype=torch.bfloat16, seed=0)
    a = {k: v.float().numpy() for k, v in inp.items()}
    rt = orc.route(a["logits"], sh.K, sh.M, orc.TR)
    O, c = orc.forward(a["X"], a["W1"], a["W2"], rt)
    grads = orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], rt)
    return sh, a, rt, O, c, grads


def test_rounded_outputs_pass(small_layer):
    _, _, _, O, c, (dX, dW1, dW2, dS) = small_layer
    for name, ref in (("O", O), ("H", c["H"]), ("dX", dX), ("dW1", dW1), ("dW2", dW2),
                      ("dS", dS)):
        fro, mx, _ = check(name, bf16(ref), ref)
        assert mx < TOL_ROW["bf16"] / 4, (name, mx)


def test_one_wrong_slot_fails_the_row_bound_only(small_layer):
    sh, a, rt, O, c, (dX, _, _, _) = small_layer
    assert rt.S == 32768
    # plant: a slot of median gate weight carries the wrong sign
    p = int(np.argsort(rt.slot_weight)[rt.S // 2])
    w = rt.slot_weight.copy()
    w[p] = -w[p]
    bad = dataclasses.replace(rt, slot_weight=w)
    O2, c2 = orc.forward(a["X"], a["W1"], a["W2"], bad)
    dX2 = orc.backward_minimal(a["dO"], a["X"], c2["H"], a["W1"], a["W2"], bad)[0]
    t = int(rt.slot_token[p])
    for name, got, ref in (("O", O2, O), ("dX", dX2, dX)):
        # the whole tensor stays inside the Frobenius bound ...
        assert rel_fro(got, ref) < TOL_FRO["bf16"], name
        # ... the token's row does not
        err = row_errors(got, ref)
        assert int(np.argmax(err)) == t and err[t] > 4 * TOL_ROW["bf16"], (name, err[t])
        with pytest.raises(AssertionError, match=f"row {t}"):
            check(name, got, ref)


def test_one_wrong_ds_slot_fails():
    # dS is checked in groups of 64 consecutive slots: one slot whose value
    # is off by the tensor's RMS size fails its group's bound
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(32768)
    got = ref.copy()
    got[12345] += np.sqrt(np.mean(ref ** 2))
    assert rel_fro(got, ref) < TOL_FRO["bf16"]
    with pytest.raises(AssertionError, match="row 192"):
        check("dS", got, ref)
