"""Readers for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def rounding_cases():
    return [tuple(int(v) for v in line.split()) for line in _lines("tr_rounding_rule.txt")]


def worked_example():
    rows, out, in_logits = [], {}, False
    for line in _lines("tr_worked_example.txt"):
        head = line.split()[0]
        if head == "logits":
            in_logits = True
            continue
        if head[0].isalpha():
            in_logits = False
            out[head] = np.array([int(v) for v in line.split()[1:]], dtype=np.int64)
        elif in_logits:
            rows.append([float(v) for v in line.split()])
    out["logits"] = np.array(rows, dtype=np.float32)
    return out


def rounding_variant_cases():
    """(section, row) pairs of tr_rounding_variants.txt."""
    out, section = [], None
    for line in _lines("tr_rounding_variants.txt"):
        if line in ("updown", "stochastic"):
            section = line
            continue
        out.append((section, tuple(int(v) for v in line.split())))
    return out
