"""Acceptance checks of the GPU outputs against the fp64 oracle.

Two bounds per output tensor:
  * the relative Frobenius error ||G - R|| / ||R|| of the whole tensor, at
    the tolerance the layer is specified to (1e-2 for bf16 inputs, 1e-5 for
    fp32);
  * a per-row bound: for every row i (a token row of O and dX, a slot row of
    H, a row of one expert's dW1 or dW2, a group of 64 consecutive slots of
    dS)
        ||G_i - R_i|| / (||R_i|| + rms_i ||R_i||)  <=  tol_row
    i.e. the row's error relative to its own size, with the tensor's RMS row
    norm as a floor so that rows near zero are not ill-conditioned.

Why the row bound (bf16): every output element is the end of a short chain
of roundings to bf16 (unit roundoff u = 2^-8) of fp32 sums: at most four in
the dH -> dX chain (H, dA', dH, dX-tilde, then dX).  A row of >= 64 such
elements has a relative error that concentrates near its RMS value, about
sqrt(c) * u / sqrt(3) <= 4.5e-3 for c = 4 roundings, so no correct row
comes near 2.5e-2.  A single wrong slot (one row of dX-tilde, of Y, or one
gate weight) moves its token's row by about the size of that row, an error
of order 0.1-1 there, while it moves the whole tensor's Frobenius error by
only about 1/sqrt(S) (~5e-3 at S = 32768) and so can hide under the
Frobenius bound alone.  For fp32 inputs the chain has no bf16 rounding and
the row bound is 1e-4.
"""
from __future__ import annotations

import numpy as np

TOL_FRO = {"bf16": 1e-2, "f32": 1e-5}
TOL_ROW = {"bf16": 2.5e-2, "f32": 1e-4}
DS_GROUP = 64  # dS is checked in groups of this many consecutive slots


def rel_fro(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def as_rows(a, width=None):
    """2-D view: a matrix keeps its last axis as rows' elements; a vector is
    cut into groups of `width` (the last group zero-padded)."""
    a = np.asarray(a, np.float64)
    if a.ndim == 1:
        w = width or DS_GROUP
        pad = (-len(a)) % w
        a = np.concatenate([a, np.zeros(pad)])
        return a.reshape(-1, w)
    return a.reshape(-1, a.shape[-1])


def row_errors(got, want, width=None):
    """Per-row error relative to the row norm plus the RMS row norm."""
    g, w = as_rows(got, width), as_rows(want, width)
    rn = np.linalg.norm(w, axis=1)
    rms = float(np.sqrt(np.mean(rn ** 2))) if len(rn) else 0.0
    den = rn + (rms if rms > 0 else 1.0)
    return np.linalg.norm(g - w, axis=1) / den


def check(name, got, want, kind="bf16", width=None):
    """Returns (frobenius error, worst row error, worst row index); raises
    AssertionError naming the tensor if either bound fails."""
    fro = rel_fro(got, want)
    err = row_errors(got, want, width)
    worst = int(np.argmax(err)) if len(err) else -1
    mx = float(err[worst]) if len(err) else 0.0
    assert fro <= TOL_FRO[kind], f"{name}: relative Frobenius error {fro:.3e}"
    assert mx <= TOL_ROW[kind], f"{name}: row {worst} error {mx:.3e}"
    return fro, mx, worst
