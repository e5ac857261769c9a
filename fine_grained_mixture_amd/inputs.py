"""Seeded synthetic workloads for the MoE layer.

This module only draws random inputs; it holds none of the layer's arithmetic
(no routing, no softmax, no projection).  Both the HIP path and the CPU checker
receive the tensors it returns, bit for bit.

The five workloads mirror the layer shapes the SonicMoE pages benchmark on: a
fine-grained 7B MoE with n = 256 (ICLR-2026 notes, main results), a
high-granularity layer (d/n = 16) and a high-sparsity layer (128 tokens per
expert on average), plus a tiny and a small layer for checking.  The pages name
no dataset for these kernel benchmarks, so seeded Gaussian data of these shapes
stands in for them.

Recipe (numpy PCG64 ``default_rng(seed)``, draws in float32, in the order X,
W1, W2, router, bias, dO):
  * tiny: X, W1, W2 and router weights W_r ~ N(0, 0.02^2); logits = X W_r
    computed in float64 from the (rounded) X and stored as float32.
  * others: X ~ N(0, 1); W1 ~ N(0, 1/d); W2 ~ N(0, 1/n) (std 1/sqrt(fan_in));
    logits z ~ N(0, 1) i.i.d., plus a per-expert bias b_e for two of them:
    b ~ N(0, 0.5^2) (the 7B layer), or b_e = -1.1 ln(pi_e) with pi a seeded
    permutation of 1..E (high sparsity; softmax of the bias is Zipf(1.1)
    over expert ranks).
  * dO ~ N(0, 1).
bf16 inputs are the float32 draws rounded to nearest even; logits stay fp32.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int      # tokens
    d: int      # model dim
    n: int      # expert intermediate dim (W1 is d x 2n for SwiGLU)
    E: int      # experts
    K: int      # experts per token (top-K)
    M: int      # M_tile the counts are rounded to
    init: str   # "tiny" or "fan_in"
    logits: str  # "router", "iid", "normal_bias" or "zipf_bias"

    @property
    def flops(self):
        """18 T n K d: what one forward+backward step is credited with."""
        return 18 * self.T * self.n * self.K * self.d


SHAPES = {
    s.name: s
    for s in [
        LayerShape("tiny", 256, 128, 64, 8, 2, 16, "tiny", "router"),
        LayerShape("small", 4096, 768, 256, 64, 8, 128, "fan_in", "iid"),
        LayerShape("7b", 16384, 1536, 256, 128, 8, 128, "fan_in", "normal_bias"),
        LayerShape("high_g", 16384, 4096, 256, 256, 16, 128, "fan_in", "iid"),
        LayerShape("high_sparsity", 8192, 2048, 384, 512, 8, 128, "fan_in",
                   "zipf_bias"),
    ]
}


def _cast(a32: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def make_layer_inputs(shape: LayerShape | str, dtype=torch.bfloat16, seed=0,
                      T=None):
    """Returns CPU tensors X [T, d], W1 [E, d, 2n], W2 [E, n, d] (dtype),
    logits [T, E] (float32) and dO [T, d] (dtype).  ``T`` overrides the
    token count (same per-token recipe) for reduced-size checks."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    T = shape.T if T is None else T
    d, n, E = shape.d, shape.n, shape.E
    rng = np.random.default_rng(seed)
    f32 = np.float32
    if shape.init == "tiny":
        X = rng.standard_normal((T, d), dtype=f32) * f32(0.02)
        W1 = rng.standard_normal((E, d, 2 * n), dtype=f32) * f32(0.02)
        W2 = rng.standard_normal((E, n, d), dtype=f32) * f32(0.02)
    else:
        X = rng.standard_normal((T, d), dtype=f32)
        W1 = rng.standard_normal((E, d, 2 * n), dtype=f32) * f32(1 / np.sqrt(d))
        W2 = rng.standard_normal((E, n, d), dtype=f32) * f32(1 / np.sqrt(n))
    Xt = _cast(X, dtype)
    if shape.logits == "router":
        Wr = rng.standard_normal((d, E), dtype=f32) * f32(0.02)
        logits = (Xt.double().numpy() @ Wr.astype(np.float64)).astype(f32)
    else:
        logits = rng.standard_normal((T, E), dtype=f32)
        if shape.logits == "normal_bias":
            logits = logits + rng.standard_normal(E, dtype=f32) * f32(0.5)
        elif shape.logits == "zipf_bias":
            ranks = rng.permutation(E) + 1
            logits = logits + (-1.1 * np.log(ranks)).astype(f32)
    dO = rng.standard_normal((T, d), dtype=f32)
    return {
        "X": Xt,
        "W1": _cast(W1, dtype),
        "W2": _cast(W2, dtype),
        "logits": torch.from_numpy(np.ascontiguousarray(logits, dtype=f32)),
        "dO": _cast(dO, dtype),
    }


ROUTING_LOGIT_KINDS = ("normal", "quantized", "constant", "duplicated", "zipf")


def make_routing_logits(T: int, E: int, kind: str, seed: int = 0) -> np.ndarray:
    """[T, E] float32 router logits for routing-only checks, from numpy PCG64
    seeded with (seed, 0x7E5):
      normal      N(0, 1);
      quantized   N(0, 1) rounded to multiples of 1/4 (many equal logits in a
                  row, and many equal probabilities across tokens);
      constant    every logit 0, except that a seeded tenth of the tokens get
                  N(0, 1) rows;
      duplicated  N(0, 1) rows, each token a copy of one of T / 8 + 1 rows;
      zipf        N(0, 1) plus -1.1 ln(rank_e) for a seeded permutation of
                  ranks 1..E (a few experts hold most tokens)."""
    rng = np.random.default_rng([seed, 0x7E5])
    f32 = np.float32
    z = rng.standard_normal((T, E), dtype=f32)
    if kind == "normal":
        out = z
    elif kind == "quantized":
        out = np.round(z * f32(4)) / f32(4)
    elif kind == "constant":
        out = np.zeros((T, E), dtype=f32)
        rows = rng.random(T) < 0.1
        out[rows] = z[rows]
    elif kind == "duplicated":
        out = z[rng.integers(0, T // 8 + 1, size=T)]
    elif kind == "zipf":
        out = z + (-1.1 * np.log(rng.permutation(E) + 1)).astype(f32)
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(out, dtype=f32)


def make_round_rand(E: int, seed: int = 0) -> np.ndarray:
    """The per-expert uniform draws of stochastic token rounding: E values in
    [0, 2**32) from numpy PCG64 seeded with (seed, 0x52D), as uint64.  The
    device takes the same values as 32-bit words (``round_rand_tensor``)."""
    rng = np.random.default_rng([seed, 0x52D])
    return rng.integers(0, 1 << 32, size=E, dtype=np.uint64)


def round_rand_tensor(rand: np.ndarray) -> torch.Tensor:
    """[E] int32 CPU tensor holding the bits of the uint32 draws."""
    return torch.from_numpy(np.ascontiguousarray(rand.astype(np.uint32).view(np.int32)))


def make_router_weight(shape: LayerShape | str, dtype=torch.bfloat16, seed=0) -> torch.Tensor:
    """Router weights Wr [E, d] (one row per expert) from their own PCG64
    stream seeded with (seed, 0x40D7): N(0, 1/d) (std 1/sqrt(fan_in)), or
    N(0, 0.02^2) for the tiny layer; rounded to `dtype` like the other
    weights.  The layer inputs above are unaffected."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    rng = np.random.default_rng([seed, 0x40D7])
    scale = 0.02 if shape.init == "tiny" else 1 / np.sqrt(shape.d)
    Wr = rng.standard_normal((shape.E, shape.d), dtype=np.float32) * np.float32(scale)
    return _cast(Wr, dtype)
