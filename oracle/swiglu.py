"""fp64 CPU oracle of one tensor-parallel rank's SwiGLU MLP shard.

TEST INFRASTRUCTURE ONLY (see ``oracle/mlp.py``): only tests, the smoke check
and the benchmark's host-baseline leg use it.

Passages followed: Megatron expert interview Level 2 (blog.cptz.space),
M027 (a GeLU or SwiGLU between the column- and row-parallel layers is
computed on each element or on paired local shards and needs no other rank)
and M031 (SwiGLU's two projections each carry the divisibility constraint).

Readings where the pages leave a step open:
  * The pages name SwiGLU without defining it.  Reading: the standard gated
    form H = SiLU(X W_g) * (X W_u), SiLU(z) = z * sigma(z), sigma the
    logistic function, then Z = H B.
  * "Paired local shards": rank r owns columns [r*f, (r+1)*f) of BOTH W_g
    and W_u (f = F / t) and the same rows of B, so the gate and the value of
    every intermediate feature sit on one rank.
  * No biases in the gated projections (the row layer keeps the optional
    output bias and residual on rank 0, as in the GeLU MLP).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit

from .mlp import ShardError, _f64, row_linear, shard_slice

__all__ = ["silu", "swiglu_mlp_full", "swiglu_mlp_shard"]


def silu(z):
    """SiLU(z) = z * sigma(z), sigma(z) = 1 / (1 + exp(-z)) (SciPy's expit,
    which does not overflow for large |z|)."""
    z = np.asarray(z, dtype=np.float64)
    return z * expit(z)


def swiglu_mlp_full(x, wg, wu, b, bias_b=None, residual=None) -> np.ndarray:
    """Unsharded gated MLP: (SiLU(X W_g) * (X W_u)) B + b + R."""
    x, wg, wu = _f64(x), _f64(wg), _f64(wu)
    h = silu(x @ wg) * (x @ wu)
    return row_linear(h, b, bias_b, residual, rank=0)


def swiglu_mlp_shard(x, wg, wu, b, t: int, rank: int, bias_b=None, residual=None) -> np.ndarray:
    """Rank ``rank``'s partial: the paired column blocks S of W_g and W_u and
    the rows S of B, with S = shard_slice(F, t, rank); FULL weights in."""
    x, wg, wu, b = _f64(x), _f64(wg), _f64(wu), _f64(b)
    ffn = wg.shape[1]
    if wu.shape[1] != ffn or b.shape[0] != ffn:
        raise ShardError("W_g, W_u and B must share the FFN width")
    s = shard_slice(ffn, t, rank)
    h_r = silu(x @ wg[:, s]) * (x @ wu[:, s])
    return row_linear(h_r, b[s, :], bias_b, residual, rank=rank)
