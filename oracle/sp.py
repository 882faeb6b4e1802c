"""fp64 CPU oracle of the sequence-parallel boundary of the MLP shard.

TEST INFRASTRUCTURE ONLY (see ``oracle/mlp.py``): only tests, the smoke check
and the benchmark's host-baseline leg use it.

Definition followed: Megatron expert interview Level 2 (blog.cptz.space),
M034.  With sequence parallelism the row-parallel layer's full-hidden
partials [s, b, h] are not All-Reduced; a SUM Reduce-Scatter both sums them
and leaves each rank the sequence shard [s/t, b, h], on which the per-token
operations that follow (bias, residual) run locally.  Following an
All-Gather, the shards re-form the summed output (the Reduce-Scatter and the
All-Gather together are the All-Reduce).

Readings where the page leaves a step open:
  * Token rows are ordered sequence-major ([s, b] flattened), so rank r's
    sequence shard is the contiguous row block [r*M/t, (r+1)*M/t) of the
    M = s*b rows; M must divide by t (rejected otherwise, like every split).
  * The output bias b and the residual are added after the reduction, each
    rank on its own rows (the residual stream is sequence-sharded too, so
    each rank passes only its [M/t, h] rows of it).
"""
from __future__ import annotations

import numpy as np

from .mlp import ShardError

__all__ = ["sp_shard_rows", "sp_reduce_scatter"]


def sp_shard_rows(tokens: int, t: int, rank: int) -> slice:
    """Rank ``rank``'s sequence shard: rows [rank*M/t, (rank+1)*M/t)."""
    if t < 1 or not (0 <= rank < t):
        raise ShardError(f"rank {rank} outside [0, {t})")
    if tokens % t != 0:
        raise ShardError(f"tokens={tokens} not divisible by t={t}")
    m = tokens // t
    return slice(rank * m, (rank + 1) * m)


def sp_reduce_scatter(partials, t: int, rank: int, bias=None, residual_r=None) -> np.ndarray:
    """Rank ``rank``'s shard of sum_j partials[j], plus the bias and the rank's
    residual rows: [M/t, h] in fp64."""
    parts = [np.asarray(p, dtype=np.float64) for p in partials]
    if len(parts) != t:
        raise ShardError(f"{len(parts)} partials for t={t}")
    rows = sp_shard_rows(parts[0].shape[0], t, rank)
    out = sum(p[rows] for p in parts)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    if residual_r is not None:
        out = out + np.asarray(residual_r, dtype=np.float64)
    return out
