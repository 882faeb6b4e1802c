"""fp64 CPU oracle of one tensor-parallel rank's share of the Transformer MLP.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's host-baseline leg may import this module; the GPU product path
never does, and this module imports nothing from it.

Everything is the plain definition, in float64, with NumPy's ``@`` as the
matmul primitive and SciPy's ``erfc`` for the normal CDF.  There is no
blocking, fusion or reordering beyond what the definitions state.

Notation (shared by the pages up to renaming):
  X [M, h]       tokens x hidden, replicated on every rank
  A [h, F]       first MLP weight, F = 4h;  A_r = columns [r*f, (r+1)*f), f = F/t
  B [F, h]       second MLP weight;         B_r = rows    [r*f, (r+1)*f)
  Y_r = X A_r,   H_r = GeLU(Y_r),           Z_r = H_r B_r   (full-hidden partial)
  Z = sum_r Z_r = GeLU(X A) B

Passages followed (page titles as printed on each page):
  * Tencent Hunyuan AI-Infra first-round interview write-up
    (mj.mianlingai.com), answer section 参考解析: column split of W by output
    columns, row split by input rows, FFN = column layer, GeLU, row layer with
    one All-Reduce at the end.
  * 列并行 tutorial (aiqz.cc/article/old-parallel.html), sections 切分原理
    (W split into p column blocks, divisibility), 数学基础 (column-concat
    identity Y = [XW^(1) || ... || XW^(p)]), MLP 应用 (GeLU(z) = z*Phi(z), block
    invariance of GeLU, final sum over ranks of Z_i B^(i)).
  * Megatron expert interview Level 2 (blog.cptz.space), items M025
    (ColumnParallelLinear shapes: W_i [h, 4h/t], Y_i [s, b, 4h/t]), M026
    (RowParallelLinear: each rank contributes a full-hidden partial, summed),
    M031 (fail fast on shapes that do not divide).
  * Distributed-parallelism overview (talentme.airsota.com), 考点 2 (MLP: GeLU
    on column shards, Z = Z_1 + Z_2 with one All-Reduce) and 第三章 (contiguous
    column slices of W1, row slices of W2 with the same indices, summed over
    ranks).
  * Backward (Megatron Level 2, M025 and M026): for Y = X W with W split by
    columns, dW_i = X^T dY_i is local and the input-gradient contributions
    dY_i W_i^T are SUM-reduced over the ranks; for the row-split layer the
    input gradient dY W_i^T is already the rank's input-block gradient and
    dW_i is local.  Chained through the elementwise GeLU with the product
    rule, d/dz [z Phi(z)] = Phi(z) + z phi(z).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
from scipy.special import erfc

__all__ = [
    "ShardError",
    "shard_width",
    "shard_slice",
    "gelu",
    "column_linear",
    "row_linear",
    "mlp_full",
    "mlp_shard",
    "mlp_partial_sum",
    "normal_pdf",
    "gelu_grad",
    "mlp_shard_bwd",
]


class ShardError(ValueError):
    """A shape that the tensor-parallel split cannot take (rejected, never padded)."""


def shard_width(ffn: int, t: int) -> int:
    """f = F / t.  The split dimension must divide evenly by the TP degree
    (列并行 tutorial, 切分原理; Megatron Level 2, M031): otherwise the ranks
    would hold blocks of different widths, which the method rejects."""
    if not isinstance(t, (int, np.integer)) or t < 1:
        raise ShardError(f"TP degree t must be a positive integer, got {t!r}")
    if ffn < 1:
        raise ShardError(f"split dimension must be positive, got {ffn}")
    if ffn % t != 0:
        raise ShardError(f"split dimension {ffn} is not divisible by t={t}")
    return ffn // t


def shard_slice(ffn: int, t: int, rank: int) -> slice:
    """Index set owned by ``rank``: the contiguous block [rank*f, (rank+1)*f).
    The same set selects A's columns and B's rows (overview page, 第三章)."""
    f = shard_width(ffn, t)
    if not (0 <= rank < t):
        raise ShardError(f"rank {rank} outside [0, {t})")
    return slice(rank * f, (rank + 1) * f)


def gelu(z):
    """Exact GeLU, z * Phi(z) with Phi the standard normal CDF (列并行
    tutorial, MLP 应用).  Phi(z) = erfc(-z / sqrt(2)) / 2, which equals
    (1 + erf(z / sqrt(2))) / 2 without its cancellation for z << 0."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * erfc(-z / math.sqrt(2.0))


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def column_linear(x, a_i, bias_i=None, apply_gelu: bool = False) -> np.ndarray:
    """Column-parallel linear on one rank: Y_i = X A_i (+ a_i), optionally
    followed by the elementwise GeLU.  X is the full input; A_i is the rank's
    [h, f] column block; the result is the rank's [M, f] column block of the
    full output (Tencent write-up, 参考解析; Megatron Level 2, M025)."""
    x, a_i = _f64(x), _f64(a_i)
    if x.ndim != 2 or a_i.ndim != 2 or x.shape[1] != a_i.shape[0]:
        raise ShardError(f"shape mismatch X{x.shape} @ A_i{a_i.shape}")
    y = x @ a_i
    if bias_i is not None:
        y = y + _f64(bias_i)[None, :]
    return gelu(y) if apply_gelu else y


def row_linear(h_i, b_i, bias=None, residual=None, rank: int = 0) -> np.ndarray:
    """Row-parallel linear on one rank: Z_i = H_i B_i, a full-hidden [M, h]
    contribution that the ranks sum (Megatron Level 2, M026; overview page,
    考点 2).  The bias and residual belong to the summed output, so only
    rank 0 adds them; this keeps sum_i Z_i equal to the unsharded layer."""
    h_i, b_i = _f64(h_i), _f64(b_i)
    if h_i.ndim != 2 or b_i.ndim != 2 or h_i.shape[1] != b_i.shape[0]:
        raise ShardError(f"shape mismatch H_i{h_i.shape} @ B_i{b_i.shape}")
    z = h_i @ b_i
    if rank == 0:
        if bias is not None:
            z = z + _f64(bias)[None, :]
        if residual is not None:
            z = z + _f64(residual)
    return z


def mlp_full(x, a, b, bias_a=None, bias_b=None, residual=None) -> np.ndarray:
    """Unsharded MLP: GeLU(X A + a) B + b + R (the single-device reference the
    pages compare the sharded computation against)."""
    h = column_linear(x, a, bias_a, apply_gelu=True)
    return row_linear(h, b, bias_b, residual, rank=0)


def mlp_shard(x, a, b, t: int, rank: int, bias_a=None, bias_b=None,
              residual=None) -> np.ndarray:
    """Rank ``rank``'s partial Z_r = GeLU(X A[:, S] + a[S]) B[S, :]
    (+ b + R on rank 0), with S = shard_slice(F, t, rank).  ``a`` and ``b``
    are the FULL weights; the rank's blocks are cut here."""
    a, b = _f64(a), _f64(b)
    ffn = a.shape[1]
    if b.shape[0] != ffn:
        raise ShardError(f"A is [h, {ffn}] but B has {b.shape[0]} rows")
    s = shard_slice(ffn, t, rank)
    bias_i = None if bias_a is None else _f64(bias_a)[s]
    h_i = column_linear(x, a[:, s], bias_i, apply_gelu=True)
    return row_linear(h_i, b[s, :], bias_b, residual, rank=rank)


def mlp_partial_sum(x, a, b, t: int, bias_a=None, bias_b=None, residual=None,
                    activation: Optional[str] = None) -> np.ndarray:
    """sum_r Z_r over all t ranks: the value the exchange step (a SUM
    All-Reduce) would hand every rank.  ``activation="relu"`` swaps GeLU for
    ReLU, as the overview page's NumPy simulation does; the identity with the
    unsharded layer holds for any elementwise activation."""
    a, b = _f64(a), _f64(b)
    total = None
    for r in range(t):
        if activation is None:
            z = mlp_shard(x, a, b, t, r, bias_a, bias_b, residual)
        elif activation == "relu":
            s = shard_slice(a.shape[1], t, r)
            y = column_linear(x, a[:, s], None if bias_a is None else _f64(bias_a)[s])
            z = row_linear(np.maximum(y, 0.0), b[s, :], bias_b, residual, rank=r)
        else:
            raise ValueError(activation)
        total = z if total is None else total + z
    return total


def normal_pdf(z):
    """Standard normal density phi(z) = exp(-z^2 / 2) / sqrt(2 pi)."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gelu_grad(z):
    """d/dz GeLU(z) = Phi(z) + z phi(z): the product rule on z * Phi(z), with
    Phi' = phi (GeLU as defined in the 列并行 tutorial, MLP 应用)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * erfc(-z / math.sqrt(2.0)) + z * normal_pdf(z)


def mlp_shard_bwd(x, a, b, dz, t: int, rank: int, bias_a=None) -> dict:
    """Backward of rank ``rank``'s MLP shard, given dz = dL/dZ of the summed
    output Z = sum_r Z_r (the same on every rank), with FULL weights ``a``
    [h, F] and ``b`` [F, h] (the rank's blocks are cut here).

    Forward values recomputed from the definition:
      Y_r = X A_r + a_r,  H_r = GeLU(Y_r).
    Row-parallel layer Z_r = H_r B_r (M026): its input gradient
      dH_r = dz B_r^T is the rank's own block, dB_r = H_r^T dz is local.
    GeLU, elementwise: dY_r = dH_r * GeLU'(Y_r).
    Column-parallel layer Y_r = X A_r (M025): dA_r = X^T dY_r is local;
      dX_r = dY_r A_r^T is the rank's contribution to dX (summed over ranks).
    Biases: a_r is added to every token row, so its gradient is the sum of
      dY_r over tokens; the output bias b (added once, on rank 0) gets the
      sum of dz over tokens, the same on every rank.

    Returns dict(y, dx, da, db, dbias_a, dbias_b) in fp64, with da [h, f] and
    db [f, h] the rank's blocks of dA and dB."""
    x, a, b, dz = _f64(x), _f64(a), _f64(b), _f64(dz)
    ffn = a.shape[1]
    if b.shape[0] != ffn:
        raise ShardError(f"A is [h, {ffn}] but B has {b.shape[0]} rows")
    if dz.shape != (x.shape[0], b.shape[1]):
        raise ShardError(f"dz is {dz.shape}, expected {(x.shape[0], b.shape[1])}")
    s = shard_slice(ffn, t, rank)
    a_r, b_r = a[:, s], b[s, :]
    bias_r = None if bias_a is None else _f64(bias_a)[s]
    y = column_linear(x, a_r, bias_r)
    h = gelu(y)
    dh = dz @ b_r.T
    dy = dh * gelu_grad(y)
    return {
        "y": y,
        "dx": dy @ a_r.T,
        "da": x.T @ dy,
        "db": h.T @ dz,
        "dbias_a": dy.sum(axis=0),
        "dbias_b": dz.sum(axis=0),
    }
