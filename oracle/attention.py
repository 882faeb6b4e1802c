"""fp64 CPU oracle of one tensor-parallel rank's head-local attention shard.

TEST INFRASTRUCTURE ONLY (see ``oracle/mlp.py``): only tests, the smoke check
and the benchmark's host-baseline leg use it.

Definition followed:
  * Tencent Hunyuan AI-Infra interview write-up (mj.mianlingai.com), 参考解析,
    attention paragraph: the Q, K, V projections are split by heads, each rank
    owning heads/t of them; every rank computes softmax(Q K^T / sqrt(d)) V for
    its own heads with no communication; with a packed QKV matrix the column
    split must keep each head's Q, K and V blocks on one rank, so the packed
    layout interleaves them per head; the output projection is row-parallel
    and its partial sums are All-Reduced.
  * Megatron expert interview Level 2 (blog.cptz.space), M028: QKV projection
    column-parallel over heads, local attention, row-parallel output
    projection; the softmax reduces over keys, not heads.

Readings where the pages leave a step open:
  * Packed QKV layout: per-head blocks [q | k | v], each head_dim wide, i.e.
    column j*3d + c*d + e of W_qkv is column j*d + e of W_c, c in (q, k, v).
    Rank r's shard is columns [r*3h/t, (r+1)*3h/t) of W_qkv.  The pages only
    say "interleaved"; any fixed per-head permutation would do.  PARITY
    UNPINNED for this convention beyond internal consistency with the full
    multi-head form (no page fixes it).
  * Scale 1/sqrt(head_dim); no mask (non-causal) unless ``causal``; no
    projection biases; no dropout.
"""
from __future__ import annotations

import math

import numpy as np

from .mlp import ShardError

__all__ = [
    "softmax_rows",
    "split_packed_qkv",
    "mha_full",
    "attn_shard",
    "attn_partial_sum",
    "local_heads",
]


def local_heads(heads: int, t: int) -> int:
    """heads / t; the head count must divide by the TP degree (Megatron
    Level 2, M031)."""
    if t < 1:
        raise ShardError(f"TP degree t must be positive, got {t}")
    if heads % t != 0:
        raise ShardError(f"heads={heads} not divisible by t={t}")
    return heads // t


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax in fp64 (max subtracted before exp; exact up to rounding)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def split_packed_qkv(wqkv: np.ndarray, heads: int, head_dim: int):
    """Undo the per-head [q|k|v] packing: return W_q, W_k, W_v, each
    [h, heads*head_dim] with head j in columns [j*d, (j+1)*d)."""
    w = np.asarray(wqkv, dtype=np.float64)
    hid, cols = w.shape
    if cols != 3 * heads * head_dim:
        raise ShardError(f"packed QKV has {cols} columns, expected {3 * heads * head_dim}")
    w3 = w.reshape(hid, heads, 3, head_dim)
    return tuple(np.ascontiguousarray(w3[:, :, c, :].reshape(hid, heads * head_dim)) for c in range(3))


def _attend(q, k, v, causal: bool, qpos=None) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v for one head; q [n, d] at sequence positions
    ``qpos`` (default 0..n-1), k, v [s, d].  Causal: query i sees keys j <= i."""
    d = q.shape[-1]
    s = (q @ k.T) / math.sqrt(d)
    if causal:
        qpos = np.arange(q.shape[0]) if qpos is None else np.asarray(qpos)
        s = np.where(np.arange(k.shape[0])[None, :] <= qpos[:, None], s, -np.inf)
    return softmax_rows(s) @ v


def mha_full(x, wq, wk, wv, wo, heads: int, causal: bool = False) -> np.ndarray:
    """Standard multi-head attention, unsharded: x [batch, seq, h]; W_q, W_k,
    W_v [h, heads*d]; W_o [heads*d, h]; out = concat_j(O_j) W_o."""
    x = np.asarray(x, dtype=np.float64)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    d = wq.shape[1] // heads
    out = np.empty((x.shape[0], x.shape[1], wo.shape[1]))
    for bi in range(x.shape[0]):
        q, k, v = x[bi] @ wq, x[bi] @ wk, x[bi] @ wv
        o = np.concatenate([_attend(q[:, j * d:(j + 1) * d], k[:, j * d:(j + 1) * d],
                                    v[:, j * d:(j + 1) * d], causal) for j in range(heads)], axis=1)
        out[bi] = o @ wo
    return out


def attn_shard(x, wqkv_i, wo_i, heads: int, head_dim: int, t: int, rank: int,
               causal: bool = False, rows=None) -> np.ndarray:
    """Rank ``rank``'s fp64 partial: its heads/t local heads from the packed
    QKV column block ``wqkv_i`` [h, 3*h_loc], local attention per head, and
    the row block ``wo_i`` [h_loc, h] of the output projection.  Returns the
    full-hidden [batch, seq, h] contribution that the ranks sum, or only the
    query positions ``rows`` ([batch, len(rows), h]; every key is still used:
    each output row is defined by its own query alone)."""
    nl = local_heads(heads, t)
    if not (0 <= rank < t):
        raise ShardError(f"rank {rank} outside [0, {t})")
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(wqkv_i, dtype=np.float64)
    wo_i = np.asarray(wo_i, dtype=np.float64)
    d = head_dim
    if w.shape[1] != 3 * nl * d or wo_i.shape[0] != nl * d:
        raise ShardError("shard weight shapes do not match heads/t x head_dim")
    qrows = np.arange(x.shape[1]) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], len(qrows), wo_i.shape[1]))
    for bi in range(x.shape[0]):
        qkv = x[bi] @ w
        heads_out = []
        for j in range(nl):
            base = j * 3 * d
            q, k, v = qkv[qrows, base:base + d], qkv[:, base + d:base + 2 * d], qkv[:, base + 2 * d:base + 3 * d]
            heads_out.append(_attend(q, k, v, causal, qrows))
        out[bi] = np.concatenate(heads_out, axis=1) @ wo_i
    return out


def attn_partial_sum(x, wqkv, wo, heads: int, head_dim: int, t: int,
                     causal: bool = False) -> np.ndarray:
    """sum over ranks of attn_shard, cutting rank r's blocks from the FULL
    packed W_qkv [h, 3h] (columns) and W_o [h, h] (rows)."""
    hid = np.asarray(wqkv).shape[0]
    nl = local_heads(heads, t)
    wcols = 3 * nl * head_dim
    wrows = nl * head_dim
    total = None
    for r in range(t):
        z = attn_shard(x, np.asarray(wqkv)[:, r * wcols:(r + 1) * wcols],
                       np.asarray(wo)[r * wrows:(r + 1) * wrows, :], heads, head_dim, t, r, causal)
        total = z if total is None else total + z
    del hid
    return total
