"""Pure-Python brute-force forms of the MLP shard and one attention head.

TEST INFRASTRUCTURE ONLY.  Written straight from the index definitions with
``math.erf`` and explicit loops (no NumPy arithmetic), so that a mistake in the
vectorised oracle (a transposed operand, a wrong block index, a dropped bias)
shows up as a disagreement.  Only for tiny sizes.
"""
from __future__ import annotations

import math

__all__ = ["mlp_shard_loops", "attention_head_loops"]


def mlp_shard_loops(x, a, b, t, rank, bias_a=None, bias_b=None, residual=None):
    """Z_r[m][n] = sum_{j in S_r} GeLU(sum_k x[m][k] a[k][j] + bias_a[j]) b[j][n]
    (+ bias_b[n] + residual[m][n] when rank == 0), S_r = [r*F/t, (r+1)*F/t).

    ``x``, ``a``, ``b`` are nested lists (or anything indexable [i][j]) of the
    FULL tensors."""
    M, K = len(x), len(x[0])
    F, N = len(a[0]), len(b[0])
    assert len(a) == K and len(b) == F and F % t == 0
    f = F // t
    cols = range(rank * f, (rank + 1) * f)
    out = [[0.0] * N for _ in range(M)]
    for m in range(M):
        hrow = {}
        for j in cols:
            acc = 0.0
            for k in range(K):
                acc += float(x[m][k]) * float(a[k][j])
            if bias_a is not None:
                acc += float(bias_a[j])
            hrow[j] = 0.5 * acc * (1.0 + math.erf(acc / math.sqrt(2.0)))
        for n in range(N):
            s = 0.0
            for j in cols:
                s += hrow[j] * float(b[j][n])
            if rank == 0:
                if bias_b is not None:
                    s += float(bias_b[n])
                if residual is not None:
                    s += float(residual[m][n])
            out[m][n] = s
    return out


def attention_head_loops(q, k, v, causal=False):
    """O[i][e] = sum_j p[i][j] v[j][e], p[i][.] = softmax_j(q_i . k_j / sqrt(d))
    over keys j (j <= i when causal)."""
    n, d = len(q), len(q[0])
    nk, dv = len(k), len(v[0])
    out = []
    for i in range(n):
        keys = range(min(i + 1, nk)) if causal else range(nk)
        logits = []
        for j in keys:
            s = 0.0
            for e in range(d):
                s += float(q[i][e]) * float(k[j][e])
            logits.append(s / math.sqrt(d))
        mx = max(logits)
        w = [math.exp(l - mx) for l in logits]
        tot = sum(w)
        row = []
        for e in range(dv):
            acc = 0.0
            for wi, j in zip(w, keys):
                acc += wi * float(v[j][e])
            row.append(acc / tot)
        out.append(row)
    return out


def swiglu_shard_loops(x, wg, wu, b, t, rank):
    """Rank ``rank``'s SwiGLU partial with explicit loops and math.exp."""
    tokens, hidden = len(x), len(x[0])
    ffn = len(wg[0])
    f = ffn // t
    cols = range(rank * f, (rank + 1) * f)
    out_w = len(b[0])
    z = [[0.0] * out_w for _ in range(tokens)]
    for m in range(tokens):
        h = []
        for c in cols:
            g = sum(x[m][k] * wg[k][c] for k in range(hidden))
            u = sum(x[m][k] * wu[k][c] for k in range(hidden))
            h.append(g / (1.0 + math.exp(-g)) * u)
        for n in range(out_w):
            z[m][n] = sum(h[j] * b[c][n] for j, c in enumerate(cols))
    return z
