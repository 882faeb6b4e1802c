"""Seeded synthetic inputs for the tensor-parallel MLP / attention shard.

This module is shared by the tests, the benchmark and the smoke check. It
draws random numbers and rounds them to bf16; it holds none of the method's
arithmetic (no matmul, no activation, no softmax, no sharding rule beyond
naming which block of a drawn tensor a seed belongs to).

Every tensor is drawn block by block from ``numpy.random.default_rng`` with a
``SeedSequence`` keyed on (workload, tensor, block).  Drawing by block lets a
caller materialise only the rows or the rank block it needs (for sampled
parity checks and the bounded host-side timing) and still get exactly the
values the full tensor holds.

Values are drawn in fp32.  For bf16 workloads they are rounded to bf16 with
round-to-nearest-even on the bit pattern; both the GPU side (as raw bf16
bits) and the oracle (widened exactly to fp64) consume the same rounded
values, so input quantisation is never counted as error.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

__all__ = [
    "MlpWorkload",
    "AttnWorkload",
    "MLP_WORKLOADS",
    "ATTN_WORKLOADS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "draw",
    "mlp_x_rows",
    "mlp_a_block",
    "mlp_b_block",
    "mlp_bias_a_block",
    "mlp_bias_b",
    "mlp_residual_rows",
    "mlp_dz_rows",
    "mlp_wg_block",
    "mlp_wu_block",
    "attn_x",
    "attn_wqkv_block",
    "attn_wo_block",
    "X_ROW_CHUNK",
]

# Rows of X (and of the residual) are drawn in chunks of this many tokens.
X_ROW_CHUNK = 256

_TENSOR_IDS = {"x": 0, "a": 1, "b": 2, "wqkv": 3, "wo": 4, "residual": 5,
               "bias_a": 6, "bias_b": 7, "dz": 8, "partial": 9,
               "wg": 10, "wu": 11}


@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    """Shapes and value distributions of one MLP workload.

    tokens = M (= seq x batch), hidden = h, ffn = F (= 4h), t = TP degree.
    ``*_std`` are standard deviations of the normal draws.
    """
    name: str
    tokens: int
    hidden: int
    ffn: int
    t: int
    dtype: str            # "bf16" or "f32": the dtype of X, A, B as handed to the path
    x_std: float
    a_std: float
    b_std: float
    out_dtype: str        # dtype of the partial Z_i the path writes

    @property
    def f(self) -> int:
        return self.ffn // self.t

    def flops_per_shard(self) -> int:
        return 4 * self.tokens * self.hidden * self.f


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    head_dim: int
    t: int
    dtype: str
    x_std: float
    w_std: float
    out_dtype: str
    wo_std: Optional[float] = None   # output projection std (default w_std)


MLP_WORKLOADS = {
    # Tiny fp32 MLP: 64 tokens (s=32, b=2), h=64, F=256, t=4, weights with
    # std 1/sqrt(fan_in) (fan_in = rows of the weight: 64 for A, 256 for B).
    "tiny_f32_t4": MlpWorkload("tiny_f32_t4", 64, 64, 256, 4, "f32",
                               1.0, 1.0 / np.sqrt(64.0), 1.0 / np.sqrt(256.0), "f32"),
    # Unsharded (t=1) bf16 MLP, 2048 tokens, h=1024: bf16 final output.
    "t1_h1024_m2048": MlpWorkload("t1_h1024_m2048", 2048, 1024, 4096, 1, "bf16",
                                  1.0, 0.02, 0.02, "bf16"),
    # Small sharded bf16 MLP, t=4: 1024 tokens, h=1024, F=4096 (f=1024), every
    # dimension a multiple of the 256 tile (backward and strided-view cases).
    "t4_h1024_m1024": MlpWorkload("t4_h1024_m1024", 1024, 1024, 4096, 4, "bf16",
                                  1.0, 0.02, 0.02, "f32"),
    # One rank of t=8 at h=8192, 4096 tokens: fp32 partial sum.
    "t8_h8192_m4096": MlpWorkload("t8_h8192_m4096", 4096, 8192, 32768, 8, "bf16",
                                  1.0, 0.02, 0.02, "f32"),
    # t=8 at h=8192, 16384 tokens: the headline shard shape.
    "t8_h8192_m16384": MlpWorkload("t8_h8192_m16384", 16384, 8192, 32768, 8, "bf16",
                                   1.0, 0.02, 0.02, "f32"),
}

ATTN_WORKLOADS = {
    # Small shards the oracle finishes in seconds: hidden 1024, 8 heads of
    # 128, t=2 (4 local heads).  QKV weight std chosen so the logits have std
    # ~3 like the large case (q std = sqrt(1024) * 0.057 ~ 1.8); output
    # projection std 0.02 * sqrt(1024 / 512) so the partial's scale (std of
    # O times sqrt(rows of W_o)) also matches the large case.
    # batch 2 x seq 384: 3 query blocks, 6 key blocks, tile-aligned projections.
    "attn_t2_h1024_b2_s384": AttnWorkload("attn_t2_h1024_b2_s384", 2, 384, 1024, 8, 128, 2,
                                          "bf16", 1.0, 0.057, "f32", 0.028),
    # batch 3 x seq 128: one query block, 384 tokens (not a multiple of 256).
    "attn_t2_h1024_b3_s128": AttnWorkload("attn_t2_h1024_b3_s128", 3, 128, 1024, 8, 128, 2,
                                          "bf16", 1.0, 0.057, "f32", 0.028),
    # Head-local attention shard: hidden 8192, 64 heads of 128, t=8 (8 local
    # heads), batch 1, seq 4096, non-causal.
    "attn_t8_h8192_s4096": AttnWorkload("attn_t8_h8192_s4096", 1, 4096, 8192, 64, 128, 8,
                                        "bf16", 1.0, 0.02, "f32"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs are finite (no NaN handling)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _seed(workload: str, tensor: str, block: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([zlib.crc32(workload.encode()), _TENSOR_IDS[tensor], block])


def draw(workload: str, tensor: str, block: int, shape, std: float, dtype: str) -> np.ndarray:
    """One seeded block: N(0, std^2) drawn in fp32, then rounded.

    Returns uint16 bf16 bit patterns for dtype "bf16", float32 for "f32".
    """
    rng = np.random.default_rng(_seed(workload, tensor, block))
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    if dtype == "f32":
        return v
    raise ValueError(f"unknown dtype {dtype!r}")


def mlp_x_rows(wl: MlpWorkload, row0: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """Rows [row0, row0+rows) of X [tokens, hidden]."""
    rows = wl.tokens - row0 if rows is None else rows
    if row0 < 0 or rows < 0 or row0 + rows > wl.tokens:
        raise ValueError("row range outside X")
    c0, c1 = row0 // X_ROW_CHUNK, (row0 + rows + X_ROW_CHUNK - 1) // X_ROW_CHUNK
    parts = []
    for c in range(c0, c1):
        n = min(X_ROW_CHUNK, wl.tokens - c * X_ROW_CHUNK)
        parts.append(draw(wl.name, "x", c, (n, wl.hidden), wl.x_std, wl.dtype))
    full = np.concatenate(parts, axis=0) if parts else np.zeros((0, wl.hidden),
                                                                 np.uint16 if wl.dtype == "bf16" else np.float32)
    off = row0 - c0 * X_ROW_CHUNK
    return np.ascontiguousarray(full[off:off + rows])


def mlp_a_block(wl: MlpWorkload, r: int) -> np.ndarray:
    """Column block r (width F/t) of A [hidden, F]; the full A is the
    concatenation of the blocks r = 0..t-1 along columns."""
    return draw(wl.name, "a", r, (wl.hidden, wl.f), wl.a_std, wl.dtype)


def mlp_b_block(wl: MlpWorkload, r: int) -> np.ndarray:
    """Row block r (height F/t) of B [F, hidden]; the full B is the
    concatenation of the blocks along rows."""
    return draw(wl.name, "b", r, (wl.f, wl.hidden), wl.b_std, wl.dtype)


def mlp_bias_a_block(wl: MlpWorkload, r: int, std: float = 0.1) -> np.ndarray:
    """Block r (length F/t) of an optional first-layer bias a [F]."""
    return draw(wl.name, "bias_a", r, (wl.f,), std, wl.dtype)


def mlp_bias_b(wl: MlpWorkload, std: float = 0.1) -> np.ndarray:
    """Optional second-layer bias b [hidden]."""
    return draw(wl.name, "bias_b", 0, (wl.hidden,), std, wl.dtype)


def mlp_residual_rows(wl: MlpWorkload, row0: int = 0, rows: Optional[int] = None,
                      std: float = 1.0) -> np.ndarray:
    """Rows of an optional residual R [tokens, hidden]."""
    rows = wl.tokens - row0 if rows is None else rows
    c0, c1 = row0 // X_ROW_CHUNK, (row0 + rows + X_ROW_CHUNK - 1) // X_ROW_CHUNK
    parts = [draw(wl.name, "residual", c, (min(X_ROW_CHUNK, wl.tokens - c * X_ROW_CHUNK), wl.hidden),
                  std, wl.dtype) for c in range(c0, c1)]
    full = np.concatenate(parts, axis=0)
    off = row0 - c0 * X_ROW_CHUNK
    return np.ascontiguousarray(full[off:off + rows])


def mlp_wg_block(wl: MlpWorkload, r: int) -> np.ndarray:
    """Column block r [hidden, f] of the SwiGLU gate projection [hidden, ffn]
    (same distribution as A)."""
    return draw(wl.name, "wg", r, (wl.hidden, wl.f), wl.a_std, wl.dtype)


def mlp_wu_block(wl: MlpWorkload, r: int) -> np.ndarray:
    """Column block r [hidden, f] of the SwiGLU value projection."""
    return draw(wl.name, "wu", r, (wl.hidden, wl.f), wl.a_std, wl.dtype)


def mlp_dz_rows(wl: MlpWorkload, row0: int = 0, rows: Optional[int] = None,
                std: float = 1.0) -> np.ndarray:
    """Rows of the output gradient dZ [tokens, hidden] fed to the backward
    (N(0, std^2), drawn in 256-row chunks like X)."""
    rows = wl.tokens - row0 if rows is None else rows
    c0, c1 = row0 // X_ROW_CHUNK, (row0 + rows + X_ROW_CHUNK - 1) // X_ROW_CHUNK
    parts = [draw(wl.name, "dz", c, (min(X_ROW_CHUNK, wl.tokens - c * X_ROW_CHUNK), wl.hidden),
                  std, wl.dtype) for c in range(c0, c1)]
    full = np.concatenate(parts, axis=0)
    off = row0 - c0 * X_ROW_CHUNK
    return np.ascontiguousarray(full[off:off + rows])


def attn_x(wl: AttnWorkload, b: int, row0: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """Rows [row0, row0+rows) of batch b of X [batch, seq, hidden]."""
    rows = wl.seq - row0 if rows is None else rows
    c0, c1 = row0 // X_ROW_CHUNK, (row0 + rows + X_ROW_CHUNK - 1) // X_ROW_CHUNK
    nchunk = (wl.seq + X_ROW_CHUNK - 1) // X_ROW_CHUNK
    parts = [draw(wl.name, "x", b * nchunk + c, (min(X_ROW_CHUNK, wl.seq - c * X_ROW_CHUNK), wl.hidden),
                  wl.x_std, wl.dtype) for c in range(c0, c1)]
    full = np.concatenate(parts, axis=0)
    off = row0 - c0 * X_ROW_CHUNK
    return np.ascontiguousarray(full[off:off + rows])


def attn_wqkv_block(wl: AttnWorkload, r: int) -> np.ndarray:
    """Column block r (width 3*hidden/t) of the packed QKV weight [hidden, 3*hidden]."""
    return draw(wl.name, "wqkv", r, (wl.hidden, 3 * wl.hidden // wl.t), wl.w_std, wl.dtype)


def attn_wo_block(wl: AttnWorkload, r: int) -> np.ndarray:
    """Row block r (height hidden/t) of the output projection [hidden, hidden]."""
    std = wl.w_std if wl.wo_std is None else wl.wo_std
    return draw(wl.name, "wo", r, (wl.hidden // wl.t, wl.hidden), std, wl.dtype)
