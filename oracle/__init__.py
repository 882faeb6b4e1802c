"""Plain, slow, fp64 CPU oracle of the tensor-parallel MLP and attention shards.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by the smoke check and by
the benchmark's host-baseline leg, never by the GPU product package, and it
imports nothing from that package.  See ``mlp.py`` and ``attention.py`` for
the passages each function follows.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
except the per-head packing convention of the QKV weight, which no page fixes
(parity unpinned for that convention; it is pinned only internally, by the
equality of the sharded form with full multi-head attention).
"""
from .mlp import (ShardError, shard_width, shard_slice, gelu, column_linear, row_linear,
                  mlp_full, mlp_shard, mlp_partial_sum, normal_pdf, gelu_grad, mlp_shard_bwd)
from .attention import (softmax_rows, split_packed_qkv, mha_full, attn_shard, attn_partial_sum,
                        local_heads)
from .brute import mlp_shard_loops, attention_head_loops, swiglu_shard_loops
from .sp import sp_shard_rows, sp_reduce_scatter
from .swiglu import silu, swiglu_mlp_full, swiglu_mlp_shard

__all__ = [
    "ShardError", "shard_width", "shard_slice", "gelu", "column_linear", "row_linear",
    "mlp_full", "mlp_shard", "mlp_partial_sum", "normal_pdf", "gelu_grad", "mlp_shard_bwd",
    "softmax_rows", "split_packed_qkv",
    "mha_full", "attn_shard", "attn_partial_sum", "local_heads", "mlp_shard_loops",
    "attention_head_loops", "sp_shard_rows", "sp_reduce_scatter", "silu", "swiglu_mlp_full",
    "swiglu_mlp_shard", "swiglu_shard_loops",
]
