"""One tensor-parallel rank's share of the Megatron Transformer MLP (and the
head-local attention shard) as hand-written HIP kernels for gfx950, behind a
C-ABI library.  ``binding`` holds the thin Python marshalling layer; it loads
the compiled library on first use and raises if it is missing.
"""
__all__ = ["binding", "inputs"]
