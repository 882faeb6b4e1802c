"""The Python binding refuses mismatched tensors before calling the library.

The C ABI sees raw pointers, so a tensor of the wrong shape, dtype or device
would turn into an out-of-bounds access inside a kernel.  Each wrapper checks
shapes and dtypes first, then that every operand lives on one GPU; all of it
runs before the library is touched, so these tests run on the CPU (host
tensors of the right shape are refused as "not a GPU tensor", which shows the
shape and dtype checks passed).
"""
import pytest
import torch

from megatron_tensor_transformer_tp_amd import binding

BF, F32 = torch.bfloat16, torch.float32


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def test_column_linear_shapes_dtypes_device():
    x, a, y = z(16, 64), z(64, 32), z(16, 32, dtype=F32)
    with pytest.raises(ValueError, match="a_i has shape"):
        binding.tp_column_linear(x, z(64, 33), y, ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="a_i has shape"):
        binding.tp_column_linear(x, z(32, 32), y, ffn=64, t=2, rank=0)   # hidden rows
    with pytest.raises(ValueError, match="y_i has shape"):
        binding.tp_column_linear(x, a, z(15, 32), ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="a_i has dtype"):
        binding.tp_column_linear(x, z(64, 32, dtype=F32), y, ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="bias_i has shape"):
        binding.tp_column_linear(x, a, y, ffn=64, t=2, rank=0, bias_i=z(64))
    with pytest.raises(ValueError, match="unsupported input dtype"):
        binding.tp_column_linear(z(16, 64, dtype=torch.float16), a, y, ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_column_linear(x, a, y, ffn=64, t=2, rank=0)


def test_row_linear_checks():
    h, b, out = z(16, 32), z(32, 64), z(16, 64, dtype=F32)
    with pytest.raises(ValueError, match="h_i has shape"):
        binding.tp_row_linear(z(16, 31), b, out, ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="b_i has shape"):
        binding.tp_row_linear(h, z(33, 64), out, ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="z_i has shape"):
        binding.tp_row_linear(h, b, z(16, 63, dtype=F32), ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="residual has shape"):
        binding.tp_row_linear(h, b, out, ffn=64, t=2, rank=0, residual=z(15, 64))
    with pytest.raises(ValueError, match="bias has dtype"):
        binding.tp_row_linear(h, b, out, ffn=64, t=2, rank=0, bias=z(64, dtype=F32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_row_linear(h, b, out, ffn=64, t=2, rank=0, bias=z(64), residual=z(16, 64))


def test_mlp_shard_fwd_checks():
    x, a, b = z(16, 64), z(64, 128), z(128, 64)
    out, ws = z(16, 64, dtype=F32), torch.zeros(16 * 128 * 2, dtype=torch.uint8)
    kw = dict(ffn=256, t=2, rank=0)
    with pytest.raises(ValueError, match="b_i has shape"):
        binding.tp_mlp_shard_fwd(x, a, z(64, 64), out, ws, **kw)
    with pytest.raises(ValueError, match="y_save has shape"):
        binding.tp_mlp_shard_fwd(x, a, b, out, ws, y_save=z(16, 64), **kw)
    with pytest.raises(ValueError, match="y_save has dtype"):
        binding.tp_mlp_shard_fwd(x, a, b, out, ws, y_save=z(16, 128, dtype=F32), **kw)
    with pytest.raises(ValueError, match="bias_a_i has shape"):
        binding.tp_mlp_shard_fwd(x, a, b, out, ws, bias_a_i=z(64), **kw)
    with pytest.raises(ValueError, match="must be contiguous"):
        binding.tp_mlp_shard_fwd(x, a, z(64, 128).t(), out, ws, **kw)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_mlp_shard_fwd(x, a, b, out, ws, **kw)
    # a split that does not divide is left to the library's own status code:
    # the shard-shape checks do not apply, the device check still does
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_mlp_shard_fwd(x, a, b, out, ws, ffn=257, t=2, rank=0)


def test_mlp_shard_bwd_checks():
    x, a, b, y, dz = z(16, 64), z(64, 128), z(128, 64), z(16, 128), z(16, 64)
    dx, da, db = z(16, 64, dtype=F32), z(64, 128, dtype=F32), z(128, 64, dtype=F32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    kw = dict(ffn=256, t=2, rank=1)
    with pytest.raises(ValueError, match="y_i has shape"):
        binding.tp_mlp_shard_bwd(x, a, b, z(16, 64), dz, dx, da, db, ws, **kw)
    with pytest.raises(ValueError, match="db_i has dtype"):
        binding.tp_mlp_shard_bwd(x, a, b, y, dz, dx, da, z(128, 64), ws, **kw)
    with pytest.raises(ValueError, match="dbias_a_i has dtype"):
        binding.tp_mlp_shard_bwd(x, a, b, y, dz, dx, da, db, ws, dbias_a_i=z(128), **kw)
    with pytest.raises(ValueError, match="dz has shape"):
        binding.tp_mlp_shard_bwd(x, a, b, y, z(17, 64), dx, da, db, ws, **kw)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_mlp_shard_bwd(x, a, b, y, dz, dx, da, db, ws, **kw)


def test_attention_and_swiglu_checks():
    x = z(2, 128, 256)
    wqkv, wo, out = z(256, 3 * 128), z(128, 256), z(2, 128, 256, dtype=F32)
    kw = dict(heads=2, head_dim=128, t=2, rank=0)
    with pytest.raises(ValueError, match="wqkv_i has shape"):
        binding.tp_attn_shard_fwd(x, z(256, 256), wo, out, None, **kw)
    with pytest.raises(ValueError, match="wo_i has shape"):
        binding.tp_attn_shard_fwd(x, wqkv, z(256, 256), out, None, **kw)
    with pytest.raises(ValueError, match="out_i has shape"):
        binding.tp_attn_shard_fwd(x, wqkv, wo, z(2, 127, 256, dtype=F32), None, **kw)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_attn_shard_fwd(x, wqkv, wo, out, None, **kw)

    x2, wg, b = z(16, 64), z(64, 32), z(32, 64)
    o2, ws = z(16, 64, dtype=F32), torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError, match="wu_i has shape"):
        binding.tp_mlp_swiglu_shard_fwd(x2, wg, z(64, 16), b, o2, ws, ffn=64, t=2, rank=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_mlp_swiglu_shard_fwd(x2, wg, wg, b, o2, ws, ffn=64, t=2, rank=0)


def test_sp_and_gelu_checks():
    parts = [z(8, 64, dtype=F32) for _ in range(4)]
    with pytest.raises(ValueError, match="partials\\[2\\] has shape"):
        binding.tp_sp_reduce_scatter(parts[:2] + [z(9, 64, dtype=F32)] + parts[3:], z(2, 64, dtype=F32),
                                     t=4, rank=0)
    with pytest.raises(ValueError, match="partials\\[0\\] has dtype"):
        binding.tp_sp_reduce_scatter([z(8, 64)] * 4, z(2, 64, dtype=F32), t=4, rank=0)
    with pytest.raises(ValueError, match="out_r has shape"):
        binding.tp_sp_reduce_scatter(parts, z(3, 64, dtype=F32), t=4, rank=0)
    with pytest.raises(ValueError, match="residual_r has shape"):
        binding.tp_sp_reduce_scatter(parts, z(2, 64, dtype=F32), t=4, rank=0, residual_r=z(8, 64))
    with pytest.raises(ValueError, match="4 partials for t=2"):
        binding.tp_sp_reduce_scatter(parts, z(4, 64, dtype=F32), t=2, rank=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_sp_reduce_scatter(parts, z(2, 64, dtype=F32), t=4, rank=0)
    with pytest.raises(ValueError, match="equal size"):
        binding.tp_gelu(z(8), z(9))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        binding.tp_gelu(z(8), z(8))
