"""tp_mlp_shard_fwd_noalloc (the MLP shard forward whose GeLU intermediate
lives in the library's fixed device array, for callers that cannot allocate)
against tp_mlp_shard_fwd with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input (the array keeps the first
call's contents), then an fp32 call: each output compared with the workspace
entry point's to the stated bounds (bf16 inputs: max |err| / (1 + |ref|) <=
2e-2 and relative Frobenius <= 5e-3; fp32: 1e-5).  The first call spans
three row chunks of the array (the last one ragged) with every optional
input; a shard width whose 256 rows of H_i would not fit is refused before
anything is enqueued.
"""
import numpy as np
import pytest
import torch

from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import assert_close, dev, nan_tensor, say, to_np

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _both(wl, rank, extras: bool, y_save: bool):
    """Outputs (z, y) of the workspace entry point and of the no-allocation one."""
    dt = wl.dtype
    x = dev(inputs.mlp_x_rows(wl), dt)
    a, b = dev(inputs.mlp_a_block(wl, rank), dt), dev(inputs.mlp_b_block(wl, rank), dt)
    kw = {}
    if extras:
        kw = dict(bias_a_i=dev(inputs.mlp_bias_a_block(wl, rank), dt), bias_b=dev(inputs.mlp_bias_b(wl), dt),
                  residual=dev(inputs.mlp_residual_rows(wl), dt))
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t, TORCH_DT[dt]),
                     dtype=torch.uint8, device="cuda")
    out = []
    for noalloc in (False, True):
        z = nan_tensor((wl.tokens, wl.hidden), TORCH_DT[wl.out_dtype])
        y = nan_tensor((wl.tokens, wl.f), TORCH_DT[dt]) if y_save else None
        if noalloc:
            binding.tp_mlp_shard_fwd_noalloc(x, a, b, z, ffn=wl.ffn, t=wl.t, rank=rank, y_save=y, **kw)
        else:
            binding.tp_mlp_shard_fwd(x, a, b, z, ws, ffn=wl.ffn, t=wl.t, rank=rank, y_save=y, **kw)
        torch.cuda.synchronize()
        out.append((z, y))
    return out


def _compare(wl, rank, extras, y_save, what):
    (z0, y0), (z1, y1) = _both(wl, rank, extras, y_save)
    dt = "bf16" if wl.dtype == "bf16" else "f32"
    say(f"{what}: outputs bit-identical to the workspace entry point: {torch.equal(z0, z1)}")
    assert_close(to_np(z1), to_np(z0), dt, f"{what} z")
    if y_save:
        assert_close(to_np(y1), to_np(y0), dt, f"{what} saved pre-activation")


def test_two_calls_second_smaller_then_f32():
    # 20000 tokens at f = 4096 (bf16): H_i rows of 8 KiB, 8192 rows per chunk
    # of the 64 MiB array -> chunks of 8192, 8192 and 3616 rows
    big = inputs.MlpWorkload("noalloc_big", 20000, 1024, 8192, 2, "bf16", 1.0, 0.03, 0.03, "f32")
    say("no-alloc call 1: 20000 tokens, hidden 1024, f 4096, rank 0, bias/residual/y_save")
    _compare(big, 0, True, True, "no-alloc 20000 tokens")
    small = inputs.MlpWorkload("noalloc_small", 300, 256, 1024, 2, "bf16", 1.0, 0.05, 0.05, "bf16")
    say("no-alloc call 2: 300 tokens, hidden 256, f 512, rank 1, bf16 out")
    _compare(small, 1, False, False, "no-alloc 300 tokens")
    wl32 = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    say("no-alloc call 3: tiny fp32 shard, rank 2")
    _compare(wl32, 2, True, True, "no-alloc fp32")


def test_width_beyond_the_array_is_refused():
    # f = 131080: 256 rows of bf16 H_i take 67.1 MB > 64 MiB
    f, hidden, tokens = 131080, 8, 300
    x = torch.zeros((tokens, hidden), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((hidden, f), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((f, hidden), dtype=torch.bfloat16, device="cuda")
    z = torch.full((tokens, hidden), 7.0, device="cuda")
    say("no-alloc: f = 131080 refused")
    with pytest.raises(binding.TpError, match="WORKSPACE"):
        binding.tp_mlp_shard_fwd_noalloc(x, a, b, z, ffn=2 * f, t=2, rank=0)
    torch.cuda.synchronize()
    assert torch.all(z == 7.0).item(), "nothing may be written when the call is refused"
