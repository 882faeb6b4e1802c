"""GPU parity of the sequence-parallel boundary (tp_sp_reduce_scatter)
against the fp64 oracle: random fp32 partials, and the whole chain (the
ranks' MLP partials without bias / residual, then the reduce-scatter with
them) against the unsharded layer.  Outputs NaN-filled before each call."""
import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import assert_close, dev, host64, nan_tensor, say, to_np

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def partials_for(name, t, tokens, hidden):
    return [inputs.draw(name, "partial", j, (tokens, hidden), 1.0, "f32") for j in range(t)]


@pytest.mark.parametrize("t,tokens,hidden,in_dt,out_dt,extras,ranks", [
    (4, 64, 64, "f32", "f32", "bias+res", None),
    (2, 74, 1000, "f32", "f32", "res", None),
    (8, 4096, 8192, "bf16", "f32", "bias+res", (0, 7)),
    (8, 4096, 8192, "bf16", "bf16", "bias+res", (3,)),
    (8, 2048, 4096, "bf16", "f32", "none", (5,)),
])
def test_random_partials(t, tokens, hidden, in_dt, out_dt, extras, ranks):
    name = f"sp_t{t}_m{tokens}_h{hidden}"
    parts = partials_for(name, t, tokens, hidden)
    parts_d = [dev(p, "f32") for p in parts]
    rows = tokens // t
    bias = inputs.draw(name, "bias_b", 0, (hidden,), 0.1, in_dt) if "bias" in extras else None
    res = inputs.draw(name, "residual", 0, (tokens, hidden), 1.0, in_dt) if "res" in extras else None
    for r in (ranks if ranks is not None else range(t)):
        say(f"{name} rank {r} {in_dt}->{out_dt} {extras}")
        res_r = None if res is None else np.ascontiguousarray(res[r * rows:(r + 1) * rows])
        out = nan_tensor((rows, hidden), TORCH_DT[out_dt])
        binding.tp_sp_reduce_scatter(parts_d, out, t=t, rank=r,
                                     bias=None if bias is None else dev(bias, in_dt),
                                     residual_r=None if res_r is None else dev(res_r, in_dt))
        torch.cuda.synchronize()
        ref = oracle.sp_reduce_scatter(parts, t, r,
                                       None if bias is None else host64(bias, in_dt),
                                       None if res_r is None else host64(res_r, in_dt))
        assert_close(to_np(out), ref, out_dt, f"{name} rank {r}")


def test_mlp_chain_with_sequence_parallel_boundary():
    """Row-parallel partials of every rank (no bias / residual in the GEMM),
    then each rank's reduce-scatter with the output bias and its residual
    rows: the shards stacked in rank order are the unsharded layer output."""
    wl = inputs.MLP_WORKLOADS["t4_h1024_m1024"]
    x = inputs.mlp_x_rows(wl)
    a_blocks = [inputs.mlp_a_block(wl, r) for r in range(wl.t)]
    b_blocks = [inputs.mlp_b_block(wl, r) for r in range(wl.t)]
    bias_b, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    xd = dev(x, "bf16")
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                          torch.bfloat16), dtype=torch.uint8, device="cuda")
    parts = []
    for r in range(wl.t):
        z = nan_tensor((wl.tokens, wl.hidden), torch.float32)
        binding.tp_mlp_shard_fwd(xd, dev(a_blocks[r], "bf16"), dev(b_blocks[r], "bf16"), z, ws,
                                 ffn=wl.ffn, t=wl.t, rank=r)
        parts.append(z)
    rows = wl.tokens // wl.t
    shards = []
    for r in range(wl.t):
        say(f"t4_h1024_m1024 sequence shard {r}")
        out = nan_tensor((rows, wl.hidden), torch.bfloat16)
        binding.tp_sp_reduce_scatter(parts, out, t=wl.t, rank=r, bias=dev(bias_b, "bf16"),
                                     residual_r=dev(np.ascontiguousarray(res[r * rows:(r + 1) * rows]), "bf16"))
        shards.append(out)
    torch.cuda.synchronize()
    got = np.concatenate([to_np(s) for s in shards], axis=0)
    ref = oracle.mlp_full(host64(x, "bf16"), host64(np.concatenate(a_blocks, axis=1), "bf16"),
                          host64(np.concatenate(b_blocks, axis=0), "bf16"), None,
                          host64(bias_b, "bf16"), host64(res, "bf16"))
    assert_close(got, ref, "bf16", "sequence shards stacked vs unsharded layer")


def test_errors():
    parts = [torch.zeros((10, 64), device="cuda") for _ in range(4)]
    out = torch.zeros((2, 64), device="cuda")
    with pytest.raises(binding.TpError, match="NOT_DIVISIBLE"):
        binding.tp_sp_reduce_scatter(parts, out, t=4, rank=0)
