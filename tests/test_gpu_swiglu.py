"""GPU parity of the SwiGLU MLP shard (tp_mlp_swiglu_shard_fwd) against the
fp64 oracle.  Outputs NaN-filled before each call.  Tolerances as for the
GeLU MLP, bf16 inputs: max |err| <= 2e-2 (s + |ref|) and relative Frobenius
<= 5e-3 per shard, s = max(1, rms(ref)): the stated bound (s = 1) for
outputs at or below unit scale, the same bound in the output's own units for
the larger ones (the gated product of two projections puts the partial at
RMS ~3 for the large shard, ~25 for the wider random shapes); the stated
figure max|err| / (1 + |ref|) is printed beside it.  The sum over ranks:
floor max(sqrt(t), rms).  fp32: both <= 1e-5, floor 1."""
import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import SHAPE_SWEEP, assert_close, dev, host64, nan_tensor, rms, say, to_np

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run(wl, r, xd, wgd, wud, bd, tokens, **extras):
    td = TORCH_DT[wl.dtype]
    ws = torch.empty(binding.tp_mlp_swiglu_shard_workspace_bytes(tokens, wl.hidden, wl.ffn, wl.t, td),
                     dtype=torch.uint8, device="cuda")
    z = nan_tensor((tokens, wl.hidden), TORCH_DT[wl.out_dtype])
    binding.tp_mlp_swiglu_shard_fwd(xd, wgd, wud, bd, z, ws, ffn=wl.ffn, t=wl.t, rank=r, **extras)
    torch.cuda.synchronize()
    return z


def full_weights(wl):
    return (np.concatenate([inputs.mlp_wg_block(wl, r) for r in range(wl.t)], axis=1),
            np.concatenate([inputs.mlp_wu_block(wl, r) for r in range(wl.t)], axis=1),
            np.concatenate([inputs.mlp_b_block(wl, r) for r in range(wl.t)], axis=0))


@pytest.mark.parametrize("name", ["tiny_f32_t4", "t4_h1024_m1024"])
def test_all_ranks_and_reconstruction(name):
    wl = inputs.MLP_WORKLOADS[name]
    dt = wl.dtype
    x = inputs.mlp_x_rows(wl)
    wg, wu, b = full_weights(wl)
    bb, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    x64, wg64, wu64, b64 = (host64(v, dt) for v in (x, wg, wu, b))
    bb64, res64 = host64(bb, dt), host64(res, dt)
    xd = dev(x, dt)
    total = None
    for r in range(wl.t):
        say(f"{name} swiglu rank {r}")
        z = to_np(run(wl, r, xd, dev(inputs.mlp_wg_block(wl, r), dt), dev(inputs.mlp_wu_block(wl, r), dt),
                      dev(inputs.mlp_b_block(wl, r), dt), wl.tokens, bias_b=dev(bb, dt),
                      residual=dev(res, dt)))
        ref = oracle.swiglu_mlp_shard(x64, wg64, wu64, b64, wl.t, r, bb64, res64)
        assert_close(z, ref, dt, f"{name} swiglu rank {r}", floor="one" if dt == "f32" else "scale")
        total = z if total is None else total + z
    full = oracle.swiglu_mlp_full(x64, wg64, wu64, b64, bb64, res64)
    if dt == "f32":
        assert_close(total, full, dt, f"{name} swiglu sum over ranks")
    else:
        # independent bf16 rounding errors of the t shards add in quadrature
        assert_close(total, full, dt, f"{name} swiglu sum over ranks",
                     floor=max(np.sqrt(wl.t), rms(full)))


@pytest.mark.parametrize("rank", [0, 6])
def test_large_shard_full(rank):
    """t = 8, hidden 8192, 16384 tokens (the shape the benchmark times):
    every element of the rank's fp32 partial against the fp64 oracle (~3.3
    TFLOP of host fp64 per shard)."""
    wl = inputs.MLP_WORKLOADS["t8_h8192_m16384"]
    x = inputs.mlp_x_rows(wl)
    wg, wu, b = inputs.mlp_wg_block(wl, rank), inputs.mlp_wu_block(wl, rank), inputs.mlp_b_block(wl, rank)
    say(f"t8_h8192_m16384 swiglu rank {rank}: all 16384 x 8192 outputs")
    z = to_np(run(wl, rank, dev(x, "bf16"), dev(wg, "bf16"), dev(wu, "bf16"), dev(b, "bf16"), wl.tokens))
    assert np.isfinite(z).all()
    # the rank's blocks with t = 1 are the whole of its shard (partition pin)
    ref = oracle.swiglu_mlp_shard(host64(x, "bf16"), host64(wg, "bf16"), host64(wu, "bf16"),
                                  host64(b, "bf16"), 1, 0)
    assert_close(z, ref, "bf16", f"t8 swiglu rank {rank} full shard", floor="scale")


def test_strided_weight_views_and_f32_ragged():
    wl = inputs.MLP_WORKLOADS["t4_h1024_m1024"]
    x = inputs.mlp_x_rows(wl)
    wg, wu, b = full_weights(wl)
    wgd, wud = dev(wg, "bf16"), dev(wu, "bf16")
    r = 2
    cols = slice(r * wl.f, (r + 1) * wl.f)
    say("t4_h1024_m1024 swiglu rank 2 from column-block views (ld = ffn)")
    z = to_np(run(wl, r, dev(x, "bf16"), wgd[:, cols], wud[:, cols], dev(inputs.mlp_b_block(wl, r), "bf16"),
                  wl.tokens))
    ref = oracle.swiglu_mlp_shard(host64(x, "bf16"), host64(wg, "bf16"), host64(wu, "bf16"),
                                  host64(b, "bf16"), wl.t, r)
    assert_close(z, ref, "bf16", "swiglu strided views", floor="scale")
    # fp32 takes any token count
    wt = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    xs = inputs.mlp_x_rows(wt, 0, 37)
    say("tiny_f32_t4 swiglu rank 1, 37 tokens")
    z = to_np(run(wt, 1, dev(xs, "f32"), dev(inputs.mlp_wg_block(wt, 1), "f32"),
                  dev(inputs.mlp_wu_block(wt, 1), "f32"), dev(inputs.mlp_b_block(wt, 1), "f32"), 37))
    fg, fu, fb = full_weights(wt)
    assert_close(z, oracle.swiglu_mlp_shard(xs, fg, fu, fb, wt.t, 1), "f32", "swiglu fp32 ragged")


@pytest.mark.parametrize("tokens,hidden,f", [(9, 24, 16), (1, 64, 64), (77, 136, 200), (300, 264, 360),
                                             (513, 1024, 520)])
def test_bf16_ragged_shapes(tokens, hidden, f):
    """bf16 shapes off every tile: ragged tokens, a feature count that ends
    inside a paired gate / value tile, and k extents (hidden, f) that end
    inside a 32-deep k-tile."""
    wl = inputs.MlpWorkload(f"swiglu_{tokens}_{hidden}_{f}", tokens, hidden, 2 * f, 2, "bf16", 1.0,
                            0.05, 0.05, "f32")
    x = inputs.mlp_x_rows(wl)
    wg, wu, b = full_weights(wl)
    bb, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    say(f"swiglu tokens={tokens} hidden={hidden} f={f} rank 0")
    z = to_np(run(wl, 0, dev(x, "bf16"), dev(inputs.mlp_wg_block(wl, 0), "bf16"),
                  dev(inputs.mlp_wu_block(wl, 0), "bf16"), dev(inputs.mlp_b_block(wl, 0), "bf16"),
                  tokens, bias_b=dev(bb, "bf16"), residual=dev(res, "bf16")))
    ref = oracle.swiglu_mlp_shard(host64(x, "bf16"), host64(wg, "bf16"), host64(wu, "bf16"),
                                  host64(b, "bf16"), wl.t, 0, host64(bb, "bf16"), host64(res, "bf16"))
    assert_close(z, ref, "bf16", f"swiglu ragged {tokens}x{hidden}x{f}", floor="scale")


def test_bf16_ragged_multiround():
    """Nearly the headline size with every extent ragged: the gated product
    (2048 paired 256 x 256 tiles, 8 rounds of resident workgroups, features
    ending inside a paired tile, K % 32 = 24) and the row GEMM (8 rounds,
    K % 32 = 24) of rank 0; every element checked.  The oracle takes rank
    0's weight blocks as a t = 1 shard, the same arithmetic."""
    tokens, hidden, f = 16376, 8184, 4088
    wl = inputs.MlpWorkload("swiglu_multiround", tokens, hidden, 2 * f, 2, "bf16", 1.0, 0.02, 0.02, "f32")
    x = inputs.mlp_x_rows(wl)
    wg, wu, b = inputs.mlp_wg_block(wl, 0), inputs.mlp_wu_block(wl, 0), inputs.mlp_b_block(wl, 0)
    bb, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    say(f"swiglu multi-round tokens={tokens} hidden={hidden} f={f} rank 0")
    z = to_np(run(wl, 0, dev(x, "bf16"), dev(wg, "bf16"), dev(wu, "bf16"), dev(b, "bf16"), tokens,
                  bias_b=dev(bb, "bf16"), residual=dev(res, "bf16")))
    assert not np.isnan(z).any(), "unwritten outputs"
    ref = oracle.swiglu_mlp_shard(host64(x, "bf16"), host64(wg, "bf16"), host64(wu, "bf16"),
                                  host64(b, "bf16"), 1, 0, host64(bb, "bf16"), host64(res, "bf16"))
    assert_close(z, ref, "bf16", "swiglu multi-round", floor="scale")


def _swiglu_shapes(seed, n):
    """n seeded shard shapes: every third at 3000-9000 tokens and 1024-5600
    wide (several rounds of paired gate / value tiles), the rest small;
    ragged everywhere, k extents (hidden) a multiple of 64 about half the
    time; rank 0 or 1 of t = 2."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 3 == 0:
            tokens, hidden, f = (int(rng.integers(3000, 9001)), 8 * int(rng.integers(128, 701)),
                                 8 * int(rng.integers(128, 701)))
        else:
            tokens, hidden, f = (int(rng.integers(1, 2000)), 8 * int(rng.integers(1, 151)),
                                 8 * int(rng.integers(1, 151)))
        if rng.random() < 0.5:
            hidden = 64 * max(1, hidden // 64)
        out.append((tokens, hidden, f, int(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("tokens,hidden,f,rank", _swiglu_shapes(31, 9 * SHAPE_SWEEP))
def test_bf16_random_shapes(tokens, hidden, f, rank):
    wl = inputs.MlpWorkload(f"swiglu_rand_{tokens}_{hidden}_{f}", tokens, hidden, 2 * f, 2, "bf16", 1.0,
                            0.05, 0.05, "f32")
    x = inputs.mlp_x_rows(wl)
    wg, wu, b = full_weights(wl)
    bb, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    say(f"swiglu random shapes: tokens={tokens} hidden={hidden} f={f} rank {rank}")
    z = to_np(run(wl, rank, dev(x, "bf16"), dev(inputs.mlp_wg_block(wl, rank), "bf16"),
                  dev(inputs.mlp_wu_block(wl, rank), "bf16"), dev(inputs.mlp_b_block(wl, rank), "bf16"),
                  tokens, bias_b=dev(bb, "bf16"), residual=dev(res, "bf16")))
    assert not np.isnan(z).any(), "unwritten outputs"
    ref = oracle.swiglu_mlp_shard(host64(x, "bf16"), host64(wg, "bf16"), host64(wu, "bf16"),
                                  host64(b, "bf16"), wl.t, rank, host64(bb, "bf16"), host64(res, "bf16"))
    assert_close(z, ref, "bf16", f"swiglu random {tokens}x{hidden}x{f} rank {rank}", floor="scale")
