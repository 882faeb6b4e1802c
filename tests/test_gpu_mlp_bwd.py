"""GPU parity of the MLP shard backward (tp_mlp_shard_bwd) and of the
forward's saved pre-activation against the fp64 oracle.

Every call goes through the C ABI.  Outputs are NaN-filled before each call.
Tolerances as for the forward, bf16 inputs: max |err| <= 2e-2 (s + |ref|) and
relative Frobenius <= 5e-3 per output; fp32: both <= 1e-5.  For the
gradients s is the output's RMS magnitude rather than 1 (they are sums over
up to 16384 tokens, far from unit scale; at unit scale it is the same bound).
The sum of the ranks' dX contributions is held to the relative Frobenius
bound, its normalised max error reported.
"""
import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import assert_close, dev, host64, nan_tensor, rms, say, to_np

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run_fwd_save(wl, r, xd, ad, bd, bias_d=None):
    """Forward of rank r with the pre-activation saved; returns (z, y)."""
    td = TORCH_DT[wl.dtype]
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(xd.shape[0], wl.hidden, wl.ffn, wl.t, td),
                     dtype=torch.uint8, device="cuda")
    z = nan_tensor((xd.shape[0], wl.hidden), TORCH_DT[wl.out_dtype])
    y = nan_tensor((xd.shape[0], wl.f), td)
    binding.tp_mlp_shard_fwd(xd, ad, bd, z, ws, ffn=wl.ffn, t=wl.t, rank=r, bias_a_i=bias_d,
                             y_save=y)
    torch.cuda.synchronize()
    return z, y


def run_bwd(wl, r, xd, ad, bd, yd, dzd, grad_dt, with_bias=True, da=None):
    td = TORCH_DT[wl.dtype]
    tokens = xd.shape[0]
    nbytes = binding.tp_mlp_shard_bwd_workspace_bytes(tokens, wl.hidden, wl.ffn, wl.t, td)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    gd = TORCH_DT[grad_dt]
    dx = nan_tensor((tokens, wl.hidden), gd)
    da = nan_tensor((wl.hidden, wl.f), gd) if da is None else da
    db = nan_tensor((wl.f, wl.hidden), gd)
    dba = nan_tensor((wl.f,), torch.float32) if with_bias else None
    dbb = nan_tensor((wl.hidden,), torch.float32) if with_bias else None
    binding.tp_mlp_shard_bwd(xd, ad, bd, yd, dzd, dx, da, db, ws, ffn=wl.ffn, t=wl.t, rank=r,
                             dbias_a_i=dba, dbias_b=dbb)
    torch.cuda.synchronize()
    return dict(dx=dx, da=da, db=db, dbias_a=dba, dbias_b=dbb)


def check_grads(got, ref, dtype, what, keys=("dx", "da", "db", "dbias_a", "dbias_b")):
    """dX (near unit scale) to the stated bound: fp32 with the floor 1, bf16
    in its own units (floor max(1, rms)); the weight and bias gradients,
    sums over all the tokens (RMS in the tens to hundreds, whose rounding
    error grows with the summands in either precision), with the RMS as the
    floor (fp32: max(1, rms), the stated bound at or below unit scale).  The
    figure with the floor 1 is always printed."""
    for k in keys:
        if got.get(k) is None:
            continue
        if dtype == "f32":
            floor = "one" if k == "dx" else "scale"
        else:
            floor = "scale" if k == "dx" else "rms"
        assert_close(to_np(got[k]), ref[k], dtype, f"{what} {k}", floor=floor)


def shard_ref(x64, a64, b64, dz64, ba64=None):
    """Oracle backward of one rank given that rank's blocks: with t = 1 the
    oracle's rank-0 block of [h, f] / [f, h] weights is the whole of them
    (the partition identity pin ties this to the sharded form)."""
    return oracle.mlp_shard_bwd(x64, a64, b64, dz64, 1, 0, bias_a=ba64)


def test_tiny_f32_all_ranks_save_and_backward():
    wl = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a_full = np.concatenate([inputs.mlp_a_block(wl, r) for r in range(wl.t)], axis=1)
    b_full = np.concatenate([inputs.mlp_b_block(wl, r) for r in range(wl.t)], axis=0)
    ba_full = np.concatenate([inputs.mlp_bias_a_block(wl, r) for r in range(wl.t)])
    xd, dzd = dev(x, "f32"), dev(dz, "f32")
    dx_sum = None
    for r in range(wl.t):
        say(f"tiny_f32_t4 backward rank {r}")
        ad, bd = dev(inputs.mlp_a_block(wl, r), "f32"), dev(inputs.mlp_b_block(wl, r), "f32")
        bias_d = dev(inputs.mlp_bias_a_block(wl, r), "f32")
        _z, y = run_fwd_save(wl, r, xd, ad, bd, bias_d)
        ref = oracle.mlp_shard_bwd(x, a_full, b_full, dz, wl.t, r, bias_a=ba_full)
        assert_close(to_np(y), ref["y"], "f32", f"tiny rank {r} saved pre-activation")
        got = run_bwd(wl, r, xd, ad, bd, y, dzd, "f32")
        check_grads(got, ref, "f32", f"tiny rank {r}")
        dx = to_np(got["dx"])
        dx_sum = dx if dx_sum is None else dx_sum + dx
    full = oracle.mlp_shard_bwd(x, a_full, b_full, dz, 1, 0, bias_a=ba_full)
    assert_close(dx_sum, full["dx"], "f32", "tiny sum over ranks of dX vs unsharded dX")


def test_f32_ragged_tokens():
    """fp32 takes any shape: 37 tokens."""
    wl = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    x, dz = inputs.mlp_x_rows(wl, 0, 37), inputs.mlp_dz_rows(wl, 0, 37)
    a, b = inputs.mlp_a_block(wl, 2), inputs.mlp_b_block(wl, 2)
    ref = shard_ref(x, a, b, dz)
    say("tiny_f32_t4 rank 2, 37 tokens")
    got = run_bwd(wl, 2, dev(x, "f32"), dev(a, "f32"), dev(b, "f32"), dev(ref["y"].astype(np.float32), "f32"),
                  dev(dz, "f32"), "f32")
    check_grads(got, ref, "f32", "ragged f32")


@pytest.mark.parametrize("tokens,hidden,f,grad_dt", [
    (9, 24, 16, "f32"),                 # every k extent below one 32-deep k-tile
    (1, 64, 64, "f32"),
    (77, 136, 200, "f32"),
    (300, 264, 360, "bf16"),
    (513, 1024, 520, "f32"),
    (16000, 2112, 1088, "f32"),         # dH / dX: paired B stages over 2 / 3 rounds, ragged M and N
])
def test_bf16_ragged_shapes(tokens, hidden, f, grad_dt):
    """bf16 shapes off every tile: token counts that are ragged against the
    256-row tiles and, as the k extent of the weight-gradient products,
    against the 32-deep k-tiles; hidden and f ragged against both."""
    wl = inputs.MlpWorkload(f"bwd_{tokens}_{hidden}_{f}", tokens, hidden, 2 * f, 2, "bf16", 1.0,
                            0.05, 0.05, "f32")
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a, b = inputs.mlp_a_block(wl, 1), inputs.mlp_b_block(wl, 1)
    xd, ad, bd = dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16")
    say(f"backward tokens={tokens} hidden={hidden} f={f} grads {grad_dt}")
    _z, y = run_fwd_save(wl, 1, xd, ad, bd)
    ref = shard_ref(host64(x, "bf16"), host64(a, "bf16"), host64(b, "bf16"), host64(dz, "bf16"))
    assert_close(to_np(y), ref["y"], "bf16", "ragged saved pre-activation")
    got = run_bwd(wl, 1, xd, ad, bd, y, dev(dz, "bf16"), grad_dt)
    check_grads(got, ref, "bf16", f"ragged {tokens}x{hidden}x{f} grads {grad_dt}")


@pytest.mark.parametrize("grad_dt", ["f32", "bf16"])
def test_t1_bf16(grad_dt):
    wl = inputs.MLP_WORKLOADS["t1_h1024_m2048"]
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a, b = inputs.mlp_a_block(wl, 0), inputs.mlp_b_block(wl, 0)
    xd, ad, bd = dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16")
    say(f"t1_h1024_m2048 backward, grads {grad_dt}")
    _z, y = run_fwd_save(wl, 0, xd, ad, bd)
    ref = shard_ref(host64(x, "bf16"), host64(a, "bf16"), host64(b, "bf16"), host64(dz, "bf16"))
    assert_close(to_np(y), ref["y"], "bf16", "t1 saved pre-activation")
    got = run_bwd(wl, 0, xd, ad, bd, y, dev(dz, "bf16"), grad_dt)
    check_grads(got, ref, "bf16", f"t1 grads {grad_dt}")


def test_t4_all_ranks_strided_weight_views_and_reconstruction():
    """A_i and dA_i as column-block views of the full [h, F] tensors (ld = F):
    the rank writes only its block.  The ranks' dX contributions sum to the
    unsharded dX."""
    wl = inputs.MLP_WORKLOADS["t4_h1024_m1024"]
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a_blocks = [inputs.mlp_a_block(wl, r) for r in range(wl.t)]
    b_blocks = [inputs.mlp_b_block(wl, r) for r in range(wl.t)]
    xd, dzd = dev(x, "bf16"), dev(dz, "bf16")
    a_full_d = dev(np.concatenate(a_blocks, axis=1), "bf16")
    da_full = nan_tensor((wl.hidden, wl.ffn), torch.float32)
    x64, dz64 = host64(x, "bf16"), host64(dz, "bf16")
    dx_sum = None
    for r in range(wl.t):
        say(f"t4_h1024_m1024 backward rank {r} (strided A_i / dA_i)")
        cols = slice(r * wl.f, (r + 1) * wl.f)
        a_view = a_full_d[:, cols]
        bd = dev(b_blocks[r], "bf16")
        _z, y = run_fwd_save(wl, r, xd, a_view, bd)
        got = run_bwd(wl, r, xd, a_view, bd, y, dzd, "f32", da=da_full[:, cols])
        ref = shard_ref(x64, host64(a_blocks[r], "bf16"), host64(b_blocks[r], "bf16"), dz64)
        check_grads(got, ref, "bf16", f"t4 rank {r}")
        if r < wl.t - 1:
            assert torch.isnan(da_full[:, (r + 1) * wl.f:]).all(), "dA columns of later ranks written"
        dx = to_np(got["dx"])
        dx_sum = dx if dx_sum is None else dx_sum + dx
    a64 = host64(np.concatenate(a_blocks, axis=1), "bf16")
    b64 = host64(np.concatenate(b_blocks, axis=0), "bf16")
    full = oracle.mlp_shard_bwd(x64, a64, b64, dz64, 1, 0)
    assert_close(to_np(da_full), full["da"], "bf16", "t4 assembled dA vs unsharded dA", floor="rms")
    # the t contributions carry independent bf16 rounding errors, which add
    # in quadrature: the floor of the max criterion grows by sqrt(t)
    assert_close(dx_sum, full["dx"], "bf16", "t4 sum over ranks of dX vs unsharded dX",
                 floor=max(np.sqrt(wl.t), rms(full["dx"])))


@pytest.mark.parametrize("name,rank", [("t8_h8192_m4096", 0), ("t8_h8192_m4096", 5),
                                       ("t8_h8192_m16384", 3)])
def test_large_rank_shards(name, rank):
    wl = inputs.MLP_WORKLOADS[name]
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a, b = inputs.mlp_a_block(wl, rank), inputs.mlp_b_block(wl, rank)
    xd, ad, bd = dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16")
    say(f"{name} backward rank {rank}")
    _z, y = run_fwd_save(wl, rank, xd, ad, bd)
    got = run_bwd(wl, rank, xd, ad, bd, y, dev(dz, "bf16"), "f32")
    del xd, ad, bd
    ref = shard_ref(host64(x, "bf16"), host64(a, "bf16"), host64(b, "bf16"), host64(dz, "bf16"))
    check_grads(got, ref, "bf16", f"{name} rank {rank}")


def test_f32_shard_on_64x64_tiles():
    """fp32 forward (saved pre-activation) and backward at 2048 tokens,
    hidden 2048, f 2048: every product has at least 1024 tiles of 64 x 64,
    the fp32 GEMM's larger tile (the small fp32 cases run on 32 x 32 tiles)."""
    wl = inputs.MlpWorkload("f32_2048", 2048, 2048, 4096, 2, "f32", 1.0, 1.0 / np.sqrt(2048),
                            1.0 / np.sqrt(4096), "f32")
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a, b = inputs.mlp_a_block(wl, 1), inputs.mlp_b_block(wl, 1)
    ba = inputs.mlp_bias_a_block(wl, 1)
    xd, ad, bd = dev(x, "f32"), dev(a, "f32"), dev(b, "f32")
    say("fp32 forward and backward, 2048 tokens, hidden 2048, f 2048")
    _z, y = run_fwd_save(wl, 1, xd, ad, bd, dev(ba, "f32"))
    ref = shard_ref(host64(x, "f32"), host64(a, "f32"), host64(b, "f32"), host64(dz, "f32"),
                    host64(ba, "f32"))
    assert_close(to_np(y), ref["y"], "f32", "fp32 2048 saved pre-activation")
    got = run_bwd(wl, 1, xd, ad, bd, y, dev(dz, "f32"), "f32")
    check_grads(got, ref, "f32", "fp32 2048")


def test_ragged_tokens_near_headline():
    """16376 tokens (not a multiple of the 32-deep k-tile) at the headline
    widths: the weight-gradient products take the K-tail path over 512
    k-tiles.  Their gradients for a seeded block of 64 of the shard's f
    columns are checked against the oracle run on that block (each column of
    A with its row of B is an independent GeLU unit, so the block's weight
    gradients do not depend on the other columns), and the launch must run
    at close to the rate of the aligned 16384-token backward (a register
    spill in the K-tail kernel once made it 2.5 times slower)."""
    wl = inputs.MlpWorkload("bwd_ragged_16376", 16376, 8192, 32768, 8, "bf16", 1.0, 0.02, 0.02, "f32")
    x, dz = inputs.mlp_x_rows(wl), inputs.mlp_dz_rows(wl)
    a, b = inputs.mlp_a_block(wl, 2), inputs.mlp_b_block(wl, 2)
    xd, ad, bd, dzd = dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16"), dev(dz, "bf16")
    say("backward 16376 tokens, h 8192, f 4096: K-tail weight gradients")
    _z, y = run_fwd_save(wl, 2, xd, ad, bd)
    got = run_bwd(wl, 2, xd, ad, bd, y, dzd, "f32", with_bias=False)
    cols = np.sort(np.random.default_rng(16376).choice(wl.f, 64, replace=False))
    ref = shard_ref(host64(x, "bf16"), host64(a, "bf16")[:, cols], host64(b, "bf16")[cols, :],
                    host64(dz, "bf16"))
    check_grads({"da": got["da"][:, torch.from_numpy(cols).cuda()],
                 "db": got["db"][torch.from_numpy(cols).cuda(), :]}, ref, "bf16",
                "16376-token column block", keys=("da", "db"))

    # rate: the same launch against an aligned 16384-token one, interleaved
    tok2 = 16384
    x2 = torch.randn(tok2, wl.hidden, device="cuda").to(torch.bfloat16)
    y2 = torch.randn(tok2, wl.f, device="cuda").to(torch.bfloat16)
    dz2 = torch.randn(tok2, wl.hidden, device="cuda").to(torch.bfloat16)
    outs = {n: (torch.empty(n, wl.hidden, device="cuda"), torch.empty(wl.hidden, wl.f, device="cuda"),
                torch.empty(wl.f, wl.hidden, device="cuda")) for n in (wl.tokens, tok2)}
    args = {wl.tokens: (xd, y, dzd), tok2: (x2, y2, dz2)}
    ws = torch.empty(binding.tp_mlp_shard_bwd_workspace_bytes(tok2, wl.hidden, wl.ffn, wl.t, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def launch(n):
        xx, yy, zz = args[n]
        binding.tp_mlp_shard_bwd(xx, ad, bd, yy, zz, *outs[n], ws, ffn=wl.ffn, t=wl.t, rank=2)

    best = {n: float("inf") for n in args}
    for n in args:
        launch(n)
    for _ in range(3):
        for n in args:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                launch(n)
            e1.record()
            torch.cuda.synchronize()
            best[n] = min(best[n], e0.elapsed_time(e1) / 3)
    ratio = best[wl.tokens] / best[tok2]
    say(f"backward 16376 tokens {best[wl.tokens]:.3f} ms, 16384 tokens {best[tok2]:.3f} ms, ratio {ratio:.3f}")
    assert ratio < 1.25, f"ragged-token backward {ratio:.2f} times the aligned one"


def test_large_token_count_sampled():
    """65536 tokens at the headline widths (rank 4): the weight-gradient
    products accumulate over 2048 k-tiles.  dA and dB are checked on a
    seeded block of 32 of the shard's f columns against the oracle run on
    that block (the columns are independent GeLU units), dX on three 64-row
    blocks against the oracle run on those rows (each token's dX depends on
    that token only); every output must be written (finite)."""
    wl = inputs.MlpWorkload("bwd_t8_h8192_m65536", 65536, 8192, 32768, 8, "bf16", 1.0, 0.02, 0.02, "f32")
    r, step = 4, 8192
    xd = torch.empty((wl.tokens, wl.hidden), dtype=torch.bfloat16, device="cuda")
    dzd = torch.empty((wl.tokens, wl.hidden), dtype=torch.bfloat16, device="cuda")
    x_parts, dz_parts = [], []
    for r0 in range(0, wl.tokens, step):
        xp, dp = inputs.mlp_x_rows(wl, r0, step), inputs.mlp_dz_rows(wl, r0, step)
        xd[r0:r0 + step], dzd[r0:r0 + step] = dev(xp, "bf16"), dev(dp, "bf16")
        x_parts.append(xp)
        dz_parts.append(dp)
    a, b = inputs.mlp_a_block(wl, r), inputs.mlp_b_block(wl, r)
    ad, bd = dev(a, "bf16"), dev(b, "bf16")
    say(f"backward 65536 tokens, rank {r}")
    _z, y = run_fwd_save(wl, r, xd, ad, bd)
    got = run_bwd(wl, r, xd, ad, bd, y, dzd, "f32", with_bias=False)
    del xd, dzd, y, _z
    for k in ("dx", "da", "db"):
        assert bool(torch.isfinite(got[k]).all()), f"{k}: unwritten or non-finite outputs"
    a64, b64 = host64(a, "bf16"), host64(b, "bf16")
    cols = np.sort(np.random.default_rng(65536).choice(wl.f, 32, replace=False))
    x64 = np.concatenate([host64(p, "bf16") for p in x_parts])
    dz64 = np.concatenate([host64(p, "bf16") for p in dz_parts])
    del x_parts, dz_parts
    ref = shard_ref(x64, a64[:, cols], b64[cols, :], dz64)
    tc = torch.from_numpy(cols).cuda()
    check_grads({"da": got["da"][:, tc], "db": got["db"][tc, :]}, ref, "bf16",
                "65536-token column block", keys=("da", "db"))
    for r0 in (0, 32768, wl.tokens - 64):
        ref_rows = shard_ref(x64[r0:r0 + 64], a64, b64, dz64[r0:r0 + 64])
        check_grads({"dx": got["dx"][r0:r0 + 64]}, ref_rows, "bf16", f"65536 tokens dX rows {r0}..",
                    keys=("dx",))


def test_zero_tokens_and_errors():
    wl = inputs.MLP_WORKLOADS["t4_h1024_m1024"]
    ad = dev(inputs.mlp_a_block(wl, 0), "bf16")
    bd = dev(inputs.mlp_b_block(wl, 0), "bf16")
    empty = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    y0 = torch.empty((0, wl.f), dtype=torch.bfloat16, device="cuda")
    say("backward with tokens = 0")
    got = run_bwd(wl, 0, empty, ad, bd, y0, empty, "f32")
    for k in ("da", "db", "dbias_a", "dbias_b"):
        assert (got[k] == 0).all(), f"{k} must be zero for zero tokens"
    # a width that is not a multiple of 8 is refused before any launch
    wm = inputs.MlpWorkload("misaligned", 16, 1028, 2 * 1028, 2, "bf16", 1.0, 0.05, 0.05, "f32")
    x = torch.zeros((16, 1028), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1028, 1028), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.TpError, match="MISALIGNED"):
        run_bwd(wm, 0, x, w, w, w[:16], x, "f32")
