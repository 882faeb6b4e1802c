"""GPU parity of the head-local attention shard (tp_attn_shard_fwd) against
the fp64 oracle.

Every call goes through the C ABI.  Outputs and workspace are NaN-filled
first, so an unwritten tile cannot pass.  Tolerance as for the bf16 MLP path:
max |err| / (1 + |ref|) <= 2e-2 and relative Frobenius <= 5e-3 per shard; the
sum over ranks to both bounds with the max criterion's floor sqrt(t) (the
shards' independent bf16 rounding errors add in quadrature; the stated-floor
figure is printed beside it).
"""
import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import SHAPE_SWEEP, assert_close, dev, host64, nan_tensor, say, to_np

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def x_all(wl):
    return np.stack([inputs.attn_x(wl, b) for b in range(wl.batch)])


def run(wl, r, xd, wqkv_d, wo_d, causal, out_dtype="f32"):
    nbytes = binding.tp_attn_shard_workspace_bytes(wl.batch, wl.seq, wl.hidden, wl.heads,
                                                   wl.head_dim, wl.t, torch.bfloat16)
    assert nbytes > 0
    ws = nan_tensor((nbytes // 2,), torch.bfloat16)
    out = nan_tensor((wl.batch, wl.seq, wl.hidden), TORCH_DT[out_dtype])
    binding.tp_attn_shard_fwd(xd, wqkv_d, wo_d, out, ws, heads=wl.heads, head_dim=wl.head_dim,
                              t=wl.t, rank=r, causal=causal)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["attn_t2_h1024_b2_s384", "attn_t2_h1024_b3_s128"])
@pytest.mark.parametrize("causal", [False, True])
def test_small_all_ranks_and_reconstruction(name, causal):
    wl = inputs.ATTN_WORKLOADS[name]
    x = x_all(wl)
    xd = dev(x, "bf16")
    wqkv = [inputs.attn_wqkv_block(wl, r) for r in range(wl.t)]
    wo = [inputs.attn_wo_block(wl, r) for r in range(wl.t)]
    x64 = host64(x, "bf16")
    total = None
    for r in range(wl.t):
        say(f"{name} rank {r} causal={causal}")
        out = to_np(run(wl, r, xd, dev(wqkv[r], "bf16"), dev(wo[r], "bf16"), causal))
        ref = oracle.attn_shard(x64, host64(wqkv[r], "bf16"), host64(wo[r], "bf16"), wl.heads,
                                wl.head_dim, wl.t, r, causal)
        assert_close(out, ref, "bf16", f"{name} rank {r} causal={causal}")
        total = out if total is None else total + out
    # The ranks' partials sum to unsharded multi-head attention with the full
    # Q, K, V, O weights (the packed per-head layout undone).
    wq, wk, wv = oracle.split_packed_qkv(host64(np.concatenate(wqkv, axis=1), "bf16"), wl.heads,
                                         wl.head_dim)
    full = oracle.mha_full(x64, wq, wk, wv, host64(np.concatenate(wo, axis=0), "bf16"), wl.heads,
                           causal)
    # the ranks' bf16 rounding errors are independent: they add in
    # quadrature, so the max criterion's floor is sqrt(t)
    assert_close(total, full, "bf16", f"{name} sum over ranks vs unsharded attention causal={causal}",
                 floor=float(np.sqrt(wl.t)))


def test_small_bf16_output():
    wl = inputs.ATTN_WORKLOADS["attn_t2_h1024_b2_s384"]
    x = x_all(wl)
    r = 1
    wqkv, wo = inputs.attn_wqkv_block(wl, r), inputs.attn_wo_block(wl, r)
    say("attn_t2_h1024_b2_s384 rank 1 bf16 out")
    out = to_np(run(wl, r, dev(x, "bf16"), dev(wqkv, "bf16"), dev(wo, "bf16"), False, "bf16"))
    ref = oracle.attn_shard(host64(x, "bf16"), host64(wqkv, "bf16"), host64(wo, "bf16"), wl.heads,
                            wl.head_dim, wl.t, r)
    assert_close(out, ref, "bf16", "bf16 output")


@pytest.mark.parametrize("rank,causal", [(0, False), (7, True)])
def test_large_full(rank, causal):
    """hidden 8192, 64 heads, t=8, seq 4096 (the attention workload the
    benchmark times): every element of the rank's fp32 partial against the
    fp64 oracle (~5 s of host time per shard)."""
    wl = inputs.ATTN_WORKLOADS["attn_t8_h8192_s4096"]
    x = x_all(wl)
    wqkv, wo = inputs.attn_wqkv_block(wl, rank), inputs.attn_wo_block(wl, rank)
    say(f"attn_t8_h8192_s4096 rank {rank} causal={causal}: all 4096 x 8192 outputs")
    out = to_np(run(wl, rank, dev(x, "bf16"), dev(wqkv, "bf16"), dev(wo, "bf16"), causal))
    assert np.isfinite(out).all()
    ref = oracle.attn_shard(host64(x, "bf16"), host64(wqkv, "bf16"), host64(wo, "bf16"), wl.heads,
                            wl.head_dim, wl.t, rank, causal)
    assert_close(out, ref, "bf16", f"large rank {rank} causal={causal} full shard")


def test_errors_and_empty():
    wl = inputs.ATTN_WORKLOADS["attn_t2_h1024_b3_s128"]
    x = dev(x_all(wl), "bf16")
    wqkv = dev(inputs.attn_wqkv_block(wl, 0), "bf16")
    wo = dev(inputs.attn_wo_block(wl, 0), "bf16")
    out = nan_tensor((wl.batch, wl.seq, wl.hidden), torch.float32)
    with pytest.raises(binding.TpError):          # no workspace
        binding.tp_attn_shard_fwd(x, wqkv, wo, out, None, heads=8, head_dim=128, t=2, rank=0)
    with pytest.raises(binding.TpError):          # heads not divisible by t
        binding.tp_attn_shard_fwd(x, wqkv, wo, out, None, heads=8, head_dim=128, t=3, rank=0)
    assert torch.isnan(out).all()
    # batch 0: nothing to do, nothing written
    x0 = torch.empty((0, 128, wl.hidden), dtype=torch.bfloat16, device="cuda")
    out0 = torch.empty((0, 128, wl.hidden), dtype=torch.float32, device="cuda")
    binding.tp_attn_shard_fwd(x0, wqkv, wo, out0, None, heads=8, head_dim=128, t=2, rank=0)
    torch.cuda.synchronize()


def test_projection_overflow_is_never_finite_and_wrong():
    """X scaled by 2^24: Q and K exceed the scaled fp16 range (|q|, |k| >=
    2^24).  Every output row is then either non-finite or still within the
    bound of the oracle's (fp64, no overflow) result: an overflow is never a
    finite wrong answer."""
    wl = inputs.ATTN_WORKLOADS["attn_t2_h1024_b3_s128"]
    x = x_all(wl)
    xs = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x) * np.float32(2.0 ** 24))
    wqkv, wo = inputs.attn_wqkv_block(wl, 0), inputs.attn_wo_block(wl, 0)
    say("attn_t2_h1024_b3_s128 rank 0 with X scaled by 2^24 (fp16 Q/K overflow)")
    out = to_np(run(wl, 0, dev(xs, "bf16"), dev(wqkv, "bf16"), dev(wo, "bf16"), False))
    ref = oracle.attn_shard(host64(xs, "bf16"), host64(wqkv, "bf16"), host64(wo, "bf16"), wl.heads,
                            wl.head_dim, wl.t, 0, False)
    rows_out, rows_ref = out.reshape(-1, wl.hidden), ref.reshape(-1, wl.hidden)
    bad = ~np.isfinite(rows_out).all(axis=1)
    assert bad.any(), "an overflow this large must reach some row"
    ok = rows_out[~bad]
    if ok.size:
        d = np.abs(ok - rows_ref[~bad]) / (1.0 + np.abs(rows_ref[~bad]))
        assert d.max() <= 2e-2, "a finite row differs from the oracle"
    say(f"overflow: {bad.sum()} of {len(bad)} rows non-finite, the rest within the bound")


def _attn_shapes(seed, n):
    """n seeded shard shapes: batch 1-3, seq a multiple of 128 up to 1152
    (1-36 key blocks of 32, so the loop unrolled by 4 ends at every phase)
    for even draws and any length from 32 to 1152 for odd ones (partial key
    and query blocks, odd block counts), 1-6 local heads, t in 1-4,
    hidden = heads x 128, causal or not."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        t = int(rng.integers(1, 5))
        hl = int(rng.integers(1, 7))
        while hl * t > 16:
            hl -= 1
        seq = 128 * int(rng.integers(1, 10)) if i % 2 == 0 else int(rng.integers(32, 1153))
        out.append((int(rng.integers(1, 4)), seq, hl, t, int(rng.integers(0, t)), bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("batch,seq,hl,t,rank,causal", _attn_shapes(11, 10 * SHAPE_SWEEP))
def test_random_shapes(batch, seq, hl, t, rank, causal):
    heads = hl * t
    hidden = heads * 128
    # QKV weight std keeps the logits' std near 3, as in the fixed workloads
    wl = inputs.AttnWorkload(f"attn_rand_{batch}_{seq}_{hl}_{t}", batch, seq, hidden, heads, 128, t,
                             "bf16", 1.0, 1.8 / np.sqrt(hidden), "f32", 0.02)
    x = x_all(wl)
    wqkv, wo = inputs.attn_wqkv_block(wl, rank), inputs.attn_wo_block(wl, rank)
    say(f"random attention: batch={batch} seq={seq} local heads={hl} t={t} rank={rank} causal={causal}")
    out = to_np(run(wl, rank, dev(x, "bf16"), dev(wqkv, "bf16"), dev(wo, "bf16"), causal))
    ref = oracle.attn_shard(host64(x, "bf16"), host64(wqkv, "bf16"), host64(wo, "bf16"), heads, 128, t,
                            rank, causal)
    assert_close(out, ref, "bf16", f"random attention {wl.name} rank {rank} causal={causal}")


def _attn_long_shapes(seed, n):
    """n seeded shard shapes of long sequences on small grids: batch 1-2,
    seq 2048-4600 (a multiple of 128 for even draws, any length for odd
    ones), 1-3 local heads, t in 1-2, causal or not; the grids of at most
    128 query blocks run each row on two workgroups."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        t = int(rng.integers(1, 3))
        hl = int(rng.integers(1, 4))
        seq = 128 * int(rng.integers(16, 36)) if i % 2 == 0 else int(rng.integers(2048, 4601))
        out.append((int(rng.integers(1, 3)), seq, hl, t, int(rng.integers(0, t)), bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("batch,seq,hl,t,rank,causal", _attn_long_shapes(13, 6 * SHAPE_SWEEP))
def test_random_long_shapes(batch, seq, hl, t, rank, causal):
    heads = hl * t
    hidden = heads * 128
    wl = inputs.AttnWorkload(f"attn_long_{batch}_{seq}_{hl}_{t}", batch, seq, hidden, heads, 128, t,
                             "bf16", 1.0, 1.8 / np.sqrt(hidden), "f32", 0.02)
    x = x_all(wl)
    wqkv, wo = inputs.attn_wqkv_block(wl, rank), inputs.attn_wo_block(wl, rank)
    say(f"random long attention: batch={batch} seq={seq} local heads={hl} t={t} rank={rank} causal={causal}")
    out = to_np(run(wl, rank, dev(x, "bf16"), dev(wqkv, "bf16"), dev(wo, "bf16"), causal))
    ref = oracle.attn_shard(host64(x, "bf16"), host64(wqkv, "bf16"), host64(wo, "bf16"), heads, 128, t,
                            rank, causal)
    assert_close(out, ref, "bf16", f"random long attention {wl.name} rank {rank} causal={causal}")


@pytest.mark.parametrize("batch,seq,hl,t,rank,causal", [
    (2, 32, 2, 2, 1, False),    # one key block, its partner a phantom block
    (2, 33, 2, 2, 0, True),     # a one-key partial block
    (1, 100, 4, 2, 1, True),    # partial query and key blocks, odd block count
    (3, 200, 2, 4, 3, False),
    (1, 1000, 8, 1, 0, True),   # the headline's local heads, 1000 tokens
    (1, 4095, 1, 8, 5, False),  # one short of the headline length
    # causal grids of more query blocks than the 256 CUs: rows not split
    (3, 1408, 8, 1, 0, True),
    (3, 1400, 8, 1, 0, True),
    # few long rows (at most 128 query blocks, 2048 keys or more): each
    # row's keys on two workgroups, merged by the second to finish
    (1, 2048, 2, 1, 0, False),
    (1, 2048, 2, 1, 0, True),
    (2, 2100, 2, 2, 1, True),
    (1, 4096, 4, 2, 1, False),
    (1, 4000, 4, 2, 0, True),
])
def test_ragged_seq(batch, seq, hl, t, rank, causal):
    """Sequence lengths that are not multiples of the 128-query or 32-key
    blocks, causal grids of more than one round, and small grids of long
    rows split over two workgroups, every output element against the
    oracle."""
    heads = hl * t
    hidden = heads * 128
    wl = inputs.AttnWorkload(f"attn_ragged_{batch}_{seq}_{hl}_{t}", batch, seq, hidden, heads, 128, t,
                             "bf16", 1.0, 1.8 / np.sqrt(hidden), "f32", 0.02)
    x = x_all(wl)
    wqkv, wo = inputs.attn_wqkv_block(wl, rank), inputs.attn_wo_block(wl, rank)
    say(f"ragged attention: batch={batch} seq={seq} local heads={hl} t={t} rank={rank} causal={causal}")
    out = to_np(run(wl, rank, dev(x, "bf16"), dev(wqkv, "bf16"), dev(wo, "bf16"), causal))
    ref = oracle.attn_shard(host64(x, "bf16"), host64(wqkv, "bf16"), host64(wo, "bf16"), heads, 128, t,
                            rank, causal)
    assert_close(out, ref, "bf16", f"ragged attention {wl.name} rank {rank} causal={causal}")


def test_short_seq_refused():
    """A sequence shorter than one 32-key block is refused before any launch."""
    wl = inputs.AttnWorkload("attn_short", 1, 31, 1024, 8, 128, 2, "bf16", 1.0, 0.02, "f32", 0.02)
    x = torch.zeros((1, 31, 1024), dtype=torch.bfloat16, device="cuda")
    wqkv = torch.zeros((1024, 3 * 4 * 128), dtype=torch.bfloat16, device="cuda")
    wo = torch.zeros((4 * 128, 1024), dtype=torch.bfloat16, device="cuda")
    out = nan_tensor((1, 31, 1024), torch.float32)
    ws = torch.empty(binding.tp_attn_shard_workspace_bytes(1, 31, 1024, 8, 128, 2, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.TpError, match="UNSUPPORTED"):
        binding.tp_attn_shard_fwd(x, wqkv, wo, out, ws, heads=8, head_dim=128, t=2, rank=0)
    assert torch.isnan(out).all()
