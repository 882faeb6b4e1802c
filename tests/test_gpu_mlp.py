"""GPU parity of the MLP shard entry points against the fp64 oracle.

Every call goes through the C ABI (via the ctypes binding).  Outputs are
NaN-filled before each call so an unwritten tile cannot pass.  Tolerances:
bf16 inputs with fp32 accumulation -- max |err| / (1 + |ref|) <= 2e-2 and
relative Frobenius <= 5e-3 per shard; fp32 path -- both <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import assert_close, dev, host64, nan_tensor, say, to_np

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def full_weights(wl):
    a = np.concatenate([inputs.mlp_a_block(wl, r) for r in range(wl.t)], axis=1)
    b = np.concatenate([inputs.mlp_b_block(wl, r) for r in range(wl.t)], axis=0)
    return a, b


def run_shard(wl, r, xd, ad, bd, out_dtype, extras=None):
    extras = extras or {}
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                          TORCH_DT[wl.dtype]),
                     dtype=torch.uint8, device="cuda")
    z = nan_tensor((wl.tokens, wl.hidden), TORCH_DT[out_dtype])
    binding.tp_mlp_shard_fwd(xd, ad, bd, z, ws, ffn=wl.ffn, t=wl.t, rank=r, **extras)
    torch.cuda.synchronize()
    return z


@pytest.mark.parametrize("with_extras", [False, True])
def test_tiny_f32_all_ranks_and_local_sum(with_extras):
    wl = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    x = inputs.mlp_x_rows(wl)
    a, b = full_weights(wl)
    ex_h, ex_d = {}, {}
    if with_extras:
        ba = np.concatenate([inputs.mlp_bias_a_block(wl, r) for r in range(wl.t)])
        bb, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
        ex_h = dict(bias_a=ba, bias_b=bb, residual=res)
        ex_d = dict(bias_b=dev(bb, "f32"), residual=dev(res, "f32"))
    total = None
    for r in range(wl.t):
        say(f"tiny_f32_t4 rank {r} extras={with_extras}")
        ed = dict(ex_d)
        if with_extras:
            ed["bias_a_i"] = dev(inputs.mlp_bias_a_block(wl, r), "f32")
        z = to_np(run_shard(wl, r, dev(x, "f32"), dev(inputs.mlp_a_block(wl, r), "f32"),
                            dev(inputs.mlp_b_block(wl, r), "f32"), "f32", ed))
        ref = oracle.mlp_shard(x, a, b, wl.t, r, **ex_h)
        assert_close(z, ref, "f32", f"tiny rank {r}")
        total = z if total is None else total + z
    assert_close(total, oracle.mlp_full(x, a, b, **ex_h), "f32", "tiny local sum of 4 ranks")


@pytest.mark.parametrize("with_extras", [False, True])
def test_t1_h1024_bf16_final_output(with_extras):
    wl = inputs.MLP_WORKLOADS["t1_h1024_m2048"]
    x = inputs.mlp_x_rows(wl)
    a, b = inputs.mlp_a_block(wl, 0), inputs.mlp_b_block(wl, 0)
    ex_h, ex_d = {}, {}
    if with_extras:
        ba, bb, res = inputs.mlp_bias_a_block(wl, 0), inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
        ex_h = dict(bias_a=host64(ba, "bf16"), bias_b=host64(bb, "bf16"), residual=host64(res, "bf16"))
        ex_d = dict(bias_a_i=dev(ba, "bf16"), bias_b=dev(bb, "bf16"), residual=dev(res, "bf16"))
    say(f"t1_h1024_m2048 extras={with_extras}")
    z = to_np(run_shard(wl, 0, dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16"), "bf16", ex_d))
    ref = oracle.mlp_shard(host64(x, "bf16"), host64(a, "bf16"), host64(b, "bf16"), 1, 0, **ex_h)
    assert_close(z, ref, "bf16", "t=1 h=1024 M=2048 bf16 out")


@pytest.mark.parametrize("tokens,hidden,f,rank,out", [
    (1, 1024, 512, 0, "f32"),
    (7, 1024, 512, 1, "f32"),
    (16, 8192, 4096, 0, "f32"),     # the headline shard's widths at 16 tokens
    (64, 2048, 1024, 0, "bf16"),
    (100, 1024, 1376, 0, "f32"),    # f = 1376: the row product's k range does not split, it stays tiled
    (128, 4096, 1024, 0, "f32"),
    (129, 1024, 512, 0, "f32"),     # 128 x 128 tiles for the split products from here on
    (200, 2048, 1024, 1, "bf16"),
    (256, 8192, 4096, 0, "f32"),    # headline widths: 4 and 2 k-slices
    (384, 2048, 1536, 0, "bf16"),
    (512, 1024, 512, 1, "f32"),
    (513, 1024, 512, 0, "f32"),     # past the split-K limit: the tiled products
])
def test_small_token_counts(tokens, hidden, f, rank, out):
    """Few tokens: the two products have few tiles and run split-K (k-slices
    written as fp32 partial products, summed in slice order by the kernel
    that applies the epilogue) up to 512 tokens; bias, residual and the
    saved pre-activation included, every element against the oracle."""
    t = 4
    wl = inputs.MlpWorkload(f"small_{tokens}_{hidden}_{f}", tokens, hidden, f * t, t, "bf16", 1.0, 0.02,
                            0.02, out)
    x, a, b = inputs.mlp_x_rows(wl), inputs.mlp_a_block(wl, rank), inputs.mlp_b_block(wl, rank)
    ba, bb, res = inputs.mlp_bias_a_block(wl, rank), inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    say(f"small token count: tokens={tokens} hidden={hidden} f={f} rank={rank} out={out}")
    y = nan_tensor((tokens, f), torch.bfloat16)
    ed = dict(bias_a_i=dev(ba, "bf16"), bias_b=dev(bb, "bf16"), residual=dev(res, "bf16"), y_save=y)
    z = to_np(run_shard(wl, rank, dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16"), out, ed))
    ref_y = oracle.column_linear(host64(x, "bf16"), host64(a, "bf16"), host64(ba, "bf16"))
    assert_close(to_np(y), ref_y, "bf16", f"small {tokens} tokens: saved pre-activation")
    ref = oracle.row_linear(oracle.column_linear(host64(x, "bf16"), host64(a, "bf16"), host64(ba, "bf16"),
                                                 apply_gelu=True),
                            host64(b, "bf16"), host64(bb, "bf16"), host64(res, "bf16"), rank=rank)
    assert_close(z, ref, out if out == "bf16" else "bf16", f"small {tokens} tokens: partial")


def test_t8_h8192_m4096_rank0_full():
    wl = inputs.MLP_WORKLOADS["t8_h8192_m4096"]
    x = inputs.mlp_x_rows(wl)
    a, b = inputs.mlp_a_block(wl, 0), inputs.mlp_b_block(wl, 0)
    say("t8_h8192_m4096 rank 0")
    z = to_np(run_shard(wl, 0, dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16"), "f32"))
    ref = oracle.row_linear(oracle.column_linear(host64(x, "bf16"), host64(a, "bf16"), apply_gelu=True),
                            host64(b, "bf16"), rank=0)
    assert_close(z, ref, "bf16", "t=8 h=8192 M=4096 rank 0 partial")


@pytest.fixture(scope="module")
def headline():
    """All 8 ranks of the t=8, h=8192, 16384-token workload, computed back to back on
    the GPU exactly as the benchmark launches them (partials stay on the device),
    and a host-side record of the oracle's partials summed so far."""
    wl = inputs.MLP_WORKLOADS["t8_h8192_m16384"]
    say("headline: generating inputs")
    xd = dev(inputs.mlp_x_rows(wl), "bf16")
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                          torch.bfloat16), dtype=torch.uint8, device="cuda")
    zs = []
    for r in range(wl.t):
        ad = dev(inputs.mlp_a_block(wl, r), "bf16")
        bd = dev(inputs.mlp_b_block(wl, r), "bf16")
        z = nan_tensor((wl.tokens, wl.hidden), torch.float32)
        say(f"headline rank {r}")
        binding.tp_mlp_shard_fwd(xd, ad, bd, z, ws, ffn=wl.ffn, t=wl.t, rank=r)
        zs.append(z)
    torch.cuda.synchronize()
    del ws, xd
    state = {"x64": host64(inputs.mlp_x_rows(wl), "bf16"), "ref_sum": None, "ranks": set()}
    return wl, zs, state


def _headline_ref(wl, state, r):
    """The oracle's partial Z_r of the whole shard (fp64, every token), added
    once into the running sum of the ranks' partials."""
    ref = oracle.row_linear(oracle.column_linear(state["x64"], host64(inputs.mlp_a_block(wl, r), "bf16"),
                                                 apply_gelu=True),
                            host64(inputs.mlp_b_block(wl, r), "bf16"), rank=r)
    if r not in state["ranks"]:
        state["ref_sum"] = ref.copy() if state["ref_sum"] is None else state["ref_sum"] + ref
        state["ranks"].add(r)
    return ref


@pytest.mark.parametrize("rank", range(8))
def test_headline_rank_full(headline, rank):
    """Every element of rank r's partial Z_r [16384, 8192] against the oracle:
    both bounds as stated, per shard."""
    wl, zs, state = headline
    say(f"headline rank {rank}: oracle over all {wl.tokens} tokens")
    ref = _headline_ref(wl, state, rank)
    got = zs[rank].cpu().numpy().astype(np.float64)
    assert_close(got, ref, "bf16", f"headline rank {rank}, all {got.size} elements")


def test_headline_reconstruction_full(headline):
    """sum_r Z_r formed on the device (the untimed local stand-in for the
    All-Reduce) against the unsharded GeLU(X A) B, every element.  Relative
    Frobenius as stated; the max criterion with floor sqrt(t): the t shards'
    bf16 rounding errors are independent and add in quadrature, so the sum's
    absolute error floor is sqrt(t) times a shard's (the stated-floor figure
    is printed beside it)."""
    wl, zs, state = headline
    for r in range(wl.t):
        if r not in state["ranks"]:
            say(f"headline reconstruction: oracle rank {r}")
            _headline_ref(wl, state, r)
    total = torch.zeros_like(zs[0])
    for z in zs:
        total += z
    got = total.cpu().numpy().astype(np.float64)
    del total
    assert_close(got, state["ref_sum"], "bf16", f"headline reconstruction of {wl.t} shards, all elements",
                 floor=float(np.sqrt(wl.t)))


def test_large_token_count_sampled():
    """65536 tokens at the headline widths (t = 8, rank 5): 16 rounds of
    256 x 256 column tiles and 32 of row tiles, a 2 GiB fp32 partial.  X
    goes up in row chunks; every output must be written (finite), and four
    64-row blocks spread over the rounds, the last rows included, are
    checked against the oracle (the shard is row-independent)."""
    wl = inputs.MlpWorkload("t8_h8192_m65536", 65536, 8192, 32768, 8, "bf16", 1.0, 0.02, 0.02, "f32")
    r = 5
    xd = torch.empty((wl.tokens, wl.hidden), dtype=torch.bfloat16, device="cuda")
    step = 8192
    for r0 in range(0, wl.tokens, step):
        xd[r0:r0 + step] = dev(inputs.mlp_x_rows(wl, r0, step), "bf16")
    a, b = inputs.mlp_a_block(wl, r), inputs.mlp_b_block(wl, r)
    say(f"65536 tokens, rank {r}")
    z = run_shard(wl, r, xd, dev(a, "bf16"), dev(b, "bf16"), "f32")
    del xd
    assert bool(torch.isfinite(z).all()), "unwritten or non-finite outputs"
    a64, b64 = host64(a, "bf16"), host64(b, "bf16")
    for r0 in (0, 21824, 43712, wl.tokens - 64):
        x64 = host64(inputs.mlp_x_rows(wl, r0, 64), "bf16")
        ref = oracle.mlp_shard(x64, a64, b64, 1, 0)
        got = z[r0:r0 + 64].cpu().numpy().astype(np.float64)
        assert_close(got, ref, "bf16", f"65536 tokens rank {r} rows {r0}..{r0 + 63}")


@pytest.mark.parametrize("tokens,hidden,f,gelu,out", [
    (5, 8, 64, True, "f32"),            # K = 8: the only k-tile is a partial one
    (33, 24, 72, False, "bf16"),        # K = 24
    (1, 64, 64, True, "bf16"),
    (77, 136, 200, True, "f32"),
    (300, 256, 1000, False, "bf16"),
    (513, 1024, 520, True, "bf16"),
    (4000, 1000, 4096, True, "bf16"),   # 256x256 tile path, ragged M and K
    (4000, 1000, 3000, True, "bf16"),   # 128x384 tile path, ragged M, N and K
    (2048, 1024, 1024, True, "bf16"),   # 64x128 tile path (128 tiles of 128x128 fill half the CUs)
    (1900, 1000, 1000, True, "f32"),    # 64x128 tiles, ragged M, N and K
])
def test_column_linear_ragged(tokens, hidden, f, gelu, out):
    t = 2
    wl = inputs.MlpWorkload(f"col_{tokens}_{hidden}_{f}", tokens, hidden, f * t, t, "bf16", 1.0, 0.05, 0.05, out)
    x, a = inputs.mlp_x_rows(wl), inputs.mlp_a_block(wl, 1)
    bias = inputs.mlp_bias_a_block(wl, 1)
    say(f"column_linear tokens={tokens} hidden={hidden} f={f} gelu={gelu} out={out}")
    y = nan_tensor((tokens, f), TORCH_DT[out])
    binding.tp_column_linear(dev(x, "bf16"), dev(a, "bf16"), y, ffn=f * t, t=t, rank=1,
                             bias_i=dev(bias, "bf16"), apply_gelu=gelu)
    torch.cuda.synchronize()
    ref = oracle.column_linear(host64(x, "bf16"), host64(a, "bf16"), host64(bias, "bf16"), apply_gelu=gelu)
    assert_close(to_np(y), ref, "bf16", "column_linear")


@pytest.mark.parametrize("tokens,f,hidden,rank,out", [
    (5, 64, 64, 0, "f32"),
    (129, 200, 136, 0, "bf16"),
    (129, 200, 136, 1, "f32"),
    (1000, 520, 1024, 0, "f32"),
    (4000, 1000, 4096, 0, "f32"),       # 256x256 tile path, ragged M and K, residual
    (4000, 1000, 3000, 0, "f32"),       # 128x384 tile path, ragged M, N and K, residual
    (2048, 4096, 1024, 0, "f32"),       # 64x128 tiles, paired A stages, fp32 restaging, residual
    (2000, 4000, 1000, 0, "f32"),       # 64x128 tiles, single stages (K % 64 != 0), ragged M and N
    (2048, 4096, 1024, 1, "bf16"),      # 64x128 tiles, bf16 out
])
def test_row_linear_ragged(tokens, f, hidden, rank, out):
    t = 2
    wl = inputs.MlpWorkload(f"row_{tokens}_{f}_{hidden}", tokens, hidden, f * t, t, "bf16", 1.0, 0.05, 0.05, out)
    h = inputs.draw(wl.name, "x", 99, (tokens, f), 1.0, "bf16")
    b = inputs.mlp_b_block(wl, rank)
    bias, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    say(f"row_linear tokens={tokens} f={f} hidden={hidden} rank={rank} out={out}")
    z = nan_tensor((tokens, hidden), TORCH_DT[out])
    binding.tp_row_linear(dev(h, "bf16"), dev(b, "bf16"), z, ffn=f * t, t=t, rank=rank,
                          bias=dev(bias, "bf16"), residual=dev(res, "bf16"))
    torch.cuda.synchronize()
    ref = oracle.row_linear(host64(h, "bf16"), host64(b, "bf16"), host64(bias, "bf16"),
                            host64(res, "bf16"), rank=rank)
    assert_close(to_np(z), ref, "bf16", f"row_linear rank {rank}")


def test_column_linear_ragged_multiround():
    """M, N and K all ragged at nearly the headline size: 256 x 256 tiles in
    four rounds of resident workgroups, edge tiles in every round, a partial
    last k-tile (K % 32 = 24), GeLU epilogue; every element checked."""
    tokens, hidden, f, t = 16376, 8184, 4088, 2
    wl = inputs.MlpWorkload("col_multiround", tokens, hidden, f * t, t, "bf16", 1.0, 0.02, 0.02, "bf16")
    x, a = inputs.mlp_x_rows(wl), inputs.mlp_a_block(wl, 0)
    bias = inputs.mlp_bias_a_block(wl, 0)
    say(f"column_linear multi-round tokens={tokens} hidden={hidden} f={f}")
    y = nan_tensor((tokens, f), torch.bfloat16)
    binding.tp_column_linear(dev(x, "bf16"), dev(a, "bf16"), y, ffn=f * t, t=t, rank=0,
                             bias_i=dev(bias, "bf16"), apply_gelu=True)
    torch.cuda.synchronize()
    got = to_np(y)
    assert not np.isnan(got).any(), "unwritten outputs"
    ref = oracle.column_linear(host64(x, "bf16"), host64(a, "bf16"), host64(bias, "bf16"),
                               apply_gelu=True)
    assert_close(got, ref, "bf16", "column_linear multi-round")


def test_row_linear_ragged_multiround():
    """As above for the row layer (fp32 out, bias and residual on rank 0):
    eight rounds, the LDS-restaged epilogue on interior tiles and the masked
    one on edge tiles, K % 32 = 24; every element checked."""
    tokens, f, hidden, t = 16376, 4088, 8184, 2
    wl = inputs.MlpWorkload("row_multiround", tokens, hidden, f * t, t, "bf16", 1.0, 0.02, 0.02, "f32")
    h = inputs.draw(wl.name, "x", 99, (tokens, f), 1.0, "bf16")
    b = inputs.mlp_b_block(wl, 0)
    bias, res = inputs.mlp_bias_b(wl), inputs.mlp_residual_rows(wl)
    say(f"row_linear multi-round tokens={tokens} f={f} hidden={hidden}")
    z = nan_tensor((tokens, hidden), torch.float32)
    binding.tp_row_linear(dev(h, "bf16"), dev(b, "bf16"), z, ffn=f * t, t=t, rank=0,
                          bias=dev(bias, "bf16"), residual=dev(res, "bf16"))
    torch.cuda.synchronize()
    got = to_np(z)
    assert not np.isnan(got).any(), "unwritten outputs"
    ref = oracle.row_linear(host64(h, "bf16"), host64(b, "bf16"), host64(bias, "bf16"),
                            host64(res, "bf16"), rank=0)
    assert_close(got, ref, "bf16", "row_linear multi-round")


@pytest.mark.parametrize("n", [1, 7, 8, 1000, (1 << 20) + 3])
@pytest.mark.parametrize("in_dt,out_dt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32"), ("bf16", "bf16")])
def test_gelu_standalone(n, in_dt, out_dt):
    v = inputs.draw(f"gelu_{n}", "x", 0, (n,), 3.0, in_dt)
    say(f"gelu n={n} {in_dt}->{out_dt}")
    y = nan_tensor((n,), TORCH_DT[out_dt])
    binding.tp_gelu(dev(v, in_dt), y)
    torch.cuda.synchronize()
    ref = oracle.gelu(host64(v, in_dt))
    got = to_np(y)
    if out_dt == "f32":
        assert np.isfinite(got).all() and np.max(np.abs(got - ref) / (1 + np.abs(ref))) <= 1e-5
    else:
        # a bf16 result is within one bf16 ulp of the exact value (absolute
        # floor for the far negative tail, where GeLU underflows towards 0)
        assert np.isfinite(got).all()
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6)


def test_gelu_in_place():
    v = inputs.draw("gelu_inplace", "x", 0, (4099,), 2.0, "f32")
    d = dev(v, "f32")
    binding.tp_gelu(d, d)
    torch.cuda.synchronize()
    ref = oracle.gelu(host64(v, "f32"))
    assert np.max(np.abs(to_np(d) - ref) / (1 + np.abs(ref))) <= 1e-5


def test_unfused_path_matches_oracle():
    """column_linear (fp32 Y) -> gelu (bf16 H) -> row_linear: the three separate
    entry points compose to the same shard as the fused call."""
    wl = inputs.MlpWorkload("unfused", 640, 512, 2048, 2, "bf16", 1.0, 0.05, 0.05, "f32")
    x, a, b = inputs.mlp_x_rows(wl), inputs.mlp_a_block(wl, 0), inputs.mlp_b_block(wl, 0)
    f = wl.f
    xd, ad, bd = dev(x, "bf16"), dev(a, "bf16"), dev(b, "bf16")
    say("unfused column -> gelu -> row")
    y = nan_tensor((wl.tokens, f), torch.float32)
    binding.tp_column_linear(xd, ad, y, ffn=wl.ffn, t=wl.t, rank=0)
    h = nan_tensor((wl.tokens, f), torch.bfloat16)
    binding.tp_gelu(y, h)
    z = nan_tensor((wl.tokens, wl.hidden), torch.float32)
    binding.tp_row_linear(h, bd, z, ffn=wl.ffn, t=wl.t, rank=0)
    zf = run_shard(wl, 0, xd, ad, bd, "f32")
    torch.cuda.synchronize()
    ref = oracle.row_linear(oracle.column_linear(host64(x, "bf16"), host64(a, "bf16"), apply_gelu=True),
                            host64(b, "bf16"))
    assert_close(to_np(z), ref, "bf16", "unfused shard")
    assert_close(to_np(zf), ref, "bf16", "fused shard")


def test_strided_views_and_lda():
    """A_i given as a column-block VIEW of the full A (lda = F) and X with ldx > hidden."""
    wl = inputs.MlpWorkload("views", 200, 128, 1024, 4, "bf16", 1.0, 0.05, 0.05, "f32")
    a_full, b_full = full_weights(wl)
    x = inputs.mlp_x_rows(wl)
    a_dev = dev(a_full, "bf16")
    xpad = torch.zeros((wl.tokens, wl.hidden + 64), dtype=torch.bfloat16, device="cuda")
    xpad[:, :wl.hidden] = dev(x, "bf16")
    xview = xpad[:, :wl.hidden]
    for r in range(wl.t):
        say(f"views rank {r}")
        a_view = a_dev[:, r * wl.f:(r + 1) * wl.f]
        y = nan_tensor((wl.tokens, wl.f), torch.bfloat16)
        binding.tp_column_linear(xview, a_view, y, ffn=wl.ffn, t=wl.t, rank=r, apply_gelu=True)
        ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                              torch.bfloat16), dtype=torch.uint8, device="cuda")
        z = nan_tensor((wl.tokens, wl.hidden), torch.float32)
        binding.tp_mlp_shard_fwd(dev(x, "bf16"), a_view, dev(inputs.mlp_b_block(wl, r), "bf16"), z, ws,
                                 ffn=wl.ffn, t=wl.t, rank=r)
        torch.cuda.synchronize()
        s = oracle.shard_slice(wl.ffn, wl.t, r)
        assert_close(to_np(y), oracle.column_linear(host64(x, "bf16"), host64(a_full, "bf16")[:, s],
                                                    apply_gelu=True), "bf16", "column on views")
        assert_close(to_np(z), oracle.mlp_shard(host64(x, "bf16"), host64(a_full, "bf16"),
                                                host64(b_full, "bf16"), wl.t, r), "bf16", "shard with lda")


def test_tokens_zero_is_noop_and_errors_raise():
    z = torch.full((4, 64), 7.0, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    binding.tp_mlp_shard_fwd(x, a, a, z[:0], ws, ffn=128, t=2, rank=0)
    torch.cuda.synchronize()
    assert torch.all(z == 7.0).item()
    with pytest.raises(binding.TpError) as e:
        binding.tp_mlp_shard_fwd(torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda"), a, a, z, ws,
                                 ffn=129, t=2, rank=0)
    assert e.value.status == 2  # not divisible
    with pytest.raises(binding.TpError):
        binding.tp_column_linear(torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda"), a,
                                 torch.empty((4, 64), device="cuda"), ffn=128, t=2, rank=2)
