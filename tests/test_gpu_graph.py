"""Graph capture of the C-ABI entry points.  Every launch the library makes
is an ordinary kernel launch on the caller's stream (no allocation, no
memset, no synchronisation), so a captured sequence of calls replays to the
same bits as the eager calls.  Each graph is replayed several times, with
outputs poisoned before each replay and eager calls of the same entry points
in between, and every replay is compared with the eager result bit for bit."""
import numpy as np
import pytest
import torch

from megatron_tensor_transformer_tp_amd import binding, inputs
from tests.gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def _replay_matches(run, outs, reps=3):
    """Eager reference, capture of `run`, then `reps` replays checked bit for
    bit against the reference with an eager `run` between replays."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    # warm-up on a side stream, as graph capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(reps):
        for t in outs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"replay {rep}: output {i} differs from the eager result"
        run()                                   # eager work between replays
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"eager call after replay {rep}: output {i} differs"


def test_mlp_forward_and_backward_replay():
    wl = inputs.MLP_WORKLOADS["t4_h1024_m1024"]
    r = 1
    say("graph: t4_h1024_m1024 rank 1 forward (pre-activation saved) + backward")
    xd, dzd = dev(inputs.mlp_x_rows(wl), "bf16"), dev(inputs.mlp_dz_rows(wl), "bf16")
    ad, bd = dev(inputs.mlp_a_block(wl, r), "bf16"), dev(inputs.mlp_b_block(wl, r), "bf16")
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    wsb = torch.empty(binding.tp_mlp_shard_bwd_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                               torch.bfloat16), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    z = torch.empty((wl.tokens, wl.hidden), **f32)
    y = torch.empty((wl.tokens, wl.f), dtype=torch.bfloat16, device="cuda")
    dx, da, db = (torch.empty(s, **f32) for s in ((wl.tokens, wl.hidden), (wl.hidden, wl.f), (wl.f, wl.hidden)))
    dba, dbb = torch.empty((wl.f,), **f32), torch.empty((wl.hidden,), **f32)

    def run():
        binding.tp_mlp_shard_fwd(xd, ad, bd, z, ws, ffn=wl.ffn, t=wl.t, rank=r, y_save=y)
        binding.tp_mlp_shard_bwd(xd, ad, bd, y, dzd, dx, da, db, wsb, ffn=wl.ffn, t=wl.t, rank=r,
                                 dbias_a_i=dba, dbias_b=dbb)

    _replay_matches(run, [z, y, dx, da, db, dba, dbb])


def test_attention_and_sp_replay():
    wl = inputs.ATTN_WORKLOADS["attn_t2_h1024_b2_s384"]
    r = 0
    say("graph: attn_t2_h1024_b2_s384 rank 0 attention shard + SP reduce-scatter of two partials")
    tokens = wl.batch * wl.seq
    xd = dev(np.stack([inputs.attn_x(wl, b) for b in range(wl.batch)]), "bf16")
    wqkv = dev(inputs.attn_wqkv_block(wl, r), "bf16")
    wo = dev(inputs.attn_wo_block(wl, r), "bf16")
    ws = torch.empty(binding.tp_attn_shard_workspace_bytes(wl.batch, wl.seq, wl.hidden, wl.heads, wl.head_dim,
                                                           wl.t, torch.bfloat16), dtype=torch.uint8, device="cuda")
    out = torch.empty((tokens, wl.hidden), dtype=torch.float32, device="cuda")
    other = torch.randn((tokens, wl.hidden), dtype=torch.float32, device="cuda")
    sp_out = torch.empty((tokens // 2, wl.hidden), dtype=torch.float32, device="cuda")

    def run():
        binding.tp_attn_shard_fwd(xd, wqkv, wo, out, ws, heads=wl.heads, head_dim=wl.head_dim, t=wl.t,
                                  rank=r)
        binding.tp_sp_reduce_scatter([out, other], sp_out, t=2, rank=1)

    _replay_matches(run, [out, sp_out])


def test_swiglu_linears_ragged_attention_and_empty_backward_replay():
    """One graph with the entry points the other captures leave out: the
    SwiGLU shard, the column linear with GeLU, the standalone GeLU, the row
    linear with bias and residual, attention at a length that is not a
    multiple of its blocks (the ragged kernel, causal), and a backward over
    zero tokens (its gradients zeroed by a fill kernel, not a memset)."""
    wl = inputs.MLP_WORKLOADS["t4_h1024_m1024"]
    r = 2
    say("graph: SwiGLU shard, column / row linears, GeLU, ragged causal attention, empty backward")
    xd = dev(inputs.mlp_x_rows(wl), "bf16")
    ad, bd = dev(inputs.mlp_a_block(wl, r), "bf16"), dev(inputs.mlp_b_block(wl, r), "bf16")
    wg, wu = dev(inputs.mlp_wg_block(wl, r), "bf16"), dev(inputs.mlp_wu_block(wl, r), "bf16")
    f32 = dict(dtype=torch.float32, device="cuda")
    zs = torch.empty((wl.tokens, wl.hidden), **f32)
    wss = torch.empty(binding.tp_mlp_swiglu_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                                  torch.bfloat16), dtype=torch.uint8, device="cuda")
    y = torch.empty((wl.tokens, wl.f), **f32)
    h = torch.empty((wl.tokens, wl.f), dtype=torch.bfloat16, device="cuda")
    bias = torch.randn((wl.hidden,), device="cuda").to(torch.bfloat16)
    res = torch.randn((wl.tokens, wl.hidden), device="cuda").to(torch.bfloat16)
    zr = torch.empty((wl.tokens, wl.hidden), **f32)

    aw = inputs.AttnWorkload("attn_graph_ragged", 2, 200, 1024, 8, 128, 2, "bf16", 1.0, 1.8 / np.sqrt(1024),
                             "f32", 0.02)
    xa = dev(np.stack([inputs.attn_x(aw, b) for b in range(aw.batch)]), "bf16")
    wqkv, wo = dev(inputs.attn_wqkv_block(aw, 1), "bf16"), dev(inputs.attn_wo_block(aw, 1), "bf16")
    wsa = torch.empty(binding.tp_attn_shard_workspace_bytes(aw.batch, aw.seq, aw.hidden, aw.heads, aw.head_dim,
                                                            aw.t, torch.bfloat16), dtype=torch.uint8, device="cuda")
    oa = torch.empty((aw.batch * aw.seq, aw.hidden), **f32)

    x0 = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    y0 = torch.empty((0, wl.f), dtype=torch.bfloat16, device="cuda")
    dx0 = torch.empty((0, wl.hidden), **f32)
    da0, db0 = torch.empty((wl.hidden, wl.f), **f32), torch.empty((wl.f, wl.hidden), **f32)
    dba0, dbb0 = torch.empty((wl.f,), **f32), torch.empty((wl.hidden,), **f32)
    wsb = torch.empty(256, dtype=torch.uint8, device="cuda")

    def run():
        binding.tp_mlp_swiglu_shard_fwd(xd, wg, wu, bd, zs, wss, ffn=wl.ffn, t=wl.t, rank=r)
        binding.tp_column_linear(xd, ad, y, ffn=wl.ffn, t=wl.t, rank=r)
        binding.tp_gelu(y, h)
        binding.tp_row_linear(h, bd, zr, ffn=wl.ffn, t=wl.t, rank=0, bias=bias, residual=res)
        binding.tp_attn_shard_fwd(xa, wqkv, wo, oa, wsa, heads=aw.heads, head_dim=aw.head_dim, t=aw.t,
                                  rank=1, causal=True)
        binding.tp_mlp_shard_bwd(x0, ad, bd, y0, x0, dx0, da0, db0, wsb, ffn=wl.ffn, t=wl.t, rank=r,
                                 dbias_a_i=dba0, dbias_b=dbb0)

    _replay_matches(run, [zs, y, h, zr, oa, da0, db0, dba0, dbb0])
    for g in (da0, db0, dba0, dbb0):
        assert bool((g == 0).all()), "gradients over zero tokens must be zero"


def test_split_attention_replay():
    """Attention over few long rows (at most half as many query blocks as
    CUs, 2048 keys or more), where each row's keys run on two workgroups and
    the second of the two to finish merges both halves: the merge is
    symmetric in the halves, so every call and replay gives the same bits
    whichever finishes last (non-causal, and causal at a ragged length)."""
    say("graph: split attention rows, non-causal seq 2048 and causal seq 2100")
    f32 = dict(dtype=torch.float32, device="cuda")
    calls, outs = [], []
    for seq, causal in ((2048, False), (2100, True)):
        aw = inputs.AttnWorkload(f"attn_graph_split_{seq}", 1, seq, 512, 4, 128, 2, "bf16", 1.0,
                                 1.8 / np.sqrt(512), "f32", 0.02)
        xa = dev(np.stack([inputs.attn_x(aw, 0)]), "bf16")
        wqkv, wo = dev(inputs.attn_wqkv_block(aw, 1), "bf16"), dev(inputs.attn_wo_block(aw, 1), "bf16")
        wsa = torch.empty(binding.tp_attn_shard_workspace_bytes(1, seq, aw.hidden, aw.heads, aw.head_dim, aw.t,
                                                                torch.bfloat16), dtype=torch.uint8, device="cuda")
        oa = torch.empty((seq, aw.hidden), **f32)
        calls.append((xa, wqkv, wo, oa, wsa, aw, causal))
        outs.append(oa)

    def run():
        for xa, wqkv, wo, oa, wsa, aw, causal in calls:
            binding.tp_attn_shard_fwd(xa, wqkv, wo, oa, wsa, heads=aw.heads, head_dim=aw.head_dim, t=aw.t,
                                      rank=1, causal=causal)

    _replay_matches(run, outs, reps=4)


def test_few_token_split_k_replay():
    """The MLP shard at few tokens, where both products run split-K (fp32
    partial products of k-slices, summed in a fixed order by the epilogue
    kernel): captured and replayed, bit for bit (16 tokens, h 2048, f 1024,
    bias, residual and the saved pre-activation)."""
    say("graph: 16-token MLP shard (split-K products)")
    t, rank = 4, 0
    wl = inputs.MlpWorkload("graph_few_tokens", 16, 2048, 1024 * t, t, "bf16", 1.0, 0.02, 0.02, "f32")
    xd = dev(inputs.mlp_x_rows(wl), "bf16")
    ad, bd = dev(inputs.mlp_a_block(wl, rank), "bf16"), dev(inputs.mlp_b_block(wl, rank), "bf16")
    ba, bb = dev(inputs.mlp_bias_a_block(wl, rank), "bf16"), dev(inputs.mlp_bias_b(wl), "bf16")
    res = dev(inputs.mlp_residual_rows(wl), "bf16")
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    z = torch.empty((wl.tokens, wl.hidden), dtype=torch.float32, device="cuda")
    y = torch.empty((wl.tokens, wl.f), dtype=torch.bfloat16, device="cuda")

    def run():
        binding.tp_mlp_shard_fwd(xd, ad, bd, z, ws, ffn=wl.ffn, t=wl.t, rank=rank, bias_a_i=ba, bias_b=bb,
                                 residual=res, y_save=y)

    _replay_matches(run, [z, y], reps=4)
