"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage (page title + section) or the closed form it
checks.  They are chosen so that a plausible slip in the oracle -- a dropped
factor in GeLU, erf(z) for erf(z/sqrt2), a transposed weight, B's rows taken
from another block than A's columns, the bias or residual added on every
rank, a 1/d softmax scale -- fails at least one of them.
"""
import math
import os

import mpmath
import numpy as np
import pytest
from scipy.special import ndtr

import oracle
from megatron_tensor_transformer_tp_amd import inputs
from tests.conftest import read_golden_table

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- GeLU
def test_gelu_matches_textbook_normal_cdf(golden_dir):
    """GeLU(z)/z = Phi(z) (列并行 tutorial, MLP 应用) against table values."""
    rows = read_golden_table(os.path.join(golden_dir, "normal_cdf.txt"))
    assert len(rows) == 12
    for z_s, phi_s in rows:
        z, phi = float(z_s), float(phi_s)
        g = float(oracle.gelu(z))
        assert g == pytest.approx(z * phi, rel=1e-13, abs=1e-300)
        if z == 0.0:
            assert g == 0.0


def test_gelu_closed_forms():
    z = np.linspace(-8.0, 8.0, 1601)
    g = oracle.gelu(z)
    # GeLU(z) - GeLU(-z) = z Phi(z) - (-z)(1 - Phi(z)) = z
    np.testing.assert_allclose(g - oracle.gelu(-z), z, rtol=0, atol=1e-14)
    # Phi via an independent library routine (ndtr, not erf)
    nz = z[z != 0]
    np.testing.assert_allclose(oracle.gelu(nz) / nz, ndtr(nz), rtol=5e-14, atol=1e-300)
    # tails: GeLU(z) -> z for z >> 0, -> 0 for z << 0
    assert abs(float(oracle.gelu(40.0)) - 40.0) == 0.0
    assert abs(float(oracle.gelu(-40.0))) < 1e-300
    assert float(oracle.gelu(0.0)) == 0.0


def test_gelu_mpmath_50_digits():
    mpmath.mp.dps = 50
    for z in (-6.5, -2.25, -1e-3, 1e-3, 0.7, 1.0, 3.3, 5.0):
        ref = mpmath.mpf(z) * mpmath.ncdf(mpmath.mpf(z))
        got = float(oracle.gelu(z))
        assert abs(got - float(ref)) <= 4e-16 * max(1.0, abs(float(ref))), (z, got, ref)


# ------------------------------------------------------------- column split
def test_column_split_demo_shapes_and_equality(golden_dir):
    """列并行 tutorial, Python 演示: p column blocks -> p partials [batch, d_out/p],
    concatenated -> [batch, d_out] equal to the unsplit product."""
    g = {r[0]: [int(v) for v in r[1:]] for r in read_golden_table(
        os.path.join(golden_dir, "column_split_demo.txt"))}
    batch, d_in, d_out, p = g["batch"][0], g["d_in"][0], g["d_out"][0], g["p"][0]
    rng = _rng(42)
    x = rng.standard_normal((batch, d_in))
    w = rng.standard_normal((d_in, d_out))
    f = oracle.shard_width(d_out, p)
    partials = [oracle.column_linear(x, w[:, oracle.shard_slice(d_out, p, r)]) for r in range(p)]
    assert [list(q.shape) for q in partials] == [g["partial_shape"]] * p
    gathered = np.concatenate(partials, axis=1)
    assert list(gathered.shape) == g["gathered_shape"]
    assert f == g["partial_shape"][1]
    # brute-force the unsplit product from the index definition
    ref = np.array([[sum(x[i, k] * w[k, j] for k in range(d_in)) for j in range(d_out)]
                    for i in range(batch)])
    np.testing.assert_allclose(gathered, ref, rtol=1e-13, atol=1e-13)


def test_column_concat_identity_and_gelu_block_invariance():
    """列并行 tutorial, 数学基础 (XW = [XW^(1)|...|XW^(p)]) and MLP 应用
    (GeLU of a column block = that block of GeLU(XW))."""
    rng = _rng(1)
    x = rng.standard_normal((37, 24))
    a = rng.standard_normal((24, 40))
    bias = rng.standard_normal(40)
    full = oracle.column_linear(x, a, bias)
    full_g = oracle.gelu(full)
    for t in (1, 2, 4, 5, 8):
        parts = []
        for r in range(t):
            s = oracle.shard_slice(40, t, r)
            y_r = oracle.column_linear(x, a[:, s], bias[s])
            np.testing.assert_allclose(y_r, full[:, s], rtol=1e-13, atol=1e-13)
            h_r = oracle.column_linear(x, a[:, s], bias[s], apply_gelu=True)
            np.testing.assert_allclose(h_r, full_g[:, s], rtol=1e-13, atol=1e-13)
            parts.append(y_r)
        np.testing.assert_allclose(np.concatenate(parts, axis=1), full, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ row split / sum
def test_hand_computed_mlp_example():
    """A 1-token MLP worked by hand with the table values of Phi.

    X = [1, 2]; A = [[1, 0, -1, 2], [0, 1, 1, -1]] -> Y = [1, 2, 1, 0];
    H = [Phi(1), 2 Phi(2), Phi(1), 0]; B rows = e_1, e_2, e_1 + e_2, 7 e_2.
    Z = [H0 + H2, H1 + H2] = [2 Phi(1), 2 Phi(2) + Phi(1)].
    With t = 2: rank 0 owns A columns {0,1} / B rows {0,1}, rank 1 owns {2,3}.
    """
    p1, p2 = 0.841344746068543, 0.977249868051821
    x = np.array([[1.0, 2.0]])
    a = np.array([[1.0, 0.0, -1.0, 2.0], [0.0, 1.0, 1.0, -1.0]])
    b = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [0.0, 7.0]])
    z0 = oracle.mlp_shard(x, a, b, 2, 0)
    z1 = oracle.mlp_shard(x, a, b, 2, 1)
    np.testing.assert_allclose(z0, [[p1, 2 * p2]], rtol=1e-14)
    np.testing.assert_allclose(z1, [[p1, p1]], rtol=1e-14)
    np.testing.assert_allclose(oracle.mlp_full(x, a, b), [[2 * p1, 2 * p2 + p1]], rtol=1e-14)


@pytest.mark.parametrize("with_extras", [False, True])
def test_row_sum_identity_tiny_workload(with_extras):
    """sum_r GeLU(X A_r) B_r = GeLU(X A) B (列并行 tutorial, MLP 应用; overview
    考点 2) on the tiny fp32 workload (t = 4), with bias/residual on rank 0."""
    wl = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    x = inputs.mlp_x_rows(wl)
    a = np.concatenate([inputs.mlp_a_block(wl, r) for r in range(wl.t)], axis=1)
    b = np.concatenate([inputs.mlp_b_block(wl, r) for r in range(wl.t)], axis=0)
    ex = {}
    if with_extras:
        ex = dict(bias_a=np.concatenate([inputs.mlp_bias_a_block(wl, r) for r in range(wl.t)]),
                  bias_b=inputs.mlp_bias_b(wl), residual=inputs.mlp_residual_rows(wl))
    full = oracle.mlp_full(x, a, b, **ex)
    summed = oracle.mlp_partial_sum(x, a, b, wl.t, **ex)
    err = np.linalg.norm(summed - full) / np.linalg.norm(full)
    assert err <= 1e-12
    assert full.shape == (wl.tokens, wl.hidden)


def test_row_sum_identity_relu_variant():
    """Overview page, 第三章: the split identity also holds with ReLU in place
    of GeLU (the page's own simulation uses ReLU)."""
    rng = _rng(7)
    x, a, b = rng.standard_normal((2, 8)), rng.standard_normal((8, 32)), rng.standard_normal((32, 8))
    summed = oracle.mlp_partial_sum(x, a, b, 2, activation="relu")
    ref = np.array([[sum(max(0.0, sum(x[i, k] * a[k, j] for k in range(8))) * b[j, n] for j in range(32))
                     for n in range(8)] for i in range(2)])
    np.testing.assert_allclose(summed, ref, rtol=1e-12, atol=1e-12)


def test_mismatched_blocks_break_the_identity():
    """Negative control: B rows from a different block than A columns, or the
    residual added by every rank, do NOT reproduce the unsharded layer."""
    rng = _rng(3)
    x, a, b = rng.standard_normal((5, 6)), rng.standard_normal((6, 12)), rng.standard_normal((12, 6))
    full = oracle.mlp_full(x, a, b)
    t = 3
    wrong = sum(oracle.row_linear(oracle.column_linear(x, a[:, oracle.shard_slice(12, t, r)], apply_gelu=True),
                                  b[oracle.shard_slice(12, t, (r + 1) % t), :]) for r in range(t))
    assert np.linalg.norm(wrong - full) > 1e-3 * np.linalg.norm(full)
    res = rng.standard_normal((5, 6))
    all_ranks = sum(oracle.row_linear(oracle.column_linear(x, a[:, oracle.shard_slice(12, t, r)], apply_gelu=True),
                                      b[oracle.shard_slice(12, t, r), :], residual=res, rank=0) for r in range(t))
    assert np.linalg.norm(all_ranks - (full + res)) > 1.0


def test_t1_shard_is_whole_mlp():
    """t = 1: the single shard is the whole MLP (Tencent write-up, FFN paragraph)."""
    rng = _rng(11)
    x, a, b = rng.standard_normal((9, 16)), rng.standard_normal((16, 64)), rng.standard_normal((64, 16))
    np.testing.assert_array_equal(oracle.mlp_shard(x, a, b, 1, 0), oracle.mlp_full(x, a, b))


@pytest.mark.parametrize("rank", [0, 1, 2])
def test_brute_force_loops_match_vectorised(rank):
    """Pure-Python index loops (math.erf) == vectorised oracle, non-square
    shapes so that a transposed operand cannot pass."""
    rng = _rng(100 + rank)
    M, h, F, t = 5, 7, 12, 3
    x, a, b = rng.standard_normal((M, h)), rng.standard_normal((h, F)), rng.standard_normal((F, h))
    ba, bb, res = rng.standard_normal(F), rng.standard_normal(h), rng.standard_normal((M, h))
    got = oracle.mlp_shard(x, a, b, t, rank, ba, bb, res)
    ref = np.array(oracle.mlp_shard_loops(x.tolist(), a.tolist(), b.tolist(), t, rank,
                                          ba.tolist(), bb.tolist(), res.tolist()))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_full_tiny_workload():
    """Brute-force loops over every rank of the tiny fp32 workload."""
    wl = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    x = inputs.mlp_x_rows(wl).astype(np.float64)
    a = np.concatenate([inputs.mlp_a_block(wl, r) for r in range(wl.t)], axis=1).astype(np.float64)
    b = np.concatenate([inputs.mlp_b_block(wl, r) for r in range(wl.t)], axis=0).astype(np.float64)
    xl, al, bl = x.tolist(), a.tolist(), b.tolist()
    for r in range(wl.t):
        got = oracle.mlp_shard(x, a, b, wl.t, r)
        ref = np.array(oracle.mlp_shard_loops(xl, al, bl, wl.t, r))
        assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


def test_divisibility_and_rank_rejected():
    """列并行 tutorial 切分原理 (h mod p = 0) and Megatron Level 2 M031 (fail fast)."""
    with pytest.raises(oracle.ShardError):
        oracle.shard_width(10, 3)
    with pytest.raises(oracle.ShardError):
        oracle.shard_width(10, 0)
    with pytest.raises(oracle.ShardError):
        oracle.shard_slice(12, 3, 3)
    with pytest.raises(oracle.ShardError):
        oracle.shard_slice(12, 3, -1)
    with pytest.raises(oracle.ShardError):
        oracle.mlp_shard(np.ones((2, 4)), np.ones((4, 10)), np.ones((10, 4)), 4, 0)
    with pytest.raises(oracle.ShardError):
        oracle.local_heads(12, 5)
    assert oracle.shard_width(32768, 8) == 4096


def test_partial_is_full_hidden_64MiB(golden_dir):
    """Overview page, 考点 2: one rank's partial at 4096 tokens x hidden 8192 in
    2-byte elements is 64 MiB, whatever t is (the partial is full-hidden)."""
    g = {r[0]: int(r[1]) for r in read_golden_table(os.path.join(golden_dir, "partial_sum_bytes.txt"))}
    f = oracle.shard_width(4 * g["hidden"], g["t"])
    # a rank's partial for a rank-1 (f = 1) stand-in: only the shape matters here
    z = oracle.row_linear(np.zeros((g["tokens"], 1)), np.zeros((1, g["hidden"])), rank=1)
    assert z.shape == (g["tokens"], g["hidden"])
    assert z.size * g["bytes_per_element"] == g["bytes"]
    assert f == 4096


# ------------------------------------------------------------------ attention
def _tiny_attn(seed=5, batch=2, seq=6, heads=4, d=3, t=2):
    rng = _rng(seed)
    h = heads * d
    x = rng.standard_normal((batch, seq, h))
    wqkv = rng.standard_normal((h, 3 * h))
    wo = rng.standard_normal((h, h))
    return x, wqkv, wo, heads, d, t


@pytest.mark.parametrize("causal", [False, True])
def test_head_local_sum_equals_full_mha(causal):
    """Tencent write-up (attention paragraph) / Megatron Level 2 M028: the sum
    of the head-local shards equals full multi-head attention."""
    for t in (1, 2, 4):
        x, wqkv, wo, heads, d, _ = _tiny_attn(t=t)
        wq, wk, wv = oracle.split_packed_qkv(wqkv, heads, d)
        full = oracle.mha_full(x, wq, wk, wv, wo, heads, causal)
        summed = oracle.attn_partial_sum(x, wqkv, wo, heads, d, t, causal)
        assert np.linalg.norm(summed - full) <= 1e-12 * np.linalg.norm(full)


def test_attention_head_matches_loops():
    rng = _rng(9)
    q, k, v = rng.standard_normal((5, 4)), rng.standard_normal((7, 4)), rng.standard_normal((7, 3))
    from oracle.attention import _attend
    for causal in (False, True):
        if causal:
            k, v = k[:5], v[:5]
        got = _attend(q, k, v, causal)
        ref = np.array(oracle.attention_head_loops(q.tolist(), k.tolist(), v.tolist(), causal))
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_softmax_special_cases():
    from oracle.attention import _attend
    rng = _rng(13)
    s = rng.standard_normal((6, 9)) * 5
    np.testing.assert_allclose(oracle.softmax_rows(s).sum(axis=1), 1.0, rtol=0, atol=1e-15)
    v = rng.standard_normal((9, 4))
    k = rng.standard_normal((9, 4))
    # q = 0 -> uniform weights -> mean of the value rows
    np.testing.assert_allclose(_attend(np.zeros((3, 4)), k, v, False), np.tile(v.mean(0), (3, 1)),
                               rtol=1e-14, atol=1e-14)
    # one key -> its value row
    np.testing.assert_allclose(_attend(rng.standard_normal((3, 4)), k[:1], v[:1], False),
                               np.tile(v[0], (3, 1)), rtol=1e-14)
    # permuting keys and values together leaves the output unchanged
    q = rng.standard_normal((3, 4))
    perm = rng.permutation(9)
    np.testing.assert_allclose(_attend(q, k[perm], v[perm], False), _attend(q, k, v, False),
                               rtol=1e-13, atol=1e-13)
    # causal first row sees only key 0
    np.testing.assert_allclose(_attend(q, k[:3], v[:3], True)[0], v[0], rtol=1e-14)


def test_softmax_scale_is_inverse_sqrt_d():
    """Two keys whose logits differ by ln 3 after the 1/sqrt(d) scale get
    weights 3/4 and 1/4 (d = 4, raw dot products 2 ln 3 and 0)."""
    from oracle.attention import _attend
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    k = np.array([[2.0 * math.log(3.0), 0, 0, 0], [0.0, 0, 0, 0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    np.testing.assert_allclose(_attend(q, k, v, False), [[0.75, 0.25]], rtol=1e-14)


def test_packed_qkv_split_layout():
    """Per-head [q|k|v] packing: column j*3d + c*d + e of W_qkv is column
    j*d + e of W_c."""
    heads, d, h = 3, 2, 5
    w = np.arange(h * 3 * heads * d, dtype=np.float64).reshape(h, 3 * heads * d)
    wq, wk, wv = oracle.split_packed_qkv(w, heads, d)
    for j in range(heads):
        for c, wc in enumerate((wq, wk, wv)):
            for e in range(d):
                np.testing.assert_array_equal(wc[:, j * d + e], w[:, j * 3 * d + c * d + e])


@pytest.mark.parametrize("causal", [False, True])
def test_attn_shard_row_subset_equals_full(causal):
    """Computing only some query rows gives exactly those rows of the full
    shard (every output row depends on its own query and all keys only)."""
    x, wqkv, wo, heads, d, t = _tiny_attn(seed=21, batch=2, seq=9, t=2)
    nl = heads // t
    wq_i, wo_i = wqkv[:, :3 * nl * d], wo[:nl * d, :]
    full = oracle.attn_shard(x, wq_i, wo_i, heads, d, t, 0, causal)
    rows = [0, 4, 8]
    np.testing.assert_array_equal(oracle.attn_shard(x, wq_i, wo_i, heads, d, t, 0, causal, rows=rows),
                                  full[:, rows, :])


# ---- backward (Megatron Level 2, M025 / M026; GeLU' by the product rule) ----

def test_gelu_grad_matches_central_differences():
    z = np.linspace(-8.0, 8.0, 161)
    h = 1e-5
    fd = (oracle.gelu(z + h) - oracle.gelu(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_grad(z), fd, rtol=0, atol=1e-9)


def test_gelu_grad_special_values(golden_dir):
    assert oracle.gelu_grad(0.0) == 0.5                      # Phi(0) + 0
    assert abs(oracle.gelu_grad(10.0) - 1.0) < 1e-15         # Phi -> 1, z phi -> 0
    assert abs(oracle.gelu_grad(-10.0)) < 1e-20
    # Phi(1) from the printed normal table, phi(1) = exp(-1/2) / sqrt(2 pi)
    table = {float(z): float(p) for z, p in read_golden_table(os.path.join(golden_dir, "normal_cdf.txt"))}
    expect = table[1.0] + math.exp(-0.5) / math.sqrt(2 * math.pi)
    assert abs(oracle.gelu_grad(1.0) - expect) < 1e-9


def _tiny_mlp_problem(seed, tokens=3, hidden=4, ffn=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((tokens, hidden)), rng.standard_normal((hidden, ffn)) * 0.7,
            rng.standard_normal((ffn, hidden)) * 0.5, rng.standard_normal(ffn) * 0.3,
            rng.standard_normal(hidden) * 0.3, rng.standard_normal((tokens, hidden)))


def _assembled_grads(x, a, b, ba, dz, t):
    """Rank gradients put back together: dX summed over ranks, dA / dB / da
    concatenated along the split dimension."""
    parts = [oracle.mlp_shard_bwd(x, a, b, dz, t, r, bias_a=ba) for r in range(t)]
    return {
        "x": sum(p["dx"] for p in parts),
        "a": np.concatenate([p["da"] for p in parts], axis=1),
        "b": np.concatenate([p["db"] for p in parts], axis=0),
        "ba": np.concatenate([p["dbias_a"] for p in parts]),
        "bb": parts[0]["dbias_b"],
    }


def _fd_grads(x, a, b, ba, bb, dz, eps=1e-6):
    """Central differences of L = sum(dz * (GeLU(X A + a) B + b))."""
    params = {"x": x, "a": a, "b": b, "ba": ba, "bb": bb}

    def loss():
        return float(np.sum(dz * oracle.mlp_full(params["x"], params["a"], params["b"],
                                                   params["ba"], params["bb"])))

    out = {}
    for name, arr in params.items():
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            up = loss()
            arr[idx] = keep - eps
            down = loss()
            arr[idx] = keep
            g[idx] = (up - down) / (2 * eps)
        out[name] = g
    return out


@pytest.mark.parametrize("t", [1, 2, 4])
def test_mlp_backward_matches_finite_differences(t):
    x, a, b, ba, bb, dz = _tiny_mlp_problem(seed=30 + t)
    got = _assembled_grads(x, a, b, ba, dz, t)
    fd = _fd_grads(x.copy(), a.copy(), b.copy(), ba.copy(), bb.copy(), dz)
    for name in fd:
        np.testing.assert_allclose(got[name], fd[name], rtol=1e-6, atol=1e-7, err_msg=name)


def test_mlp_backward_fd_check_catches_a_dropped_term(monkeypatch):
    """Negative control: GeLU' without its z * phi(z) term must fail the
    finite-difference comparison."""
    import oracle.mlp as om
    x, a, b, ba, bb, dz = _tiny_mlp_problem(seed=41)
    fd = _fd_grads(x.copy(), a.copy(), b.copy(), ba.copy(), bb.copy(), dz)
    monkeypatch.setattr(om, "gelu_grad", lambda z: 0.5 * om.erfc(-np.asarray(z) / math.sqrt(2.0)))
    bad = _assembled_grads(x, a, b, ba, dz, 2)
    assert not np.allclose(bad["x"], fd["x"], rtol=1e-6, atol=1e-7)
    assert not np.allclose(bad["a"], fd["a"], rtol=1e-6, atol=1e-7)
    assert np.allclose(bad["b"], fd["b"], rtol=1e-6, atol=1e-7)   # dB does not use GeLU'


def test_mlp_backward_partition_identity():
    """The ranks' dX contributions sum to the unsharded dX, and their weight
    gradients are the blocks of the unsharded ones (M025 / M026)."""
    x, a, b, ba, _bb, dz = _tiny_mlp_problem(seed=43, tokens=5, hidden=8, ffn=32)
    full = _assembled_grads(x, a, b, ba, dz, 1)
    for t in (2, 4, 8):
        parts = _assembled_grads(x, a, b, ba, dz, t)
        for name in full:
            np.testing.assert_allclose(parts[name], full[name], rtol=1e-12, atol=1e-12)


# ---- sequence-parallel boundary (Megatron Level 2, M034) ----

def test_sp_shards_gather_to_the_layer_output():
    """Reduce-scatter then gather = the summed output: the shards of the t
    partials, stacked in rank order, equal GeLU(X A + a) B + b + R."""
    rng = np.random.default_rng(50)
    tokens, hidden, ffn, t = 12, 6, 16, 4
    x, a, b = rng.standard_normal((tokens, hidden)), rng.standard_normal((hidden, ffn)), \
        rng.standard_normal((ffn, hidden))
    ba, bb, res = rng.standard_normal(ffn), rng.standard_normal(hidden), rng.standard_normal((tokens, hidden))
    parts = [oracle.mlp_shard(x, a, b, t, r, bias_a=ba) for r in range(t)]
    shards = [oracle.sp_reduce_scatter(parts, t, r, bias=bb,
                                       residual_r=res[oracle.sp_shard_rows(tokens, t, r)])
              for r in range(t)]
    np.testing.assert_allclose(np.concatenate(shards, axis=0),
                               oracle.mlp_full(x, a, b, ba, bb, res), rtol=1e-12, atol=1e-12)


def test_sp_reduce_scatter_by_hand():
    """Two ranks, four tokens, one column: each rank sums its two rows."""
    p0 = np.array([[1.0], [2.0], [3.0], [4.0]])
    p1 = np.array([[10.0], [20.0], [30.0], [40.0]])
    assert oracle.sp_reduce_scatter([p0, p1], 2, 0).tolist() == [[11.0], [22.0]]
    assert oracle.sp_reduce_scatter([p0, p1], 2, 1, bias=[0.5]).tolist() == [[33.5], [44.5]]


def test_sp_rejects_tokens_not_divisible():
    with pytest.raises(oracle.ShardError):
        oracle.sp_shard_rows(10, 4, 0)
    with pytest.raises(oracle.ShardError):
        oracle.sp_shard_rows(8, 4, 4)


# ---- SwiGLU variant (Megatron Level 2, M027 / M031) ----

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    z = np.linspace(-30, 30, 121)
    # sigma(z) + sigma(-z) = 1  =>  SiLU(z) - SiLU(-z) = z
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu(-40.0)) < 1e-15
    # mpmath at 50 digits
    mpmath.mp.dps = 50
    for v in (-3.7, -0.2, 0.9, 5.5):
        assert abs(oracle.silu(v) - float(v / (1 + mpmath.e ** (-v)))) < 1e-15


def test_swiglu_partition_identity_and_pairing():
    """sum over ranks of the paired shards = the unsharded gated MLP; pairing
    the gate block of one rank with the value block of another breaks it."""
    rng = np.random.default_rng(60)
    x = rng.standard_normal((7, 8))
    wg, wu = rng.standard_normal((8, 24)), rng.standard_normal((8, 24))
    b = rng.standard_normal((24, 8))
    bb, res = rng.standard_normal(8), rng.standard_normal((7, 8))
    full = oracle.swiglu_mlp_full(x, wg, wu, b, bb, res)
    for t in (1, 2, 3, 4, 6):
        total = sum(oracle.swiglu_mlp_shard(x, wg, wu, b, t, r, bb, res) for r in range(t))
        np.testing.assert_allclose(total, full, rtol=1e-12, atol=1e-12)
    # negative control: value columns of the neighbouring block
    wu_shift = np.concatenate([wu[:, 6:], wu[:, :6]], axis=1)
    bad = sum(oracle.swiglu_mlp_shard(x, wg, wu_shift, b, 4, r, bb, res) for r in range(4))
    assert not np.allclose(bad, full, rtol=1e-6, atol=1e-6)


def test_swiglu_brute_force():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((3, 5))
    wg, wu = rng.standard_normal((5, 6)), rng.standard_normal((5, 6))
    b = rng.standard_normal((6, 4))
    for r in range(3):
        np.testing.assert_allclose(oracle.swiglu_mlp_shard(x, wg, wu, b, 3, r),
                                   np.array(oracle.swiglu_shard_loops(x.tolist(), wg.tolist(),
                                                                      wu.tolist(), b.tolist(), 3, r)),
                                   rtol=1e-12, atol=1e-12)


def test_swiglu_rejects_undivisible():
    x = np.zeros((2, 4))
    with pytest.raises(oracle.ShardError):
        oracle.swiglu_mlp_shard(x, np.zeros((4, 10)), np.zeros((4, 10)), np.zeros((10, 4)), 4, 0)
