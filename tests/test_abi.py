"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments before anything reaches the GPU.

Every call here fails validation (or has tokens == 0), so no HIP call is
made; the pointers are fake integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")

OK, INVALID, NOT_DIV, BAD_RANK, DTYPE, MISALIGNED, WORKSPACE, UNSUPPORTED, HIP = range(9)
F32, BF16 = 0, 1
P = 0x10000  # a fake, 16-byte aligned "device pointer"; never dereferenced


@pytest.fixture(scope="module")
def lib():
    from megatron_tensor_transformer_tp_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from megatron_tensor_transformer_tp_amd.build import build
        build()
    return binding.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    from megatron_tensor_transformer_tp_amd import binding
    names = header_functions()
    assert {"tp_column_linear", "tp_gelu", "tp_row_linear", "tp_mlp_shard_fwd",
            "tp_attn_shard_fwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in binding.SIGNATURES, f"binding lacks {n}"
    assert set(binding.SIGNATURES) == set(names)


def test_status_strings_and_version(lib):
    for s in range(9):
        assert lib.tp_status_string(s).decode().startswith(
            ["TP_OK", "TP_ERR_INVALID_ARG", "TP_ERR_NOT_DIVISIBLE", "TP_ERR_BAD_RANK", "TP_ERR_DTYPE",
             "TP_ERR_MISALIGNED", "TP_ERR_WORKSPACE", "TP_ERR_UNSUPPORTED", "TP_ERR_HIP"][s])
    assert lib.tp_version() >= 100


def col(lib, **kw):
    a = dict(x=P, ldx=1024, a=P, lda=512, bias=None, y=P, ldy=512, tokens=16, hidden=1024,
             ffn=4096, t=8, rank=0, in_dt=BF16, out_dt=BF16, gelu=1)
    a.update(kw)
    return lib.tp_column_linear(a["x"], a["ldx"], a["a"], a["lda"], a["bias"], a["y"], a["ldy"],
                                a["tokens"], a["hidden"], a["ffn"], a["t"], a["rank"], a["in_dt"],
                                a["out_dt"], a["gelu"], None)


def test_column_linear_validation(lib):
    assert col(lib, ffn=4100) == NOT_DIV          # F mod t != 0
    assert col(lib, t=0) == BAD_RANK
    assert col(lib, rank=8) == BAD_RANK
    assert col(lib, rank=-1) == BAD_RANK
    assert col(lib, x=None) == INVALID
    assert col(lib, ldy=256) == INVALID           # ld < width
    assert col(lib, tokens=-1) == INVALID
    assert col(lib, gelu=2) == INVALID
    assert col(lib, x=P + 8) == MISALIGNED        # not 16-byte aligned
    assert col(lib, hidden=1020, ldx=1020) == MISALIGNED  # row width not a multiple of 8
    assert col(lib, lda=516) == MISALIGNED
    assert col(lib, bias=P + 2) == MISALIGNED
    assert col(lib, in_dt=F32, out_dt=BF16) == DTYPE
    assert col(lib, in_dt=7) == DTYPE
    assert col(lib, tokens=0) == OK               # empty input: nothing enqueued
    assert col(lib, tokens=0, ffn=4100) == NOT_DIV  # config still validated when empty
    # fp32 rows need 4-element alignment only
    assert col(lib, tokens=0, in_dt=F32, out_dt=F32, hidden=1020, ldx=1020) == OK


def row(lib, **kw):
    a = dict(h=P, ldh=512, b=P, ldb=1024, bias=None, res=None, ldr=0, z=P, ldz=1024, tokens=16,
             ffn=4096, hidden=1024, t=8, rank=0, in_dt=BF16, out_dt=F32)
    a.update(kw)
    return lib.tp_row_linear(a["h"], a["ldh"], a["b"], a["ldb"], a["bias"], a["res"], a["ldr"],
                             a["z"], a["ldz"], a["tokens"], a["ffn"], a["hidden"], a["t"], a["rank"],
                             a["in_dt"], a["out_dt"], None)


def test_row_linear_validation(lib):
    assert row(lib, ffn=30, t=4) == NOT_DIV
    assert row(lib, rank=8) == BAD_RANK
    assert row(lib, b=None) == INVALID
    assert row(lib, res=P, ldr=100) == INVALID    # residual ld < hidden
    assert row(lib, res=P + 4, ldr=1024) == MISALIGNED
    # ranks != 0 ignore bias / residual entirely (even malformed ones)
    assert row(lib, rank=3, res=P + 4, ldr=100, bias=P + 2, tokens=0) == OK
    assert row(lib, z=P + 8) == MISALIGNED
    assert row(lib, in_dt=F32, out_dt=BF16) == DTYPE
    assert row(lib, tokens=0) == OK


def test_gelu_validation(lib):
    assert lib.tp_gelu(P, P + 4096, -1, BF16, BF16, None) == INVALID
    assert lib.tp_gelu(None, P, 10, BF16, BF16, None) == INVALID
    assert lib.tp_gelu(P + 2, P + 4096, 10, BF16, BF16, None) == MISALIGNED
    assert lib.tp_gelu(P, P + 16, 100, BF16, BF16, None) == INVALID  # partial overlap
    assert lib.tp_gelu(P, P, 100, F32, BF16, None) == INVALID        # in place, sizes differ
    assert lib.tp_gelu(P, P + 4096, 10, 3, BF16, None) == DTYPE
    assert lib.tp_gelu(P, P, 0, BF16, BF16, None) == OK


def mlp(lib, **kw):
    a = dict(x=P, a=P, lda=512, b=P, bias_a=None, bias_b=None, res=None, z=P, y=None, ws=P,
             ws_bytes=1 << 30, tokens=16, hidden=1024, ffn=4096, t=8, rank=0, in_dt=BF16, out_dt=F32)
    a.update(kw)
    return lib.tp_mlp_shard_fwd(a["x"], a["a"], a["lda"], a["b"], a["bias_a"], a["bias_b"], a["res"],
                                a["z"], a["y"], a["ws"], a["ws_bytes"], a["tokens"], a["hidden"],
                                a["ffn"], a["t"], a["rank"], a["in_dt"], a["out_dt"], None)


def test_mlp_shard_validation(lib):
    need = lib.tp_mlp_shard_workspace_bytes(16, 1024, 4096, 8, BF16)
    # H_i [16, 512] bf16, then (bf16, at most 512 tokens) the split-K partial
    # products: 8 slices x 16 tokens x max(f, hidden) = 1024 floats
    assert need == 16 * 512 * 2 + 8 * 16 * 1024 * 4
    assert lib.tp_mlp_shard_workspace_bytes(512, 1024, 4096, 8, BF16) == 512 * 512 * 2 + 8 * 512 * 1024 * 4
    assert lib.tp_mlp_shard_workspace_bytes(513, 1024, 4096, 8, BF16) == 513 * 512 * 2   # no split part
    assert lib.tp_mlp_shard_workspace_bytes(3, 1024, 4096, 8, F32) == 3 * 512 * 4
    assert lib.tp_mlp_shard_workspace_bytes(3, 1024, 40, 8, F32) == 256  # 60 B rounded up
    assert lib.tp_mlp_shard_workspace_bytes(16, 1024, 4100, 8, BF16) == 0
    assert mlp(lib, ws_bytes=need - 1) == WORKSPACE
    assert mlp(lib, ws=None) == WORKSPACE
    assert mlp(lib, ws=P + 16) == MISALIGNED      # workspace must be 256-byte aligned
    assert mlp(lib, ffn=4097) == NOT_DIV
    assert mlp(lib, t=3, ffn=4096, rank=0) == NOT_DIV
    assert mlp(lib, t=3, ffn=4095, rank=0, lda=1368) == MISALIGNED  # f = 1365, not a multiple of 8
    assert mlp(lib, rank=9) == BAD_RANK
    assert mlp(lib, x=None) == INVALID
    assert mlp(lib, lda=500) == INVALID
    assert mlp(lib, bias_a=P + 2) == MISALIGNED
    assert mlp(lib, in_dt=F32, out_dt=BF16) == DTYPE
    assert mlp(lib, tokens=0, ws=None) == OK
    assert mlp(lib, y=P + 8) == MISALIGNED        # the saved pre-activation must be aligned
    # sizes past 2^30 are refused before anything is enqueued
    assert mlp(lib, tokens=(1 << 30) + 8) == UNSUPPORTED
    assert mlp(lib, hidden=(1 << 30) + 8, ws_bytes=1 << 62) == UNSUPPORTED
    assert bwd(lib, tokens=(1 << 30) + 8) == UNSUPPORTED


def bwd(lib, **kw):
    a = dict(x=P, a=P, lda=512, b=P, y=P, dz=P, dx=P, da=P, db=P, dba=None, dbb=None, ws=P,
             ws_bytes=1 << 30, tokens=256, hidden=1024, ffn=4096, t=8, rank=0, in_dt=BF16,
             g_dt=F32)
    a.update(kw)
    return lib.tp_mlp_shard_bwd(a["x"], a["a"], a["lda"], a["b"], a["y"], a["dz"], a["dx"], a["da"],
                                a["db"], a["dba"], a["dbb"], a["ws"], a["ws_bytes"], a["tokens"],
                                a["hidden"], a["ffn"], a["t"], a["rank"], a["in_dt"], a["g_dt"], None)


def test_mlp_shard_bwd_validation(lib):
    need = lib.tp_mlp_shard_bwd_workspace_bytes(256, 1024, 4096, 8, BF16)
    # dY and H [256, 512] bf16, then four 64-row chunks of fp32 partial sums over max(f, hidden)
    assert need == 2 * 256 * 512 * 2 + 4 * 1024 * 4
    assert lib.tp_mlp_shard_bwd_workspace_bytes(256, 1024, 4100, 8, BF16) == 0
    assert bwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, ws=P + 16) == MISALIGNED
    assert bwd(lib, ffn=4097) == NOT_DIV
    assert bwd(lib, rank=8) == BAD_RANK
    assert bwd(lib, in_dt=F32, g_dt=BF16) == DTYPE
    assert bwd(lib, y=None) == INVALID
    assert bwd(lib, dz=None) == INVALID
    assert bwd(lib, da=None) == INVALID
    assert bwd(lib, lda=500) == INVALID
    assert bwd(lib, dba=P + 4) == MISALIGNED
    # widths must be multiples of 8 (bf16) / 4 (fp32)
    assert bwd(lib, hidden=1028) == MISALIGNED
    assert bwd(lib, ffn=8 * 260, lda=260) == MISALIGNED
    # any token count and 8-aligned widths get past the shape checks (and
    # stop at the workspace size, before any launch)
    assert bwd(lib, tokens=300, hidden=1032, ffn=8 * 264, lda=264, ws_bytes=1) == WORKSPACE
    assert bwd(lib, in_dt=F32, tokens=300, hidden=1000, ffn=4000, lda=500, ws_bytes=1) == WORKSPACE


def attn(lib, **kw):
    a = dict(x=P, wqkv=P, wo=P, out=P, ws=P, ws_bytes=1 << 30, batch=1, seq=256, hidden=1024, heads=8,
             head_dim=128, causal=0, t=2, rank=0, in_dt=BF16, out_dt=F32)
    a.update(kw)
    return lib.tp_attn_shard_fwd(a["x"], a["wqkv"], a["wo"], a["out"], a["ws"], a["ws_bytes"], a["batch"],
                                 a["seq"], a["hidden"], a["heads"], a["head_dim"], a["causal"], a["t"],
                                 a["rank"], a["in_dt"], a["out_dt"], None)


def test_attn_shard_validation(lib):
    assert attn(lib, t=3) == NOT_DIV                      # heads mod t != 0
    assert attn(lib, rank=2) == BAD_RANK
    assert attn(lib, hidden=1000) == INVALID               # hidden != heads * head_dim
    assert attn(lib, head_dim=64, hidden=512) == UNSUPPORTED
    assert attn(lib, seq=31) == UNSUPPORTED                # shorter than one key block
    assert attn(lib, seq=200, ws_bytes=1) == WORKSPACE     # any seq >= 32 passes the shape checks
    assert attn(lib, batch=0, seq=16, ws=None) == OK        # nothing to do
    assert attn(lib, in_dt=F32) == DTYPE
    assert attn(lib, causal=2) == INVALID
    assert attn(lib, x=None) == INVALID
    assert attn(lib, out=P + 8) == MISALIGNED
    need = lib.tp_attn_shard_workspace_bytes(1, 256, 1024, 8, 128, 2, BF16)
    # packed projection [256, 3*4*128] (16-bit) + output [256, 4*128] bf16
    # + split-row partial states (2 halves x 256 tokens x 4 heads x 130
    # floats) + arrival counters (1 x 4 heads x 2 query blocks, one 256-byte
    # unit)
    assert need == 256 * 1536 * 2 + 256 * 512 * 2 + 2 * 256 * 4 * 130 * 4 + 256
    assert attn(lib, ws_bytes=need - 1) == WORKSPACE
    assert attn(lib, ws=P + 16) == MISALIGNED
    assert attn(lib, batch=0, ws=None) == OK
    assert lib.tp_attn_shard_workspace_bytes(1, 256, 1024, 8, 128, 3, BF16) == 0
    # a grid of more than 512 query blocks never splits its rows: no split
    # scratch (batch 4 x 8 local heads x 64 blocks of 128 = 2048 blocks)
    big = lib.tp_attn_shard_workspace_bytes(4, 8192, 8192, 64, 128, 8, BF16)
    assert big == 32768 * 3 * 1024 * 2 + 32768 * 1024 * 2
    # 512 query blocks still carry it (batch 1 x 8 heads x 64 blocks)
    edge = lib.tp_attn_shard_workspace_bytes(1, 8192, 8192, 64, 128, 8, BF16)
    assert edge == 8192 * 3 * 1024 * 2 + 8192 * 1024 * 2 + 2 * 8192 * 8 * 130 * 4 + 2048


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "megatron_tensor_transformer_tp_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), fn
                assert "oracle." not in text.replace("the oracle.", ""), fn


def sp(lib, t=4, parts=None, **kw):
    a = dict(rank=0, bias=None, res=None, out=P, tokens=256, hidden=1024, in_dt=BF16, out_dt=F32)
    a.update(kw)
    ptrs = (ctypes.c_void_p * max(t, 1))(*(parts if parts is not None else [P + 4096 * j for j in range(t)]))
    return lib.tp_sp_reduce_scatter(ptrs, t, a["rank"], a["bias"], a["res"], a["out"], a["tokens"],
                                    a["hidden"], a["in_dt"], a["out_dt"], None)


def test_sp_reduce_scatter_validation(lib):
    assert sp(lib, t=0, parts=[P]) == BAD_RANK
    assert sp(lib, rank=4) == BAD_RANK
    assert sp(lib, t=17) == UNSUPPORTED
    assert sp(lib, tokens=250) == NOT_DIV
    assert sp(lib, hidden=1022) == MISALIGNED
    assert sp(lib, in_dt=5) == DTYPE
    assert sp(lib, parts=[P, None, P, P]) == INVALID
    assert sp(lib, parts=[P, P + 8, P, P]) == MISALIGNED
    assert sp(lib, out=None) == INVALID                 # every partial passed its checks
    assert sp(lib, bias=P + 2, out=P) == MISALIGNED
    assert sp(lib, tokens=0) == OK
    assert lib.tp_sp_reduce_scatter(None, 4, 0, None, None, P, 256, 1024, BF16, F32, None) == INVALID


def swiglu(lib, **kw):
    a = dict(x=P, wg=P, wu=P, lda=512, b=P, bias_b=None, res=None, z=P, ws=P, ws_bytes=1 << 30,
             tokens=256, hidden=1024, ffn=4096, t=8, rank=0, in_dt=BF16, out_dt=F32)
    a.update(kw)
    return lib.tp_mlp_swiglu_shard_fwd(a["x"], a["wg"], a["wu"], a["lda"], a["b"], a["bias_b"],
                                       a["res"], a["z"], a["ws"], a["ws_bytes"], a["tokens"],
                                       a["hidden"], a["ffn"], a["t"], a["rank"], a["in_dt"],
                                       a["out_dt"], None)


def test_swiglu_validation(lib):
    need = lib.tp_mlp_swiglu_shard_workspace_bytes(256, 1024, 4096, 8, BF16)
    assert need == 256 * 512 * 2
    assert lib.tp_mlp_swiglu_shard_workspace_bytes(64, 64, 256, 4, F32) == 3 * 64 * 64 * 4
    assert swiglu(lib, ffn=4097) == NOT_DIV
    assert swiglu(lib, rank=8) == BAD_RANK
    assert swiglu(lib, wu=None) == INVALID
    assert swiglu(lib, wg=P + 8) == MISALIGNED
    assert swiglu(lib, in_dt=F32, out_dt=BF16) == DTYPE
    assert swiglu(lib, ffn=8 * 132, lda=132) == MISALIGNED   # f % 8
    # any token count and 8-aligned widths get past the shape checks
    assert swiglu(lib, tokens=300, ffn=8 * 136, lda=136, hidden=1000, ws_bytes=1) == WORKSPACE
    assert swiglu(lib, ws_bytes=need - 1) == WORKSPACE
    assert swiglu(lib, in_dt=F32, tokens=300, ws_bytes=1) == WORKSPACE   # fp32: any shape
    assert swiglu(lib, tokens=0, ws=None) == OK
