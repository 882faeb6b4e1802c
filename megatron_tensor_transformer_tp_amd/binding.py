"""Thin ctypes binding of ``libtp_shard.so`` (C ABI in ``include/tp_shard.h``).

Argument marshalling only: shapes, leading dimensions, dtypes and the current
HIP stream are read off torch tensors and handed to the C entry points of the
same names; every step of the computation runs in the library's kernels.
torch is used for device memory and streams, nothing else.  There is no
fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtp_shard.so")

TP_F32, TP_BF16 = 0, 1

STATUS_NAMES = {
    0: "TP_OK", 1: "TP_ERR_INVALID_ARG", 2: "TP_ERR_NOT_DIVISIBLE", 3: "TP_ERR_BAD_RANK",
    4: "TP_ERR_DTYPE", 5: "TP_ERR_MISALIGNED", 6: "TP_ERR_WORKSPACE", 7: "TP_ERR_UNSUPPORTED",
    8: "TP_ERR_HIP",
}

_I64, _INT, _VP, _SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tp_shard.h
SIGNATURES = {
    "tp_status_string": (ctypes.c_char_p, [_INT]),
    "tp_version": (_INT, []),
    "tp_column_linear": (_INT, [_VP, _I64, _VP, _I64, _VP, _VP, _I64, _I64, _I64, _I64, _INT,
                                _INT, _INT, _INT, _INT, _VP]),
    "tp_gelu": (_INT, [_VP, _VP, _I64, _INT, _INT, _VP]),
    "tp_row_linear": (_INT, [_VP, _I64, _VP, _I64, _VP, _VP, _I64, _VP, _I64, _I64, _I64, _I64,
                             _INT, _INT, _INT, _INT, _VP]),
    "tp_mlp_shard_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT, _INT]),
    "tp_mlp_shard_fwd": (_INT, [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I64,
                                _I64, _I64, _INT, _INT, _INT, _INT, _VP]),
    "tp_mlp_shard_fwd_noalloc": (_INT, [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64,
                                        _I64, _INT, _INT, _INT, _INT, _VP]),
    "tp_mlp_swiglu_shard_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT, _INT]),
    "tp_mlp_swiglu_shard_fwd": (_INT, [_VP, _VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _SZ, _I64,
                                       _I64, _I64, _INT, _INT, _INT, _INT, _VP]),
    "tp_mlp_shard_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT, _INT]),
    "tp_mlp_shard_bwd": (_INT, [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                _I64, _I64, _I64, _INT, _INT, _INT, _INT, _VP]),
    "tp_sp_reduce_scatter": (_INT, [_VP, _INT, _INT, _VP, _VP, _VP, _I64, _I64, _INT, _INT, _VP]),
    "tp_attn_shard_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _INT, _INT]),
    "tp_attn_shard_fwd": (_INT, [_VP, _VP, _VP, _VP, _VP, _SZ, _I64, _I64, _I64, _I64, _I64,
                                 _INT, _INT, _INT, _INT, _INT, _VP]),
}

_lib: Optional[ctypes.CDLL] = None


class TpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m megatron_tensor_transformer_tp_amd.build` "
                "(or __graft_entry__.build()); there is no CPU fallback")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _rows(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D row-major view (rows may be strided, columns not)."""
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise TpError(status, where)


# ---- argument checks done here, before the library is called ---------------
# The C ABI sees raw pointers: a tensor of the wrong shape, dtype or device
# would become an out-of-bounds access inside a kernel.  Each wrapper checks
# every tensor's shape and dtype against the sizes it passes, then that all
# of them live on one GPU, and raises ValueError before anything reaches the
# library.  Splits that do not divide (or a bad t / rank) are left to the
# library, which rejects them with its own status code before enqueueing
# anything; the shard-shape checks then do not apply.

def _shard(total: int, t: int) -> Optional[int]:
    """total / t when the split is valid, else None (the library reports it)."""
    return total // t if t >= 1 and total >= 1 and total % t == 0 else None


def _expect(ten: Optional[torch.Tensor], name: str, shape, dtype=None, where: str = "") -> None:
    """``ten`` (if given) has this shape (None entries: any size) and dtype."""
    if ten is None:
        return
    if not isinstance(ten, torch.Tensor):
        raise ValueError(f"{where}: {name} must be a torch.Tensor")
    if ten.dim() != len(shape) or any(w is not None and g != w for g, w in zip(ten.shape, shape)):
        want = "x".join("*" if w is None else str(w) for w in shape)
        raise ValueError(f"{where}: {name} has shape {tuple(ten.shape)}, expected [{want}]")
    if dtype is not None and ten.dtype != dtype:
        raise ValueError(f"{where}: {name} has dtype {ten.dtype}, expected {dtype}")


def _contiguous(where: str, **tensors) -> None:
    for name, ten in tensors.items():
        if ten is not None and not ten.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")


def _on_one_gpu(where: str, **tensors) -> None:
    """Every given tensor is a GPU tensor, all on the same device."""
    device = None
    for name, ten in tensors.items():
        if ten is None:
            continue
        if not ten.is_cuda:
            raise ValueError(f"{where}: {name} must be a GPU tensor (got device {ten.device})")
        if device is None:
            device = ten.device
        elif ten.device != device:
            raise ValueError(f"{where}: {name} is on {ten.device}, the other operands on {device}")


def _in_dtype(ten: torch.Tensor, where: str) -> torch.dtype:
    if ten.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"{where}: unsupported input dtype {ten.dtype} (bfloat16 or float32)")
    return ten.dtype


def tp_column_linear(x: torch.Tensor, a_i: torch.Tensor, y_i: torch.Tensor, *, ffn: int, t: int,
                     rank: int, bias_i: Optional[torch.Tensor] = None, apply_gelu: bool = False,
                     stream=None) -> torch.Tensor:
    """y_i <- X A_i (+ a_i) [then GeLU]; x [tokens, hidden], a_i [hidden, ffn/t]."""
    w = "tp_column_linear"
    _expect(x, "x", (None, None), where=w)
    tokens, hidden = x.shape
    dt = _in_dtype(x, w)
    f = _shard(ffn, t)
    _expect(a_i, "a_i", (hidden, f), dt, w)
    _expect(y_i, "y_i", (tokens, f), None, w)
    _expect(bias_i, "bias_i", (f,), dt, w)
    _contiguous(w, bias_i=bias_i)
    _on_one_gpu(w, x=x, a_i=a_i, y_i=y_i, bias_i=bias_i)
    _check(lib().tp_column_linear(_ptr(x), _rows(x, "x"), _ptr(a_i), _rows(a_i, "a_i"),
                                  _ptr(bias_i), _ptr(y_i), _rows(y_i, "y_i"), tokens, hidden, ffn,
                                  t, rank, _dt(x), _dt(y_i), int(apply_gelu), _stream(stream)), w)
    return y_i


def tp_gelu(inp: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """out <- GeLU(inp), elementwise over contiguous tensors of equal numel."""
    w = "tp_gelu"
    if not (inp.is_contiguous() and out.is_contiguous()) or inp.numel() != out.numel():
        raise ValueError(f"{w}: needs contiguous tensors of equal size")
    _in_dtype(inp, w)
    _in_dtype(out, w)
    _on_one_gpu(w, inp=inp, out=out)
    _check(lib().tp_gelu(_ptr(inp), _ptr(out), inp.numel(), _dt(inp), _dt(out), _stream(stream)), w)
    return out


def tp_row_linear(h_i: torch.Tensor, b_i: torch.Tensor, z_i: torch.Tensor, *, ffn: int, t: int,
                  rank: int, bias: Optional[torch.Tensor] = None,
                  residual: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """z_i <- H_i B_i (+ bias + residual on rank 0); h_i [tokens, ffn/t], b_i [ffn/t, hidden]."""
    w = "tp_row_linear"
    _expect(h_i, "h_i", (None, None), where=w)
    _expect(b_i, "b_i", (None, None), where=w)
    tokens, hidden = h_i.shape[0], b_i.shape[1]
    dt = _in_dtype(h_i, w)
    f = _shard(ffn, t)
    _expect(h_i, "h_i", (tokens, f), dt, w)
    _expect(b_i, "b_i", (f, hidden), dt, w)
    _expect(z_i, "z_i", (tokens, hidden), None, w)
    _expect(bias, "bias", (hidden,), dt, w)
    _expect(residual, "residual", (tokens, hidden), dt, w)
    _contiguous(w, bias=bias)
    _on_one_gpu(w, h_i=h_i, b_i=b_i, z_i=z_i, bias=bias, residual=residual)
    ldr = _rows(residual, "residual") if residual is not None else 0
    _check(lib().tp_row_linear(_ptr(h_i), _rows(h_i, "h_i"), _ptr(b_i), _rows(b_i, "b_i"),
                               _ptr(bias), _ptr(residual), ldr, _ptr(z_i), _rows(z_i, "z_i"),
                               tokens, ffn, hidden, t, rank, _dt(h_i), _dt(z_i), _stream(stream)), w)
    return z_i


def _workspace(ws: Optional[torch.Tensor], where: str) -> None:
    if ws is not None and not ws.is_contiguous():
        raise ValueError(f"{where}: workspace must be contiguous")


def tp_mlp_shard_workspace_bytes(tokens: int, hidden: int, ffn: int, t: int, dtype) -> int:
    dt = TP_BF16 if dtype == torch.bfloat16 else TP_F32
    return int(lib().tp_mlp_shard_workspace_bytes(tokens, hidden, ffn, t, dt))


def _mlp_fwd_checks(w, x, a_i, b_i, z_i, workspace, ffn, t, bias_a_i, bias_b, residual, y_save):
    _expect(x, "x", (None, None), where=w)
    tokens, hidden = x.shape
    dt = _in_dtype(x, w)
    f = _shard(ffn, t)
    _expect(a_i, "a_i", (hidden, f), dt, w)
    _expect(b_i, "b_i", (f, hidden), dt, w)
    _expect(z_i, "z_i", (tokens, hidden), None, w)
    _expect(bias_a_i, "bias_a_i", (f,), dt, w)
    _expect(bias_b, "bias_b", (hidden,), dt, w)
    _expect(residual, "residual", (tokens, hidden), dt, w)
    _expect(y_save, "y_save", (tokens, f), dt, w)
    _contiguous(w, x=x, b_i=b_i, z_i=z_i, bias_a_i=bias_a_i, bias_b=bias_b, residual=residual,
                y_save=y_save)
    _workspace(workspace, w)
    _on_one_gpu(w, x=x, a_i=a_i, b_i=b_i, z_i=z_i, workspace=workspace, bias_a_i=bias_a_i,
                bias_b=bias_b, residual=residual, y_save=y_save)
    return tokens, hidden


def tp_mlp_shard_fwd(x: torch.Tensor, a_i: torch.Tensor, b_i: torch.Tensor, z_i: torch.Tensor,
                     workspace: torch.Tensor, *, ffn: int, t: int, rank: int,
                     bias_a_i: Optional[torch.Tensor] = None, bias_b: Optional[torch.Tensor] = None,
                     residual: Optional[torch.Tensor] = None, y_save: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """z_i <- GeLU(X A_i + a_i) B_i (+ b + R on rank 0), H_i kept in ``workspace``;
    the pre-activation X A_i + a_i also goes to ``y_save`` if given."""
    w = "tp_mlp_shard_fwd"
    tokens, hidden = _mlp_fwd_checks(w, x, a_i, b_i, z_i, workspace, ffn, t, bias_a_i, bias_b,
                                     residual, y_save)
    _check(lib().tp_mlp_shard_fwd(_ptr(x), _ptr(a_i), _rows(a_i, "a_i"), _ptr(b_i), _ptr(bias_a_i),
                                  _ptr(bias_b), _ptr(residual), _ptr(z_i), _ptr(y_save),
                                  _ptr(workspace), _nbytes(workspace), tokens, hidden, ffn,
                                  t, rank, _dt(x), _dt(z_i), _stream(stream)), w)
    return z_i


def tp_mlp_shard_fwd_noalloc(x: torch.Tensor, a_i: torch.Tensor, b_i: torch.Tensor, z_i: torch.Tensor,
                             *, ffn: int, t: int, rank: int, bias_a_i: Optional[torch.Tensor] = None,
                             bias_b: Optional[torch.Tensor] = None,
                             residual: Optional[torch.Tensor] = None,
                             y_save: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """As tp_mlp_shard_fwd, with H_i in the library's fixed device array instead of a
    workspace (allocates nothing; calls overlapping on one GPU race)."""
    w = "tp_mlp_shard_fwd_noalloc"
    tokens, hidden = _mlp_fwd_checks(w, x, a_i, b_i, z_i, None, ffn, t, bias_a_i, bias_b,
                                     residual, y_save)
    _check(lib().tp_mlp_shard_fwd_noalloc(_ptr(x), _ptr(a_i), _rows(a_i, "a_i"), _ptr(b_i),
                                          _ptr(bias_a_i), _ptr(bias_b), _ptr(residual), _ptr(z_i),
                                          _ptr(y_save), tokens, hidden, ffn, t, rank, _dt(x), _dt(z_i),
                                          _stream(stream)), w)
    return z_i


def tp_mlp_shard_bwd_workspace_bytes(tokens: int, hidden: int, ffn: int, t: int, dtype) -> int:
    dt = TP_BF16 if dtype == torch.bfloat16 else TP_F32
    return int(lib().tp_mlp_shard_bwd_workspace_bytes(tokens, hidden, ffn, t, dt))


def tp_mlp_shard_bwd(x: torch.Tensor, a_i: torch.Tensor, b_i: torch.Tensor, y_i: torch.Tensor,
                     dz: torch.Tensor, dx_i: torch.Tensor, da_i: torch.Tensor, db_i: torch.Tensor,
                     workspace: Optional[torch.Tensor], *, ffn: int, t: int, rank: int,
                     dbias_a_i: Optional[torch.Tensor] = None,
                     dbias_b: Optional[torch.Tensor] = None, stream=None):
    """Backward of the MLP shard: dx_i (the rank's contribution to dX), da_i,
    db_i and optionally the fp32 bias gradients, from dz and the saved y_i."""
    w = "tp_mlp_shard_bwd"
    _expect(x, "x", (None, None), where=w)
    tokens, hidden = x.shape
    dt = _in_dtype(x, w)
    gt = _in_dtype(dx_i, w)
    f = _shard(ffn, t)
    _expect(a_i, "a_i", (hidden, f), dt, w)
    _expect(b_i, "b_i", (f, hidden), dt, w)
    _expect(y_i, "y_i", (tokens, f), dt, w)
    _expect(dz, "dz", (tokens, hidden), dt, w)
    _expect(dx_i, "dx_i", (tokens, hidden), gt, w)
    _expect(da_i, "da_i", (hidden, f), gt, w)
    _expect(db_i, "db_i", (f, hidden), gt, w)
    _expect(dbias_a_i, "dbias_a_i", (f,), torch.float32, w)
    _expect(dbias_b, "dbias_b", (hidden,), torch.float32, w)
    _contiguous(w, x=x, b_i=b_i, y_i=y_i, dz=dz, dx_i=dx_i, db_i=db_i, dbias_a_i=dbias_a_i,
                dbias_b=dbias_b)
    if _rows(da_i, "da_i") != _rows(a_i, "a_i"):
        raise ValueError(f"{w}: da_i must have a_i's row stride")
    _workspace(workspace, w)
    _on_one_gpu(w, x=x, a_i=a_i, b_i=b_i, y_i=y_i, dz=dz, dx_i=dx_i, da_i=da_i, db_i=db_i,
                workspace=workspace, dbias_a_i=dbias_a_i, dbias_b=dbias_b)
    _check(lib().tp_mlp_shard_bwd(_ptr(x), _ptr(a_i), _rows(a_i, "a_i"), _ptr(b_i), _ptr(y_i),
                                  _ptr(dz), _ptr(dx_i), _ptr(da_i), _ptr(db_i), _ptr(dbias_a_i),
                                  _ptr(dbias_b), _ptr(workspace), _nbytes(workspace), tokens,
                                  hidden, ffn, t, rank, _dt(x), _dt(dx_i), _stream(stream)), w)
    return dx_i, da_i, db_i


def tp_attn_shard_workspace_bytes(batch: int, seq: int, hidden: int, heads: int, head_dim: int,
                                  t: int, dtype) -> int:
    dt = TP_BF16 if dtype == torch.bfloat16 else TP_F32
    return int(lib().tp_attn_shard_workspace_bytes(batch, seq, hidden, heads, head_dim, t, dt))


def tp_attn_shard_fwd(x: torch.Tensor, wqkv_i: torch.Tensor, wo_i: torch.Tensor, out_i: torch.Tensor,
                      workspace: Optional[torch.Tensor], *, heads: int, head_dim: int, t: int,
                      rank: int, causal: bool = False, stream=None) -> torch.Tensor:
    """out_i <- head-local attention of the rank's heads, projected by wo_i (fp32 partial)."""
    w = "tp_attn_shard_fwd"
    _expect(x, "x", (None, None, None), where=w)
    batch, seq, hidden = x.shape
    dt = _in_dtype(x, w)
    hl = _shard(heads, t)
    dl = None if hl is None else hl * head_dim
    _expect(wqkv_i, "wqkv_i", (hidden, None if dl is None else 3 * dl), dt, w)
    _expect(wo_i, "wo_i", (dl, hidden), dt, w)
    # out_i: [batch, seq, hidden] or the same memory viewed as [batch*seq, hidden]
    if out_i.shape[-1:] != (hidden,) or out_i.numel() != batch * seq * hidden:
        raise ValueError(f"{w}: out_i has shape {tuple(out_i.shape)}, expected "
                         f"[{batch}x{seq}x{hidden}] (or [{batch * seq}x{hidden}])")
    _contiguous(w, x=x, wqkv_i=wqkv_i, wo_i=wo_i, out_i=out_i)
    _workspace(workspace, w)
    _on_one_gpu(w, x=x, wqkv_i=wqkv_i, wo_i=wo_i, out_i=out_i, workspace=workspace)
    _check(lib().tp_attn_shard_fwd(_ptr(x), _ptr(wqkv_i), _ptr(wo_i), _ptr(out_i), _ptr(workspace),
                                   _nbytes(workspace), batch, seq, hidden, heads, head_dim,
                                   int(causal), t, rank, _dt(x), _dt(out_i), _stream(stream)), w)
    return out_i


def tp_sp_reduce_scatter(partials, out_r: torch.Tensor, *, t: int, rank: int,
                         bias: Optional[torch.Tensor] = None,
                         residual_r: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out_r <- rank's sequence shard of sum(partials) (+ bias + residual_r)."""
    w = "tp_sp_reduce_scatter"
    if len(partials) != t:
        raise ValueError(f"{w}: {len(partials)} partials for t={t}")
    _expect(partials[0], "partials[0]", (None, None), torch.float32, w)
    tokens, hidden = partials[0].shape
    for j, p in enumerate(partials):
        _expect(p, f"partials[{j}]", (tokens, hidden), torch.float32, w)
    rows = _shard(tokens, t) if tokens > 0 else 0
    if bias is not None and residual_r is not None and bias.dtype != residual_r.dtype:
        raise ValueError(f"{w}: bias and residual_r must share a dtype")
    in_ref = bias if bias is not None else residual_r
    _expect(bias, "bias", (hidden,), None, w)
    _expect(residual_r, "residual_r", (rows, hidden), None, w)
    _expect(out_r, "out_r", (rows, hidden), None, w)
    _contiguous(w, out_r=out_r, residual_r=residual_r, bias=bias,
                **{f"partials[{j}]": p for j, p in enumerate(partials)})
    _on_one_gpu(w, out_r=out_r, bias=bias, residual_r=residual_r,
                **{f"partials[{j}]": p for j, p in enumerate(partials)})
    ptrs = (ctypes.c_void_p * t)(*[p.data_ptr() for p in partials])
    _check(lib().tp_sp_reduce_scatter(ptrs, t, rank, _ptr(bias), _ptr(residual_r), _ptr(out_r),
                                      tokens, hidden, _dt(in_ref) if in_ref is not None else TP_F32,
                                      _dt(out_r), _stream(stream)), w)
    return out_r


def tp_mlp_swiglu_shard_workspace_bytes(tokens: int, hidden: int, ffn: int, t: int, dtype) -> int:
    dt = TP_BF16 if dtype == torch.bfloat16 else TP_F32
    return int(lib().tp_mlp_swiglu_shard_workspace_bytes(tokens, hidden, ffn, t, dt))


def tp_mlp_swiglu_shard_fwd(x: torch.Tensor, wg_i: torch.Tensor, wu_i: torch.Tensor,
                            b_i: torch.Tensor, z_i: torch.Tensor, workspace: torch.Tensor, *,
                            ffn: int, t: int, rank: int, bias_b: Optional[torch.Tensor] = None,
                            residual: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """z_i <- (SiLU(X Wg_i) * (X Wu_i)) B_i (+ b + R on rank 0)."""
    w = "tp_mlp_swiglu_shard_fwd"
    _expect(x, "x", (None, None), where=w)
    tokens, hidden = x.shape
    dt = _in_dtype(x, w)
    f = _shard(ffn, t)
    _expect(wg_i, "wg_i", (hidden, f), dt, w)
    _expect(wu_i, "wu_i", (hidden, f), dt, w)
    _expect(b_i, "b_i", (f, hidden), dt, w)
    _expect(z_i, "z_i", (tokens, hidden), None, w)
    _expect(bias_b, "bias_b", (hidden,), dt, w)
    _expect(residual, "residual", (tokens, hidden), dt, w)
    _contiguous(w, x=x, b_i=b_i, z_i=z_i, bias_b=bias_b, residual=residual)
    lda = _rows(wg_i, "wg_i")
    if _rows(wu_i, "wu_i") != lda:
        raise ValueError(f"{w}: wg_i and wu_i must share their row stride")
    _workspace(workspace, w)
    _on_one_gpu(w, x=x, wg_i=wg_i, wu_i=wu_i, b_i=b_i, z_i=z_i, workspace=workspace,
                bias_b=bias_b, residual=residual)
    _check(lib().tp_mlp_swiglu_shard_fwd(_ptr(x), _ptr(wg_i), _ptr(wu_i), lda, _ptr(b_i),
                                         _ptr(bias_b), _ptr(residual), _ptr(z_i), _ptr(workspace),
                                         _nbytes(workspace), tokens, hidden, ffn, t, rank, _dt(x),
                                         _dt(z_i), _stream(stream)), w)
    return z_i
