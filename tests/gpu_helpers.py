"""Shared helpers for the GPU parity tests (host <-> device marshalling and
the error metrics the tolerances are stated in)."""
import numpy as np
import torch

from megatron_tensor_transformer_tp_amd import inputs

# bf16 inputs, fp32 accumulation: max |err| / (1 + |ref|) and relative Frobenius.
BF16_MAX, BF16_FRO = 2e-2, 5e-3
# fp32 path: relative 1e-5, read as both bounds.
F32_MAX, F32_FRO = 1e-5, 1e-5


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 bf16 bits -> cuda bfloat16; float32 -> cuda float32."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda")


def host64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values the GPU sees, widened to fp64 for the oracle."""
    if dtype == "bf16":
        return inputs.bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray, floor: float = 1.0):
    """(max |err| / (floor + |ref|), relative Frobenius error)."""
    d = got - ref
    mx = float(np.max(np.abs(d) / (floor + np.abs(ref)))) if d.size else 0.0
    nr = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d))
    return mx, fro


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str,
                 rms_floor: bool = False) -> None:
    """Both bounds.  The max criterion is max |err| / (1 + |ref|); with
    rms_floor the "1" is the output's RMS magnitude instead (for outputs far
    from unit scale, e.g. weight gradients summed over thousands of tokens:
    the same bound at unit scale)."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values (unwritten tile?)"
    floor = float(np.sqrt(np.mean(ref * ref))) if rms_floor and ref.size else 1.0
    mx, fro = errors(got, ref, floor)
    lim_mx, lim_fro = (BF16_MAX, BF16_FRO) if dtype == "bf16" else (F32_MAX, F32_FRO)
    label = f"max|e|/({floor:.3g}+|r|)" if rms_floor else "max|e|/(1+|r|)"
    say(f"{what}: {label} = {mx:.3e} (<= {lim_mx}), rel-fro = {fro:.3e} (<= {lim_fro})")
    assert mx <= lim_mx and fro <= lim_fro, what


def nan_tensor(shape, dtype) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")
