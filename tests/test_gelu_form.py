"""The GPU epilogue's GeLU evaluation, checked on the CPU.

The kernels evaluate GeLU(v) = v Phi(v) (exact erf form; 列并行 tutorial, MLP
应用) in fp32 by the Abramowitz & Stegun 7.1.26 approximation of erfc with
folded constants (csrc/device_common.h, `normal_tail` / `gelu_f32`).  This
test reads those constants from the header, emulates the same sequence of
float32 operations (each fma rounded once) and compares with SciPy's erfc in
fp64: the documented error bound, and the limits at +-inf.  It exercises the
kernel's formula only, not the oracle.
"""
import os
import re

import numpy as np
import pytest
from scipy.special import erfc

HEADER = os.path.join(os.path.dirname(__file__), "..", "megatron_tensor_transformer_tp_amd", "csrc",
                      "device_common.h")
F32 = np.float32


def _literals():
    src = open(HEADER).read()
    body = src[src.index("NormalTail normal_tail(float v)"):src.index("d/dv GeLU(v)")]
    return [float(x) for x in re.findall(r"(-?\d+\.\d+(?:e\d+)?)f", body)]


def _fma(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F32)


def _mul(a, b):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)).astype(F32)


def _kernel_gelu(v):
    c, p0, one, a5h, a4h, a3h, a2h, a1h, fmax = _literals()
    assert one == 1.0
    with np.errstate(all="ignore"):
        z = _mul(np.abs(v), F32(c))
        t = (1.0 / _fma(F32(p0), z, F32(1.0)).astype(np.float64)).astype(F32)
        p = _fma(t, F32(a5h), F32(a4h))
        for a in (a3h, a2h, a1h):
            p = _fma(t, p, F32(a))
        e = np.exp2(-_mul(z, z).astype(np.float64)).astype(F32)
        tail = _mul(_mul(p, t), e)
        # max(v, 0) as the kernel takes it: a signed-integer max of the bits
        pos = np.maximum(np.asarray(v, F32).view(np.int32), 0).view(F32)
        return _fma(-np.minimum(np.abs(v), F32(fmax)), tail, pos)


def test_constants_are_the_folded_published_ones():
    c, p0, _one, a5h, a4h, a3h, a2h, a1h, fmax = _literals()
    l2e = 1.0 / np.log(2.0)
    # A&S 7.1.26: p = 0.3275911, a1..a5 as published
    a = [0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429]
    assert c == pytest.approx(np.sqrt(l2e / 2.0), rel=1e-15)
    assert p0 == pytest.approx(0.3275911 / np.sqrt(l2e), rel=1e-15)
    assert [a1h, a2h, a3h, a4h, a5h] == pytest.approx([x / 2 for x in a], rel=1e-15)
    assert fmax == pytest.approx(float(np.finfo(np.float32).max), rel=1e-9)


def test_error_bound_and_limits():
    v = np.linspace(-12.0, 12.0, 400_001).astype(F32)
    x = v.astype(np.float64)
    tail = 0.5 * erfc(np.abs(x) / np.sqrt(2.0))
    exact = x * np.where(x >= 0, 1.0 - tail, tail)
    err = np.abs(_kernel_gelu(v).astype(np.float64) - exact)
    assert err.max() < 5e-7                       # A&S 7.1.26 |error| 1.5e-7 in erf, times |v| / 2
    special = _kernel_gelu(np.array([np.inf, -np.inf, 0.0, -0.0, 3e38, -3e38], dtype=F32))
    assert special[0] == np.inf and special[1] == 0.0 and special[2] == 0.0 and special[3] == 0.0
    assert special[4] == F32(3e38) and special[5] == 0.0
    assert np.isnan(_kernel_gelu(np.array([np.nan], dtype=F32)))[0]
