"""The seeded input generator: bf16 rounding, determinism, block consistency."""
import numpy as np
import torch

from megatron_tensor_transformer_tp_amd import inputs


def test_bf16_rne_matches_torch_cpu_conversion():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1.0, 50.0)])
    # exact ties: mantissa low half 0x8000 with even and odd kept bit
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, ties])
    ours = inputs.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_draw_is_deterministic_and_blocked():
    wl = inputs.MLP_WORKLOADS["t1_h1024_m2048"]
    x1 = inputs.mlp_x_rows(wl, 0, 600)
    x2 = inputs.mlp_x_rows(wl, 0, 600)
    np.testing.assert_array_equal(x1, x2)
    np.testing.assert_array_equal(inputs.mlp_x_rows(wl, 300, 100), x1[300:400])
    assert x1.dtype == np.uint16 and x1.shape == (600, 1024)
    a0 = inputs.mlp_a_block(wl, 0)
    assert a0.shape == (1024, 4096)
    f = inputs.bf16_bits_to_f32(a0)
    assert abs(float(f.std()) - 0.02) < 1e-3 and abs(float(f.mean())) < 1e-3


def test_tiny_workload_is_fp32_with_fan_in_std():
    wl = inputs.MLP_WORKLOADS["tiny_f32_t4"]
    a = np.concatenate([inputs.mlp_a_block(wl, r) for r in range(wl.t)], axis=1)
    b = np.concatenate([inputs.mlp_b_block(wl, r) for r in range(wl.t)], axis=0)
    assert a.dtype == np.float32 and a.shape == (64, 256) and b.shape == (256, 64)
    assert abs(a.std() - 1 / 8) < 0.01 and abs(b.std() - 1 / 16) < 0.005
