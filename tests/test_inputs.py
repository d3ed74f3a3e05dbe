"""Seeded input generator (CPU): determinism, bf16 rounding, QK-norm + RoPE shaping."""
import numpy as np
import torch

from bwd_head_rms_amd import inputs


def test_deterministic_and_seeded():
    a = inputs.generate(2, 8, 2, 1, 16, seed=7)
    b = inputs.generate(2, 8, 2, 1, 16, seed=7)
    c = inputs.generate(2, 8, 2, 1, 16, seed=8)
    for n in a:
        assert a[n].dtype == np.float32
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    ours = inputs.bf16_round(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, theirs)


def test_shaping_unit_rms_and_norm_preserving_rope():
    g = inputs.generate(1, 64, 2, 2, 32, seed=3, shaped=True)
    for n in ("q", "k"):
        rms = np.sqrt(np.mean(g[n].astype(np.float64) ** 2, axis=-1))
        assert np.allclose(rms, 1.0, atol=1e-5)
    # RoPE at position 0 is the identity
    raw = inputs.rms_qk_norm(np.random.default_rng(1).standard_normal((3, 16)))
    assert np.allclose(inputs.rope(raw)[0], raw[0])


def test_workload_table():
    w = inputs.WORKLOADS[inputs.LONG_CONTEXT]
    assert (w.B, w.S, w.H, w.Hkv, w.hd, w.dtype) == (4, 2048, 16, 16, 64, "bf16")
    assert inputs.WORKLOADS["gqa_b16_s1024_h8_kv2_hd64_f32"].group == 4
