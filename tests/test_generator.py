"""The seeded input generator: determinism, per-head regeneration, precision, structure."""
import numpy as np
import torch

from workloads import CONFIGS, custom_config, head_steps, all_steps, position_term
from workloads.gen import HeadStream


def test_deterministic_and_head_independent():
    cfg = custom_config(heads=3, head_dim=16, frames=3, grid_h=2, grid_w=3, steps=3,
                        qkv_dtype="bf16", cache_dtype="bf16")
    a = all_steps(cfg)
    b = all_steps(cfg, workers=2)
    for s in range(cfg.steps):
        for t in range(3):
            assert np.array_equal(a[s][t], b[s][t])
    h1 = head_steps(cfg, 0, 1)
    for s in range(cfg.steps):
        for t in range(3):
            assert np.array_equal(h1[s][t], a[s][t][0, 1])


def test_bf16_values_are_representable_and_drift_is_small():
    cfg = custom_config(head_dim=16, frames=3, grid_h=2, grid_w=3, steps=3,
                        qkv_dtype="bf16", cache_dtype="bf16")
    st = head_steps(cfg, 0, 0)
    for q, k, v in st:
        for x in (q, k, v):
            assert np.array_equal(x, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    d = st[1][0] - st[0][0]
    assert 0.02 < np.std(d) < 0.08


def test_position_term_blocks():
    cfg = CONFIGS[3]
    pe = position_term(cfg)
    assert pe.shape == (cfg.tokens, 64)
    # channel 0 = sin(t), channel 1 = cos(t): constant inside a frame
    F = cfg.frame_tokens
    assert np.allclose(pe[:F, 1], 1.0) and np.allclose(pe[F:2 * F, 0], np.sin(1.0))
    # y block starts at d_t = 24, x block at 44
    assert np.allclose(pe[80, 24], np.sin(1.0)) and np.allclose(pe[1, 44], np.sin(1.0))
    pe2 = position_term(CONFIGS[2])
    assert np.allclose(pe2[64, 0], np.sin(1.0)) and np.allclose(pe2[1, 36], np.sin(1.0))


def test_cfg_batch_structure():
    cfg = custom_config(batch=2, head_dim=16, frames=2, grid_h=2, grid_w=2, steps=3,
                        qkv_dtype="f32", cache_dtype="f32", cfg_v_offset=0.1)
    s0, s1 = head_steps(cfg, 0, 0), head_steps(cfg, 1, 0)
    eps = None
    for a, b in zip(s0, s1):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        d = b[2] - a[2]
        if eps is None:
            eps = d
        assert np.allclose(d, eps, atol=1e-6)
    assert 0.05 < np.std(eps) < 0.15


def test_steps_must_be_consecutive():
    hs = HeadStream(custom_config(), 0, 0)
    hs.step_tensors(1)
    try:
        hs.step_tensors(3)
    except ValueError:
        return
    raise AssertionError("expected ValueError")
