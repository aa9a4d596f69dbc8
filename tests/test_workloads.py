"""The seeded input generator: determinism, shapes, bf16 rounding, mask recipe."""
import numpy as np
import torch

from workloads import CONFIGS, get_config, make_qkv, random_block_mask, rep_head_flags, to_bf16_array
from workloads.generator import head_densities, phi_features


def test_config_shapes():
    assert get_config(0).seq_len == 256 and get_config(0).nb == 8
    assert get_config(1).seq_len == 32760 and get_config(1).nb == 256
    assert get_config(2).seq_len == 75600 and get_config(2).nb == 591
    assert get_config(3).seq_len == 256 + 44520 and get_config(3).n_prefix_blocks == 2
    assert get_config(4).seq_len == 118800 and get_config(4).nb == 929
    for cfg in CONFIGS.values():
        assert cfg.n_prefix % cfg.block == 0


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # ties to even
    ours = to_bf16_array(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_qkv_deterministic_and_head_independent():
    cfg = get_config(0)
    q1, k1, v1 = make_qkv(cfg, draw=0)
    q2, k2, v2 = make_qkv(cfg, draw=0, heads=[1])
    np.testing.assert_array_equal(q1[1], q2[0])
    np.testing.assert_array_equal(v1[1], v2[0])
    q3, _, _ = make_qkv(cfg, draw=1)
    assert not np.array_equal(q1, q3)
    assert q1.shape == (2, 256, 64) and q1.dtype == np.float32


def test_bf16_workload_values_are_bf16():
    cfg = get_config(1)
    q, k, v = make_qkv(cfg, draw=0, heads=[0])
    for x in (q, k, v):
        np.testing.assert_array_equal(x, to_bf16_array(x))


def test_phi_fixed_across_draws_and_text_rows_plain():
    cfg = get_config(3)
    phi = phi_features(cfg, head=2)
    assert (phi[: cfg.n_prefix] == 0).all()
    np.testing.assert_allclose((phi[cfg.n_prefix:] ** 2).mean(), 1.0, atol=0.05)


def test_masks_and_rep_heads():
    cfg = get_config(2)
    m = random_block_mask(cfg)
    assert m.shape == (40, 591, 591)
    assert (m[:, np.arange(591), np.arange(591)] == 1).all()
    dens = head_densities(cfg)
    assert ((dens >= 0.2) & (dens <= 0.5)).all()
    np.testing.assert_allclose(m.mean(axis=(1, 2)), dens, atol=0.02)
    flags = rep_head_flags(cfg)
    assert flags.sum() == 10
    assert rep_head_flags(get_config(0)).tolist() == [0, 1]
