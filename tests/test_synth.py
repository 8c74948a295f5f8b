"""The seeded input generator: bf16 rounding and the recipe's structure."""
import numpy as np
import torch

from synth import WORKLOADS, bf16_bits_to_f32, clustered_head, cross_head, f32_to_bf16_bits


def test_bf16_round_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_clustered_is_deterministic_per_head():
    a = clustered_head(256, 32, 64, 4, 0.5, seed=9, h=3)
    b = clustered_head(256, 32, 64, 4, 0.5, seed=9, h=3)
    c = clustered_head(256, 32, 64, 4, 0.5, seed=9, h=4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_clustered_structure():
    """Keys of a block share a centre, so the within-block spread is the noise."""
    q, k, v = clustered_head(1024, 128, 64, 16, 0.5, seed=0, h=0)
    kf = bf16_bits_to_f32(k).reshape(16, 64, 128)
    within = kf.std(axis=1).mean()
    assert 0.45 < within < 0.55
    qf = bf16_bits_to_f32(q).reshape(16, 64, 128)
    assert 0.45 < qf.std(axis=1).mean() < 0.55


def test_workload_sizes():
    assert WORKLOADS["4k"].n == 130686
    assert WORKLOADS["stage2"].n == 24702
    assert WORKLOADS["stage1"].n == 6144
    assert WORKLOADS["tiny"].n == 2048


def test_cross_head_shapes():
    q, k, v = cross_head(126, 300, 128, seed=2, h=0)
    assert q.shape == (126, 128) and k.shape == (300, 128) and v.shape == (300, 128)


def test_per_token_variant():
    """The stress variant draws a centre per query token: keys and values are the
    default recipe's, and query rows of one block no longer share a centre."""
    base = clustered_head(1024, 128, 64, 16, 0.5, seed=0, h=0)
    pt = clustered_head(1024, 128, 64, 16, 0.5, seed=0, h=0, per_token=True)
    np.testing.assert_array_equal(base[1], pt[1])  # keys: drawn before the query centres
    qb = bf16_bits_to_f32(base[0]).reshape(16, 64, 128)
    qt = bf16_bits_to_f32(pt[0]).reshape(16, 64, 128)
    assert 0.45 < qb.std(axis=1).mean() < 0.55        # one centre per block
    assert qt.std(axis=1).mean() > 1.0                  # centres differ within a block
    # the per-token centres follow the recipe's draw order
    rng = np.random.default_rng(np.random.SeedSequence([0, 0]))
    c = rng.standard_normal((16, 128), dtype=np.float32)
    rng.standard_normal((1024, 128), dtype=np.float32)
    u = rng.integers(0, 16, size=1024)
    q = c[u] + np.float32(0.5) * rng.standard_normal((1024, 128), dtype=np.float32)
    np.testing.assert_array_equal(pt[0], f32_to_bf16_bits(q))
