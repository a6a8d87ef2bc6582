"""The seeded generator: determinism, shapes, bf16 rounding (CPU only)."""

import numpy as np
import torch

from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_head, scaled_config


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 0.0], np.float32)])
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(bf16_bits_to_f32(bits), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_heads_are_deterministic_and_distinct():
    cfg = scaled_config("acausal_8k", N=512)
    a = make_head(cfg, 0, 1)
    b = make_head(cfg, 0, 1)
    c = make_head(cfg, 1, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    for t in a:
        assert t.dtype == np.float32 and t.shape == (512, 64)
        assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(t)), t)   # bf16-representable


def test_outliers_and_drift():
    cfg = scaled_config("retrieval_16k", N=2048)
    q, k, v = make_head(cfg, 0, 0)
    norms = np.linalg.norm(k, axis=1)
    n_out = int(0.01 * 2048)
    assert np.sum(norms > 3 * np.median(norms)) == n_out
    c4 = scaled_config("causal_64k_d128", N=1024, drift=1.0)  # exaggerated drift is visible in the mean
    q4, _, _ = make_head(c4, 0, 0)
    base = make_head(scaled_config("causal_64k_d128", N=1024, drift=0.0), 0, 0)[0]
    d = (q4 - base).mean(axis=1)
    assert np.allclose(d, np.sin(np.arange(1024) / 4096.0), atol=2e-2)


def test_config_table():
    assert CONFIGS["acausal_8k"].tokens == 32768 and CONFIGS["causal_64k_d128"].N == 65536 and CONFIGS["causal_64k_d128"].D == 128
    assert CONFIGS["retrieval_16k"].topk_clusters == 4 and CONFIGS["retrieval_16k"].topk_blocks == 2
    assert all(c.N % c.block == 0 for c in CONFIGS.values() if c.causal)
