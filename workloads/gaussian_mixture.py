"""Seeded Gaussian-mixture Q/K/V generator for the MuSe forward workloads.

The pages measure MuSe on isolated attention layers at 8k and 64k context
(fugumt.com v2 abstract; pith.science review, referee "Significance") on trained
activations that are not available here. These synthetic mixtures stand in for
them: queries and keys drawn around shared per-head component means (so that
K-means has semantic structure to find), values drawn independently.

Recipe, per (config, batch b, head h):
  * seed streams: numpy ``default_rng(SeedSequence([2026, cfg_id, b, h, stream]))``
    with stream 0 = component means, 1 = query component ids, 2 = query noise,
    3 = key component ids, 4 = key noise, 5 = values, 6 = outlier positions;
  * means mu ~ N(0, D**-0.5 * I) (per-coordinate std D**-0.25), shape [M, D];
  * q_n = mu[z_n] + sigma * eps_n, k_n likewise with independent ids and noise;
  * v ~ N(0, 1);
  * optional drift: ``drift * sin(n / drift_period)`` added to every coordinate
    of q_n and k_n;
  * optional outliers: ``floor(outlier_frac * N)`` distinct key positions
    scaled by ``outlier_scale``;
  * everything is generated in float32 and, for bf16 workloads, rounded to
    bfloat16 with round-to-nearest-even. Both sides read these rounded values.

Nothing here computes attention, clustering or summaries.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    cfg_id: int
    B: int
    H: int
    N: int
    D: int
    dtype: str  # "f32" or "bf16"
    M: int  # mixture components per head
    sigma: float
    Cq: int
    Ck: int
    iters: int
    causal: bool
    block: int  # 0 when acausal
    topk_clusters: int = 0
    topk_blocks: int = 0
    drift: float = 0.0
    drift_period: float = 4096.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def tokens(self) -> int:
        return self.B * self.N


CONFIGS: Dict[str, WorkloadConfig] = {
    # 1k acausal, fp32, one head.
    "acausal_1k_f32": WorkloadConfig("acausal_1k_f32", 1, 1, 1, 1024, 64, "f32", 32, 0.10, 8, 32, 5, False, 0),
    # 8k acausal isolated-layer shape.
    "acausal_8k": WorkloadConfig("acausal_8k", 2, 4, 8, 8192, 64, "bf16", 128, 0.15, 32, 128, 5, False, 0),
    # 16k causal, block 1024.
    "causal_16k": WorkloadConfig("causal_16k", 3, 8, 8, 16384, 64, "bf16", 256, 0.20, 16, 64, 5, True, 1024),
    # 64k causal, D=128, block 2048, slow positional drift.
    "causal_64k_d128": WorkloadConfig("causal_64k_d128", 4, 1, 16, 65536, 128, "bf16", 512, 0.20, 32, 128, 5, True, 2048,
                         drift=0.01, drift_period=4096.0),
    # 16k causal with retrieval (k1=4 clusters, k2=2 blocks) and 1% planted 5x outlier keys.
    "retrieval_16k": WorkloadConfig("retrieval_16k", 5, 2, 8, 16384, 64, "bf16", 256, 0.20, 16, 64, 5, True, 1024,
                         topk_clusters=4, topk_blocks=2, outlier_frac=0.01, outlier_scale=5.0),
}


def scaled_config(name: str, **overrides) -> WorkloadConfig:
    """A named workload with some fields replaced (smaller N, fewer heads ...).

    The seed stream keeps the named config's id, so a reduced case draws from the
    same mixture family as the full one.
    """
    return dataclasses.replace(CONFIGS[name], **overrides)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg: WorkloadConfig, b: int, h: int, stream: int, seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg.cfg_id, b, h, stream]))


def make_head(cfg: WorkloadConfig, b: int, h: int, seed: int = 2026) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One (b, h) head: float32 arrays q, k, v of shape [N, D] (bf16-representable if dtype bf16)."""
    N, D, M = cfg.N, cfg.D, cfg.M
    mu = _rng(cfg, b, h, 0, seed).standard_normal((M, D), dtype=np.float32) * np.float32(D ** -0.25)
    zq = _rng(cfg, b, h, 1, seed).integers(0, M, size=N)
    q = mu[zq] + np.float32(cfg.sigma) * _rng(cfg, b, h, 2, seed).standard_normal((N, D), dtype=np.float32)
    zk = _rng(cfg, b, h, 3, seed).integers(0, M, size=N)
    k = mu[zk] + np.float32(cfg.sigma) * _rng(cfg, b, h, 4, seed).standard_normal((N, D), dtype=np.float32)
    v = _rng(cfg, b, h, 5, seed).standard_normal((N, D), dtype=np.float32)
    if cfg.drift:
        drift = (np.float32(cfg.drift) * np.sin(np.arange(N, dtype=np.float64) / cfg.drift_period)).astype(np.float32)
        q = q + drift[:, None]
        k = k + drift[:, None]
    if cfg.outlier_frac:
        n_out = int(np.floor(cfg.outlier_frac * N))
        pos = _rng(cfg, b, h, 6, seed).choice(N, size=n_out, replace=False)
        k[pos] *= np.float32(cfg.outlier_scale)
    q, k, v = (np.ascontiguousarray(t, dtype=np.float32) for t in (q, k, v))
    if cfg.dtype == "bf16":
        q, k, v = (bf16_bits_to_f32(f32_to_bf16_bits(t)) for t in (q, k, v))
    return q, k, v


def make_inputs(cfg: WorkloadConfig, seed: int = 2026, heads: Optional[list] = None):
    """Full [B, H, N, D] float32 tensors q, k, v (bf16-representable values for bf16 configs).

    ``heads``: optional list of (b, h) to generate; others are left zero (used when
    only a few heads are checked against the oracle).
    """
    shape = (cfg.B, cfg.H, cfg.N, cfg.D)
    q = np.zeros(shape, np.float32)
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    for b, h in todo:
        q[b, h], k[b, h], v[b, h] = make_head(cfg, b, h, seed)
    return q, k, v
