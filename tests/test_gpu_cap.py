"""GPU parity of the key cluster size cap (cap_ratio; pith.science review, "Assumptions &
free parameters": ratio 1.5, 1.25 to 4.0 explored), through the C-ABI binding, against
the oracle's capped forward (cap_key_labels: cluster j keeps its first ceil(ratio N / Ck)
members in position order in the stage-1 summaries).

Acausal and causal (prefix and hierarchical far field), fp32 and bf16, D = 64 and 128,
the three dipole modes, one and five Lloyd iterations, and the full-size timed shapes
with one iteration (the paper's speed setting). Every case asserts that the cap leaves
keys out, so that it is not vacuous. A cap above every cluster size gives the uncapped
result bitwise. Tolerances as everywhere: relative L2 <= 1e-5 (fp32), <= 3e-3 (bf16).
"""

import pytest
import torch

from parity_util import check_config, log, run_gpu
from workloads import CONFIGS, make_inputs, scaled_config

pytestmark = pytest.mark.gpu


def _heads(cfg):
    return [(0, 0)] if cfg.B * cfg.H == 1 else [(0, 0), (cfg.B - 1, cfg.H - 1)]


def _check(cfg, ratio, **kw):
    res = check_config(cfg, _heads(cfg), cap_ratio=ratio, **kw)
    assert all(r.dropped_k > 0 for r in res), "the cap left no key out: the case tests nothing"


@pytest.mark.parametrize("ratio", [1.5, 1.25])
@pytest.mark.parametrize("dipole", [True, "untilted", False])
def test_acausal_bf16(muse_lib, ratio, dipole):
    _check(scaled_config("acausal_8k", B=1, H=2, N=2048), ratio, dipole=dipole)


@pytest.mark.parametrize("ratio,dipole", [(1.0, True), (1.5, "untilted"), (1.25, False)])
def test_acausal_f32(muse_lib, ratio, dipole):
    _check(CONFIGS["acausal_1k_f32"], ratio, dipole=dipole)


@pytest.mark.parametrize("name,over,ratio,dipole", [
    ("causal_16k", {"B": 1, "H": 2, "N": 4096, "block": 1024}, 1.5, True),
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 512}, 1.25, "untilted"),
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 256}, 1.5, False),
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 4096, "block": 1024}, 1.5, True),
    ("acausal_1k_f32", {"causal": True, "block": 256}, 1.25, True),
    ("acausal_1k_f32", {"causal": True, "block": 128}, 1.5, "untilted"),
])
def test_causal(muse_lib, name, over, ratio, dipole):
    _check(scaled_config(name, **over), ratio, dipole=dipole)


@pytest.mark.parametrize("name,over", [
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 256}),
    ("acausal_1k_f32", {"causal": True, "block": 128}),
])
def test_causal_hierarchical(muse_lib, name, over):
    _check(scaled_config(name, **over), 1.5, hierarchy=True)


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 2048, "iters": 1}),
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 1024, "iters": 1}),
])
def test_one_lloyd_iteration(muse_lib, name, over):
    _check(scaled_config(name, **over), 1.5)


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 2048}),
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 1024}),
    ("acausal_1k_f32", {}),
])
def test_cap_above_every_cluster_is_no_cap(muse_lib, name, over):
    # ratio Ck: U = N, which no cluster exceeds; the capped call is the uncapped one bitwise
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    q, k, v = make_inputs(cfg)
    a, _ = run_gpu(cfg, q, k, v)
    b, _ = run_gpu(cfg, q, k, v, cap_ratio=float(cfg.Ck))
    log(f"[{cfg.name}] cap ratio {cfg.Ck} vs no cap: max |diff| {float((a - b).abs().max()):.3e}")
    assert torch.equal(a, b)


def test_acausal_8k_full_size_one_iteration(muse_lib):
    cfg = scaled_config("acausal_8k", iters=1)
    res = check_config(cfg, [(1, 3)], cap_ratio=1.5, out_dtype=torch.bfloat16)
    assert res[0].dropped_k > 0


def test_causal_64k_d128_full_size_one_iteration(muse_lib):
    cfg = scaled_config("causal_64k_d128", iters=1)
    res = check_config(cfg, [(0, 5)], blocks=[1, 17, 31], cap_ratio=1.5, out_dtype=torch.bfloat16)
    assert res[0].dropped_k > 0
