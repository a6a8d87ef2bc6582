"""The allocation-free entry point (muse_attn_fwd_noalloc) against muse_attn_fwd_ex,
through the C-ABI binding: both run the same kernels, the first on the library's fixed
per-device scratch and the caller's stream only, the second on a stream-ordered workspace
with the stage-1 side stream. Outputs (and the other returned tensors) must be equal
bitwise, over consecutive calls of decreasing size, which reuse the scratch that the
previous call left behind."""

import pytest
import torch

from parity_util import log, to_device
from workloads import make_inputs, scaled_config

pytestmark = pytest.mark.gpu

# largest first: every later call runs on scratch holding the previous call's values
CALLS = [
    ("acausal_8k", {"B": 1, "H": 1, "N": 8192}, {}),
    ("causal_16k", {"B": 1, "H": 2, "N": 4096, "block": 1024}, {}),
    ("retrieval_16k", {"B": 1, "H": 1, "N": 4096}, {}),
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 512}, {"hierarchy": True}),
    ("acausal_8k", {"B": 1, "H": 1, "N": 1000, "Cq": 20, "Ck": 40}, {"dipole": "untilted"}),
    ("acausal_1k_f32", {"N": 700}, {}),
]


def _run(fn, cfg, Q, K, V, extra):
    out, ex = fn(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                 out_dtype=torch.float32, return_lse=True, return_trace=True, return_centroids=True,
                 topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks, **extra)
    torch.cuda.synchronize()
    return out, ex


def test_noalloc_matches_the_workspace_entry(muse_lib):
    from clustered_softmax_attention_amd import binding
    for name, over, extra in CALLS:
        cfg = scaled_config(name, **over)
        need = binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal, cfg.block,
                                       1 if cfg.dtype == "bf16" else 0, cfg.topk_clusters, cfg.topk_blocks,
                                       dipole=extra.get("dipole", True), hierarchy=extra.get("hierarchy", False))
        assert need <= binding.NOALLOC_SCRATCH_BYTES, (name, need)
        q, k, v = make_inputs(cfg)
        Q, K, V = (to_device(t, cfg.dtype) for t in (q, k, v))
        log(f"[noalloc] {name} {over} {extra}: workspace {need / 2**20:.1f} MiB")
        o_ref, ex_ref = _run(binding.attn_fwd, cfg, Q, K, V, extra)
        o_na, ex_na = _run(binding.attn_fwd_noalloc, cfg, Q, K, V, extra)
        assert torch.equal(o_na, o_ref), name
        for key in ex_ref:
            assert torch.equal(ex_na[key], ex_ref[key]), (name, key)
        # a second allocation-free call on the same inputs reproduces itself bitwise
        o_again, _ = _run(binding.attn_fwd_noalloc, cfg, Q, K, V, extra)
        assert torch.equal(o_again, o_na), name


def test_noalloc_refuses_oversize_shapes(muse_lib):
    from clustered_softmax_attention_amd import binding
    cfg = scaled_config("acausal_8k", B=2, H=8, N=8192)
    Q, K, V = (torch.zeros((cfg.B, cfg.H, cfg.N, cfg.D), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    with pytest.raises(binding.MuseError, match="scratch") as err:
        binding.attn_fwd_noalloc(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters)
    assert err.value.code == -5  # MUSE_ERR_WORKSPACE
